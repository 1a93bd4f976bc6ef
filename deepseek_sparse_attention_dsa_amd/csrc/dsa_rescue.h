// Exact top-k of one row from its dense scores (internal header): the
// rescue passes of the combined indexer + top-k (bf16 and FP8 inputs) score a
// queued row into a spill row, then select from it here.
#pragma once

#include "dsa_device.h"
#include "dsa_rowsel.h"
#include "dsa_select.h"

namespace dsa {

// Row r's top fa.k of spill[0..n) (scores of keys s0 .. s0+n-1), with the
// order rule of the other top-k paths (greater first, then equal values in
// column order), their logits, softmax and the row's LSE: theta by radix
// passes over the row, then each thread counts its run of columns above and
// equal to theta and, after a scan of the counts, places its selected
// columns. Every thread of the workgroup (WAVES waves) calls it; it ends
// with a barrier, after which the spill row may be overwritten.
template <int WAVES>
__device__ void select_spill_row(const float* spill, int n, int32_t s0, const FusedArgs& fa,
                                 int64_t r, uint32_t* hist, uint32_t* s_wave, uint32_t* s_sel,
                                 float* s_fsum) {
  constexpr int NT = WAVES * 64;
  constexpr float kLog2e = 1.4426950408889634f;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto block_sum = [&](float v) -> float {
    v = wave_sum_f32(v);
    if (lane == 0) s_fsum[wave] = v;
    __syncthreads();
    v = 0.0f;
#pragma unroll
    for (int i = 0; i < WAVES; ++i) v += s_fsum[i];
    __syncthreads();
    return v;
  };
  int32_t* oi = fa.idx + r * fa.ld_idx;
  float* ol = fa.logit ? fa.logit + r * fa.ld_idx : nullptr;
  float* os = fa.soft ? fa.soft + r * fa.ld_idx : nullptr;
  const uint32_t kk = (uint32_t)fa.k;
  uint32_t kmax = 0u;
  for (int i = tid; i < n; i += NT) kmax = max(kmax, float_to_key(spill[i]));
  kmax = block_max<WAVES>(kmax, s_wave);
  const float vmax = key_to_float(kmax);
  uint32_t theta = 0u, need_eq = 0u;
  if ((uint32_t)n > kk)  // uniform
    theta = radix_select<WAVES>(kk, hist, s_wave, s_sel, &need_eq, [&](auto&& f) {
      for (int i = tid; i < n; i += NT) f(float_to_key(spill[i]));
    });
  // (n <= k: theta = 0 takes every column, need_eq = 0)
  float s = 0.0f;
  for (int i = tid; i < n; i += NT) {
    const uint32_t key = float_to_key(spill[i]);
    if (key > theta) s += __builtin_amdgcn_exp2f((key_to_float(key) - vmax) * kLog2e);
  }
  float ssum = block_sum(s);
  if (need_eq) ssum += (float)need_eq * __builtin_amdgcn_exp2f((key_to_float(theta) - vmax) * kLog2e);
  const uint32_t m = min((uint32_t)n, kk);
  const float lse = m ? vmax + __logf(ssum) : __builtin_inff();
  // Thread tid owns columns [c0, c1), in column order.
  const int P = (n + NT - 1) / NT;
  const int c0 = min(tid * P, n), c1 = min(c0 + P, n);
  uint32_t ngt = 0u, neq = 0u;
  for (int i = c0; i < c1; ++i) {
    const uint32_t key = float_to_key(spill[i]);
    ngt += key > theta;
    neq += key == theta;
  }
  uint32_t tot;
  uint32_t g = block_exclusive_scan<WAVES>(ngt, s_wave, &tot);
  uint32_t qn = block_exclusive_scan<WAVES>(neq, s_wave, &tot);
  for (int i = c0; i < c1; ++i) {
    const uint32_t key = float_to_key(spill[i]);
    const bool is_gt = key > theta, is_eq = key == theta;
    const uint32_t pos = g + min(qn, need_eq);
    if ((is_gt || (is_eq && qn < need_eq)) && pos < kk) {
      const float v = key_to_float(key);
      oi[pos] = s0 + i;
      if (ol) ol[pos] = v;
      if (os) os[pos] = __builtin_amdgcn_exp2f((v - lse) * kLog2e);
    }
    g += is_gt;
    qn += is_eq;
  }
  for (uint32_t i = m + tid; i < kk; i += NT) {
    oi[i] = -1;
    if (ol) ol[i] = -__builtin_inff();
    if (os) os[i] = 0.0f;
  }
  if (tid == 0) {
    if (fa.len) fa.len[r] = (int32_t)m;
    if (fa.lse) fa.lse[r] = lse;
  }
  __syncthreads();  // the spill row is read before the next row overwrites it
}

}  // namespace dsa
