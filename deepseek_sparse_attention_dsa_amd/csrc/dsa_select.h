// Per-wave exact top-K of one score row held in LDS (internal header), for
// the combined indexer + top-K kernels.
//
// The selection rules are those of dsa_topk (cuDNN Frontend DSA page,
// sections 4 and 5): the k largest of the row's first n scores, exact ties at
// the k-th value going to the lower columns, -0.0 equal to +0.0, every
// column taken when n <= k; the output is the canonical compact form
// (ascending global ids, -1 suffix). The combined path also returns the
// selected scores (logits), their softmax and its natural-log normaliser
// (section 4; section 6 defines the softmax over the top-K entries);
// padded slots are -1 / -inf / 0, an empty row has lse = +inf.
#pragma once

#include "dsa_device.h"

namespace dsa {

constexpr int kFuseMaxCols = 4096;                // longest row the combined path selects on
constexpr int kFuseChunks = kFuseMaxCols / 256;   // 4-column groups per lane
constexpr int kFuseRowStride = kFuseMaxCols + 4;  // floats per LDS row; slot 4096 takes dropped writes

// Order-preserving uint32 key of a score (-0.0 folded onto +0.0). Key 0 is
// reserved for columns past the row end.
__device__ __forceinline__ uint32_t fused_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float fused_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

struct FusedArgs {
  int k;               // top-k, 1..2048
  int32_t* idx;        // [n_rows, ld_idx] global ids
  int64_t ld_idx;
  int32_t* len;        // [n_rows] or null
  float* logit;        // [n_rows, ld_idx] or null
  float* soft;         // [n_rows, ld_idx] or null
  float* lse;          // [n_rows] or null
};

// Orders the wave's earlier LDS accesses before its later ones (a wave's LDS
// instructions execute in issue order; this keeps the compiler from moving
// them across).
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Top-k of row[0..n) (LDS, n <= kFuseMaxCols) by the calling wave; hist is
// 256 words of LDS private to the wave. Writes row r_out of the outputs.
__device__ void wave_topk_row(const float* row, int n, int32_t base, uint32_t* hist,
                              const FusedArgs& a, int64_t r_out) {
  const int lane = threadIdx.x & 63;
  const uint32_t k = (uint32_t)a.k;
  // Column 256c + 4*lane + e of the row is key kreg[c][e] (0 past the end).
  u32x4 kreg[kFuseChunks];
  uint32_t kmax = 0;
#pragma unroll
  for (int c = 0; c < kFuseChunks; ++c) {
    const int col = 256 * c + 4 * lane;
    const float4 v = *reinterpret_cast<const float4*>(row + col);
    kreg[c] = u32x4{col + 0 < n ? fused_key(v.x) : 0u, col + 1 < n ? fused_key(v.y) : 0u,
                    col + 2 < n ? fused_key(v.z) : 0u, col + 3 < n ? fused_key(v.w) : 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) kmax = max(kmax, kreg[c][e]);
  }
  kmax = wave_max_u32(kmax);

  // theta: the k-th largest key; need_eq: how many keys equal to it are
  // taken. With n <= k every valid key (> 0) is taken.
  //
  // Histogram passes (256 bins in LDS, lane l owning bins 255-4l .. 252-4l)
  // find the bin holding the remaining-th largest member key; bin_of(key)
  // gives a member's bin, or -1 for a non-member. visit(f) calls f on every
  // key the pass looks at (the lane's columns, or a member list).
  auto find_bin = [&](uint32_t remaining, uint32_t* above_out, auto&& visit,
                      auto&& bin_of) -> uint32_t {
    *reinterpret_cast<u32x4*>(hist + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
    wave_lds_order();
    visit([&](uint32_t key) {
      const int b = bin_of(key);
      if (b >= 0) atomicAdd(&hist[b], 1u);
    });
    wave_lds_order();
    const u32x4 h = *reinterpret_cast<const u32x4*>(hist + 252 - 4 * lane);
    const uint32_t local = h.x + h.y + h.z + h.w;
    const uint32_t incl = wave_incl_scan_dpp(local, [](uint32_t a, uint32_t b) { return a + b; }, 0u);
    const uint32_t above = incl - local;
    const bool cross = above < remaining && remaining <= incl;
    uint32_t bin = 0, before = above;
    if (cross) {
      const uint32_t hb[4] = {h.w, h.z, h.y, h.x};  // bins 255-4l, 254-4l, ...
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (before + hb[i] >= remaining) {
          bin = 255 - 4 * lane - i;
          break;
        }
        before += hb[i];
      }
    }
    const int src = __builtin_ctzll(ballot(cross));  // wave-uniform
    *above_out = (uint32_t)__builtin_amdgcn_readlane((int)before, src);
    wave_lds_order();  // the next pass clears the bins
    return (uint32_t)__builtin_amdgcn_readlane((int)bin, src);
  };
  auto visit_cols = [&](auto&& f) {
#pragma unroll
    for (int c = 0; c < kFuseChunks; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) f(kreg[c][e]);
  };
  uint32_t theta = 0, need_eq = 0;
  if ((uint32_t)n > k) {
    // First pass: 256 buckets linear in the score between the row's minimum
    // and maximum (monotone in the key, so a bucket is a range of keys, and
    // the keys spread over the bins instead of piling onto a few exponents).
    // Then four 8-bit radix passes over the members of the chosen bucket.
    uint32_t kmin = 0xffffffffu;
#pragma unroll
    for (int c = 0; c < kFuseChunks; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) kmin = min(kmin, kreg[c][e] ? kreg[c][e] : 0xffffffffu);
    kmin = wave_min_u32(kmin);
    const float lo = fused_value(kmin), span = fused_value(kmax) - lo;
    const float scale = 256.0f / span;
    const bool linear = span > 0.0f && span < 3.0e38f && scale < 3.0e38f;  // finite, non-empty
    uint32_t remaining = k;
    int bucket = -1;
    if (linear) {
      auto lin = [&](uint32_t key) -> int {
        if (key == 0u) return -1;
        const int b = (int)((fused_value(key) - lo) * scale);
        return b > 255 ? 255 : b;
      };
      uint32_t above;
      bucket = (int)find_bin(remaining, &above, visit_cols, lin);
      remaining -= above;
    }
    // The chosen bucket's members (every valid key without the linear pass)
    // move, in column order, to a list in the row's own LDS, which is free
    // once the keys sit in registers: the radix passes then visit the
    // members only, instead of every column four times.
    uint32_t* list = reinterpret_cast<uint32_t*>(const_cast<float*>(row));
    uint32_t n_mem = 0;
    wave_lds_order();  // every lane has read its keys from the row
#pragma unroll
    for (int c = 0; c < kFuseChunks; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = kreg[c][e];
        bool mem = key != 0u;
        if (bucket >= 0) {
          const int b = (int)((fused_value(key) - lo) * scale);
          mem = mem && (b > 255 ? 255 : b) == bucket;
        }
        const uint64_t bm = ballot(mem);
        if (mem) list[n_mem + popc_below(bm)] = key;
        n_mem += (uint32_t)__popcll(bm);
      }
    wave_lds_order();
    auto visit_list = [&](auto&& f) {
      for (uint32_t i = lane; i < n_mem; i += 64) f(list[i]);
    };
    uint32_t prefix = 0, pmask = 0;
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      uint32_t above;
      const uint32_t bin = find_bin(remaining, &above, visit_list, [&](uint32_t key) -> int {
        if ((key & pmask) != prefix) return -1;
        return (int)((key >> shift) & 255u);
      });
      remaining -= above;
      prefix |= bin << shift;
      pmask |= 0xffu << shift;
    }
    theta = prefix;
    need_eq = remaining;
  }

  // Ordered compaction: a taken key's slot is #greater-before +
  // min(#equal-before, need_eq) in column order (chunk, lane, element).
  int32_t* oi = a.idx + r_out * a.ld_idx;
  float* ol = a.logit ? a.logit + r_out * a.ld_idx : nullptr;
  float* os = a.soft ? a.soft + r_out * a.ld_idx : nullptr;
  const float vmax = fused_value(kmax);
  constexpr float kLog2e = 1.4426950408889634f;
  auto place = [&](auto&& f) {
    uint32_t gt_run = 0, eq_run = 0;
#pragma unroll
    for (int c = 0; c < kFuseChunks; ++c) {
      const u32x4 kv = kreg[c];
      uint32_t below_gt = 0, below_eq = 0, tot_gt = 0, tot_eq = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint64_t bg = ballot(kv[e] > theta);
        const uint64_t be = ballot(kv[e] == theta && kv[e] != 0u);
        below_gt += popc_below(bg);
        below_eq += popc_below(be);
        tot_gt += __popcll(bg);
        tot_eq += __popcll(be);
      }
      uint32_t g = gt_run + below_gt, q = eq_run + below_eq;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool is_gt = kv[e] > theta;
        const bool is_eq = kv[e] == theta && kv[e] != 0u;
        const uint32_t pos = g + min(q, need_eq);
        if ((is_gt || (is_eq && q < need_eq)) && pos < k)
          f(pos, base + 256 * c + 4 * lane + e, fused_value(kv[e]));
        g += is_gt;
        q += is_eq;
      }
      gt_run += tot_gt;
      eq_run += tot_eq;
    }
  };
  // The selected set is every key above theta plus need_eq keys equal to
  // it, so the softmax normaliser needs no placement: one pass sums it.
  const uint32_t m = min((uint32_t)n, k);
  float ssum = 0.0f;
#pragma unroll
  for (int c = 0; c < kFuseChunks; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (kreg[c][e] > theta)
        ssum += __builtin_amdgcn_exp2f((fused_value(kreg[c][e]) - vmax) * kLog2e);
  ssum = wave_sum_f32(ssum);
  if (need_eq) ssum += (float)need_eq * __builtin_amdgcn_exp2f((fused_value(theta) - vmax) * kLog2e);
  const float lse = m ? vmax + __logf(ssum) : __builtin_inff();
  place([&](uint32_t pos, int32_t gcol, float v) {
    oi[pos] = gcol;
    if (ol) ol[pos] = v;
    if (os) os[pos] = __builtin_amdgcn_exp2f((v - lse) * kLog2e);
  });
  for (uint32_t i = m + lane; i < k; i += 64) {
    oi[i] = -1;
    if (ol) ol[i] = -__builtin_inff();
    if (os) os[i] = 0.0f;
  }
  if (lane == 0) {
    if (a.len) a.len[r_out] = (int32_t)m;
    if (a.lse) a.lse[r_out] = lse;
  }
}

}  // namespace dsa
