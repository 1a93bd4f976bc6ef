// Per-row radix top-K with per-row length, ordered compaction and
// local -> global conversion, for gfx950.
//
// Semantics: cuDNN Frontend DSA page, section 5 "Indexer Top-K" (radix top-K
// with a per-row effective length, top_k <= 2048) and section 4 (the
// deterministic tie-break: exact ties at the K-th boundary go to the smallest
// column); NeMo cudnn_dsa page (global coordinates, ascending valid prefix,
// -1 suffix).
//
// One workgroup owns one row and keeps all of it on chip: wave w holds a
// contiguous column range, read with 16-byte loads so that every load
// instruction covers 1 KiB of the row; rows up to 32K columns sit in VGPRs,
// 64K-column rows keep half of each wave's range in LDS. Scores become
// order-preserving uint32 keys (-0.0 folded onto +0.0, so they tie as equal
// values). Three LDS-histogram passes over 11/11/10-bit digits find the K-th
// largest key theta and how many keys equal to theta are taken. A final pass
// walks the columns in ascending order, using wave ballots and mbcnt prefix
// counts, and drops each selected column straight into its output slot:
// position = (#greater before it) + min(#equal before it, #equal taken).
// The score row is read from HBM exactly once.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {
namespace {

__device__ __forceinline__ uint32_t float_to_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;  // -0.0 == +0.0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t key) {
  uint32_t b = (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
  return __uint_as_float(b);
}

// Exclusive prefix sum over the threads of the workgroup (tid order).
template <int WAVES>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wave,
                                                         uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    uint32_t o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (WAVES == 1) {
    *total = __shfl(incl, 63, 64);
    return incl - v;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) {
    uint32_t t = s_wave[w];
    before += (w < wave) ? t : 0u;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// CR / CL: 4-column chunks per lane held in VGPRs / in LDS. Wave w owns the
// columns [w * 256 * (CR + CL), (w + 1) * 256 * (CR + CL)); chunk c of a wave
// covers 256 consecutive columns, 4 per lane.
template <int WAVES, int CR, int CL>
__global__ __launch_bounds__(64 * WAVES) void topk_kernel(
    const float* __restrict__ scores, int64_t ld, int64_t n_cols,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ row_starts, int k,
    int32_t* __restrict__ indices, int64_t ld_idx, int32_t* __restrict__ topk_length,
    float* __restrict__ values) {
  constexpr int NT = 64 * WAVES;
  constexpr int NCH = CR + CL;
  constexpr int NBINS = 2048;
  constexpr int BPT = NBINS / NT;  // histogram bins owned per thread in the scan
  static_assert(NBINS % NT == 0, "bins must split evenly over threads");

  __shared__ uint32_t hist[NBINS];
  __shared__ int32_t s_idx[2048];
  __shared__ float s_val[2048];
  __shared__ uint32_t s_wave[2][WAVES > 1 ? WAVES : 1];
  __shared__ uint32_t s_sel[2];
  __shared__ u32x4 lkeys[CL > 0 ? WAVES * CL * 64 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t r = blockIdx.x;
  const float* row = scores + r * ld;
  int32_t* out_idx = indices + r * ld_idx;
  float* out_val = values ? values + r * ld_idx : nullptr;

  int64_t n64 = seq_lens[r];
  n64 = n64 < 0 ? 0 : (n64 > n_cols ? n_cols : n64);
  const int n = (int)n64;
  const int32_t base = row_starts ? row_starts[r] : 0;

  if (n <= k) {
    // Every causal column is selected; no select needed.
    for (int i = tid; i < k; i += NT) {
      out_idx[i] = i < n ? base + i : -1;
      if (out_val) out_val[i] = i < n ? row[i] : -__builtin_inff();
    }
    if (tid == 0 && topk_length) topk_length[r] = n;
    return;
  }

  // ---- load the row as order-preserving keys (0 = past the row end) ----
  const int wbase = wave * 256 * NCH;
  u32x4 kreg[CR > 0 ? CR : 1];
  auto lds_slot = [&](int c) -> u32x4* { return &lkeys[(wave * CL + (c - CR)) * 64 + lane]; };
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int col = wbase + c * 256 + lane * 4;
    u32x4 kv;
    if (col + 3 < n) {
      const float4 v = *reinterpret_cast<const float4*>(row + col);
      kv = u32x4{float_to_key(v.x), float_to_key(v.y), float_to_key(v.z), float_to_key(v.w)};
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) kv[e] = (col + e < n) ? float_to_key(row[col + e]) : 0u;
    }
    if (c < CR) kreg[c] = kv; else *lds_slot(c) = kv;
  }
  auto chunk = [&](int c) -> u32x4 { return c < CR ? kreg[c] : *lds_slot(c); };

  // ---- radix select of the K-th largest key ----
  if (tid == 0) {
    s_sel[0] = 0u;
    s_sel[1] = 0u;
  }
  uint32_t prefix = 0, pmask = 0;
  uint32_t remaining = (uint32_t)k;  // keys still to take among prefix matches
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 0x3ffu : 0x7ffu;
    for (int i = tid; i < NBINS; i += NT) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const u32x4 kv = chunk(c);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((kv[e] & pmask) == prefix) atomicAdd(&hist[(kv[e] >> shift) & dmask], 1u);
    }
    __syncthreads();
    // Thread tid owns bins [hi_bin - BPT + 1, hi_bin], highest bins first.
    const int hi_bin = NBINS - 1 - tid * BPT;
    uint32_t local = 0;
#pragma unroll
    for (int b = 0; b < BPT; ++b) local += hist[hi_bin - b];
    uint32_t total;
    uint32_t above = block_exclusive_scan<WAVES>(local, s_wave[0], &total);
    if (above < remaining && remaining <= above + local) {
      uint32_t acc = above;
      for (int b = 0; b < BPT; ++b) {
        const uint32_t h = hist[hi_bin - b];
        if (acc + h >= remaining) {
          s_sel[0] = (uint32_t)(hi_bin - b);
          s_sel[1] = acc;
          break;
        }
        acc += h;
      }
    }
    __syncthreads();
    const uint32_t bin = s_sel[0];
    remaining -= s_sel[1];
    prefix |= bin << shift;
    pmask |= dmask << shift;
    __syncthreads();
  }
  const uint32_t theta = prefix;
  const uint32_t need_eq = remaining;  // >= 1 keys equal to theta to take

  // ---- per-wave counts of keys above / equal to theta ----
  uint32_t lgt = 0, leq = 0;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const u32x4 kv = chunk(c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lgt += kv[e] > theta;
      leq += kv[e] == theta;
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    lgt += __shfl_xor(lgt, d, 64);
    leq += __shfl_xor(leq, d, 64);
  }
  uint32_t gt_run = 0, eq_run = 0;
  if (WAVES > 1) {
    if (lane == 0) {
      s_wave[0][wave] = lgt;
      s_wave[1][wave] = leq;
    }
    __syncthreads();
    for (int w = 0; w < wave; ++w) {
      gt_run += s_wave[0][w];
      eq_run += s_wave[1][w];
    }
  }

  // ---- ordered compaction into LDS ----
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const u32x4 kv = chunk(c);
    uint32_t below_gt = 0, below_eq = 0, tot_gt = 0, tot_eq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint64_t bg = ballot(kv[e] > theta);
      const uint64_t be = ballot(kv[e] == theta);
      below_gt += popc_below(bg);
      below_eq += popc_below(be);
      tot_gt += __popcll(bg);
      tot_eq += __popcll(be);
    }
    uint32_t g = gt_run + below_gt, q = eq_run + below_eq;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t kk = kv[e];
      const bool is_gt = kk > theta, is_eq = kk == theta;
      const uint32_t pos = g + min(q, need_eq);
      if ((is_gt || (is_eq && q < need_eq)) && pos < (uint32_t)k) {
        const int col = wbase + c * 256 + lane * 4 + e;
        s_idx[pos] = base + col;
        s_val[pos] = key_to_float(kk);
      }
      g += is_gt;
      q += is_eq;
    }
    gt_run += tot_gt;
    eq_run += tot_eq;
  }
  __syncthreads();
  for (int i = tid; i < k; i += NT) {
    out_idx[i] = s_idx[i];
    if (out_val) out_val[i] = s_val[i];
  }
  if (tid == 0 && topk_length) topk_length[r] = k;
}

template <int WAVES, int CR, int CL>
hipError_t launch_topk_cfg(const float* scores, int64_t ld, int64_t n_rows, int64_t n_cols,
                           const int32_t* sl, const int32_t* rs, int k, int32_t* idx,
                           int64_t ld_idx, int32_t* tl, float* vals, hipStream_t st) {
  dim3 grid((unsigned)n_rows), block(64 * WAVES);
  hipLaunchKernelGGL((topk_kernel<WAVES, CR, CL>), grid, block, 0, st, scores, ld, n_cols, sl, rs,
                     k, idx, ld_idx, tl, vals);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const float* scores, int64_t ld, int64_t n_rows, int64_t n_cols,
                       const int32_t* seq_lens, const int32_t* row_starts, int k, int32_t* indices,
                       int64_t ld_idx, int32_t* topk_length, float* values, hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
#define DSA_TOPK_CFG(W, CR, CL)                                                                \
  return launch_topk_cfg<W, CR, CL>(scores, ld, n_rows, n_cols, seq_lens, row_starts, k, indices, \
                                    ld_idx, topk_length, values, st)
  if (n_cols <= 256) DSA_TOPK_CFG(1, 1, 0);
  if (n_cols <= 1024) DSA_TOPK_CFG(1, 4, 0);
  if (n_cols <= 4096) DSA_TOPK_CFG(1, 16, 0);
  if (n_cols <= 16384) DSA_TOPK_CFG(4, 16, 0);
  if (n_cols <= 32768) DSA_TOPK_CFG(8, 16, 0);
  if (n_cols <= 65536) DSA_TOPK_CFG(16, 8, 8);
#undef DSA_TOPK_CFG
  return hipErrorInvalidValue;
}

}  // namespace dsa
