// Workgroup-level pieces of an exact per-row top-k (internal header): the
// order-preserving key of a score, block scans and reductions, radix passes
// over the keys, buckets linear in the score, and the ordered placement rule.
//
// Selection rules (cuDNN Frontend DSA page, sections 4 and 5): the k largest
// scores of a row, exact ties at the k-th value going to the lower columns,
// -0.0 equal to +0.0. A selected column's output slot is
// (#greater before it) + min(#equal before it, #equal taken), in column
// order.
#pragma once

#include "dsa_device.h"

namespace dsa {

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
  const uint32_t incl = wave_incl_scan_dpp(v, [](uint32_t a, uint32_t b) { return a + b; }, 0u);
  if (WAVES == 1) {
    *total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
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

constexpr int kBins = 2048;  // histogram bins

// Radix passes (11/11/10 bits) that find theta, the remaining-th largest key
// among the keys offered by `offer(f)`, which calls f(key) for every key of
// the calling thread that takes part. Returns theta; *need_eq receives how
// many keys equal to theta are taken.
template <int WAVES, typename Offer>
__device__ __forceinline__ uint32_t radix_select(uint32_t remaining, uint32_t* hist,
                                                 uint32_t* s_wave, uint32_t* s_sel,
                                                 uint32_t* need_eq, Offer&& offer) {
  constexpr int NT = 64 * WAVES;
  constexpr int BPT = kBins / NT;
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 0x3ffu : 0x7ffu;
    for (int i = tid; i < kBins; i += NT) hist[i] = 0u;
    __syncthreads();
    offer([&](uint32_t key) {
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
    });
    __syncthreads();
    // Thread tid owns bins [hi_bin - BPT + 1, hi_bin], highest bins first.
    const int hi_bin = kBins - 1 - tid * BPT;
    uint32_t local = 0;
#pragma unroll
    for (int b = 0; b < BPT; ++b) local += hist[hi_bin - b];
    uint32_t total;
    const uint32_t above = block_exclusive_scan<WAVES>(local, s_wave, &total);
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
    remaining -= s_sel[1];
    prefix |= s_sel[0] << shift;
    pmask |= dmask << shift;
    __syncthreads();
  }
  *need_eq = remaining;
  return prefix;
}

// Bucket of a key on a scale linear in the score value: monotone in the key,
// so the buckets split the keys into ordered ranges.
struct LinearBuckets {
  float lo, scale;
  // (-0.0 and +0.0 land in the same bucket, as their keys are equal)
  __device__ __forceinline__ int of_value(float v) const {
    const float x = (v - lo) * scale;
    if (!(x > 0.0f)) return 0;  // also NaN (inf * 0 when lo = -inf)
    return x >= (float)(kBins - 1) ? kBins - 1 : (int)x;
  }
  __device__ __forceinline__ int operator()(uint32_t key) const { return of_value(key_to_float(key)); }
};

// Max over the workgroup (s_red: WAVES words).
template <int WAVES>
__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* s_red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_max_u32(v);
  if (WAVES > 1) {
    if (lane == 0) s_red[wave] = v;
    __syncthreads();
    v = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) v = max(v, s_red[w]);
    __syncthreads();
  }
  return v;
}

// Finds the bucket holding the `want`-th largest of the keys counted in
// hist (1 <= want <= their number): s_sel[0] = bucket, s_sel[1] = count in
// the buckets above it. Ends with a barrier.
template <int WAVES>
__device__ __forceinline__ void find_bucket(const uint32_t* hist, uint32_t want, uint32_t* s_wave,
                                            uint32_t* s_sel) {
  constexpr int BPT = kBins / (64 * WAVES);
  const int hi_bin = kBins - 1 - (int)threadIdx.x * BPT;  // thread owns [hi_bin - BPT + 1, hi_bin]
  uint32_t local = 0;
#pragma unroll
  for (int b = 0; b < BPT; ++b) local += hist[hi_bin - b];
  uint32_t total;
  const uint32_t above = block_exclusive_scan<WAVES>(local, s_wave, &total);
  if (above < want && want <= above + local) {
    uint32_t acc = above;
    for (int b = 0; b < BPT; ++b) {
      const uint32_t h = hist[hi_bin - b];
      if (acc + h >= want) {
        s_sel[0] = (uint32_t)(hi_bin - b);
        s_sel[1] = acc;
        break;
      }
      acc += h;
    }
  }
  __syncthreads();
}

// Ordered write of the selected keys of one thread's run, given the counts
// of keys above / equal to theta before the run (in column order).
struct Placer {
  uint32_t theta, need_eq, k;
  int32_t* out_idx;
  float* out_val;
  __device__ __forceinline__ void operator()(uint32_t key, int32_t gcol, uint32_t& g,
                                             uint32_t& q) const {
    const bool is_gt = key > theta, is_eq = key == theta;
    const uint32_t pos = g + min(q, need_eq);
    if ((is_gt || (is_eq && q < need_eq)) && pos < k) {
      out_idx[pos] = gcol;
      if (out_val) out_val[pos] = key_to_float(key);
    }
    g += is_gt;
    q += is_eq;
  }
};

}  // namespace dsa
