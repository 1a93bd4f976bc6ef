// Packed-THD metadata and lightning-indexer score kernels for gfx950.
//
// Indexer scores follow the cuDNN Frontend DSA page, section 3 "Indexer
// Forward": S[t, j] = sum_h W[t,h] * ReLU(Q[t,h,:] . K[start(t)+j, :]) with a
// causal mask (ratio 1, no offsets), materialised as fp32 with local columns.
//
// Mapping: one workgroup = 4 waves = 8 consecutive query rows (2 per wave).
// For each query the product Q_t[H x D] . K_tile^T[D x 64] runs on
// v_mfma_f32_16x16x32_bf16 with heads on the M dimension, so each lane ends up
// holding 4 heads x 1 key per 16x16 block; the ReLU * W head reduction is then
// an in-lane FMA chain plus two cross-lane adds. Q fragments stay in VGPRs for
// the whole key loop; each 64-key tile of K is staged once in LDS and shared
// by the 8 queries of the workgroup. Workgroups are issued longest-row first
// so the causal triangle's short rows fill the tail.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

__global__ void packed_metadata_kernel(const int32_t* __restrict__ cu, int32_t n_seq, int64_t T,
                                       int32_t* __restrict__ row_starts,
                                       int32_t* __restrict__ seq_lens) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  // largest d with cu[d] <= t (skips empty documents)
  int lo = 0, hi = n_seq;  // invariant: cu[lo] <= t, answer in [lo, hi]
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  int32_t s = cu[lo];
  row_starts[t] = s;
  seq_lens[t] = (int32_t)(t - s + 1);
}

namespace {

constexpr int kIdxWaves = 4;
constexpr int kIdxQPerWave = 2;
constexpr int kIdxRows = kIdxWaves * kIdxQPerWave;  // query rows per workgroup
constexpr int kIdxTile = 64;                        // keys per LDS tile

template <typename WT>
__device__ __forceinline__ float load_w(const WT* w, int64_t i);
template <>
__device__ __forceinline__ float load_w<uint16_t>(const uint16_t* w, int64_t i) {
  return bf16_bits_to_f32(w[i]);
}
template <>
__device__ __forceinline__ float load_w<float>(const float* w, int64_t i) {
  return w[i];
}

// D: indexer head dim (64 or 128). MB: number of 16-head blocks (H <= 16*MB).
template <int D, int MB, typename WT>
__global__ __launch_bounds__(256, 2) void indexer_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const WT* __restrict__ w,
    const int32_t* __restrict__ row_starts, const int32_t* __restrict__ seq_lens, int64_t T,
    int H, int64_t row_begin, int64_t n_rows, float* __restrict__ scores, int64_t ld) {
  constexpr int KS = D / 32;                 // MFMA k-steps over the head dim
  constexpr int ROW_U32 = D / 2 + 4;         // LDS row stride in u32 (16 B pad)
  __shared__ uint32_t ktile[kIdxTile * ROW_U32];
  __shared__ int32_t s_range[2];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t n_qblk = (n_rows + kIdxRows - 1) / kIdxRows;
  const int64_t qblk = n_qblk - 1 - blockIdx.x;   // longest rows first
  const int64_t r0 = qblk * kIdxRows;

  // Key range of the workgroup: union of [start, start + len) of its rows.
  if (threadIdx.x == 0) {
    int32_t kb = INT32_MAX, ke = 0;
    for (int i = 0; i < kIdxRows; ++i) {
      int64_t r = r0 + i;
      if (r < n_rows) {
        int64_t t = row_begin + r;
        int32_t s = row_starts[t];
        int32_t n = seq_lens[t];
        if (n > 0) {
          kb = min(kb, s);
          ke = max(ke, s + n);
        }
      }
    }
    s_range[0] = kb;
    s_range[1] = ke;
  }

  // Per-query registers: Q fragments (A operand, heads as rows), weights of
  // the 4 output rows this lane holds per head block, start and length.
  u32x4 qa[kIdxQPerWave][MB][KS];
  float wv[kIdxQPerWave][MB][4];
  int32_t qstart[kIdxQPerWave], qlen[kIdxQPerWave];
  int64_t qrow[kIdxQPerWave];
#pragma unroll
  for (int qi = 0; qi < kIdxQPerWave; ++qi) {
    const int64_t r = r0 + wave * kIdxQPerWave + qi;
    qrow[qi] = r;
    const bool live = r < n_rows;
    const int64_t t = row_begin + (live ? r : 0);
    qstart[qi] = live ? row_starts[t] : 0;
    int32_t n = live ? seq_lens[t] : 0;
    qlen[qi] = (int32_t)min((int64_t)n, ld);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int head = mb * 16 + (lane & 15);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (live && head < H)
          qa[qi][mb][ks] = load16(q + ((t * H + head) * D + ks * 32 + 8 * (lane >> 4)));
        else
          qa[qi][mb][ks] = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int oh = mb * 16 + 4 * (lane >> 4) + i;
        wv[qi][mb][i] = (live && oh < H) ? load_w<WT>(w, t * H + oh) : 0.0f;
      }
    }
  }
  __syncthreads();
  const int32_t kb = s_range[0];
  const int32_t ke = s_range[1];

  for (int32_t k0 = kb; k0 < ke; k0 += kIdxTile) {
    // Stage keys [k0, k0 + 64) in LDS; rows past the range are zero.
    constexpr int CHUNKS = kIdxTile * D / 8;  // 16-byte chunks per tile
#pragma unroll
    for (int c = threadIdx.x; c < CHUNKS; c += 256) {
      const int row = c / (D / 8);
      const int col = c % (D / 8);
      const int32_t key = k0 + row;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (key < ke && key >= 0 && key < T) v = load16(k + (int64_t)key * D + col * 8);
      *reinterpret_cast<u32x4*>(&ktile[row * ROW_U32 + col * 4]) = v;
    }
    __syncthreads();

    float res[kIdxQPerWave];
#pragma unroll
    for (int qi = 0; qi < kIdxQPerWave; ++qi) res[qi] = 0.0f;

#pragma unroll
    for (int nb = 0; nb < kIdxTile / 16; ++nb) {
      u32x4 kb_frag[KS];
      const int krow = nb * 16 + (lane & 15);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kb_frag[ks] = *reinterpret_cast<const u32x4*>(&ktile[krow * ROW_U32 + ks * 16 + 4 * (lane >> 4)]);
#pragma unroll
      for (int qi = 0; qi < kIdxQPerWave; ++qi) {
        float part = 0.0f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(qa[qi][mb][ks], kb_frag[ks], acc);
#pragma unroll
          for (int i = 0; i < 4; ++i) part = fmaf(wv[qi][mb][i], fmaxf(acc[i], 0.0f), part);
        }
        part += shfl_xor_f(part, 16);
        part += shfl_xor_f(part, 32);
        if ((lane >> 4) == nb) res[qi] = part;
      }
    }

    // Lane l now holds the score of key k0 + l for each of its queries.
#pragma unroll
    for (int qi = 0; qi < kIdxQPerWave; ++qi) {
      const int64_t j = (int64_t)(k0 + lane) - qstart[qi];
      if (qrow[qi] < n_rows && j >= 0 && j < qlen[qi])
        scores[qrow[qi] * ld + j] = res[qi];
    }
    __syncthreads();
  }
}

template <int D, int MB>
hipError_t launch_indexer_w(const void* q, const void* k, const void* w, int w_dtype,
                            const int32_t* rs, const int32_t* sl, int64_t T, int H,
                            int64_t row_begin, int64_t n_rows, float* scores, int64_t ld,
                            hipStream_t st) {
  const int64_t nblk = (n_rows + kIdxRows - 1) / kIdxRows;
  dim3 grid((unsigned)nblk), block(256);
  if (w_dtype == 0)
    hipLaunchKernelGGL((indexer_kernel<D, MB, uint16_t>), grid, block, 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)w, rs, sl, T, H,
                       row_begin, n_rows, scores, ld);
  else
    hipLaunchKernelGGL((indexer_kernel<D, MB, float>), grid, block, 0, st, (const uint16_t*)q,
                       (const uint16_t*)k, (const float*)w, rs, sl, T, H, row_begin, n_rows,
                       scores, ld);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_packed_metadata(const int32_t* cu, int32_t n_seq, int64_t T, int32_t* rs,
                                  int32_t* sl, hipStream_t st) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)((T + 255) / 256)), block(256);
  hipLaunchKernelGGL(packed_metadata_kernel, grid, block, 0, st, cu, n_seq, T, rs, sl);
  return hipGetLastError();
}

hipError_t launch_indexer(const void* q, const void* k, const void* w, int w_dtype,
                          const int32_t* rs, const int32_t* sl, int64_t T, int H, int D,
                          int64_t row_begin, int64_t n_rows, float* scores, int64_t ld,
                          hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  const int mb = (H + 15) / 16;
#define DSA_IDX_CASE(DD, MM)                                                                   \
  if (D == DD && mb == MM)                                                                     \
    return launch_indexer_w<DD, MM>(q, k, w, w_dtype, rs, sl, T, H, row_begin, n_rows, scores, \
                                    ld, st);
  DSA_IDX_CASE(128, 1) DSA_IDX_CASE(128, 2) DSA_IDX_CASE(128, 3) DSA_IDX_CASE(128, 4)
  DSA_IDX_CASE(64, 1) DSA_IDX_CASE(64, 2) DSA_IDX_CASE(64, 3) DSA_IDX_CASE(64, 4)
#undef DSA_IDX_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsa
