// Lightning-indexer scores from FP8 inputs on gfx950.
//
// The cuDNN Frontend DSA page, section 3, gives two FP8 forms of the indexer
// input: E4M3 Q and K with fp32 descales per token (and head, for Q), and
// E4M3 Q and K with one E8M0 scale per 32 elements of the head dimension
// (MXFP8). The score is the section's definition on the dequantized values:
// S[t, j] = sum_h W[t,h] * ReLU(Q[t,h,:] . K[start(t)+j, :]), head dim 128.
//
// The mapping is the one of the bf16 indexer kernel (one query row per wave,
// 8 waves per workgroup, 64-key tiles of K in a double-buffered LDS ring, the
// epilogue of each 32-key block under the MFMAs of the next), with the dot
// products on v_mfma_(scale_)f32_32x32x64_f8f6f4: two k-steps of 64 over the
// head dim instead of eight of 16, at twice the bf16 rate per FLOP.
// - Per-token descales: ReLU(a * x) = a * ReLU(x) for a >= 0, so the query
//   descale of head h folds into W[t,h] and the key descale multiplies the
//   finished score of its key; the MFMAs run unscaled.
// - MXFP8: the scaled MFMA applies the E8M0 scales of Q and K per 32-element
//   block itself; the block scales of the tile's keys are staged in LDS with
//   their rows.
#include "dsa_device.h"
#include "dsa_launch.h"
#include "dsa_select.h"

namespace dsa {
namespace {

constexpr int kF8Waves = 8;     // query rows per workgroup
constexpr int kF8Pairs = 2;    // 64-key pairs of 32-key blocks per LDS tile (scores to HBM)
constexpr int kF8D = 128;       // head dim (bytes per FP8 row)
constexpr int kF8KS = kF8D / 64;  // MFMA k-steps over the head dim
constexpr int kF8RowB = kF8D + 16;  // LDS row stride in bytes (16 B pad: conflict-free b128 reads)

__device__ __forceinline__ float relu_f8(float x) {
  return __builtin_amdgcn_fmed3f(x, 0.0f, 3.40282347e38f);
}

template <typename WT>
__device__ __forceinline__ float load_wf(const WT* w, int64_t i);
template <>
__device__ __forceinline__ float load_wf<uint16_t>(const uint16_t* w, int64_t i) {
  return bf16_bits_to_f32(w[i]);
}
template <>
__device__ __forceinline__ float load_wf<float>(const float* w, int64_t i) {
  return w[i];
}

// MB: number of 32-head blocks (H <= 32*MB). MX: block-scaled (true) or
// per-token descales (false). qs / ks: fp32 descales [T, H] / [T_kv]
// (per-token) or E8M0 bytes [T, H, 4] / [T_kv, 4] (MX). P: 64-key pairs per
// LDS tile. FUSE: the scores of each row stay in LDS (ld is then the column
// cap, at most kFuseMaxCols) and the wave selects its row's top-k into `fa`
// instead of writing scores.
template <int MB, typename WT, bool MX, int P, bool FUSE>
__global__ __launch_bounds__(kF8Waves * 64, 1) void indexer_fp8_kernel(
    const uint8_t* __restrict__ q, const void* __restrict__ qs, const uint8_t* __restrict__ k,
    const void* __restrict__ ks, const WT* __restrict__ w, const int32_t* __restrict__ row_starts,
    const int32_t* __restrict__ seq_lens, int64_t T_kv, int H, int64_t row_begin, int64_t n_rows,
    float* __restrict__ scores, int64_t ld, FusedArgs fa) {
  constexpr int kF8Tile = 64 * P;  // keys per LDS tile
  constexpr int TILE_B = kF8Tile * kF8RowB;
  constexpr int CHUNKS = kF8Tile * kF8D / 16;   // 16-byte chunks per tile
  constexpr int NT = kF8Waves * 64;
  constexpr int LOADS = CHUNKS / NT;            // 16-byte chunks per thread and tile
  static_assert(CHUNKS % NT == 0 && kF8Tile <= NT, "whole chunks per thread");
  __shared__ __attribute__((aligned(16))) unsigned char ktile[2 * TILE_B];
  __shared__ uint32_t kscale[2][kF8Tile];  // per key: fp32 descale bits, or 4 E8M0 bytes
  __shared__ int32_t s_range[2];
  __shared__ __attribute__((aligned(16))) float s_rows[FUSE ? kF8Waves * kFuseRowStride : 4];
  static_assert(!FUSE || 2 * TILE_B >= kF8Waves * 256 * 4, "select histograms fit the tile ring");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int64_t n_qblk = (n_rows + kF8Waves - 1) / kF8Waves;
  const int64_t qblk = n_qblk - 1 - blockIdx.x;   // longest rows first
  const int64_t r0 = qblk * kF8Waves;
  const int64_t cap = T_kv > 0 ? ld : 0;  // longest row length taken (no keys: none)

  // This wave's query. A operand of k-step s for head 32*mb + l%32: bytes
  // 64s + 16*half .. +15 and 64s + 32 + 16*half .. +15 of the head's row.
  const int64_t r = r0 + wave;
  const bool live = r < n_rows;
  const int64_t t = row_begin + (live ? r : 0);
  const int32_t qstart = live ? row_starts[t] : 0;
  // valid columns of the row, >= 0 (the range checks of the score writes rely on it)
  const int32_t qlen = live ? (int32_t)max((int64_t)0, min((int64_t)seq_lens[t], cap)) : 0;
  i32x8 qa[MB][kF8KS];
  int qsc[MB][kF8KS];  // MX: E8M0 byte of block 2s + half of the lane's head
  float wv[MB][16];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int head = mb * 32 + (lane & 31);
    const bool hv = live && head < H;
    const uint8_t* qrow = q + (t * H + head) * kF8D;
#pragma unroll
    for (int s = 0; s < kF8KS; ++s) {
      const u32x4 lo = hv ? load16(qrow + 64 * s + 16 * half) : u32x4{0u, 0u, 0u, 0u};
      const u32x4 hi = hv ? load16(qrow + 64 * s + 32 + 16 * half) : u32x4{0u, 0u, 0u, 0u};
      qa[mb][s] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                        (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      if constexpr (MX)
        qsc[mb][s] = hv ? (int)((const uint8_t*)qs)[(t * H + head) * 4 + 2 * s + half] : 127;
      else
        qsc[mb][s] = 0;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int oh = mb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
      float wf = (live && oh < H) ? load_wf<WT>(w, t * H + oh) : 0.0f;
      if constexpr (!MX) wf *= (live && oh < H) ? ((const float*)qs)[t * H + oh] : 0.0f;
      wv[mb][i] = wf;
    }
  }
  // Key range of the workgroup (after the Q loads, so that wave 0's loads of
  // both are in flight together).
  if (threadIdx.x < 64)
    wave_key_range(row_starts, seq_lens, row_begin, r0, n_rows, kF8Waves, cap, s_range);
  __syncthreads();
  const int32_t kb = s_range[0];
  const int32_t ke = s_range[1];
  if (kb >= ke) {  // uniform: no row of the workgroup has a key
    if constexpr (FUSE)
      if (live)
        wave_topk_row(s_rows, 0, 0, nullptr, fa, r);  // writes the empty row
    return;
  }

  // Staging of keys [k0, k0 + kF8Tile): thread -> 16-byte chunks
  // c = tid + NT*i (key c / 8); threads below kF8Tile also fetch the scale
  // word of key k0 + tid. Loads past the range come from a clamped row and
  // are zeroed when stored.
  u32x4 stage[LOADS];
  uint32_t stage_sc = 0;
  uint32_t stage_ok = 0;
  bool stage_sc_ok = false;
  auto load_tile = [&](int32_t k0) {
    stage_ok = 0;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = threadIdx.x + NT * i;
      const int32_t key = k0 + c / (kF8D / 16);
      const bool ok = key < ke && key >= 0 && key < T_kv;
      const int32_t kc = ok ? key : (int32_t)(T_kv - 1);
      stage[i] = load16(k + (int64_t)kc * kF8D + (c % (kF8D / 16)) * 16);
      stage_ok |= ok ? (1u << i) : 0u;
    }
    const int c = threadIdx.x;
    if (c < kF8Tile) {
      const int32_t key2 = k0 + c;
      stage_sc_ok = key2 < ke && key2 >= 0 && key2 < T_kv;
      const int32_t kc2 = stage_sc_ok ? key2 : (int32_t)(T_kv - 1);
      stage_sc = ((const uint32_t*)ks)[kc2];
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = threadIdx.x + NT * i;
      *reinterpret_cast<u32x4*>(ktile + buf * TILE_B + (c / (kF8D / 16)) * kF8RowB +
                                (c % (kF8D / 16)) * 16) =
          ((stage_ok >> i) & 1u) ? stage[i] : u32x4{0u, 0u, 0u, 0u};
    }
    const int c = threadIdx.x;
    if (c < kF8Tile) kscale[buf][c] = stage_sc_ok ? stage_sc : 0u;
  };

  f32x16 acc0[MB], acc1[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc0[mb][i] = acc1[mb][i] = 0.0f;
  auto epilogue = [&](const f32x16* acc) -> float {
    float p = 0.0f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) p = fmaf(wv[mb][i], relu_f8(acc[mb][i]), p);
    return p;
  };
  // B operand of k-step s: key 32*nb + l%32, bytes as for A. A block's
  // operands are read from LDS one block ahead of its MFMAs.
  struct BOp {
    i32x8 kf[kF8KS];
    uint32_t sw;  // MX: the key's four E8M0 block scales
  };
  auto read_block = [&](int buf, int nb, BOp& o) {
    const unsigned char* kt = ktile + buf * TILE_B + (32 * nb + (lane & 31)) * kF8RowB;
#pragma unroll
    for (int s = 0; s < kF8KS; ++s) {
      const u32x4 lo = *reinterpret_cast<const u32x4*>(kt + 64 * s + 16 * half);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(kt + 64 * s + 32 + 16 * half);
      o.kf[s] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                      (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    o.sw = MX ? kscale[buf][32 * nb + (lane & 31)] : 0u;
  };
  auto block_mfma = [&](const BOp& o, f32x16* acc) {
    if constexpr (MX) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int s = 0; s < kF8KS; ++s)
          acc[mb] = mfma32x32x64_mxfp8(qa[mb][s], qsc[mb][s], o.kf[s],
                                       (int)(o.sw >> (8 * (2 * s + half))),
                                       s == 0 ? f32x16{} : acc[mb]);
    } else {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int s = 0; s < kF8KS; ++s)
          acc[mb] = mfma32x32x64_fp8(qa[mb][s], o.kf[s], s == 0 ? f32x16{} : acc[mb]);
    }
  };
  auto interleave = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kF8KS + (MX ? 1 : 0), 0);  // DS reads
#pragma unroll
    for (int i = 0; i < MB * kF8KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);             // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 32 / kF8KS, 0);     // VALU
    }
  };
  // Lane l < 32 sums key l of block 0 over both half-waves, lane l >= 32 key
  // l - 32 of block 1; the key descale (per-token form) multiplies the sum.
  // Scores go through a buffer descriptor of the wave's row whose range is
  // the row's valid columns: stores of other columns are dropped by the
  // hardware range check, so the tile loop has no branches.
  // (FUSE: the row lives in LDS; columns outside the row go to a spare slot.)
  const __amdgpu_buffer_rsrc_t srow =
      raw_buffer(FUSE ? (const void*)scores : (const void*)(scores + r * ld),
                 FUSE ? 0u : (uint32_t)qlen * 4u);
  float* const lrow = s_rows + (FUSE ? wave * kFuseRowStride : 0);
  auto write_scores = [&](int32_t k0, float p0, float p1, float kscl) {
    float score = halfwave_sums(p0, p1);
    if constexpr (!MX) score *= kscl;
    const uint32_t j = (uint32_t)(k0 + lane - qstart);
    if constexpr (FUSE)
      lrow[j < (uint32_t)qlen ? j : (uint32_t)kFuseMaxCols] = score;
    else
      buffer_store_f32(score, srow, j * 4u);  // negative: dropped
  };

  // Every wave runs every tile of the workgroup's key range (a row's keys
  // outside its own range are computed and their stores dropped). The first
  // pending write targets columns before the row, so it is dropped too.
  load_tile(kb);
  store_tile(0);
  __syncthreads();
  int buf = 0;
  int32_t pend_k0 = qstart - 64;
  float pend_p0 = 0.0f;
  float pend_ks = 0.0f;  // descale of key pend_k0 + lane
  for (int32_t k0 = kb; k0 < ke; k0 += kF8Tile) {
    load_tile(k0 + kF8Tile);  // zeroed past the range, so the last one is harmless

    BOp cur, nxt;
    read_block(buf, 0, cur);
#pragma unroll
    for (int pr = 0; pr < P; ++pr) {
      const int32_t kp = k0 + 64 * pr;
      const float kscl = MX ? 0.0f : __uint_as_float(kscale[buf][64 * pr + lane]);
      read_block(buf, 2 * pr + 1, nxt);
      // Each group pairs a block's MFMAs with the previous block's epilogue;
      // the fences keep the scheduler from filling the VALU slots with the
      // epilogue that waits on these very MFMAs.
      block_mfma(cur, acc0);
      const float p1_prev = epilogue(acc1);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      write_scores(pend_k0, pend_p0, p1_prev, pend_ks);
      if (pr + 1 < P) read_block(buf, 2 * pr + 2, cur);
      block_mfma(nxt, acc1);
      pend_p0 = epilogue(acc0);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      pend_k0 = kp;
      pend_ks = kscl;
    }

    store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  write_scores(pend_k0, pend_p0, epilogue(acc1), pend_ks);
  if constexpr (FUSE) {
    __syncthreads();  // the tile ring is free: it holds the select histograms now
    if (live)
      wave_topk_row(lrow, qlen, row_starts[t], reinterpret_cast<uint32_t*>(ktile) + 256 * wave,
                    fa, r);
  }
}

template <int MB, bool MX, bool FUSE>
hipError_t launch_fp8_w(const void* q, const void* qs, const void* k, const void* ks,
                        const void* w, int w_dtype, const int32_t* rs, const int32_t* sl,
                        int64_t T_kv, int H, int64_t row_begin, int64_t n_rows, float* scores,
                        int64_t ld, const FusedArgs& fa, hipStream_t st) {
  constexpr int P = FUSE ? 1 : kF8Pairs;
  const int64_t nblk = (n_rows + kF8Waves - 1) / kF8Waves;
  dim3 grid((unsigned)nblk), block(kF8Waves * 64);
  if (w_dtype == 0)
    hipLaunchKernelGGL((indexer_fp8_kernel<MB, uint16_t, MX, P, FUSE>), grid, block, 0, st,
                       (const uint8_t*)q, qs, (const uint8_t*)k, ks, (const uint16_t*)w, rs, sl,
                       T_kv, H, row_begin, n_rows, scores, ld, fa);
  else
    hipLaunchKernelGGL((indexer_fp8_kernel<MB, float, MX, P, FUSE>), grid, block, 0, st,
                       (const uint8_t*)q, qs, (const uint8_t*)k, ks, (const float*)w, rs, sl, T_kv,
                       H, row_begin, n_rows, scores, ld, fa);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_fp8(const void* q, const void* qs, const void* k, const void* ks,
                              bool mx, const void* w, int w_dtype, const int32_t* rs,
                              const int32_t* sl, int64_t T_kv, int H, int64_t row_begin,
                              int64_t n_rows, float* scores, int64_t ld, hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  const int mb = (H + 31) / 32;
  const FusedArgs none{};
#define DSA_F8_CASE(MM, XX)                                                                    \
  if (mb == MM && mx == XX)                                                                    \
    return launch_fp8_w<MM, XX, false>(q, qs, k, ks, w, w_dtype, rs, sl, T_kv, H, row_begin, \
                                       n_rows, scores, ld, none, st);
  DSA_F8_CASE(1, false) DSA_F8_CASE(2, false) DSA_F8_CASE(1, true) DSA_F8_CASE(2, true)
#undef DSA_F8_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_indexer_topk_fp8(const void* q, const void* qs, const void* k, const void* ks,
                                   bool mx, const void* w, int w_dtype, const int32_t* rs,
                                   const int32_t* sl, int64_t T_kv, int H, int64_t row_begin,
                                   int64_t n_rows, int64_t n_cols, const FusedArgs& fa,
                                   hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  const int mb = (H + 31) / 32;
#define DSA_F8_CASE(MM, XX)                                                                  \
  if (mb == MM && mx == XX)                                                                  \
    return launch_fp8_w<MM, XX, true>(q, qs, k, ks, w, w_dtype, rs, sl, T_kv, H, row_begin, \
                                      n_rows, nullptr, n_cols, fa, st);
  DSA_F8_CASE(1, false) DSA_F8_CASE(2, false) DSA_F8_CASE(1, true) DSA_F8_CASE(2, true)
#undef DSA_F8_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsa
