// Lightning-indexer scores from FP8 inputs on gfx950.
//
// The cuDNN Frontend DSA page, section 3, gives two FP8 forms of the indexer
// input: E4M3 Q and K with fp32 descales per token (and head, for Q), and
// E4M3 Q and K with one E8M0 scale per 32 elements of the head dimension
// (MXFP8). The score is the section's definition on the dequantized values:
// S[t, j] = sum_h W[t,h] * ReLU(Q[t,h,:] . K[start(t)+j, :]), head dim 128.
//
// The mapping is the one of the bf16 indexer kernel (one query row per wave,
// 8 waves per workgroup, key tiles in a double-buffered LDS ring, the
// epilogue of each 32-key block under the MFMAs of the next), with the dot
// products on v_mfma_(scale_)f32_32x32x64_f8f6f4: two k-steps of 64 over the
// head dim instead of eight of 16, at twice the bf16 rate per FLOP. A tile is
// 256 keys (one barrier per 256 keys: the FP8 MFMAs of a tile take half the
// time of the bf16 ones, so the per-tile cost weighs twice as much), 64 in
// the combined launch whose LDS holds the rows' scores.
// - Per-token descales: ReLU(a * x) = a * ReLU(x) for a >= 0, so the query
//   descale of head h folds into W[t,h] and the key descale multiplies the
//   finished score of its key; the MFMAs run unscaled.
// - MXFP8: the scaled MFMA applies the E8M0 scales of Q and K per 32-element
//   block itself; the block scales of the tile's keys are staged in LDS with
//   their rows.
#include "dsa_device.h"
#include "dsa_launch.h"
#include "dsa_rescue.h"
#include "dsa_select.h"

namespace dsa {
namespace {

constexpr int kF8Waves = 8;     // query rows per workgroup
constexpr int kF8Pairs = 4;    // 64-key pairs of 32-key blocks per LDS tile (scores, candidates)
constexpr int kF8D = 128;       // head dim (bytes per FP8 row)
constexpr int kF8KS = kF8D / 64;  // MFMA k-steps over the head dim
constexpr int kF8RowB = kF8D + 16;  // LDS row stride in bytes (16 B pad: conflict-free b128 reads)
constexpr int kF8SampleTiles = 8;   // CAND: key tiles sampled for the lower bound

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
// Four consecutive weights w[i .. i+3] (i a multiple of 4, w aligned to 4 weights).
template <typename WT>
__device__ __forceinline__ f32x4 load_wf4(const WT* w, int64_t i);
template <>
__device__ __forceinline__ f32x4 load_wf4<uint16_t>(const uint16_t* w, int64_t i) {
  const u32x2 v = *reinterpret_cast<const u32x2*>(w + i);
  return f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xffff0000u),
               __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xffff0000u)};
}
template <>
__device__ __forceinline__ f32x4 load_wf4<float>(const float* w, int64_t i) {
  return *reinterpret_cast<const f32x4*>(w + i);
}

// MB: number of 32-head blocks (H <= 32*MB). MX: block-scaled (true) or
// per-token descales (false). qs / ks: fp32 descales [T, H] / [T_kv]
// (per-token) or E8M0 bytes [T, H, 4] / [T_kv, 4] (MX). P: 64-key pairs per
// LDS tile. FUSE: the scores of each row stay in LDS (ld is then the column
// cap, at most kFuseMaxCols) and the wave selects its row's top-k into `fa`
// instead of writing scores. CAND: the row's candidates are appended to
// `ca` (the combined path's stage 1 for long rows, as the bf16 kernel's
// candidate mode: sampled lower bound, appends in column order; ld is then
// the column cap).
template <int MB, typename WT, bool MX, int P, bool FUSE, bool CAND>
__global__ __launch_bounds__(kF8Waves * 64, 1) void indexer_fp8_kernel(
    const uint8_t* __restrict__ q, const void* __restrict__ qs, const uint8_t* __restrict__ k,
    const void* __restrict__ ks, const WT* __restrict__ w, const int32_t* __restrict__ row_starts,
    const int32_t* __restrict__ seq_lens, int64_t T_kv, int H, int64_t row_begin, int64_t n_rows,
    float* __restrict__ scores, int64_t ld, FusedArgs fa, CandArgs ca, bool w_vec) {
  constexpr int kF8Tile = 64 * P;  // keys per LDS tile
  constexpr int TILE_B = kF8Tile * kF8RowB;
  constexpr int CHUNKS = kF8Tile * kF8D / 16;   // 16-byte chunks per tile
  constexpr int NT = kF8Waves * 64;
  constexpr int LOADS = CHUNKS / NT;            // 16-byte chunks per thread and tile
  static_assert(CHUNKS % NT == 0 && kF8Tile <= NT, "whole chunks per thread");
  __shared__ __attribute__((aligned(16))) unsigned char ktile[2 * TILE_B];
  // per key: fp32 descale bits, or its 4 E8M0 block scales; stored
  // transposed so that a lane reads the words of all its keys in a tile with
  // one or two 16-byte reads: MX word of block nb for key 32*nb + l at
  // l*2P + nb, per-token descale of key 64*p + l at l*P + p
  constexpr int NSC = MX ? 2 * P : P;  // scale words per lane and tile
  __shared__ __attribute__((aligned(16))) uint32_t kscale[2][kF8Tile];
  __shared__ __attribute__((aligned(16))) float s_rows[FUSE ? kF8Waves * kFuseRowStride : 4];
  static_assert(!FUSE || 2 * TILE_B >= kF8Waves * 256 * 4, "select histograms fit the tile ring");
  static_assert(!(FUSE && CAND), "one output mode");
  // CAND: the sampled keys of each wave's row, lane-major (slot 64 i + lane),
  // and the rows' valid lengths
  __shared__ uint32_t s_samp[CAND ? kF8Waves * P * kF8SampleTiles * 64 : 1];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int64_t n_qblk = (n_rows + kF8Waves - 1) / kF8Waves;
  const int64_t qblk = n_qblk - 1 - blockIdx.x;   // longest rows first
  const int64_t r0 = qblk * kF8Waves;
  const int64_t cap = T_kv > 0 ? ld : 0;  // longest row length taken (no keys: none)

  // Rows of the workgroup: lane i < kF8Waves holds row r0 + i's start and
  // valid length (>= 0; the range checks of the score writes rely on it).
  // Every wave forms the workgroup's key range [kb, ke), the union of its
  // rows' ranges, and the longest row from them, so that the first key tile
  // is requested before the query loads and without a barrier.
  const int64_t r = r0 + wave;
  const bool live = r < n_rows;
  const int64_t t = row_begin + (live ? r : 0);
  int32_t m_s0 = 0, m_n = 0;
  if (lane < kF8Waves && r0 + lane < n_rows) {
    const int64_t tt = row_begin + r0 + lane;
    m_s0 = row_starts[tt];
    m_n = (int32_t)max((int64_t)0, min((int64_t)seq_lens[tt], cap));
  }
  int32_t kb = m_n > 0 ? m_s0 : INT32_MAX, ke = m_n > 0 ? m_s0 + m_n : 0, nmax = m_n;
#pragma unroll
  for (int m = 1; m < kF8Waves; m <<= 1) {
    kb = min(kb, __shfl_xor(kb, m, kWave));
    ke = max(ke, __shfl_xor(ke, m, kWave));
    nmax = max(nmax, __shfl_xor(nmax, m, kWave));
  }
  kb = __builtin_amdgcn_readfirstlane(kb);
  ke = __builtin_amdgcn_readfirstlane(ke);
  nmax = __builtin_amdgcn_readfirstlane(nmax);
  const int32_t qstart = __shfl(m_s0, wave, kWave);
  const int32_t qlen = __shfl(m_n, wave, kWave);
  if constexpr (CAND)
    if (blockIdx.x == 0 && threadIdx.x == 0) *ca.n_queued = 0u;  // the stage-2 queue starts empty
  if (kb >= ke) {  // uniform: no row of the workgroup has a key
    if constexpr (FUSE)
      if (live)
        wave_topk_row(s_rows, 0, 0, nullptr, fa, r);  // writes the empty row
    if constexpr (CAND)
      if (live && lane == 0) ca.count[r] = 0;
    return;
  }
  // This wave's query (loaded after the first key tile is requested). A
  // operand of k-step s for head 32*mb + l%32: bytes 64s + 16*half .. +15 and
  // 64s + 32 + 16*half .. +15 of the head's row.
  i32x8 qa[MB][kF8KS];
  int qsc[MB][kF8KS];  // MX: E8M0 byte of block 2s + half of the lane's head
  float wv[MB][16];

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
    if (c < kF8Tile)
      kscale[buf][MX ? (c % 32) * NSC + c / 32 : (c % 64) * NSC + c / 64] =
          stage_sc_ok ? stage_sc : 0u;
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
  // The lane's scale words of the tile in buffer buf (read once per tile).
  uint32_t tsc[NSC];
  auto read_scales = [&](int buf) {
    const uint32_t* src = kscale[buf] + (MX ? (lane & 31) : lane) * NSC;
    if constexpr (NSC % 4 == 0) {
#pragma unroll
      for (int i = 0; i < NSC / 4; ++i) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + 4 * i);
        tsc[4 * i] = v.x;
        tsc[4 * i + 1] = v.y;
        tsc[4 * i + 2] = v.z;
        tsc[4 * i + 3] = v.w;
      }
    } else if constexpr (NSC == 2) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(src);
      tsc[0] = v.x;
      tsc[1] = v.y;
    } else {
      tsc[0] = src[0];
    }
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
    o.sw = MX ? tsc[nb] : 0u;
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
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kF8KS, 0);  // DS reads
#pragma unroll
    for (int i = 0; i < MB * kF8KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);             // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 32 / kF8KS, 0);     // VALU
    }
  };
  // Lane l < 32 sums key l of block 0 over both half-waves, lane l >= 32 key
  // l - 32 of block 1; the key descale (per-token form) multiplies the sum.
  // Scores go through a buffer descriptor of the wave's row whose range is
  // the row's valid columns; a column outside the row takes an offset past
  // the range (a select, so the tile loop has no branches), whose store the
  // hardware drops. The offset is selected rather than left to wrap below
  // zero: the compiler may move a constant part of it into the instruction's
  // offset field, and the range check then sees a wrapped register part and
  // drops valid stores too.
  // (FUSE: the row lives in LDS; columns outside the row go to a spare slot.)
  const __amdgpu_buffer_rsrc_t srow =
      raw_buffer((FUSE || CAND) ? (const void*)scores : (const void*)(scores + r * ld),
                 (FUSE || CAND) ? 0u : (uint32_t)qlen * 4u);
  float* const lrow = s_rows + (FUSE ? wave * kFuseRowStride : 0);
  // CAND: the row's lower bound and its candidates so far (wave-uniform),
  // appended in column order as (score bits, local column) through a buffer
  // descriptor of the row's cap entries: the hardware drops stores past the
  // cap (the count still grows) and those of lanes that take nothing (an
  // offset past the range). A score passes when its order-preserving signed
  // form ord() is at least t_lo: the lower bound's form, INT32_MIN for every
  // column, -1 for a bound of 0.0 (so that -0.0, form -1, passes).
  int32_t t_lo = INT32_MIN;
  uint32_t n_cand = 0u;
  const __amdgpu_buffer_rsrc_t crow =
      raw_buffer(CAND ? (const void*)(ca.cand + 2 * r * ca.cap) : (const void*)scores,
                 CAND ? (uint32_t)(ca.cap * 8) : 0u);
  auto ord = [](uint32_t b) -> int32_t {
    return (int32_t)(b ^ ((uint32_t)((int32_t)b >> 31) >> 1));
  };
  auto append = [&](uint32_t bits, uint32_t j) {
    const bool take = j < (uint32_t)qlen && ord(bits) >= t_lo;
    const uint64_t tm = ballot(take);
    const uint32_t off = take ? (n_cand + popc_below(tm)) * 8u : 0x80000000u;
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{bits, j}, crow, (int)off, 0, 0);
    n_cand += (uint32_t)__popcll(tm);
  };
  auto write_scores = [&](int32_t k0, float p0, float p1, float kscl) {
    float score = halfwave_sums(p0, p1);
    if constexpr (!MX) score *= kscl;
    const uint32_t j = (uint32_t)(k0 + lane - qstart);
    if constexpr (FUSE)
      lrow[j < (uint32_t)qlen ? j : (uint32_t)kFuseMaxCols] = score;
    else if constexpr (CAND)
      append(__float_as_uint(score), j);
    else
      buffer_store_f32(score, srow, j < (uint32_t)qlen ? j * 4u : 0x80000000u);
  };
  // CAND: whether the workgroup samples (a row longer than the capacity),
  // and the first key of sample tile i (tiles of the workgroup's range).
  const bool sample = CAND && nmax > (int32_t)ca.cap;  // uniform
  const int32_t n_tiles = (ke - kb + kF8Tile - 1) / kF8Tile;
  auto sample_start = [&](int i) -> int32_t {
    return kb + kF8Tile * (int32_t)(((int64_t)i * n_tiles) / kF8SampleTiles);
  };

  // Every wave runs every tile of the workgroup's key range (a row's keys
  // outside its own range are computed and their stores dropped). The first
  // pending write targets columns before the row, so it is dropped too.
  load_tile(kb);

  // Query fragments, MX block scales and the weights of the 16 heads whose
  // scores the lane receives per head block (32*mb + 8*(i/4) + 4*half +
  // i%4; per-token: times the query descale). The loads are unconditional
  // (clamped head, then zeroed) and all issued before any of their values is
  // used, so they are in flight together.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int head = mb * 32 + (lane & 31);
    const int hq = head < H ? head : H - 1;
    const uint8_t* qrow = q + (t * H + hq) * kF8D;
#pragma unroll
    for (int s = 0; s < kF8KS; ++s) {
      const u32x4 lo = load16(qrow + 64 * s + 16 * half);
      const u32x4 hi = load16(qrow + 64 * s + 32 + 16 * half);
      qa[mb][s] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                        (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      if constexpr (MX)
        qsc[mb][s] = (int)((const uint8_t*)qs)[(t * H + hq) * 4 + 2 * s + half];
      else
        qsc[mb][s] = 0;
    }
  }
  if (w_vec) {  // uniform: runs of 4 heads are whole, w (and qs) aligned to 4 entries
    f32x4 wr[MB][4], dr[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int oh0 = mb * 32 + 8 * j + 4 * half;
        const int64_t i0 = t * H + (oh0 < H ? oh0 : 0);
        wr[mb][j] = load_wf4<WT>(w, i0);
        if constexpr (!MX) dr[mb][j] = *reinterpret_cast<const f32x4*>((const float*)qs + i0);
      }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          wv[mb][4 * j + c] = MX ? wr[mb][j][c] : wr[mb][j][c] * dr[mb][j][c];
  } else {
    float dr[MB][16];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int oh = mb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
        const int64_t i0 = t * H + (oh < H ? oh : 0);
        wv[mb][i] = load_wf<WT>(w, i0);
        if constexpr (!MX) dr[mb][i] = ((const float*)qs)[i0];
      }
    if constexpr (!MX)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) wv[mb][i] *= dr[mb][i];
  }
  if (!live || 32 * MB > H) {  // uniform per wave: zero what is past the row or the heads
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int head = mb * 32 + (lane & 31);
#pragma unroll
      for (int s = 0; s < kF8KS; ++s)
        if (!live || head >= H) {
          qa[mb][s] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
          if constexpr (MX) qsc[mb][s] = 127;
        }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int oh = mb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
        if (!live || oh >= H) wv[mb][i] = 0.0f;
      }
    }
  }

  store_tile(0);
  __syncthreads();
  // CAND: the sample tiles are scored once; the tile loop skips them and
  // appends their saved keys in their place. Sample tile 0 is the range's
  // first tile, the others are at least 4 tiles apart (a sampling workgroup
  // has more than 32 tiles of 256 keys).
  uint32_t* const wsamp = s_samp + (CAND ? wave * P * kF8SampleTiles * 64 + lane : 0);
  auto append_saved = [&](int i) {
#pragma unroll
    for (int hp = 0; hp < P; ++hp)
      append(wsamp[64 * (P * i + hp)], (uint32_t)(sample_start(i) + 64 * hp + lane - qstart));
  };
  if constexpr (CAND) {
    if (sample) {  // uniform
      // The sample tiles go through the ring in turn (the last prefetch is
      // the tile loop's first tile, the one after sample tile 0, which lands
      // in buffer 0); lane l keeps the scores of keys s + 64 p + l (p < P)
      // of each sample tile s in the wave's LDS slots.
      static_assert(kF8SampleTiles % 2 == 0, "sample layout");
#pragma unroll 1
      for (int i = 0; i < kF8SampleTiles; ++i) {
        load_tile(i + 1 < kF8SampleTiles ? sample_start(i + 1) : kb + kF8Tile);
        const int sb = i & 1;
        const int32_t s0 = sample_start(i);
        read_scales(sb);
#pragma unroll
        for (int pr = 0; pr < P; ++pr) {
          BOp b0, b1;
          read_block(sb, 2 * pr, b0);
          read_block(sb, 2 * pr + 1, b1);
          block_mfma(b0, acc0);
          block_mfma(b1, acc1);
          float score = halfwave_sums(epilogue(acc0), epilogue(acc1));
          if constexpr (!MX) score *= __uint_as_float(tsc[pr]);
          const uint32_t j = (uint32_t)(s0 + 64 * pr + lane - qstart);
          // (invalid: all-ones bits, whose key is 0)
          wsamp[64 * (P * i + pr)] = j < (uint32_t)qlen ? __float_as_uint(score) : 0xffffffffu;
        }
        store_tile((i + 1) & 1);
        __syncthreads();
      }
      // The tile loop's first pending epilogue reads acc1 (its write is
      // dropped); zeroed, the accumulators hold nothing across the search.
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc0[mb][i] = acc1[mb][i] = 0.0f;
      if (qlen > (int32_t)ca.cap) {  // uniform per wave
        uint32_t samp[P * kF8SampleTiles];
#pragma unroll
        for (int i = 0; i < P * kF8SampleTiles; ++i)
          samp[i] = fused_key(__uint_as_float(wsamp[64 * i]));
        uint32_t nv = 0u;
#pragma unroll
        for (int i = 0; i < P * kF8SampleTiles; ++i) nv += samp[i] != 0u ? 1u : 0u;
        nv = wave_sum_u32(nv);
        const float e = (float)fa.k * (float)nv / (float)qlen;
        const uint32_t rank = (uint32_t)ceilf(e + 6.0f * sqrtf(e) + 4.0f);
        if (nv >= rank) {
          // lo = the largest key v with at least `rank` samples >= v
          uint32_t v = 0u;
#pragma unroll 1
          for (int b = 31; b >= 0; --b) {
            const uint32_t c = v | (1u << b);
            uint32_t n_ge = 0u;
#pragma unroll
            for (int i = 0; i < P * kF8SampleTiles; ++i) n_ge += samp[i] >= c ? 1u : 0u;
            if (wave_sum_u32(n_ge) >= rank) v = c;
          }
          t_lo = v == fused_key(0.0f) ? -1 : ord(__float_as_uint(fused_value(v)));
        }
      }
      append_saved(0);
    }
  }
  int buf = 0;
  int32_t pend_k0 = qstart - 64;
  float pend_p0 = 0.0f;
  float pend_ks = 0.0f;  // descale of key pend_k0 + lane
  int ns = 1;            // CAND: the next sample tile the loop has not passed
  int32_t ns_start = sample ? sample_start(1) : INT32_MAX;
  for (int32_t k0 = sample ? kb + kF8Tile : kb; k0 < ke;) {
    int32_t k_next = k0 + kF8Tile;
    if constexpr (CAND)
      if (k_next == ns_start) k_next += kF8Tile;  // uniform
    load_tile(k_next);  // zeroed past the range, so the last one is harmless

    BOp cur, nxt;
    read_scales(buf);
    read_block(buf, 0, cur);
#pragma unroll
    for (int pr = 0; pr < P; ++pr) {
      const int32_t kp = k0 + 64 * pr;
      const float kscl = MX ? 0.0f : __uint_as_float(tsc[pr]);
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

    if constexpr (CAND) {
      if (k0 + kF8Tile == ns_start) {  // uniform: a sample tile comes next
        write_scores(pend_k0, pend_p0, epilogue(acc1), pend_ks);
        append_saved(ns);
        pend_k0 = qstart - 64;  // the next tile's first pending write is dropped
        ++ns;
        ns_start = ns < kF8SampleTiles ? sample_start(ns) : INT32_MAX;
      }
    }
    store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    k0 = k_next;
  }
  write_scores(pend_k0, pend_p0, epilogue(acc1), pend_ks);
  if constexpr (CAND)
    if (live && lane == 0) ca.count[r] = (int32_t)n_cand;
  if constexpr (FUSE) {
    __syncthreads();  // the tile ring is free: it holds the select histograms now
    if (live)
      wave_topk_row(lrow, qlen, row_starts[t], reinterpret_cast<uint32_t*>(ktile) + 256 * wave,
                    fa, r);
  }
}

// Rescue pass of the combined path for long FP8 rows (the rows stage 2
// queued): workgroup g takes queued rows g, g + G, ...; for each it scores
// the row into its own spill row with the arithmetic of the indexer pass
// (per 32-key block the MFMA chain over the two 64-byte k-steps from zero,
// the ReLU * weight chain over the heads in the same order, the same
// half-wave sum, then the key's descale), so every score is bit-identical to
// the pass's, and selects exactly from them (select_spill_row).
template <int MB, typename WT, bool MX>
__global__ __launch_bounds__(kF8Waves * 64) void indexer_rescue_fp8_kernel(
    const uint8_t* __restrict__ q, const void* __restrict__ qs, const uint8_t* __restrict__ k,
    const void* __restrict__ ks, const WT* __restrict__ w, const int32_t* __restrict__ row_starts,
    const int32_t* __restrict__ seq_lens, int64_t T_kv, int H, int64_t row_begin, int64_t n_cols,
    FusedArgs fa, CandArgs ca) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t s_wave[kF8Waves];
  __shared__ uint32_t s_sel[2];
  __shared__ float s_fsum[kF8Waves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
  const uint32_t n_queued = *ca.n_queued;
  float* const spill = ca.spill + (int64_t)blockIdx.x * ca.spill_ld;
  const int64_t col_cap = T_kv > 0 ? n_cols : 0;

  for (uint32_t qi = blockIdx.x; qi < n_queued; qi += gridDim.x) {
    const int64_t r = ca.queue[qi];
    const int64_t t = row_begin + r;
    const int32_t s0 = row_starts[t];
    const int n = (int)max((int64_t)0, min((int64_t)seq_lens[t], col_cap));

    // Query fragments, block scales and weights as the indexer pass loads them.
    i32x8 qa[MB][kF8KS];
    int qsc[MB][kF8KS];
    float wv[MB][16];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int head = mb * 32 + (lane & 31);
      const bool hv = head < H;
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
        float wf = oh < H ? load_wf<WT>(w, t * H + oh) : 0.0f;
        if constexpr (!MX) wf *= oh < H ? ((const float*)qs)[t * H + oh] : 0.0f;
        wv[mb][i] = wf;
      }
    }
    // Scores of keys s0 + 64 g + [0, 64) by wave g % 8: block 0 holds keys
    // [0, 32), block 1 keys [32, 64) of the group. Keys outside [0, T_kv)
    // read zero rows and a zero scale word, as the indexer pass stages them.
    for (int g = wave; 64 * g < n; g += kF8Waves) {
      float p[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int col = 64 * g + 32 * nb + (lane & 31);
        const int64_t key = (int64_t)s0 + col;
        const bool ok = col < n && key >= 0 && key < T_kv;
        const uint8_t* krow = k + (ok ? key : 0) * kF8D;
        i32x8 kf[kF8KS];
#pragma unroll
        for (int s = 0; s < kF8KS; ++s) {
          u32x4 lo = load16(krow + 64 * s + 16 * half);
          u32x4 hi = load16(krow + 64 * s + 32 + 16 * half);
          if (!ok) lo = hi = u32x4{0u, 0u, 0u, 0u};
          kf[s] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                        (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
        const uint32_t sw = (MX && ok) ? ((const uint32_t*)ks)[key] : 0u;
        f32x16 acc[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
          for (int s = 0; s < kF8KS; ++s) {
            if constexpr (MX)
              acc[mb] = mfma32x32x64_mxfp8(qa[mb][s], qsc[mb][s], kf[s], (int)(sw >> (8 * (2 * s + half))),
                                           s == 0 ? f32x16{} : acc[mb]);
            else
              acc[mb] = mfma32x32x64_fp8(qa[mb][s], kf[s], s == 0 ? f32x16{} : acc[mb]);
          }
        }
        float sum = 0.0f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) sum = fmaf(wv[mb][i], relu_f8(acc[mb][i]), sum);
        p[nb] = sum;
      }
      float score = halfwave_sums(p[0], p[1]);
      const int colw = 64 * g + lane;  // the key this lane's score belongs to
      if constexpr (!MX) {
        const int64_t key = (int64_t)s0 + colw;
        const bool ok = colw < n && key >= 0 && key < T_kv;
        score *= ok ? ((const float*)ks)[key] : 0.0f;
      }
      if (colw < n) spill[colw] = score;
    }
    __syncthreads();  // the spill row is complete
    select_spill_row<kF8Waves>(spill, n, s0, fa, r, hist, s_wave, s_sel, s_fsum);
  }
}

template <int MB, bool MX, bool FUSE, bool CAND>
hipError_t launch_fp8_w(const void* q, const void* qs, const void* k, const void* ks,
                        const void* w, int w_dtype, const int32_t* rs, const int32_t* sl,
                        int64_t T_kv, int H, int64_t row_begin, int64_t n_rows, float* scores,
                        int64_t ld, const FusedArgs& fa, const CandArgs& ca, hipStream_t st) {
  constexpr int P = FUSE ? 1 : kF8Pairs;
  const int64_t nblk = (n_rows + kF8Waves - 1) / kF8Waves;
  dim3 grid((unsigned)nblk), block(kF8Waves * 64);
  // vector loads of 4 weights (and, per-token, 4 query descales) per run of heads
  const uintptr_t wbytes = w_dtype == 0 ? 2 : 4;
  const bool w_vec = H % 4 == 0 && (uintptr_t)w % (4 * wbytes) == 0 &&
                     (MX || (uintptr_t)qs % 16 == 0);
  if (w_dtype == 0)
    hipLaunchKernelGGL((indexer_fp8_kernel<MB, uint16_t, MX, P, FUSE, CAND>), grid, block, 0, st,
                       (const uint8_t*)q, qs, (const uint8_t*)k, ks, (const uint16_t*)w, rs, sl,
                       T_kv, H, row_begin, n_rows, scores, ld, fa, ca, w_vec);
  else
    hipLaunchKernelGGL((indexer_fp8_kernel<MB, float, MX, P, FUSE, CAND>), grid, block, 0, st,
                       (const uint8_t*)q, qs, (const uint8_t*)k, ks, (const float*)w, rs, sl, T_kv,
                       H, row_begin, n_rows, scores, ld, fa, ca, w_vec);
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
    return launch_fp8_w<MM, XX, false, false>(q, qs, k, ks, w, w_dtype, rs, sl, T_kv, H,      \
                                              row_begin, n_rows, scores, ld, none, CandArgs{}, st);
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
    return launch_fp8_w<MM, XX, true, false>(q, qs, k, ks, w, w_dtype, rs, sl, T_kv, H,      \
                                             row_begin, n_rows, nullptr, n_cols, fa, CandArgs{},  \
                                             st);
  DSA_F8_CASE(1, false) DSA_F8_CASE(2, false) DSA_F8_CASE(1, true) DSA_F8_CASE(2, true)
#undef DSA_F8_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_indexer_cand_fp8(const void* q, const void* qs, const void* k, const void* ks,
                                   bool mx, const void* w, int w_dtype, const int32_t* rs,
                                   const int32_t* sl, int64_t T_kv, int H, int64_t row_begin,
                                   int64_t n_rows, int64_t n_cols, int top_k, const CandArgs& ca,
                                   hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  const int mb = (H + 31) / 32;
  FusedArgs fa{};
  fa.k = top_k;
#define DSA_F8_CASE(MM, XX)                                                                 \
  if (mb == MM && mx == XX)                                                                 \
    return launch_fp8_w<MM, XX, false, true>(q, qs, k, ks, w, w_dtype, rs, sl, T_kv, H,     \
                                             row_begin, n_rows, nullptr, n_cols, fa, ca, st);
  DSA_F8_CASE(1, false) DSA_F8_CASE(2, false) DSA_F8_CASE(1, true) DSA_F8_CASE(2, true)
#undef DSA_F8_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_indexer_rescue_fp8(const void* q, const void* qs, const void* k, const void* ks,
                                     bool mx, const void* w, int w_dtype, const int32_t* rs,
                                     const int32_t* sl, int64_t T_kv, int H, int64_t row_begin,
                                     int64_t n_rows, int64_t n_cols, const FusedArgs& fa,
                                     const CandArgs& ca, hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  const int mb = (H + 31) / 32;
  dim3 grid((unsigned)std::min<int64_t>(ca.n_spill, n_rows)), block(kF8Waves * 64);
#define DSA_F8_CASE(MM, XX)                                                                     \
  if (mb == MM && mx == XX) {                                                                   \
    if (w_dtype == 0)                                                                           \
      hipLaunchKernelGGL((indexer_rescue_fp8_kernel<MM, uint16_t, XX>), grid, block, 0, st,     \
                         (const uint8_t*)q, qs, (const uint8_t*)k, ks, (const uint16_t*)w, rs,  \
                         sl, T_kv, H, row_begin, n_cols, fa, ca);                               \
    else                                                                                        \
      hipLaunchKernelGGL((indexer_rescue_fp8_kernel<MM, float, XX>), grid, block, 0, st,        \
                         (const uint8_t*)q, qs, (const uint8_t*)k, ks, (const float*)w, rs, sl, \
                         T_kv, H, row_begin, n_cols, fa, ca);                                   \
    return hipGetLastError();                                                                   \
  }
  DSA_F8_CASE(1, false) DSA_F8_CASE(2, false) DSA_F8_CASE(1, true) DSA_F8_CASE(2, true)
#undef DSA_F8_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsa
