// Packed-THD metadata and lightning-indexer score kernels for gfx950.
//
// Indexer scores follow the cuDNN Frontend DSA page, section 3 "Indexer
// Forward": S[t, j] = sum_h W[t,h] * ReLU(Q[t,h,:] . K[start(t)+j, :]) for
// j < len(t), materialised as fp32 with local columns. start(t) and len(t)
// come from one of the two metadata kernels: the plain causal mask of packed
// documents, or the section's ratio-causal mask with per-segment query
// causal offsets.
//
// Mapping: one workgroup = 8 waves = 8 consecutive query rows, one per wave
// (two waves per SIMD, so one wave's epilogue overlaps the other's MFMAs).
// For its query, a wave computes Q_t[H x D] . K_tile^T[D x 32] on
// v_mfma_f32_32x32x16_bf16 with heads on the M dimension (32 heads per MFMA
// block): lane l ends up with key l % 32 and 16 of the block's heads, so the
// ReLU * W head reduction is an in-lane max + FMA chain plus one exchange
// between the two half-waves. Q fragments and the lane's 16 weights per head
// block stay in registers for the whole key loop; 128-key tiles of K are
// staged in a double-buffered LDS ring (16-byte padded rows, conflict-free
// operand reads) and shared by the 8 queries. Each wave writes its 64 scores
// of a tile as one contiguous 256-byte run. Workgroups are issued longest row
// first so the causal triangle's short rows fill the tail.
#include "dsa_device.h"
#include "dsa_launch.h"
#include "dsa_rescue.h"
#include "dsa_rowsel.h"
#include "dsa_select.h"

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

// Ratio-causal mask (DSA page, section 3): query row t of segment b sees the
// first clamp(floor((off[b] + t - cu_q[b] + 1) / ratio), 0, |K segment b|)
// compressed keys of its segment, which start at key row cu_k[b].
__global__ void ratio_metadata_kernel(const int32_t* __restrict__ cu_q,
                                      const int32_t* __restrict__ cu_k,
                                      const int32_t* __restrict__ offsets, int32_t n_seq,
                                      int64_t T_q, int32_t ratio,
                                      int32_t* __restrict__ row_starts,
                                      int32_t* __restrict__ seq_lens) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T_q) return;
  // largest segment b in [0, n_seq) with cu_q[b] <= t (skips empty segments)
  int lo = 0, hi = n_seq - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu_q[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int64_t kb = cu_k[lo];
  const int64_t klen = (int64_t)cu_k[lo + 1] - kb;
  // global position of the query, plus one; non-positive sees nothing
  const int64_t g1 = (offsets ? (int64_t)offsets[lo] : 0) + (t - cu_q[lo]) + 1;
  int64_t n = g1 > 0 ? g1 / ratio : 0;
  n = n < klen ? n : klen;
  row_starts[t] = (int32_t)kb;
  seq_lens[t] = (int32_t)(n > 0 ? n : 0);
}

namespace {

constexpr int kIdxWaves = 8;                        // = query rows per workgroup
constexpr int kIdxHalf = 64;                        // keys per pipelined pair of 32-key blocks

// max(x, 0) for finite x as one v_med3_f32 (clamp to [0, FLT_MAX]); fmaxf
// would first quiet a possible NaN in x with a second instruction.
__device__ __forceinline__ float relu(float x) {
  return __builtin_amdgcn_fmed3f(x, 0.0f, 3.40282347e38f);
}

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
// Four consecutive weights w[i .. i+3] (i a multiple of 4, w 16-byte aligned).
template <typename WT>
__device__ __forceinline__ f32x4 load_w4(const WT* w, int64_t i);
template <>
__device__ __forceinline__ f32x4 load_w4<uint16_t>(const uint16_t* w, int64_t i) {
  const u32x2 v = *reinterpret_cast<const u32x2*>(w + i);
  return f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xffff0000u),
               __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xffff0000u)};
}
template <>
__device__ __forceinline__ f32x4 load_w4<float>(const float* w, int64_t i) {
  return *reinterpret_cast<const f32x4*>(w + i);
}

// What the indexer pass does with the scores of its rows.
enum : int {
  kModeScores = 0,  // writes them to a dense score matrix
  kModeFused = 1,   // keeps each row in LDS and selects its top-k there
  kModeCand = 2,    // appends the columns at or above a per-row lower bound
};
constexpr int kSampleTiles = 8;  // key tiles sampled for the lower bound

// D: indexer head dim (64 or 128). MB: number of 32-head blocks (H <= 32*MB).
// kModeFused: the scores of each row stay in LDS (ld is then the column cap,
// at most kFuseMaxCols) and the wave selects its row's top-k into `fa`
// instead of writing scores; with D = 128 the key tile is then
// single-buffered so that eight 4096-column rows fit next to it.
// kModeCand (stage 1 of the combined path for long rows; ld is the column
// cap): when a row of the workgroup is longer than the candidate capacity,
// kSampleTiles key tiles spread over the workgroup's key range are scored
// first, and each such row takes as its lower bound lo the sample of rank
// e + 6 sqrt(e) + 4 from the top, e = k * (valid samples) / (row length)
// being the expected sample rank of the row's k-th largest score (about six
// standard deviations of the sampling noise above it); shorter rows take
// every column. The tile loop then appends each column whose score is at or
// above lo to the row's candidate list as (order-preserving key, local
// column), in column order, counting them all (also those past the cap).
template <int D, int MB, typename WT, int MODE>
__global__ __launch_bounds__(kIdxWaves * 64, 1) void indexer_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const WT* __restrict__ w,
    const int32_t* __restrict__ row_starts, const int32_t* __restrict__ seq_lens, int64_t T_kv,
    int H, int64_t row_begin, int64_t n_rows, float* __restrict__ scores, int64_t ld,
    FusedArgs fa, CandArgs ca, bool w_vec) {
  constexpr bool FUSE = MODE == kModeFused;
  constexpr bool CAND = MODE == kModeCand;
  constexpr int KS = D / 16;                      // MFMA k-steps over the head dim
  constexpr int ROW_B = 2 * D + 16;               // LDS row stride in bytes (16 B pad)
  // keys per LDS tile: 128 (one barrier per 128 keys); 64 when the rows'
  // scores share the LDS
  constexpr int TILE = FUSE ? 64 : 128;
  constexpr int TILE_B = TILE * ROW_B;
  constexpr int CHUNKS = TILE * D / 8;            // 16-byte chunks per tile
  constexpr int NT = kIdxWaves * 64;
  constexpr int LOADS = (CHUNKS + NT - 1) / NT;   // 16-byte loads per thread and tile
  constexpr int NBUF = (FUSE && D == 128) ? 1 : 2;  // key tiles in the LDS ring
  __shared__ __attribute__((aligned(16))) unsigned char ktile[NBUF * TILE_B];
  __shared__ __attribute__((aligned(16))) float s_rows[FUSE ? kIdxWaves * kFuseRowStride : 4];
  // CAND: the sampled keys of each wave's row, lane-major (slot 64 i + lane)
  __shared__ uint32_t s_samp[CAND ? kIdxWaves * 2 * kSampleTiles * 64 : 1];
  static_assert(!FUSE || NBUF * TILE_B >= kIdxWaves * 256 * 4, "select histograms fit the ring");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int64_t n_qblk = (n_rows + kIdxWaves - 1) / kIdxWaves;
  const int64_t qblk = n_qblk - 1 - blockIdx.x;   // longest rows first
  const int64_t r0 = qblk * kIdxWaves;
  const int64_t cap = T_kv > 0 ? ld : 0;  // longest row length taken (no keys: none)

  // Rows of the workgroup: lane i < kIdxWaves holds row r0 + i's start and
  // valid length (>= 0; the range checks of the score writes rely on it).
  // Every wave forms the key range [kb, kb) of the workgroup from them, the
  // union of its rows' ranges, so the first key tile is requested before
  // anything else and without a barrier.
  const int64_t r = r0 + wave;
  const bool live = r < n_rows;
  const int64_t t = row_begin + (live ? r : 0);
  int32_t m_s0 = 0, m_n = 0;
  if (lane < kIdxWaves && r0 + lane < n_rows) {
    const int64_t tt = row_begin + r0 + lane;
    m_s0 = row_starts[tt];
    m_n = (int32_t)max((int64_t)0, min((int64_t)seq_lens[tt], cap));
  }
  int32_t kb = m_n > 0 ? m_s0 : INT32_MAX, ke = m_n > 0 ? m_s0 + m_n : 0, nmax = m_n;
#pragma unroll
  for (int m = 1; m < kIdxWaves; m <<= 1) {
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

  u32x4 qa[MB][KS];  // filled after the first key tile is requested
  float wv[MB][16];

  // Staging of keys [k0, k0 + 64): thread -> chunks c = tid + NT*i.
  u32x4 stage[LOADS];
  // The staging has no branches: keys past the range are loaded from a
  // clamped row (the validity bit is kept, not applied to the value of the
  // load, which is still in flight) and zeroed when stored to LDS.
  uint32_t stage_ok = 0;
  auto load_tile = [&](int32_t k0) {
    stage_ok = 0;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = threadIdx.x + NT * i;
      if (c < CHUNKS) {
        const int32_t key = k0 + c / (D / 8);
        const bool ok = key < ke && key >= 0 && key < T_kv;
        const int32_t kc = ok ? key : (int32_t)(T_kv - 1);
        stage[i] = load16(k + (int64_t)kc * D + (c % (D / 8)) * 8);
        stage_ok |= ok ? (1u << i) : 0u;
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = threadIdx.x + NT * i;
      if (c < CHUNKS)
        *reinterpret_cast<u32x4*>(ktile + buf * TILE_B + (c / (D / 8)) * ROW_B +
                                  (c % (D / 8)) * 16) =
            ((stage_ok >> i) & 1u) ? stage[i] : u32x4{0u, 0u, 0u, 0u};
    }
  };

  // The epilogue of each 32-key block runs under the MFMAs of the next one:
  // block 0 of tile i overlaps the epilogue of block 1 of tile i-1, block 1
  // overlaps the epilogue of block 0 of tile i.
  f32x16 acc0[MB], acc1[MB];  // block 0 / block 1 of the current tile
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc0[mb][i] = acc1[mb][i] = 0.0f;
  auto epilogue = [&](const f32x16* acc) -> float {
    float p = 0.0f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) p = fmaf(wv[mb][i], relu(acc[mb][i]), p);
    return p;
  };
  // B operand: lane -> key 32*nb + l%32, dims 16*ks + 8*half .. +7
  auto block_mfma = [&](const unsigned char* kt, int nb, f32x16* acc) {
    u32x4 kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kf[ks] = *reinterpret_cast<const u32x4*>(kt + (32 * nb + (lane & 31)) * ROW_B + ks * 32 +
                                               16 * half);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc[mb] = mfma32x32x16(qa[mb][ks], kf[ks], ks == 0 ? f32x16{} : acc[mb]);
    }
  };
  // Interleave: the block's operand reads first, then one MFMA per 4 VALU ops.
  auto interleave = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);  // DS reads
#pragma unroll
    for (int i = 0; i < MB * KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 32 / KS, 0);  // VALU
    }
  };
  // Lane l < 32 sums key l of block 0 over both half-waves, lane l >= 32
  // key l - 32 of block 1: one exchange between the half-waves. Scores go
  // through a buffer descriptor of the wave's row whose range is the row's
  // valid columns; a column outside the row takes an offset past the range
  // (a select, so the tile loop has no branches), whose store the hardware
  // drops. The offset is selected rather than left to wrap below zero: the
  // compiler may move a constant part of it into the instruction's offset
  // field, and the range check then sees a wrapped register part and drops
  // valid stores too.
  // (FUSE: the row lives in LDS; columns outside the row go to a spare slot.)
  const __amdgpu_buffer_rsrc_t srow =
      raw_buffer(MODE != kModeScores ? (const void*)scores : (const void*)(scores + r * ld),
                 MODE != kModeScores ? 0u : (uint32_t)qlen * 4u);
  float* const lrow = s_rows + (FUSE ? wave * kFuseRowStride : 0);
  // CAND: the row's lower bound and its candidates so far (wave-uniform),
  // appended in column order as (score bits, local column) through a buffer
  // descriptor of the row's cap entries: the hardware drops stores past the
  // cap (the count still grows) and those of lanes that take nothing (an
  // offset past the range). A score passes when its order-preserving signed
  // form ord() is at least t_lo: the lower bound's form, INT32_MIN for
  // every column, -1 for a bound of 0.0 (so that -0.0, form -1, passes).
  int32_t t_lo = INT32_MIN;
  uint32_t n_cand = 0u;
  const __amdgpu_buffer_rsrc_t crow =
      raw_buffer(CAND ? (const void*)(ca.cand + 2 * r * ca.cap) : (const void*)scores,
                 CAND ? (uint32_t)(ca.cap * 8) : 0u);
  auto ord = [](uint32_t b) -> int32_t {
    return (int32_t)(b ^ ((uint32_t)((int32_t)b >> 31) >> 1));
  };
  // one column per lane: local column j of the row, its score's bits
  auto append = [&](uint32_t bits, uint32_t j) {
    const bool take = j < (uint32_t)qlen && ord(bits) >= t_lo;
    const uint64_t tm = ballot(take);
    const uint32_t off = take ? (n_cand + popc_below(tm)) * 8u : 0x80000000u;
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{bits, j}, crow, (int)off, 0, 0);
    n_cand += (uint32_t)__popcll(tm);
  };
  auto write_scores = [&](int32_t k0, float p0, float p1) {
    const float score = halfwave_sums(p0, p1);
    const uint32_t j = (uint32_t)(k0 + lane - qstart);
    if constexpr (FUSE) {
      lrow[j < (uint32_t)qlen ? j : (uint32_t)kFuseMaxCols] = score;
    } else if constexpr (CAND) {
      append(__float_as_uint(score), j);
    } else {
      buffer_store_f32(score, srow, j < (uint32_t)qlen ? j * 4u : 0x80000000u);
    }
  };

  // CAND: whether the workgroup samples (a row longer than the capacity),
  // and the first key of sample tile i (tiles of the workgroup's range).
  const bool sample = CAND && nmax > (int32_t)ca.cap;  // uniform
  const int32_t n_tiles = (ke - kb + TILE - 1) / TILE;
  auto sample_start = [&](int i) -> int32_t {
    return kb + TILE * (int32_t)(((int64_t)i * n_tiles) / kSampleTiles);
  };

  // Every wave runs every tile of the workgroup's key range (a row's keys
  // outside its own range are computed and their stores dropped). The first
  // pending write targets columns before the row, so it is dropped too.
  load_tile(sample ? sample_start(0) : kb);

  // This wave's query: Q fragments (A operand: lane -> head 32*mb + l%32,
  // dims 16*ks + 8*half .. +7) and the weights of the 16 heads whose scores
  // the lane receives per head block: 32*mb + 8*(i/4) + 4*half + i%4. The
  // loads are unconditional (clamped head, then zeroed), so that waiting
  // for the key tile does not wait for them.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int head = mb * 32 + (lane & 31);
    const int hq = head < H ? head : H - 1;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qa[mb][ks] = load16(q + ((t * H + hq) * D + ks * 16 + 8 * half));
    if (w_vec) {  // uniform: runs of 4 heads are whole, w aligned to 4 weights
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int oh0 = mb * 32 + 8 * j + 4 * half;
        const f32x4 v = load_w4<WT>(w, t * H + (oh0 < H ? oh0 : 0));
#pragma unroll
        for (int c = 0; c < 4; ++c) wv[mb][4 * j + c] = v[c];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int oh = mb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
        wv[mb][i] = load_w<WT>(w, t * H + (oh < H ? oh : 0));
      }
    }
  }
  if (!live || 32 * MB > H) {  // uniform per wave: zero what is past the row or the heads
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int head = mb * 32 + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        if (!live || head >= H) qa[mb][ks] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int oh = mb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
        if (!live || oh >= H) wv[mb][i] = 0.0f;
      }
    }
  }

  // Every prologue load (the first tile, then the query and the weights) is
  // complete before the tile loop. Left to the compiler, the waits for the
  // query fragments land inside the loop, where their counts then also wait
  // for the next tile's prefetch on every iteration.
  wait_vmcnt0();
  store_tile(0);
  __syncthreads();
  // CAND: the sample tiles are scored once; the tile loop skips them and
  // appends their saved keys in their place. Sample tile 0 is the range's
  // first tile, the others are at least 8 tiles apart (a sampling workgroup
  // has more than 64 tiles).
  uint32_t* const wsamp = s_samp + (CAND ? wave * 2 * kSampleTiles * 64 + lane : 0);
  auto append_saved = [&](int i) {
#pragma unroll
    for (int hp = 0; hp < 2; ++hp)
      append(wsamp[64 * (2 * i + hp)],
             (uint32_t)(sample_start(i) + kIdxHalf * hp + lane - qstart));
  };
  if constexpr (CAND) {
    if (sample) {  // uniform
      // The sample tiles go through the ring in turn (the last prefetch is
      // the tile loop's first tile, the one after sample tile 0, which lands
      // in buffer 0); lane l keeps the scores of keys s + l and s + 64 + l of
      // each sample tile s in the wave's LDS slots.
      static_assert(TILE == 2 * kIdxHalf && NBUF == 2 && kSampleTiles % 2 == 0, "sample layout");
#pragma unroll 1
      for (int i = 0; i < kSampleTiles; ++i) {
        load_tile(i + 1 < kSampleTiles ? sample_start(i + 1) : kb + TILE);
        const unsigned char* kt = ktile + (i & 1) * TILE_B;
        const int32_t s0 = sample_start(i);
#pragma unroll
        for (int hp = 0; hp < 2; ++hp) {
          block_mfma(kt, 2 * hp, acc0);
          block_mfma(kt, 2 * hp + 1, acc1);
          const float score = halfwave_sums(epilogue(acc0), epilogue(acc1));
          const uint32_t j = (uint32_t)(s0 + kIdxHalf * hp + lane - qstart);
          // (invalid: all-ones bits, whose key is 0)
          wsamp[64 * (2 * i + hp)] = j < (uint32_t)qlen ? __float_as_uint(score) : 0xffffffffu;
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
        uint32_t samp[2 * kSampleTiles];
#pragma unroll
        for (int i = 0; i < 2 * kSampleTiles; ++i)
          samp[i] = fused_key(__uint_as_float(wsamp[64 * i]));
        uint32_t nv = 0u;
#pragma unroll
        for (int i = 0; i < 2 * kSampleTiles; ++i) nv += samp[i] != 0u ? 1u : 0u;
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
            for (int i = 0; i < 2 * kSampleTiles; ++i) n_ge += samp[i] >= c ? 1u : 0u;
            if (wave_sum_u32(n_ge) >= rank) v = c;
          }
          t_lo = v == fused_key(0.0f) ? -1 : ord(__float_as_uint(fused_value(v)));
        }
      }
      append_saved(0);
    }
  }
  int buf = 0;
  int32_t pend_k0 = qstart - 64;  // the second block of the pair at pend_k0 awaits its epilogue
  float pend_p0 = 0.0f;           // its block-0 partial
  int ns = 1;                     // CAND: the next sample tile the loop has not passed
  int32_t ns_start = sample ? sample_start(1) : INT32_MAX;
  for (int32_t k0 = sample ? kb + TILE : kb; k0 < ke;) {
    int32_t k_next = k0 + TILE;
    if constexpr (CAND)
      if (k_next == ns_start) k_next += TILE;  // uniform
    load_tile(k_next);  // zeroed past the range, so the last one is harmless
    const unsigned char* kt = ktile + buf * TILE_B;
    // Each group pairs a block's MFMAs with the previous block's epilogue;
    // the fences keep the scheduler from filling the VALU slots with the
    // epilogue that waits on these very MFMAs. A tile is two or four blocks
    // of 32 keys, taken in pairs; a pair wholly past the range is skipped.
    auto pair = [&](int hp) {
      block_mfma(kt, 2 * hp, acc0);
      const float p1_prev = epilogue(acc1);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      write_scores(pend_k0, pend_p0, p1_prev);
      block_mfma(kt, 2 * hp + 1, acc1);
      pend_p0 = epilogue(acc0);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      pend_k0 = k0 + kIdxHalf * hp;
    };
    if constexpr (TILE == kIdxHalf) {
      pair(0);
    } else {
#pragma unroll
      for (int hp = 0; hp < TILE / kIdxHalf; ++hp) {
        if (hp > 0 && k0 + kIdxHalf * hp >= ke) break;  // uniform
        pair(hp);
      }
    }

    if constexpr (CAND) {
      if (k0 + TILE == ns_start) {  // uniform: a sample tile comes next
        write_scores(pend_k0, pend_p0, epilogue(acc1));
        append_saved(ns);
        pend_k0 = qstart - 64;  // the next tile's first pending write is dropped
        ++ns;
        ns_start = ns < kSampleTiles ? sample_start(ns) : INT32_MAX;
      }
    }

    if constexpr (NBUF == 2) {
      store_tile(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    } else {
      __syncthreads();  // every wave is done with the tile
      store_tile(0);
      __syncthreads();
    }
    k0 = k_next;
  }
  write_scores(pend_k0, pend_p0, epilogue(acc1));
  if constexpr (CAND)
    if (live && lane == 0) ca.count[r] = (int32_t)n_cand;
  if constexpr (FUSE) {
    __syncthreads();  // the tile ring is free: it holds the select histograms now
    if (live)
      wave_topk_row(lrow, qlen, row_starts[t], reinterpret_cast<uint32_t*>(ktile) + 256 * wave,
                    fa, r);
  }
}

// Rescue pass of the combined path for long rows: the rows whose candidate
// list could not hold their top k (too few or too many candidates, queued by
// stage 2). Workgroup g takes queued rows g, g + G, ... (G workgroups); for
// each it recomputes the row's dense scores into its own spill row, with the
// arithmetic of the indexer pass (per 32-key block the MFMA chain over the
// head dim from zero, the ReLU * weight chain over the heads in the same
// order, the same half-wave sum, so every score is bit-identical to the
// pass's), then selects exactly from them: theta by radix passes over the
// row, then each thread counts its run of columns above and equal to theta
// and, after a scan of the counts, places its selected columns.
template <int D, int MB, typename WT>
__global__ __launch_bounds__(kIdxWaves * 64) void indexer_rescue_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const WT* __restrict__ w,
    const int32_t* __restrict__ row_starts, const int32_t* __restrict__ seq_lens, int64_t T_kv,
    int H, int64_t row_begin, int64_t n_cols, FusedArgs fa, CandArgs ca, bool w_vec) {
  constexpr int KS = D / 16;
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t s_wave[kIdxWaves];
  __shared__ uint32_t s_sel[2];
  __shared__ float s_fsum[kIdxWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
  const uint32_t n_queued = *ca.n_queued;
  float* const spill = ca.spill + (int64_t)blockIdx.x * ca.spill_ld;
  const int64_t col_cap = T_kv > 0 ? n_cols : 0;

  for (uint32_t qi = blockIdx.x; qi < n_queued; qi += gridDim.x) {
    const int64_t r = ca.queue[qi];
    const int64_t t = row_begin + r;
    const int32_t s0 = row_starts[t];
    const int n = (int)max((int64_t)0, min((int64_t)seq_lens[t], col_cap));

    // Query fragments and weights as the indexer pass loads them.
    u32x4 qa[MB][KS];
    float wv[MB][16];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int head = mb * 32 + (lane & 31);
      const int hq = head < H ? head : H - 1;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qa[mb][ks] = head < H ? load16(q + ((t * H + hq) * D + ks * 16 + 8 * half))
                              : u32x4{0u, 0u, 0u, 0u};
      if (w_vec) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int oh0 = mb * 32 + 8 * j + 4 * half;
          const f32x4 v = load_w4<WT>(w, t * H + (oh0 < H ? oh0 : 0));
#pragma unroll
          for (int c = 0; c < 4; ++c) wv[mb][4 * j + c] = oh0 + c < H ? v[c] : 0.0f;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int oh = mb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
          wv[mb][i] = oh < H ? load_w<WT>(w, t * H + oh) : 0.0f;
        }
      }
    }
    // Scores of keys s0 + 64 g + [0, 64) by wave g % 8: block 0 holds keys
    // [0, 32), block 1 keys [32, 64) of the group.
    for (int g = wave; 64 * g < n; g += kIdxWaves) {
      float p[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        // (keys outside [0, T_kv) score 0, as the indexer pass zeroes them)
        const int col = 64 * g + 32 * nb + (lane & 31);
        const int64_t key = (int64_t)s0 + col;
        const bool ok = col < n && key >= 0 && key < T_kv;
        u32x4 kf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          kf[ks] = load16(k + (ok ? key : 0) * D + ks * 16 + 8 * half);
          if (!ok) kf[ks] = u32x4{0u, 0u, 0u, 0u};
        }
        f32x16 acc[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            acc[mb] = mfma32x32x16(qa[mb][ks], kf[ks], ks == 0 ? f32x16{} : acc[mb]);
        float s = 0.0f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) s = fmaf(wv[mb][i], relu(acc[mb][i]), s);
        p[nb] = s;
      }
      const float score = halfwave_sums(p[0], p[1]);
      if (64 * g + lane < n) spill[64 * g + lane] = score;
    }
    __syncthreads();  // the spill row is complete

    select_spill_row<kIdxWaves>(spill, n, s0, fa, r, hist, s_wave, s_sel, s_fsum);
  }
}

template <int D, int MB, int MODE>
hipError_t launch_indexer_w(const void* q, const void* k, const void* w, int w_dtype,
                            const int32_t* rs, const int32_t* sl, int64_t T_kv, int H,
                            int64_t row_begin, int64_t n_rows, float* scores, int64_t ld,
                            const FusedArgs& fa, const CandArgs& ca, hipStream_t st) {
  const int64_t nblk = (n_rows + kIdxWaves - 1) / kIdxWaves;
  dim3 grid((unsigned)nblk), block(kIdxWaves * 64);
  // Four weights per load when every run of four heads starts at a multiple
  // of four weights from an address aligned to four weights; otherwise one
  // weight per load (w only needs its element alignment).
  const size_t wbytes = w_dtype == 0 ? 2 : 4;
  const bool w_vec = H % 4 == 0 && (uintptr_t)w % (4 * wbytes) == 0;
  if (w_dtype == 0)
    hipLaunchKernelGGL((indexer_kernel<D, MB, uint16_t, MODE>), grid, block, 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)w, rs, sl, T_kv, H,
                       row_begin, n_rows, scores, ld, fa, ca, w_vec);
  else
    hipLaunchKernelGGL((indexer_kernel<D, MB, float, MODE>), grid, block, 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const float*)w, rs, sl, T_kv, H,
                       row_begin, n_rows, scores, ld, fa, ca, w_vec);
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

hipError_t launch_ratio_metadata(const int32_t* cu_q, const int32_t* cu_k, const int32_t* offsets,
                                 int32_t n_seq, int64_t T_q, int32_t ratio, int32_t* rs,
                                 int32_t* sl, hipStream_t st) {
  if (T_q == 0) return hipSuccess;
  dim3 grid((unsigned)((T_q + 255) / 256)), block(256);
  hipLaunchKernelGGL(ratio_metadata_kernel, grid, block, 0, st, cu_q, cu_k, offsets, n_seq, T_q,
                     ratio, rs, sl);
  return hipGetLastError();
}

hipError_t launch_indexer(const void* q, const void* k, const void* w, int w_dtype,
                          const int32_t* rs, const int32_t* sl, int64_t T_kv, int H, int D,
                          int64_t row_begin, int64_t n_rows, float* scores, int64_t ld,
                          hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  const int mb = (H + 31) / 32;
  const FusedArgs none{};
#define DSA_IDX_CASE(DD, MM)                                                                  \
  if (D == DD && mb == MM)                                                                    \
    return launch_indexer_w<DD, MM, kModeScores>(q, k, w, w_dtype, rs, sl, T_kv, H,          \
                                                 row_begin, n_rows, scores, ld, none, CandArgs{}, \
                                                 st);
  DSA_IDX_CASE(128, 1) DSA_IDX_CASE(128, 2) DSA_IDX_CASE(64, 1) DSA_IDX_CASE(64, 2)
#undef DSA_IDX_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_indexer_topk(const void* q, const void* k, const void* w, int w_dtype,
                               const int32_t* rs, const int32_t* sl, int64_t T_kv, int H, int D,
                               int64_t row_begin, int64_t n_rows, int64_t n_cols,
                               const FusedArgs& fa, hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  const int mb = (H + 31) / 32;
#define DSA_IDX_CASE(DD, MM)                                                                 \
  if (D == DD && mb == MM)                                                                   \
    return launch_indexer_w<DD, MM, kModeFused>(q, k, w, w_dtype, rs, sl, T_kv, H, row_begin, \
                                                n_rows, nullptr, n_cols, fa, CandArgs{}, st);
  DSA_IDX_CASE(128, 1) DSA_IDX_CASE(128, 2) DSA_IDX_CASE(64, 1) DSA_IDX_CASE(64, 2)
#undef DSA_IDX_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_indexer_cand(const void* q, const void* k, const void* w, int w_dtype,
                               const int32_t* rs, const int32_t* sl, int64_t T_kv, int H, int D,
                               int64_t row_begin, int64_t n_rows, int64_t n_cols, int top_k,
                               const CandArgs& ca, hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  const int mb = (H + 31) / 32;
  FusedArgs fa{};
  fa.k = top_k;
#define DSA_IDX_CASE(DD, MM)                                                                 \
  if (D == DD && mb == MM)                                                                   \
    return launch_indexer_w<DD, MM, kModeCand>(q, k, w, w_dtype, rs, sl, T_kv, H, row_begin, \
                                               n_rows, nullptr, n_cols, fa, ca, st);
  DSA_IDX_CASE(128, 1) DSA_IDX_CASE(128, 2) DSA_IDX_CASE(64, 1) DSA_IDX_CASE(64, 2)
#undef DSA_IDX_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_indexer_rescue(const void* q, const void* k, const void* w, int w_dtype,
                                 const int32_t* rs, const int32_t* sl, int64_t T_kv, int H, int D,
                                 int64_t row_begin, int64_t n_rows, int64_t n_cols,
                                 const FusedArgs& fa, const CandArgs& ca, hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  const int mb = (H + 31) / 32;
  dim3 grid((unsigned)std::min<int64_t>(ca.n_spill, n_rows)), block(kIdxWaves * 64);
  const size_t wbytes = w_dtype == 0 ? 2 : 4;
  const bool w_vec = H % 4 == 0 && (uintptr_t)w % (4 * wbytes) == 0;
#define DSA_RESCUE_CASE(DD, MM)                                                               \
  if (D == DD && mb == MM) {                                                                  \
    if (w_dtype == 0)                                                                         \
      hipLaunchKernelGGL((indexer_rescue_kernel<DD, MM, uint16_t>), grid, block, 0, st,       \
                         (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)w, rs, sl,  \
                         T_kv, H, row_begin, n_cols, fa, ca, w_vec);                          \
    else                                                                                      \
      hipLaunchKernelGGL((indexer_rescue_kernel<DD, MM, float>), grid, block, 0, st,          \
                         (const uint16_t*)q, (const uint16_t*)k, (const float*)w, rs, sl,     \
                         T_kv, H, row_begin, n_cols, fa, ca, w_vec);                          \
    return hipGetLastError();                                                                 \
  }
  DSA_RESCUE_CASE(128, 1) DSA_RESCUE_CASE(128, 2) DSA_RESCUE_CASE(64, 1) DSA_RESCUE_CASE(64, 2)
#undef DSA_RESCUE_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsa
