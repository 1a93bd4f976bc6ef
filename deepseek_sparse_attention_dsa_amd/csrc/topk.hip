// Per-row top-K with per-row length, ordered compaction and local -> global
// conversion, for gfx950.
//
// Semantics: cuDNN Frontend DSA page, section 5 "Indexer Top-K" (radix top-K
// with a per-row effective length, top_k <= 2048) and section 4 (the
// deterministic tie-break: exact ties at the K-th boundary go to the smallest
// column); NeMo cudnn_dsa page (global coordinates, ascending valid prefix,
// -1 suffix).
//
// One workgroup per row; workgroups take the rows in reverse order, so a
// causal sequence's long rows (the ones that need a selection) start first
// and the short closed-form rows fill the tail.
//
// Scores become order-preserving uint32 keys (-0.0 folded onto +0.0, so they
// tie as equal values; key 0 marks columns past the row end). Output
// positions come from one rule: a selected column goes to
// (#greater before it) + min(#equal before it, #equal taken).
//
// Rows of up to 8192 columns (topk_radix_kernel): one workgroup (four waves
// from 1025 columns up, eight from 4097) keeps the row in VGPRs, counts its
// keys into 2048 buckets linear in the score between the row's extremes,
// ranks the few members of the bucket holding the K-th largest key exactly to
// find theta (radix passes over 11/11/10-bit digits when a bucket holds more
// than 64), then places the selected columns in ascending order from
// per-lane counts scanned on DPP lane moves.
//
// Longer rows (topk_stream_kernel) are streamed once and never held on chip,
// so several rows share a CU and one row's loads overlap another's work:
//  1. Sampled lower bound lo: 64 runs of 64 contiguous columns spread over
//     the row (4096 samples); lo is the sample of rank e + 4 sqrt(e) + 2 from
//     the top, e = K * 4096 / n being the expected rank of the K-th largest
//     key, i.e. about 4 standard deviations of the sampling noise above it.
//     Rows of at most kCap columns take every column as a candidate.
//  2. One streaming pass compares every score with lo and appends the
//     columns at or above it, chunk by chunk (256 columns per wave load), to
//     an LDS candidate list: wave w takes chunks w, w + 4, ... and appends to
//     its own quarter of the list with a counter in a register (no shared
//     counter); a direct-mapped table of chunks records where each chunk's
//     candidates went, which restores column order later. If fewer than K
//     columns pass, or more than a quarter's kCap / 4 in some wave, the row
//     is redone with radix passes that re-stream it (correct for any input,
//     slow).
//  3. theta among the candidates: a histogram over 2048 buckets linear in
//     the score value between lo and the largest candidate (dense score
//     ranges spread over many bins instead of piling onto a few exponent
//     digits), then an exact rank inside the bucket holding the K-th largest
//     (one wave when it has at most 64 members, radix passes otherwise).
//  4. Output: a scan of the chunk counts gives each chunk's first position
//     in column order; every thread takes an equal share of the positions
//     (its first chunk by binary search), counts the keys above and equal to
//     theta, and after a scan of those counts places its selected keys,
//     staged in LDS for 16-byte stores when no values are written.
#include "dsa.h"
#include "dsa_device.h"
#include "dsa_launch.h"
#include "dsa_rowsel.h"

namespace dsa {
namespace {

// ------------------------------------------------ rows of <= 8192 columns --
// CH: 4-column chunks per lane, held in VGPRs. Wave w owns the columns
// [w * 256 * CH, (w + 1) * 256 * CH); chunk c of a wave covers 256
// consecutive columns, 4 per lane.
//
// CAND: stage 2 of the combined indexer + top-k for long rows (DSA page
// section 4). The row is not a score row but its candidate list from the
// indexer pass: (score, local column) pairs in column order,
// every column whose score reached the row's lower bound. The list holds the
// row's top k when it has between k and cap entries (or, for a row of at most
// k columns, all of them); any other row is queued for the rescue pass and
// left alone here. The selected scores, their softmax and its log-sum-exp
// are written as well.
struct CandSel {
  const uint32_t* cand;  // [n_rows, cap] (score bits, local column) pairs
  int64_t cap;           // = 64 * WAVES * 4 * CH
  const int32_t* count;  // [n_rows] candidates found (may exceed cap)
  int32_t* queue;        // [n_rows] rows left to the rescue pass
  uint32_t* n_queued;    // their number (zeroed by the indexer pass)
  float* soft;           // [n_rows, ld_idx] or null
  float* lse;            // [n_rows] or null
};

// (CAND: six waves per SIMD, three workgroups per CU, hide the list loads)
template <int WAVES, int CH, bool CAND>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(CAND ? 6 : 1)))
void topk_radix_kernel(
    const float* __restrict__ scores, int64_t ld, int64_t n_cols,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ row_starts, int k,
    int32_t* __restrict__ indices, int64_t ld_idx, int32_t* __restrict__ topk_length,
    float* __restrict__ values, CandSel cs) {
  constexpr int NT = 64 * WAVES;
  constexpr float kLog2e = 1.4426950408889634f;
  static_assert(kBins % NT == 0, "bins must split evenly over threads");
  __shared__ uint32_t hist[kBins + 64];  // + a spare output slot per lane
  __shared__ uint32_t s_wave[2][WAVES > 1 ? WAVES : 1];
  __shared__ float s_fsum[WAVES];
  __shared__ uint32_t s_sel[2];
  __shared__ uint32_t s_mem[64];
  __shared__ uint32_t s_cnt;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t r = (int64_t)gridDim.x - 1 - blockIdx.x;  // long rows first
  const float* row = CAND ? nullptr : scores + r * ld;
  int32_t* out_idx = indices + r * ld_idx;
  float* out_val = values ? values + r * ld_idx : nullptr;
  int64_t n64 = seq_lens[r];
  n64 = n64 < 0 ? 0 : (n64 > n_cols ? n_cols : n64);
  const int n = (int)n64;
  const int32_t base = row_starts ? row_starts[r] : 0;
  float* out_soft = nullptr;
  const uint32_t* crow = nullptr;
  int nsel = n;  // entries to select from
  if constexpr (CAND) {
    out_soft = cs.soft ? cs.soft + r * ld_idx : nullptr;
    crow = cs.cand + 2 * r * cs.cap;
    const int32_t c = cs.count[r];
    if (n <= k ? c != n : (c < k || c > cs.cap)) {  // uniform
      if (tid == 0) cs.queue[atomicAdd(cs.n_queued, 1u)] = (int32_t)r;
      return;
    }
    nsel = c;
  }
  // Sum over the workgroup of one float per thread.
  auto block_sum = [&](float v) -> float {
    v = wave_sum_f32(v);
    if (WAVES == 1) return v;
    if (lane == 0) s_fsum[wave] = v;
    __syncthreads();
    v = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) v += s_fsum[w];
    __syncthreads();
    return v;
  };

  if (CAND && n <= k) {
    // Every column is selected, in the list's (column) order.
    uint32_t kmax = 0u;
    for (int i = tid; i < nsel; i += NT) kmax = max(kmax, float_to_key(__uint_as_float(crow[2 * i])));
    kmax = block_max<WAVES>(kmax, s_wave[0]);
    const float vmax = key_to_float(kmax);
    float s = 0.0f;
    for (int i = tid; i < nsel; i += NT)
      s += __builtin_amdgcn_exp2f((key_to_float(float_to_key(__uint_as_float(crow[2 * i]))) - vmax) *
                                  kLog2e);
    const float ssum = block_sum(s);
    const float lse = nsel ? vmax + __logf(ssum) : __builtin_inff();
    for (int i = tid; i < k; i += NT) {
      const float v =
          i < nsel ? key_to_float(float_to_key(__uint_as_float(crow[2 * i]))) : -__builtin_inff();
      out_idx[i] = i < nsel ? base + (int32_t)crow[2 * i + 1] : -1;
      if (out_val) out_val[i] = v;
      if (out_soft) out_soft[i] = i < nsel ? __builtin_amdgcn_exp2f((v - lse) * kLog2e) : 0.0f;
    }
    if (tid == 0) {
      if (topk_length) topk_length[r] = nsel;
      if (cs.lse) cs.lse[r] = lse;
    }
    return;
  }
  if (!CAND && n <= k) {
    // Every causal column is selected; no select needed.
    if (!out_val && (k & 3) == 0 && ((uintptr_t)out_idx & 15u) == 0) {
      // 16-byte stores of four consecutive slots
      for (int i = 4 * tid; i < k; i += 4 * NT)
        *reinterpret_cast<i32x4*>(out_idx + i) =
            i32x4{i + 0 < n ? base + i + 0 : -1, i + 1 < n ? base + i + 1 : -1,
                  i + 2 < n ? base + i + 2 : -1, i + 3 < n ? base + i + 3 : -1};
    } else {
      for (int i = tid; i < k; i += NT) {
        out_idx[i] = i < n ? base + i : -1;
        if (out_val) out_val[i] = i < n ? row[i] : -__builtin_inff();
      }
    }
    if (tid == 0 && topk_length) topk_length[r] = n;
    return;
  }

  // All loads are issued before any is used. Every load is a full 16-byte
  // chunk inside the row's ld columns (ld is a multiple of 4 and >= n):
  // chunks past the row read a clamped address and columns >= n become key 0.
  // CAND: the entries are read as two 16-byte (key, column) pairs per lane
  // and chunk, inside the row's cap entries; entries >= nsel become key 0.
  const int wbase = wave * 256 * CH;
  float4 raw[CAND ? 1 : CH];  // the scores (CAND: formed from the keys where used)
  u32x4 kreg[CH];
  u32x2 creg[CAND ? CH : 1];  // CAND: the entries' columns, two 16-bit ones per word
  if constexpr (CAND) {
    u32x4 pr[CH][2];  // only the filled entries are read
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int e0 = wbase + c * 256 + lane * 4 + 2 * h;
        pr[c][h] = e0 < nsel ? *reinterpret_cast<const u32x4*>(crow + 2 * e0) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int col = wbase + c * 256 + lane * 4;
      kreg[c] = u32x4{col + 0 < nsel ? float_to_key(__uint_as_float(pr[c][0][0])) : 0u,
                      col + 1 < nsel ? float_to_key(__uint_as_float(pr[c][0][2])) : 0u,
                      col + 2 < nsel ? float_to_key(__uint_as_float(pr[c][1][0])) : 0u,
                      col + 3 < nsel ? float_to_key(__uint_as_float(pr[c][1][2])) : 0u};
      creg[c] = u32x2{(pr[c][0][1] & 0xffffu) | (pr[c][0][3] << 16),
                      (pr[c][1][1] & 0xffffu) | (pr[c][1][3] << 16)};
    }
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int col = wbase + c * 256 + lane * 4;
      const int64_t colc = col < ld - 4 ? (int64_t)col : ld - 4;
      raw[c] = *reinterpret_cast<const float4*>(row + colc);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int col = wbase + c * 256 + lane * 4;
      kreg[c] = u32x4{col + 0 < n ? float_to_key(raw[c].x) : 0u, col + 1 < n ? float_to_key(raw[c].y) : 0u,
                      col + 2 < n ? float_to_key(raw[c].z) : 0u, col + 3 < n ? float_to_key(raw[c].w) : 0u};
    }
  }

  // theta: one histogram over kBins buckets linear in the score between the
  // row's smallest and largest valid scores (monotone in the key), then the
  // members of the bucket holding the k-th largest key are ranked exactly:
  // by one wave when there are at most 64 of them, else by radix passes
  // restricted to the bucket (heavy ties, infinite scores). Wave-wide
  // reductions and scans run on DPP lane moves; the waves meet in LDS.
  uint32_t kmax = 0u, knmax = 0u;
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = kreg[c][e];
      kmax = max(kmax, key);
      knmax = max(knmax, key != 0u ? ~key : 0u);
    }
  kmax = wave_max_u32(kmax);
  knmax = wave_max_u32(knmax);
  for (int i = tid; i < kBins; i += NT) hist[i] = 0u;
  if (tid == 0) s_cnt = 0u;
  if (WAVES > 1 && lane == 0) {
    s_wave[0][wave] = kmax;
    s_wave[1][wave] = knmax;
  }
  __syncthreads();
  if (WAVES > 1) {
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      kmax = max(kmax, s_wave[0][w]);
      knmax = max(knmax, s_wave[1][w]);
    }
  }
  const float flo = key_to_float(~knmax), span = key_to_float(kmax) - flo;
  const LinearBuckets lb{flo, span > 0.0f ? (float)kBins / span : 0.0f};
  // bucket of entry (c, e): stored, or (CAND, fewer registers) formed again
  uint16_t bk[CAND ? 1 : CH][4];
  auto bucket = [&](int c, int e) -> uint32_t {
    if constexpr (CAND) return (uint32_t)lb.of_value(key_to_float(kreg[c][e]));
    else return bk[c][e];
  };
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (!CAND) bk[c][e] = (uint16_t)lb.of_value(raw[c][e]);
      if (kreg[c][e] != 0u) atomicAdd(&hist[bucket(c, e)], 1u);
    }
  __syncthreads();
  find_bucket<WAVES>(hist, (uint32_t)k, s_wave[0], s_sel);
  const uint32_t bstar = s_sel[0];
  const uint32_t rem = (uint32_t)k - s_sel[1];  // >= 1 keys to take from bucket bstar
  // members of bucket bstar into a small list (order does not matter here)
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool mem = kreg[c][e] != 0u && bucket(c, e) == bstar;
      const uint64_t bal = ballot(mem);
      if (bal != 0u) {  // uniform
        uint32_t at = 0u;
        if (lane == 0) at = atomicAdd(&s_cnt, (uint32_t)__popcll(bal));
        at = (uint32_t)__builtin_amdgcn_readlane((int)at, 0) + popc_below(bal);
        if (mem && at < 64u) s_mem[at] = kreg[c][e];
      }
    }
  __syncthreads();
  const uint32_t m = s_cnt;
  uint32_t theta, need_eq;
  if (m <= 64u) {  // uniform
    if (wave == 0) {
      const uint32_t x = lane < (int)m ? s_mem[lane] : 0u;
      uint32_t gt = 0u, eq = 0u;
      for (uint32_t j = 0; j < m; ++j) {  // member j broadcast from lane j
        const uint32_t y = (uint32_t)__builtin_amdgcn_readlane((int)x, (int)j);
        gt += y > x;
        eq += y == x;
      }
      if (lane < (int)m && gt < rem && rem <= gt + eq) {  // equal members write equal values
        s_sel[0] = x;
        s_sel[1] = rem - gt;
      }
    }
    __syncthreads();
    theta = s_sel[0];
    need_eq = s_sel[1];
  } else {
    theta = radix_select<WAVES>(rem, hist, s_wave[0], s_sel, &need_eq, [&](auto&& f) {
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (kreg[c][e] != 0u && bucket(c, e) == bstar) f(kreg[c][e]);
    });
  }

  // CAND: the softmax normaliser of the selected set (every key above theta
  // and need_eq keys equal to it), as the on-chip combined path forms it.
  float lse = 0.0f;
  if (CAND && (out_soft || cs.lse)) {  // uniform
    const float vmax = key_to_float(kmax);
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (kreg[c][e] > theta)
          s += __builtin_amdgcn_exp2f((key_to_float(kreg[c][e]) - vmax) * kLog2e);
    float ssum = block_sum(s);
    if (need_eq)
      ssum += (float)need_eq * __builtin_amdgcn_exp2f((key_to_float(theta) - vmax) * kLog2e);
    lse = vmax + __logf(ssum);
  }

  // Output positions follow column order (wave, chunk, lane, element). Per
  // chunk, each lane counts its keys above and equal to theta, packed as
  // (above | equal << 16) (both < 2^16), and the wave scans the packed counts
  // over its lanes; the waves' totals meet in LDS.
  uint32_t excl[CH], chunk_base[CH];
  uint32_t wave_tot = 0u;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    uint32_t p = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      p += (kreg[c][e] > theta ? 1u : 0u) + (kreg[c][e] == theta ? 0x10000u : 0u);
    const uint32_t incl = wave_incl_scan_dpp(p, [](uint32_t a, uint32_t b) { return a + b; }, 0u);
    excl[c] = incl - p;
    chunk_base[c] = wave_tot;
    wave_tot += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  }
  uint32_t wave_base = 0u;
  if (WAVES > 1) {
    __syncthreads();  // every wave has read theta from s_sel and left the scans of s_wave
    if (lane == 0) s_wave[1][wave] = wave_tot;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < WAVES; ++w) wave_base += w < wave ? s_wave[1][w] : 0u;
  }
  // Without values and with 16-byte aligned output rows, the k slots are
  // staged in LDS (the histogram is free now; k <= kBins; unselected columns
  // write a spare slot of their lane) and leave in 16-byte stores; otherwise
  // they are written in place.
  const bool staged =
      !out_val && !out_soft && (k & 3) == 0 && ((uintptr_t)out_idx & 15u) == 0;  // uniform
  if (staged) __syncthreads();  // the histogram's last readers are done
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    uint32_t cnt = wave_base + chunk_base[c] + excl[c];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = kreg[c][e];
      const bool is_gt = key > theta, is_eq = key == theta;
      const uint32_t ng = cnt & 0xffffu, nq = cnt >> 16;
      const uint32_t pos = ng + min(nq, need_eq);
      const bool take = (is_gt || (is_eq && nq < need_eq)) && pos < (uint32_t)k;
      const int32_t gcol =
          base + (CAND ? (int32_t)((creg[c][e >> 1] >> (16 * (e & 1))) & 0xffffu)
                       : wbase + c * 256 + lane * 4 + e);
      if (staged) {
        hist[take ? pos : (uint32_t)(kBins + lane)] = (uint32_t)gcol;
      } else if (take) {
        out_idx[pos] = gcol;
        if (out_val) out_val[pos] = key_to_float(key);
        if (out_soft) out_soft[pos] = __builtin_amdgcn_exp2f((key_to_float(key) - lse) * kLog2e);
      }
      cnt += (is_gt ? 1u : 0u) + (is_eq ? 0x10000u : 0u);
    }
  }
  if (staged) {
    __syncthreads();
    for (int i = 4 * tid; i < k; i += 4 * NT)
      *reinterpret_cast<u32x4*>(out_idx + i) = *reinterpret_cast<const u32x4*>(hist + i);
  }
  if (tid == 0) {
    if (topk_length) topk_length[r] = k;
    if (CAND && cs.lse) cs.lse[r] = lse;
  }
}

// ------------------------------------------------- rows of > 8192 columns --
constexpr int kSWaves = 4;
constexpr int kSThreads = 64 * kSWaves;
constexpr int kMaxChunks = 65536 / 256;  // 256-column chunks of the longest row
constexpr int kCap = 4096;               // candidate list capacity
constexpr int kWaveCap = kCap / kSWaves;  // ... in each wave's quarter
constexpr int kBatch = 8;                // chunk loads in flight per wave
static_assert(kMaxChunks == kSThreads, "one thread per chunk in the output walk");
static_assert(kBins >= DSA_MAX_TOPK, "the histogram holds the staged output of a row");

__global__ __launch_bounds__(kSThreads) void topk_stream_kernel(
    const float* __restrict__ scores, int64_t ld, int64_t n_cols,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ row_starts, int k,
    int32_t* __restrict__ indices, int64_t ld_idx, int32_t* __restrict__ topk_length,
    float* __restrict__ values) {
  constexpr int NT = kSThreads;
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t s_ckey[kCap];
  __shared__ uint8_t s_ccol[kCap];         // column within its 256-column chunk
  __shared__ uint16_t s_cbase[kMaxChunks];  // chunk -> first candidate slot
  __shared__ uint16_t s_ccnt[kMaxChunks + 1];  // chunk -> candidate count, later its start
  __shared__ uint32_t s_wave[kSWaves];
  __shared__ uint32_t s_red[kSWaves];
  __shared__ uint32_t s_sel[2];
  __shared__ uint32_t s_wcnt[kSWaves];     // candidates of each wave's quarter

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t r = (int64_t)gridDim.x - 1 - blockIdx.x;  // long rows first
  const float* row = scores + r * ld;
  int32_t* out_idx = indices + r * ld_idx;
  float* out_val = values ? values + r * ld_idx : nullptr;
  int64_t n64 = seq_lens[r];
  n64 = n64 < 0 ? 0 : (n64 > n_cols ? n_cols : n64);
  const int n = (int)n64;
  const int32_t base = row_starts ? row_starts[r] : 0;

  if (n <= k) {
    if (!out_val && (k & 3) == 0 && ((uintptr_t)out_idx & 15u) == 0) {
      for (int i = 4 * tid; i < k; i += 4 * NT)
        *reinterpret_cast<i32x4*>(out_idx + i) =
            i32x4{i + 0 < n ? base + i + 0 : -1, i + 1 < n ? base + i + 1 : -1,
                  i + 2 < n ? base + i + 2 : -1, i + 3 < n ? base + i + 3 : -1};
    } else {
      for (int i = tid; i < k; i += NT) {
        out_idx[i] = i < n ? base + i : -1;
        if (out_val) out_val[i] = i < n ? row[i] : -__builtin_inff();
      }
    }
    if (tid == 0 && topk_length) topk_length[r] = n;
    return;
  }
  const int nchunks = (n + 255) / 256;

  // the bucket holding the want-th largest of the histogrammed keys:
  // s_sel[0] = bucket, s_sel[1] = count in the buckets above it
  auto find_bucket_s = [&](uint32_t want) { find_bucket<kSWaves>(hist, want, s_wave, s_sel); };

  // The streaming pass's first batch is requested now, so that its loads
  // are in flight while the sample is taken.
  float4 v[kBatch];
  auto load_batch = [&](int c0) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int ch = c0 + kSWaves * i;
      const int64_t col = ch < nchunks ? (int64_t)ch * 256 + lane * 4 : 0;
      const int64_t colc = col < ld - 4 ? col : ld - 4;
      v[i] = *reinterpret_cast<const float4*>(row + colc);
    }
  };
  load_batch(wave);

  // ---- 1. sampled lower bound (rows of more than kCap columns) ----
  uint32_t lo_key = 1u;  // the smallest valid key: every column is a candidate
  if (n > kCap) {        // uniform; n > kCap >= 64 keeps every run inside the row
    constexpr int S = 4096;  // 64 runs x 64 columns; n > 4096 keeps runs apart
    const float e = (float)k * (float)S / (float)n;
    const int rank = (int)ceilf(e + 4.0f * sqrtf(e) + 2.0f);
    uint32_t skey[16];
    uint32_t smax = 0, snmax = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = (tid >> 4) + 16 * j;  // run 0..63
      const int64_t start = ((int64_t)q * (n - 64) / 63) & ~(int64_t)3;
      const float4 v = *reinterpret_cast<const float4*>(row + start + 4 * (tid & 15));
      skey[4 * j + 0] = float_to_key(v.x);
      skey[4 * j + 1] = float_to_key(v.y);
      skey[4 * j + 2] = float_to_key(v.z);
      skey[4 * j + 3] = float_to_key(v.w);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      smax = max(smax, skey[i]);
      snmax = max(snmax, ~skey[i]);
    }
    smax = block_max<kSWaves>(smax, s_red);
    const uint32_t smin = ~block_max<kSWaves>(snmax, s_red);
    const float flo = key_to_float(smin), span = key_to_float(smax) - flo;
    const LinearBuckets sb{flo, span > 0.0f ? (float)kBins / span : 0.0f};
    for (int i = tid; i < kBins; i += NT) hist[i] = 0u;
    if (tid == 0) s_red[0] = 0xffffffffu;
    __syncthreads();
    int sbk[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sbk[i] = sb(skey[i]);
      atomicAdd(&hist[sbk[i]], 1u);
    }
    __syncthreads();
    if (rank < S) {  // uniform
      find_bucket_s((uint32_t)rank);
      // lo = the smallest sample key in the bucket: >= `rank` samples are >= lo
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (sbk[i] == (int)s_sel[0]) atomicMin(&s_red[0], skey[i]);
      __syncthreads();
      lo_key = s_red[0];
    } else {
      lo_key = smin;
    }
    __syncthreads();
  }

  // ---- 2. one streaming pass: candidates (score >= lo) by chunk ----
  // key >= lo_key <=> score >= lo_f for every non-NaN score
  const float lo_f = lo_key == 1u ? -__builtin_inff() : key_to_float(lo_key);
  // Each wave appends the candidates of its chunks to its own quarter of
  // the list, counting in a register: no shared counter, no broadcast.
  const uint32_t wbase = (uint32_t)(wave * kWaveCap);
  uint32_t wcnt = 0;  // uniform; keeps counting past the quarter (overflow)
  for (int c0 = wave; c0 < nchunks; c0 += kSWaves * kBatch) {
    if (c0 != wave) load_batch(c0);  // the first batch is already in flight
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int ch = c0 + kSWaves * i;  // uniform
      if (ch < nchunks) {
        const int col = ch * 256 + lane * 4;
        const float x[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        uint64_t bal[4];
        uint32_t below = 0, cnt = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bal[e] = ballot(col + e < n && x[e] >= lo_f);
          below += popc_below(bal[e]);
          cnt += __popcll(bal[e]);
        }
        const uint32_t slot = wbase + wcnt;
        if (cnt > 0u && wcnt + cnt <= (uint32_t)kWaveCap) {  // uniform
          uint32_t pos = slot + below;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if ((bal[e] >> lane) & 1u) {
              s_ckey[pos] = float_to_key(x[e]);
              s_ccol[pos] = (uint8_t)(4 * lane + e);
              ++pos;
            }
        }
        if (lane == 0) {
          s_cbase[ch] = (uint16_t)(wcnt + cnt <= (uint32_t)kWaveCap ? slot : 0u);
          s_ccnt[ch] = (uint16_t)cnt;
        }
        wcnt += cnt;
      }
    }
  }
  if (lane == 0) s_wcnt[wave] = wcnt;
  __syncthreads();
  uint32_t ccount = 0;
  bool spill = false;  // some quarter overflowed
#pragma unroll
  for (int w = 0; w < kSWaves; ++w) {
    ccount += s_wcnt[w];
    spill |= s_wcnt[w] > (uint32_t)kWaveCap;
  }
  // f(key) for every candidate of the calling thread (the quarters in turn)
  auto for_cands = [&](auto&& f) {
#pragma unroll
    for (int w = 0; w < kSWaves; ++w) {
      const int cw = (int)s_wcnt[w];
      for (int i = tid; i < cw; i += NT) f(s_ckey[w * kWaveCap + i]);
    }
  };

  uint32_t theta, need_eq;
  const Placer place{0u, 0u, (uint32_t)k, out_idx, out_val};
  if (ccount >= (uint32_t)k && !spill) {  // uniform
    const int nc = (int)ccount;
    // ---- 3. theta among the candidates ----
    uint32_t cmax = 0;
    for_cands([&](uint32_t key) { cmax = max(cmax, key); });
    cmax = block_max<kSWaves>(cmax, s_red);
    const float span = key_to_float(cmax) - lo_f;
    const LinearBuckets cb{lo_f, span > 0.0f ? (float)kBins / span : 0.0f};
    for (int i = tid; i < kBins; i += NT) hist[i] = 0u;
    __syncthreads();
    for_cands([&](uint32_t key) { atomicAdd(&hist[cb(key)], 1u); });
    __syncthreads();
    find_bucket_s((uint32_t)k);
    const int bstar = (int)s_sel[0];
    const uint32_t rem = (uint32_t)k - s_sel[1];  // >= 1 keys to take from bucket b*
    __syncthreads();
    // Members of bucket b* into a small list (order does not matter here).
    if (tid == 0) s_sel[1] = 0u;
    __syncthreads();
    for_cands([&](uint32_t key) {
      if (cb(key) == bstar) {
        const uint32_t at = atomicAdd(&s_sel[1], 1u);
        if (at < 64u) hist[at] = key;  // the histogram is no longer needed
      }
    });
    __syncthreads();
    const uint32_t m = s_sel[1];
    if (m <= 64u) {  // uniform: rank the members against each other in one wave
      if (wave == 0) {
        const uint32_t x = lane < (int)m ? hist[lane] : 0u;
        uint32_t gt = 0, eq = 0;
        for (uint32_t j = 0; j < m; ++j) {  // member j from its lane, not from LDS
          const uint32_t y = (uint32_t)__builtin_amdgcn_readlane((int)x, (int)j);
          gt += y > x;
          eq += y == x;
        }
        if (lane < (int)m && gt < rem && rem <= gt + eq) {
          s_red[0] = x;
          s_red[1] = rem - gt;
        }
      }
      __syncthreads();
      theta = s_red[0];
      need_eq = s_red[1];
      __syncthreads();
    } else {
      theta = radix_select<kSWaves>(rem, hist, s_wave, s_sel, &need_eq, [&](auto&& f) {
        for_cands([&](uint32_t key) {
          if (cb(key) == bstar) f(key);
        });
      });
    }

    // ---- 4. output: the candidates in column order, an equal share each ----
    // Chunk starts in column order (an exclusive scan of the chunk counts)
    // replace the counts: chunk ch holds column-order positions
    // [s_ccnt[ch], s_ccnt[ch + 1]), its candidates at slots s_cbase[ch] + ...
    {
      const uint32_t c = tid < nchunks ? (uint32_t)s_ccnt[tid] : 0u;
      uint32_t tot;
      const uint32_t cst = block_exclusive_scan<kSWaves>(c, s_wave, &tot);  // ends with a barrier
      if (tid < nchunks) s_ccnt[tid] = (uint16_t)cst;
      if (tid == 0) s_ccnt[nchunks] = (uint16_t)tot;
      __syncthreads();
    }
    // thread t: positions [p0, p1); ch0 = the last chunk starting at or
    // before p0 (empty chunks share the next one's start)
    const int p0 = nc * tid / NT, p1 = nc * (tid + 1) / NT;
    int lo = 0, hi = nchunks - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int)s_ccnt[mid] <= p0) lo = mid; else hi = mid - 1;
    }
    const int ch0 = lo;
    // f(slot, chunk) for the thread's positions in order
    auto walk = [&](auto&& f) {
      int ch = ch0, cend = s_ccnt[ch + 1];
      int slot = s_cbase[ch] + (p0 - (int)s_ccnt[ch]);
      for (int p = p0; p < p1; ++p, ++slot) {
        while (p >= cend) {  // next non-empty chunk (p < nc keeps ch < nchunks)
          ++ch;
          cend = s_ccnt[ch + 1];
          slot = s_cbase[ch];
        }
        f(slot, ch);
      }
    };
    uint32_t ngt = 0, neq = 0;
    walk([&](int slot, int) {
      const uint32_t key = s_ckey[slot];
      ngt += key > theta;
      neq += key == theta;
    });
    uint32_t total;
    const uint32_t before = block_exclusive_scan<kSWaves>(ngt | (neq << 16), s_wave, &total);
    uint32_t g = before & 0xffffu, q = before >> 16;
    const bool staged = !out_val && (k & 3) == 0 && ((uintptr_t)out_idx & 15u) == 0;
    const Placer pl{theta, need_eq, (uint32_t)k, staged ? reinterpret_cast<int32_t*>(hist) : out_idx,
                    out_val};
    walk([&](int slot, int ch) { pl(s_ckey[slot], base + 256 * ch + (int32_t)s_ccol[slot], g, q); });
    if (staged) {
      __syncthreads();
      for (int i = 4 * tid; i < k; i += 4 * NT)
        *reinterpret_cast<u32x4*>(out_idx + i) = *reinterpret_cast<const u32x4*>(hist + i);
    }
  } else {
    // ---- fallback: radix passes that re-stream the row ----
    const int nq = (n + 3) / 4;  // 16-byte groups of the row
    auto keys_of = [&](int gq, uint32_t* kk) {
      const float4 v = *reinterpret_cast<const float4*>(row + 4 * (int64_t)gq);
      const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) kk[e] = 4 * gq + e < n ? float_to_key(x[e]) : 0u;
    };
    theta = radix_select<kSWaves>((uint32_t)k, hist, s_wave, s_sel, &need_eq, [&](auto&& f) {
      for (int gq = tid; gq < nq; gq += NT) {
        uint32_t kk[4];
        keys_of(gq, kk);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (kk[e] != 0u) f(kk[e]);
      }
    });
    // thread t owns groups [t * P, t * P + P), in column order
    const int P = (nq + NT - 1) / NT;
    const int g0 = min(tid * P, nq), g1 = min(g0 + P, nq);
    uint32_t ngt = 0, neq = 0;
    for (int gq = g0; gq < g1; ++gq) {
      uint32_t kk[4];
      keys_of(gq, kk);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ngt += kk[e] > theta;
        neq += kk[e] == theta;
      }
    }
    uint32_t total;
    const uint32_t before = block_exclusive_scan<kSWaves>(ngt | (neq << 16), s_wave, &total);
    uint32_t g = before & 0xffffu, q = before >> 16;
    const Placer pl{theta, need_eq, (uint32_t)k, out_idx, out_val};
    for (int gq = g0; gq < g1; ++gq) {
      uint32_t kk[4];
      keys_of(gq, kk);
#pragma unroll
      for (int e = 0; e < 4; ++e) pl(kk[e], base + 4 * gq + e, g, q);
    }
  }
  (void)place;
  if (tid == 0 && topk_length) topk_length[r] = k;
}

template <int WAVES, int CH>
hipError_t launch_radix(const float* scores, int64_t ld, int64_t n_rows, int64_t n_cols,
                        const int32_t* sl, const int32_t* rs, int k, int32_t* idx,
                        int64_t ld_idx, int32_t* tl, float* vals, hipStream_t st) {
  dim3 grid((unsigned)n_rows), block(64 * WAVES);
  hipLaunchKernelGGL((topk_radix_kernel<WAVES, CH, false>), grid, block, 0, st, scores, ld, n_cols,
                     sl, rs, k, idx, ld_idx, tl, vals, CandSel{});
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const float* scores, int64_t ld, int64_t n_rows, int64_t n_cols,
                       const int32_t* seq_lens, const int32_t* row_starts, int k, int32_t* indices,
                       int64_t ld_idx, int32_t* topk_length, float* values, hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  if (n_cols <= 256)
    return launch_radix<1, 1>(scores, ld, n_rows, n_cols, seq_lens, row_starts, k, indices, ld_idx,
                              topk_length, values, st);
  if (n_cols <= 1024)
    return launch_radix<1, 4>(scores, ld, n_rows, n_cols, seq_lens, row_starts, k, indices, ld_idx,
                              topk_length, values, st);
  if (n_cols <= 4096)
    return launch_radix<4, 4>(scores, ld, n_rows, n_cols, seq_lens, row_starts, k, indices,
                              ld_idx, topk_length, values, st);
  if (n_cols <= 8192)
    return launch_radix<8, 4>(scores, ld, n_rows, n_cols, seq_lens, row_starts, k, indices,
                              ld_idx, topk_length, values, st);
  if (n_cols <= 65536) {
    dim3 grid((unsigned)n_rows), block(kSThreads);
    hipLaunchKernelGGL(topk_stream_kernel, grid, block, 0, st, scores, ld, n_cols, seq_lens,
                       row_starts, k, indices, ld_idx, topk_length, values);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

hipError_t launch_topk_cand(const int32_t* seq_lens, const int32_t* row_starts, int64_t n_rows,
                            int64_t n_cols, int k, int32_t* indices, int64_t ld_idx,
                            int32_t* topk_length, float* logits, float* softmax, float* lse,
                            const CandArgs& ca, hipStream_t st) {
  constexpr int kW = 8, kCh = 4;
  static_assert(64 * kW * 4 * kCh == kCandCap, "one workgroup holds a full candidate list");
  if (n_rows == 0) return hipSuccess;
  const CandSel cs{ca.cand, ca.cap, ca.count, ca.queue, ca.n_queued, softmax, lse};
  dim3 grid((unsigned)n_rows), block(64 * kW);
  hipLaunchKernelGGL((topk_radix_kernel<kW, kCh, true>), grid, block, 0, st, nullptr, 0, n_cols,
                     seq_lens, row_starts, k, indices, ld_idx, topk_length, logits, cs);
  return hipGetLastError();
}

}  // namespace dsa
