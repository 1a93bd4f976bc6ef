// Sparse MQA attention backward (shared latent KV) for gfx950.
//
// Semantics: cuDNN Frontend DSA page, section 2 "Sparse Attention Backward",
// the gradient of section 1's forward. For query row t, head h and valid slot
// j (key row k_j = kv[idx[t,j]], value v_j = its first D_v dims):
//   P_j  = exp(s_j - log Z),  log Z = log(sum_i exp(s_i) + exp(sink_h))
//        = log(exp(lse) + exp(sink_h))            (lse: the forward's KV-only LSE)
//   dP_j = dout . v_j,  D = dout . out,  dS_j = P_j (dP_j - D)
//   dq   = scale sum_j dS_j k_j
//   dkv[idx_j]       += scale dS_j q          (all D_qk dims)
//   dkv[idx_j, :D_v] += P_j dout              (the value dims)
//   d_sink_h = -sum_t exp(sink_h - log Z) D
// Duplicate slots contribute separately; invalid slots contribute nothing.
//
// Kernels (one pass each, over chunks of query rows; bf16 MFMA
// v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//  * bwd_prep_kernel: D and log Z per (t, h), one wave per pair.
//  * bwd_sink_kernel: d_sink by a fixed-order reduction over t (deterministic).
//  * bwd_pds_kernel: gathers 32 selected KV rows per tile into an LDS ring
//    with asynchronous copies and computes S = q . K^T and dP = dout . V^T
//    from the same fragment reads; stores P and dS = scale * P * (dP - D)
//    (scale folded in) as bf16, in 16-head chunks ([row][head / 16][slot]
//    [head % 16]): with ascending ids, the slots of a run of KV rows are
//    consecutive, and so are their chunks.
//  * bwd_dq_ring_kernel: dq = dS . K with both operands read transposed from
//    LDS (ds_read_b64_tr_b16), two waves per 32-head block splitting the
//    dims; K gathered into the same copy ring as bwd_pds_kernel.
//  * dkv, when rows select a large share of the KV rows (KV tiles):
//    bwd_map_kernel: each row's slot per KV row (int16) and the queue of rows
//    with repeated ids; bwd_merge_kernel: their repeated slots folded into
//    the lowest one (ascending slot order); bwd_dkv_tile_kernel: per tile of
//    128 KV rows and part of 64 query rows, dS^T . q + P^T . dout over the
//    part's rows and heads, accumulated in registers (an fp32 partial per
//    part); bwd_tile_reduce_kernel: the parts summed in ascending order.
//  * dkv otherwise (per-slot rows): bwd_dkv_kernel: per tile, dS^T . q +
//    P^T . dout (the query's q and dout staged in LDS), each slot's row
//    written once as bf16 (per 64-head part); the slots per KV row, counted
//    by bwd_pds_kernel, and bwd_scan: the offsets of their lists;
//    bwd_sort_{hist,scan,scatter}: a
//    stable radix sort of the chunk's valid slots by KV row, giving each KV
//    row the ascending list of the slot rows written for it;
//    bwd_reduce_kernel: one workgroup per KV row sums its list (and parts) in
//    fp32 into the dkv workspace.
//  * bwd_convert_kernel: fp32 workspace -> bf16 dkv.
// No atomics decide the order of any sum, so dkv is reproducible.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {
namespace {

constexpr int kBT = 32;  // slots per tile
constexpr float kLog2eB = 1.442695040888963387f;

// Element offset of (slot, head h) in one row's P or dS: [h / 16][Kw][h % 16].
__device__ __forceinline__ int64_t pds_off(int slot, int h, int Kw) {
  return ((int64_t)(h >> 4) * Kw + slot) * 16 + (h & 15);
}

// C-layout row of value i of a 32x32 MFMA result for lane half `half`.
__device__ __forceinline__ int crow(int i, int half) { return 8 * (i >> 2) + 4 * half + (i & 3); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// ---------------------------------------------------------------- D, log Z --
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t p = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (p >= a.T_q * a.H) return;
  const int64_t t = p / a.H;
  const int h = (int)(p - t * a.H);
  // dout . out over the D_v dims, 8 per lane per step
  float acc = 0.0f;
  for (int d = 8 * lane; d < a.D_v; d += 512) {
    const u32x4 g = load16(a.dout + (t * a.H + h) * a.D_v + d);
    const u32x4 o = load16(a.out + (t * a.H + h) * a.D_v + d);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(bf16_bits_to_f32(g[e] & 0xffffu), bf16_bits_to_f32(o[e] & 0xffffu), acc);
      acc = fmaf(bf16_bits_to_f32(g[e] >> 16), bf16_bits_to_f32(o[e] >> 16), acc);
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) {
    const float lse = a.lse[t * a.H + h];
    float lz = lse;
    if (a.sink && lse < __builtin_inff()) {
      const float s = a.sink[h];
      const float m = fmaxf(lse, s);
      lz = m + logf(expf(lse - m) + expf(s - m));
    }
    a.logZ[t * a.H + h] = lz;  // +inf for an empty row
    a.Dsum[t * a.H + h] = acc;
  }
}

// d_sink[h] = -sum_t exp(sink_h - logZ[t,h]) * D[t,h], fixed summation order.
__global__ __launch_bounds__(256) void bwd_sink_kernel(BwdArgs a) {
  __shared__ float s_part[256];
  const int h = blockIdx.x;
  const float s = a.sink[h];
  float acc = 0.0f;
  for (int64_t t = threadIdx.x; t < a.T_q; t += 256) {
    const float lz = a.logZ[t * a.H + h];
    if (lz < __builtin_inff()) acc += expf(s - lz) * a.Dsum[t * a.H + h];
  }
  s_part[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) s_part[threadIdx.x] += s_part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.d_sink[h] = -s_part[0];
}

// s_waitcnt vmcnt(N): at most N vector-memory operations of the wave still
// in flight (they complete in issue order), through the builtin so that the
// compiler's own wait tracking knows it.
template <int N>
__device__ __forceinline__ void wait_vmcnt_le() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ int row_len(const BwdArgs& a, int64_t t) {
  if (!a.topk_length) return a.k_width;
  const int32_t L = a.topk_length[t];
  return L < 0 ? 0 : (L > a.k_width ? a.k_width : L);
}

// ---------------------------------------------------------- P and dS, fused --
// One workgroup per query row of the chunk; wave w < NW owns heads
// 32w .. 32w+31 (NWC waves are launched: NW, or 4 when NW = 3, the extra wave
// only copying). Per tile of 32 slots, with the gathered rows as the B operand
// (lane -> slot l%32, k = dims) of v_mfma_f32_32x32x16_bf16:
//   S  = q . K^T     A = q of the wave's heads, held in AGPRs   (DQK/16 k-steps)
//   dP = dout . V^T  A = dout of the wave's heads, in VGPRs     (32 k-steps)
// Each fragment read from LDS feeds both products (V is the first 512 dims
// of K). C lane -> slot column l%32, head rows crow(i). Then
//   P = exp2(S scale log2e - log Z log2e),  dS = scale P (dP - D)
// both written as bf16 to the workspaces in 16-head chunks (pds_off);
// invalid slots and heads past H write zeros. The S chain uses the compiler's
// MFMA (its accumulator in AGPRs, q where the allocator puts it); the dP chain
// is written inline with its accumulator in AGPRs, and the wait states the
// compiler would insert before reads of dP are given after the chain. Two
// sets of both accumulators alternate between tiles: P and dS of tile i - 1
// are computed and stored between the MFMAs of tile i.
//
// The tiles are gathered as in the forward kernel: asynchronous LDS copies
// into a 2-stage ring, the copies of tile i+1 interleaved with the MFMAs of
// tile i. Rows 8g .. 8g+7 and dims 64s .. 64s+63 of a tile form the 1 KiB
// block 4s + g, copied as eight 128-byte row segments; chunk c of row 8g + r
// sits in slot 8r + (c ^ f(r, g)), f = 4*((r>>1)&1) + (r>>2) + 2*(g&1), which
// keeps the fragment reads (16 lanes: 16 rows, one chunk) conflict-free. With
// BUF the copies go through a buffer descriptor over kv with 32-bit row
// offsets and masked rows read as zeros past its range; else through 64-bit
// addresses with masked rows read from a zero constant.
__device__ const u32x4 g_bwd_zero_row[128] = {};

template <int DQK, int NW, int NWC, bool BUF>
__global__ __launch_bounds__(NWC * 64, 1) void bwd_pds_kernel(BwdArgs a) {
  constexpr int KS = DQK / 16;            // S k-steps
  constexpr int KV = 512 / 16;            // dP k-steps (the value dims)
  constexpr int K_SEG = DQK / 64;         // 64-dim segments of a row
  constexpr int GPW = 4 / NWC;            // row groups copied per wave
  constexpr int NCOPY = GPW * K_SEG;      // copies per wave and tile
  constexpr int STAGE = 4 * K_SEG * 1024;
  constexpr int HP = NW * 32;
  static_assert(NWC == 1 || NWC == 2 || NWC == 4, "row groups split evenly over waves");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5, r32 = lane & 31;
  const int64_t rc = blockIdx.x;
  const int64_t t = a.row0 + rc;
  const int L = row_len(a, t);
  const int n_tiles = (L + kBT - 1) / kBT;
  const bool comp = NW == NWC || wave < NW;  // uniform; every wave when NW == NWC
  const int h0 = 32 * wave;
  const int hA = h0 + r32;

  const int key_row = lane & 31;
  const int crw = lane >> 3;
  auto swz = [](int r, int g) -> int { return 4 * ((r >> 1) & 1) + (r >> 2) + 2 * (g & 1); };
  auto load_id = [&](int j0, int row) -> int32_t {  // L > 0
    // unconditional (clamped) load, replaced past L afterwards: a predicated
    // load is waited for at its branch's end
    const int j = j0 + row;
    const int32_t raw = a.indices[t * a.ld_idx + (j < L ? j : L - 1)];
    return j < L ? raw : -1;
  };
  auto load_id_raw = [&](int j0, int row) -> int32_t {  // L > 0; checked against L at use
    const int j = j0 + row;
    return a.indices[t * a.ld_idx + (j < L ? j : L - 1)];
  };
  auto valid_id = [&](int32_t raw) -> int32_t {
    return (raw >= 0 && (int64_t)raw < a.T_kv) ? raw : -1;
  };
  // ids of the first two tiles before anything else
  const int32_t id_first = n_tiles > 0 ? load_id(0, key_row) : -1;
  const int32_t id_second = n_tiles > 1 ? load_id(kBT, key_row) : -1;

  const uint32_t smem_base = lds_addr(smem);
  struct CopySrc {
    const uint16_t* k[BUF ? 1 : GPW];
    uint32_t ko[BUF ? GPW : 1];
    uint32_t m0;
  };
  i32x4 rsrc{};
  if constexpr (BUF) rsrc = buffer_rsrc_words(a.kv, a.span_kv);
  constexpr uint32_t kPastRange = 0x80000000u;
  auto prep_copy = [&](uint32_t stage, int32_t idv) -> CopySrc {
    CopySrc cs;
    int32_t idg[GPW];
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) idg[gi] = __shfl(idv, 8 * (GPW * wave + gi) + crw, kWave);
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      const int g = GPW * wave + gi;
      const int chunk = (lane & 7) ^ swz(crw, g);
      const bool ok = idg[gi] >= 0;
      if constexpr (BUF) {
        cs.ko[gi] = ok ? __umul24((uint32_t)idg[gi], a.row_bytes) + 16u * chunk : kPastRange;
      } else {
        const uint16_t* zero = reinterpret_cast<const uint16_t*>(g_bwd_zero_row);
        const uint64_t row = ok ? (uint64_t)(uint32_t)idg[gi] : 0ull;
        cs.k[gi] = (ok ? a.kv : zero) + row * (uint64_t)a.ld_kv + 8 * chunk;
      }
    }
    cs.m0 = __builtin_amdgcn_readfirstlane(stage + 1024u * (uint32_t)(GPW * wave));
    return cs;
  };
  auto copy_one = [&](const CopySrc& cs, auto jc) {
    constexpr int J = decltype(jc)::value;
    constexpr int GI = J % GPW, S = J / GPW;
    const uint32_t m0 = cs.m0 + (uint32_t)(1024 * (4 * S + GI) - 128 * S);
    if constexpr (BUF) dma16_buf_imm<128 * S>(cs.ko[GI], rsrc, m0);
    else dma16_imm<128 * S>(cs.k[GI], m0);
  };

  // A operands: lane -> head hA, dims 16*ks + 8*half .. +7 (clamped head,
  // zeroed past H).
  u32x4 qa[KS], ga[KV];
  {
    const int hq = hA < a.H ? hA : a.H - 1;
    const uint16_t* qs = a.q + (t * a.H + hq) * (int64_t)DQK + 8 * half;
    const uint16_t* gs = a.dout + (t * a.H + hq) * (int64_t)512 + 8 * half;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qa[ks] = load16(qs + 16 * ks);
#pragma unroll
    for (int ks = 0; ks < KV; ++ks) ga[ks] = load16(gs + 16 * ks);
    if (hA >= a.H) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qa[ks] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int ks = 0; ks < KV; ++ks) ga[ks] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  // log Z and D of the lane's 16 heads: unconditional loads (clamped head)
  // replaced past H afterwards, so that all are in flight together
  float lz2[16], dd[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int h = h0 + crow(i, half);
    const int64_t o = t * a.H + (h < a.H ? h : a.H - 1);
    lz2[i] = a.logZ[o];
    dd[i] = a.Dsum[o];
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const bool hv = h0 + crow(i, half) < a.H;
    lz2[i] = hv ? lz2[i] * kLog2eB : __builtin_inff();
    dd[i] = hv ? dd[i] : 0.0f;
  }
  const float c2 = a.scale * kLog2eB;
  uint16_t* wsP = a.wsP + rc * (int64_t)a.Kw * HP;
  uint16_t* wsD = a.wsD + rc * (int64_t)a.Kw * HP;

  int32_t id_next = id_second;
  uint32_t mask_cur = 0;
  // Per-slot dkv rows: the slots per KV row are counted here, as the ids are
  // validated (one lane per slot, non-returning atomics issued before the
  // tile's copies); with KV tiles nothing is counted.
  const bool count = !a.tiles && wave == 0 && lane < 32;
  if (n_tiles > 0) {
    const int32_t id0 = valid_id(id_first);
    if (count && id0 >= 0) atomicAdd(a.cnt + id0, 1);
    mask_cur = (uint32_t)ballot(id0 >= 0);
    const CopySrc cs0 = prep_copy(smem_base, id0);
    static_for<NCOPY>([&](auto jc) { copy_one(cs0, jc); });
    wait_vmcnt0();
    __syncthreads();  // tile 0 has landed in every wave's share
  }
  // The epilogue of tile it - 1 (P and dS from its S and dP) runs between
  // the MFMAs of tile it: two accumulator sets alternate, so the VALU work
  // and the stores overlap the matrix work instead of following it.
  auto epi_part = [&](uint32_t mask, const f32x16& sa, const f32x16& da, uint32_t (&pw)[4][2],
                      uint32_t (&dw)[4][2], auto gc) {
    constexpr int g = decltype(gc)::value;
    const bool valid = (mask >> r32) & 1u;
    float pv[4], dv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * g + e;
      const float p = valid ? fast_exp2(fmaf(sa[i], c2, -lz2[i])) : 0.0f;
      pv[e] = p;
      dv[e] = a.scale * p * (da[i] - dd[i]);
    }
    pw[g][0] = pack_bf16x2(pv[0], pv[1]);
    pw[g][1] = pack_bf16x2(pv[2], pv[3]);
    dw[g][0] = pack_bf16x2(dv[0], dv[1]);
    dw[g][1] = pack_bf16x2(dv[2], dv[3]);
  };
  // lane (slot, half) holds heads 8g + 4*half + 0..3 of its slot for
  // g = 0..3 (the C layout); one v_permlane32_swap per word and pair of
  // groups (2pi, 2pi + 1) gives half 0 heads 16pi + 0..7 and half 1 heads
  // 16pi + 8..15, stored as 16-byte runs through buffer descriptors of the
  // row's P and dS. The stores of the first tile step (no previous tile) take
  // an offset past the range and are dropped, so every step issues the same
  // four stores. They are streaming (nontemporal: aux bit 1): P and dS are
  // read again only by the later passes, and at long rows far exceed the
  // caches.
  const __amdgpu_buffer_rsrc_t rP = raw_buffer(wsP, (uint32_t)(a.Kw * HP * 2));
  const __amdgpu_buffer_rsrc_t rD = raw_buffer(wsD, (uint32_t)(a.Kw * HP * 2));
  auto epi_store = [&](int te, bool live, const uint32_t (&pw)[4][2], const uint32_t (&dw)[4][2],
                       auto pc) {
    constexpr int pi = decltype(pc)::value;
    u32x4 po, dq4;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const auto sp = __builtin_amdgcn_permlane32_swap(pw[2 * pi][w], pw[2 * pi + 1][w], false, false);
      const auto sd = __builtin_amdgcn_permlane32_swap(dw[2 * pi][w], dw[2 * pi + 1][w], false, false);
      po[w] = sp[0];
      po[2 + w] = sp[1];
      dq4[w] = sd[0];
      dq4[2 + w] = sd[1];
    }
    // 8 consecutive heads
    const uint32_t off = live ? (uint32_t)pds_off(te * kBT + r32, h0 + 16 * pi + 8 * half, a.Kw) * 2u
                              : 0x80000000u;
    __builtin_amdgcn_raw_buffer_store_b128(po, rP, (int)off, 0, 2);
    __builtin_amdgcn_raw_buffer_store_b128(dq4, rD, (int)off, 0, 2);
  };
  uint32_t mask_prev = 0;
  auto tile_step = [&](int it, f32x16& sacc, f32x16& dacc, const f32x16& sprev, const f32x16& dprev) {
    uint32_t mask_next = 0;
    const bool copy_next = it + 1 < n_tiles;  // uniform
    const bool has_prev = it > 0;            // uniform
    CopySrc cs{};
    if (copy_next) {
      // (the ids' row check happens here, at their first use, after the
      // previous tile's barrier wait has covered their load)
      const int32_t idv = (it + 1) * kBT + key_row < L ? valid_id(id_next) : -1;
      if (count && idv >= 0) atomicAdd(a.cnt + idv, 1);
      mask_next = (uint32_t)ballot(idv >= 0);
      cs = prep_copy(smem_base + ((it + 1) & 1) * STAGE, idv);
    }
    // ids of tile it + 2 (clamped to the row, checked at their use), loaded
    // ahead of this tile's copies and stores so that the wait at the tile's
    // end covers them
    const int32_t id_after = load_id_raw((it + 2) * kBT, key_row);
    // copies spread over the first two thirds of the S k-steps, so that
    // most have landed by the wait after the k-loop
    auto copies_at = [&](auto kc) {
      constexpr int ks = decltype(kc)::value;
      constexpr int KF = KS * 2 / 3;
      constexpr int j0 = ks < KF ? (ks * NCOPY + KF - 1) / KF : NCOPY;
      constexpr int j1 = ks < KF ? ((ks + 1) * NCOPY + KF - 1) / KF : NCOPY;
      if (copy_next)
        static_for<j1 - j0>([&](auto dj) {
          copy_one(cs, std::integral_constant<int, j0 + decltype(dj)::value>{});
        });
    };
    const unsigned char* tile = smem + (it & 1) * STAGE;
    if (comp) {
      // fragment of k-step ks: row r32 (group kg, row kr), chunk 2*(ks%4) + half of
      // segment ks/4 at slot 8*kr + (chunk ^ f)
      const int kg = r32 >> 3, kr = r32 & 7, kf = swz(kr, kg);
      const unsigned char* kbase = tile + kg * 1024 + kr * 128 + 16 * (half ^ (kf & 1));
      const unsigned char* kq[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) kq[q] = kbase + 32 * (q ^ (kf >> 1));
      auto kread = [&](int ks) -> u32x4 {
        return *reinterpret_cast<const u32x4*>(kq[ks & 3] + (ks >> 2) * 4096);
      };
      constexpr int PF = 4;
      u32x4 bf[PF];
#pragma unroll
      for (int i = 0; i < PF; ++i) bf[i] = kread(i);
      uint32_t pw[4][2], dw[4][2];
      static_for<KS>([&](auto kc) {
        constexpr int ks = decltype(kc)::value;
        const u32x4 cur = bf[ks % PF];
        if constexpr (ks + PF < KS) bf[ks % PF] = kread(ks + PF);
        sacc = mfma32x32x16(qa[ks], cur, ks == 0 ? f32x16{} : sacc);
        if constexpr (ks == 0)
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=a"(dacc) : "v"(ga[0]), "v"(cur));
        else if constexpr (ks < KV)
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(dacc) : "v"(ga[ks]), "v"(cur));
        copies_at(kc);
        // the previous tile's P / dS: values at k-steps 2, 6, 10, 14, the
        // stores at 26 and 30, after this tile's last copy
        if constexpr (ks % 4 == 2 && ks / 4 < 4) {
          constexpr int g = ks / 4;
          epi_part(mask_prev, sprev, dprev, pw, dw, std::integral_constant<int, g>{});
          // a use here, so that the values are not sunk towards the stores
          asm volatile("" ::"v"(pw[g][0]), "v"(pw[g][1]), "v"(dw[g][0]), "v"(dw[g][1]));
        }
        if constexpr (ks == 26 || ks == 30)
          epi_store(it - 1, has_prev, pw, dw, std::integral_constant<int, (ks - 26) / 4>{});
      });
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(dacc));
    } else {
      static_for<KS>([&](auto kc) { copies_at(kc); });
    }
    id_next = id_after;
    mask_prev = mask_cur;
    mask_cur = mask_next;
    if (copy_next) {  // uniform
      // Tile it + 1 has landed in this wave's share; the four P / dS stores,
      // issued after its copies, may stay in flight.
      if (comp) wait_vmcnt_le<4>();  // uniform
      else wait_vmcnt0();
      __syncthreads();  // every wave's share has landed; tile it is consumed
    }
  };
  f32x16 s0{}, d0{}, s1{}, d1{};
  for (int it = 0; it < n_tiles; it += 2) {
    tile_step(it, s0, d0, s1, d1);
    if (it + 1 < n_tiles) tile_step(it + 1, s1, d1, s0, d0);  // uniform
  }
  if (comp && n_tiles > 0) {  // the last tile's epilogue
    const int te = n_tiles - 1;
    const f32x16& sl = (te & 1) ? s1 : s0;
    const f32x16& dl = (te & 1) ? d1 : d0;
    uint32_t pw[4][2], dw[4][2];
    static_for<4>([&](auto gc) { epi_part(mask_prev, sl, dl, pw, dw, gc); });
    static_for<2>([&](auto pc) { epi_store(te, true, pw, dw, pc); });
  }
}

// ---------------------------------------------------------- dq, ring --
// One workgroup per query row, waves (head block hb = w/2, dim half dh = w%2).
// dq[h][d] on 32x32x16 with k = slots: A = dS (heads x slots) and B = K
// (slots x dims), both read transposed (ds_read_b64_tr_b16). The K tiles are
// gathered into the same swizzled 2-stage ring as bwd_pds_kernel (copies of
// tile i+1 issued by the first min(2*NW, 4) waves between the MFMAs of tile
// i); each tile's dS (32 slots x 16 heads contiguous per 16-head chunk in
// the workspace) is loaded one tile ahead into registers and stored to a
// padded [slot][head] LDS tile.
// Lane half h of an MFMA operand covers slots 16*st + 4h + 0..3 and
// 16*st + 8 + 4h + 0..3 of k-step st, in both operands.
template <int DQK, int NW, bool BUF>
__global__ __launch_bounds__(NW * 128, NW <= 2 ? 2 : 1) void bwd_dq_ring_kernel(BwdArgs a) {
  constexpr int NWQ = 2 * NW;             // waves
  constexpr int NCW = NWQ < 4 ? NWQ : 4;  // copying waves
  constexpr int GPW = 4 / NCW;            // row groups copied per copying wave
  constexpr int K_SEG = DQK / 64;
  constexpr int NCOPY = GPW * K_SEG;
  constexpr int STAGE = 4 * K_SEG * 1024;
  constexpr int HP = NW * 32;
  constexpr int RSD = HP + 8;             // dS tile row stride (bf16): conflict-free reads
  constexpr int NBW = DQK / 64;           // 32-dim blocks per wave (half the dims)
  static_assert(NWQ * 64 == kBT * HP / 8, "one 16-byte dS chunk per thread and tile");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t sds[kBT * RSD];

  const int lane = threadIdx.x & 63, half = lane >> 5, r32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // scalar
  const int hb = wave >> 1, dh = wave & 1;
  const bool copier = wave < NCW;  // uniform
  const int64_t rc = blockIdx.x;
  const int64_t t = a.row0 + rc;
  const int L = row_len(a, t);
  const int n_tiles = (L + kBT - 1) / kBT;
  const uint16_t* wsD = a.wsD + rc * (int64_t)a.Kw * HP;

  const int key_row = lane & 31;
  const int crw = lane >> 3;
  auto swz = [](int r, int g) -> int { return 4 * ((r >> 1) & 1) + (r >> 2) + 2 * (g & 1); };
  auto load_id = [&](int j0, int row) -> int32_t {
    const int j = j0 + row;
    int32_t raw = -1;
    if (j < L) raw = a.indices[t * a.ld_idx + j];
    return raw;
  };
  auto valid_id = [&](int32_t raw) -> int32_t {
    return (raw >= 0 && (int64_t)raw < a.T_kv) ? raw : -1;
  };
  const int32_t id_first = n_tiles > 0 ? load_id(0, key_row) : -1;
  const int32_t id_second = n_tiles > 1 ? load_id(kBT, key_row) : -1;
  // this thread's 16-byte chunk of a tile's dS rows
  const int dslot = threadIdx.x / (HP / 8), dch = threadIdx.x % (HP / 8);
  auto load_ds = [&](int tl) -> u32x4 { return load16(wsD + pds_off(tl * kBT + dslot, 8 * dch, a.Kw)); };
  u32x4 ds_next = n_tiles > 0 ? load_ds(0) : u32x4{0u, 0u, 0u, 0u};

  const uint32_t smem_base = lds_addr(smem);
  struct CopySrc {
    const uint16_t* k[BUF ? 1 : GPW];
    uint32_t ko[BUF ? GPW : 1];
    uint32_t m0;
  };
  i32x4 rsrc{};
  if constexpr (BUF) rsrc = buffer_rsrc_words(a.kv, a.span_kv);
  constexpr uint32_t kPastRange = 0x80000000u;
  auto prep_copy = [&](uint32_t stage, int32_t idv) -> CopySrc {
    CopySrc cs;
    int32_t idg[GPW];
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) idg[gi] = __shfl(idv, 8 * (GPW * wave + gi) + crw, kWave);
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      const int g = GPW * wave + gi;
      const int chunk = (lane & 7) ^ swz(crw, g);
      const bool ok = idg[gi] >= 0;
      if constexpr (BUF) {
        cs.ko[gi] = ok ? __umul24((uint32_t)idg[gi], a.row_bytes) + 16u * chunk : kPastRange;
      } else {
        const uint16_t* zero = reinterpret_cast<const uint16_t*>(g_bwd_zero_row);
        const uint64_t row = ok ? (uint64_t)(uint32_t)idg[gi] : 0ull;
        cs.k[gi] = (ok ? a.kv : zero) + row * (uint64_t)a.ld_kv + 8 * chunk;
      }
    }
    cs.m0 = __builtin_amdgcn_readfirstlane(stage + 1024u * (uint32_t)(GPW * wave));
    return cs;
  };
  auto copy_one = [&](const CopySrc& cs, auto jc) {
    constexpr int J = decltype(jc)::value;
    constexpr int GI = J % GPW, S = J / GPW;
    const uint32_t m0 = cs.m0 + (uint32_t)(1024 * (4 * S + GI) - 128 * S);
    if constexpr (BUF) dma16_buf_imm<128 * S>(cs.ko[GI], rsrc, m0);
    else dma16_imm<128 * S>(cs.k[GI], m0);
  };

  // Transposed-read addressing (16-lane group G = lane/16, lane li = lane%16):
  // dS: rows (slots) 16*st + 4*(G/2) + li/4 (+8), columns 32*hb + 16*(G%2) +
  // 4*(li%4); K: the forward kernel's V reads on the swizzled tile (column
  // block nb = 32 dims, key half st).
  const int G = lane >> 4, li = lane & 15;
  const uint16_t* dsa_ptr = sds + (4 * (G >> 1) + (li >> 2)) * RSD + 32 * hb + 16 * (G & 1) + 4 * (li & 3);
  const int vr = 4 * (G >> 1) + (li >> 2);
  const int vb0 = vr * 128 + 16 * (((li >> 1) & 1) ^ (G >> 1)) + 8 * (li & 1);
  int voff[2][2];  // [nb % 2][b]
#pragma unroll
  for (int pp = 0; pp < 2; ++pp)
#pragma unroll
    for (int b = 0; b < 2; ++b) voff[pp][b] = vb0 + 1024 * b + 16 * (4 * (pp ^ (li >> 3)) + 2 * ((G & 1) ^ b));

  f32x16 acc[NBW];
#pragma unroll
  for (int b = 0; b < NBW; ++b) acc[b] = f32x16{};

  int32_t id_next = id_second;
  if (n_tiles > 0 && copier) {
    const CopySrc cs0 = prep_copy(smem_base, valid_id(id_first));
    static_for<NCOPY>([&](auto jc) { copy_one(cs0, jc); });
  }
  for (int it = 0; it < n_tiles; ++it) {
    wait_vmcnt0();
    __syncthreads();  // K tile it landed; every wave is done with tile it-1 and the dS tile
    *reinterpret_cast<u32x4*>(sds + dslot * RSD + 8 * dch) = ds_next;
    if (it + 1 < n_tiles) ds_next = load_ds(it + 1);
    __syncthreads();  // dS of tile it visible
    const bool copy_next = it + 1 < n_tiles;  // uniform
    CopySrc cs{};
    if (copy_next && copier) cs = prep_copy(smem_base + ((it + 1) & 1) * STAGE, valid_id(id_next));
    auto copies_at = [&](auto fc) {  // copies spread over the wave's 2*NBW MFMAs
      constexpr int f = decltype(fc)::value;
      constexpr int NS = 2 * NBW;
      constexpr int j0 = (f * NCOPY + NS - 1) / NS, j1 = ((f + 1) * NCOPY + NS - 1) / NS;
      if (copy_next && copier)
        static_for<j1 - j0>([&](auto dj) {
          copy_one(cs, std::integral_constant<int, j0 + decltype(dj)::value>{});
        });
    };
    const unsigned char* tile = smem + (it & 1) * STAGE;
    auto kfrag = [&](int nb, int st) -> u32x4 {
      const int so = (nb >> 1) * 4096 + st * 2048;
      const u32x2 x0 = lds_read_tr16(tile + voff[nb & 1][0] + so);
      const u32x2 x1 = lds_read_tr16(tile + voff[nb & 1][1] + so);
      return u32x4{x0.x, x0.y, x1.x, x1.y};
    };
    static_for<2>([&](auto stc) {
      constexpr int st = decltype(stc)::value;
      const u32x2 a0 = lds_read_tr16(dsa_ptr + 16 * st * RSD);
      const u32x2 a1 = lds_read_tr16(dsa_ptr + (16 * st + 8) * RSD);
      const u32x4 av = u32x4{a0.x, a0.y, a1.x, a1.y};
      u32x4 kb = kfrag(dh * NBW, st);
      static_for<NBW>([&](auto bc) {
        constexpr int b = decltype(bc)::value;
        const u32x4 cur = kb;
        if constexpr (b + 1 < NBW) kb = kfrag(dh * NBW + b + 1, st);
        acc[b] = mfma32x32x16(av, cur, acc[b]);
        copies_at(std::integral_constant<int, st * NBW + b>{});
      });
    });
    if (copy_next) id_next = (it + 2 < n_tiles) ? load_id((it + 2) * kBT, key_row) : -1;
  }
  // C: lane -> dim column, head rows crow(i); dS already carries the scale
#pragma unroll
  for (int b = 0; b < NBW; ++b) {
    const int d = (dh * NBW + b) * 32 + r32;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int h = 32 * hb + crow(i, half);
      if (h < a.H) a.dq[(t * a.H + h) * DQK + d] = (uint16_t)f32_to_bf16_bits(acc[b][i]);
    }
  }
}

// ------------------------------------------------------------------ dkv --
// One workgroup per (query row, 64-head chunk); NWD waves each own BPW
// 32-dim blocks. C^T[d][s] on 32x32x16 with k = heads: A = q^T / dout^T of
// the chunk's heads (dims x heads, read transposed once per row from the
// staged [head][dim] rows into registers), B = dS^T / P^T (16 heads of 32
// slots contiguous in the workspace). Lane (slot l%32, half) then holds runs
// of 4 consecutive dims of its slot, written as 8-byte words into an LDS
// tile of the 32 slot rows; after a barrier the waves store that tile as
// whole rows, 16 bytes per lane on consecutive addresses. (Stored straight
// from the MFMA layout, 2 bytes per lane, the kernel took 1.6 times as long.)
template <int DQK, int NW, int NWD>
__global__ __launch_bounds__(NWD * 64) void bwd_dkv_kernel(BwdArgs a) {
  constexpr int HP = NW * 32;
  constexpr int HC = HP % 64 == 0 ? 64 : 32;  // heads per chunk (divides HP)
  constexpr int RQ = DQK + 8, RG = 512 + 8;
  constexpr int NBLK = DQK / 32;
  constexpr int BPW = NBLK / NWD;
  static_assert(NBLK % NWD == 0, "dim blocks split evenly over waves");
  // C tile rows: DQK bf16 + 16 bytes, so that the 8-byte writes of 16 lanes
  // (16 rows, one column) fall on distinct banks; two tiles alternate.
  constexpr int RCB = DQK * 2 + 16;
  constexpr int STAGE_B = HC * (RQ + RG) * 2, CT_B = 2 * kBT * RCB;
  static_assert((RCB / 4) % 64 == 36 || (RCB / 4) % 64 == 4, "C tile row stride");
  __shared__ __attribute__((aligned(16))) unsigned char smem[STAGE_B > CT_B ? STAGE_B : CT_B];
  uint16_t* const sq = reinterpret_cast<uint16_t*>(smem);
  uint16_t* const sg = sq + HC * RQ;

  const int lane = threadIdx.x & 63, half = lane >> 5, r32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // scalar
  const int64_t rc = blockIdx.x / (HP / HC);
  const int hc0 = (int)(blockIdx.x % (HP / HC)) * HC;
  const int64_t t = a.row0 + rc;
  const int L = row_len(a, t);
  if (L == 0) return;
  // stage q and dout of the chunk's heads (zeros past H)
  for (int c = threadIdx.x; c < HC * (DQK / 8); c += blockDim.x) {
    const int h = c / (DQK / 8), ch = c - h * (DQK / 8);
    const int hh = hc0 + h;
    *reinterpret_cast<u32x4*>(sq + h * RQ + 8 * ch) =
        hh < a.H ? load16(a.q + (t * a.H + hh) * DQK + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
  }
  for (int c = threadIdx.x; c < HC * 64; c += blockDim.x) {
    const int h = c / 64, ch = c - h * 64;
    const int hh = hc0 + h;
    *reinterpret_cast<u32x4*>(sg + h * RG + 8 * ch) =
        hh < a.H ? load16(a.dout + (t * a.H + hh) * 512 + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
  }
  const uint16_t* wsP = a.wsP + rc * (int64_t)a.Kw * HP;
  const uint16_t* wsD = a.wsD + rc * (int64_t)a.Kw * HP;
  const int G = lane >> 4, li = lane & 15;
  const int rsel = 8 * (G >> 1) + (li >> 2);
  const int csel = 16 * (G & 1) + 4 * (li & 3);
  constexpr int NK = HC / 16;

  // this wave's q and dout fragments for the whole row (dims 512.. have no
  // dout), then the staging area is free for the C tiles
  __syncthreads();  // q and dout staged
  u32x4 qf[NK][BPW], gf[NK][BPW];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
#pragma unroll
    for (int b = 0; b < BPW; ++b) {
      const int col = (wave * BPW + b) * 32;
      const uint16_t* qb = sq + (16 * kk + rsel) * RQ + col + csel;
      const u32x2 q0 = lds_read_tr16(qb), q1 = lds_read_tr16(qb + 4 * RQ);
      qf[kk][b] = u32x4{q0.x, q0.y, q1.x, q1.y};
      if (col < 512) {
        const uint16_t* gb = sg + (16 * kk + rsel) * RG + col + csel;
        const u32x2 g0 = lds_read_tr16(gb), g1 = lds_read_tr16(gb + 4 * RG);
        gf[kk][b] = u32x4{g0.x, g0.y, g1.x, g1.y};
      } else {
        gf[kk][b] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  __syncthreads();  // every wave holds its fragments: the LDS holds C tiles from here

  // Per tile: wait for this tile's B fragments (loaded during the previous
  // tile; its row stores, issued after them, may stay in flight), multiply,
  // load the next tile's fragments into the same registers, write C^T into
  // the tile's LDS rows; after the barrier store the tile's rows.
  const int ntiles = (L + kBT - 1) / kBT;
  u32x4 ad[NK], ap[NK];
  auto load_b = [&](int tl, u32x4* ad, u32x4* ap) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const int64_t o = pds_off(tl * kBT + r32, hc0 + 16 * kk + 8 * half, a.Kw);
      ad[kk] = load16(wsD + o);
      ap[kk] = load16(wsP + o);
    }
  };
  // the row of slot s of this head part goes to wsC[part][rc][s] (bf16)
  uint16_t* crow_base = a.wsC + ((int64_t)(hc0 / HC) * a.chunk_rows + rc) * a.Kw * DQK;
  constexpr int CH = DQK / 8;                    // 16-byte chunks per row
  constexpr int NST = kBT * CH / (NWD * 64);  // row stores per thread and tile
  static_assert(kBT * CH % (NWD * 64) == 0, "every thread issues the same stores");
  if (ntiles > 0) load_b(0, ad, ap);
  for (int tl = 0; tl < ntiles; ++tl) {
    if (tl > 0) wait_vmcnt_le<NST>();  // uniform
    else wait_vmcnt0();
    f32x16 acc[BPW];
#pragma unroll
    for (int b = 0; b < BPW; ++b) acc[b] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)   // 16-head k-steps
#pragma unroll
      for (int b = 0; b < BPW; ++b) {
        acc[b] = mfma32x32x16(qf[kk][b], ad[kk], acc[b]);
        if ((wave * BPW + b) * 32 < 512) acc[b] = mfma32x32x16(gf[kk][b], ap[kk], acc[b]);
      }
    if (tl + 1 < ntiles) load_b(tl + 1, ad, ap);  // uniform
    unsigned char* ct = smem + (tl & 1) * (kBT * RCB);
#pragma unroll
    for (int b = 0; b < BPW; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = (wave * BPW + b) * 32 + 8 * g + 4 * half;  // dims d .. d+3 of slot r32
        const u32x2 w = {pack_bf16x2(acc[b][4 * g], acc[b][4 * g + 1]),
                         pack_bf16x2(acc[b][4 * g + 2], acc[b][4 * g + 3])};
        *reinterpret_cast<u32x2*>(ct + r32 * RCB + 2 * d) = w;
      }
    __syncthreads();  // the tile's rows are in LDS; tile tl - 1's were stored
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const int c = i * NWD * 64 + (int)threadIdx.x;
      const int r = c / CH, ch = c - r * CH;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ct + r * RCB + 16 * ch);
      // streaming store: the row is read back once, by the reduce, long after
      __builtin_nontemporal_store(
          v, reinterpret_cast<u32x4*>(crow_base + (int64_t)(tl * kBT + r) * DQK + 8 * ch));
    }
  }
}

// ---------------------------------------------- sort of the slots by KV row --
// offs = exclusive prefix sum of cnt (T_kv + 1 entries). One workgroup; per
// round of 1024 * PT entries the counts pass through LDS (coalesced loads
// and stores), each thread sums a run of PT consecutive entries, the
// threads' totals are scanned across the workgroup, and a carry links the
// rounds.
__global__ __launch_bounds__(1024) void bwd_scan_kernel(BwdArgs a) {
  constexpr int PT = 16;
  constexpr int N = 1024 * PT;
  __shared__ int32_t s_v[N + N / 32];  // entry i at i + i / 32 (spreads the runs over banks)
  __shared__ int32_t s_w[16];
  __shared__ int32_t s_carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto at = [](int i) { return i + (i >> 5); };
  if (tid == 0) s_carry = 0;
  for (int64_t base = 0; base <= a.T_kv; base += N) {
#pragma unroll
    for (int k = 0; k < PT; ++k) {
      const int i = k * 1024 + tid;
      s_v[at(i)] = base + i < a.T_kv ? a.cnt[base + i] : 0;
    }
    __syncthreads();  // the round's counts are in LDS; the carry is set
    int32_t v[PT];
    int32_t tot = 0;
#pragma unroll
    for (int k = 0; k < PT; ++k) {
      v[k] = s_v[at(tid * PT + k)];
      tot += v[k];
    }
    int32_t incl = tot;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    if (lane == 63) s_w[wave] = incl;
    __syncthreads();
    int32_t before = s_carry;
    for (int w = 0; w < wave; ++w) before += s_w[w];
    int32_t run = before + incl - tot;  // entries before this thread's first
#pragma unroll
    for (int k = 0; k < PT; ++k) {
      s_v[at(tid * PT + k)] = run;
      run += v[k];
    }
    __syncthreads();  // the offsets are in LDS; every thread has read the carry
    if (tid == 1023) s_carry = before + incl;
#pragma unroll
    for (int k = 0; k < PT; ++k) {
      const int i = k * 1024 + tid;
      if (base + i <= a.T_kv) a.offs[base + i] = s_v[at(i)];
    }
    __syncthreads();  // the round's offsets are stored before the next round's counts
  }
}

// Stable LSD radix sort of the chunk's valid slots by KV row, 8 bits a pass:
// the items are the slot numbers c = rc * Kw + s in ascending order, so each
// KV row's list comes out in ascending c and the per-row sums of
// bwd_reduce_kernel run in an order fixed by the inputs alone. Per pass a
// digit histogram per tile of 4096 items (bwd_sort_hist_kernel), a scan per
// digit over the tiles (bwd_sort_scan_kernel) and a scatter that ranks each
// item among the equal digits before it in its tile (bwd_sort_scatter_kernel).
constexpr int kSortWaves = 4, kSortIter = 16;
constexpr int kSortTile = kSortWaves * kSortIter * 64;

struct SortPass {
  const int32_t* key_in;  // null on the first pass: the items are the index rows
  const int32_t* val_in;
  int32_t* key_out;       // null on the last pass
  int32_t* val_out;
  int64_t n_items;        // first pass: rows * Kw slot numbers
  int shift;
  int nblk;
};

// Item i of a pass: its key (KV row) and value (slot number) when valid.
__device__ __forceinline__ bool sort_item(const BwdArgs& a, const SortPass& p, int64_t i,
                                          int32_t n_valid, int32_t& key, int32_t& val) {
  if (!p.key_in) {
    if (i >= p.n_items) return false;
    const int64_t rc = i / a.Kw;
    const int s = (int)(i - rc * a.Kw);
    const int64_t t = a.row0 + rc;
    if (s >= row_len(a, t)) return false;
    key = a.indices[t * a.ld_idx + s];
    val = (int32_t)i;
    return key >= 0 && key < a.T_kv;
  }
  if (i >= n_valid) return false;
  key = p.key_in[i];
  val = p.val_in[i];
  return true;
}

__global__ __launch_bounds__(256) void bwd_sort_hist_kernel(BwdArgs a, SortPass p) {
  __shared__ uint32_t s_h[256];
  const int tid = threadIdx.x;
  s_h[tid] = 0;
  __syncthreads();
  const int32_t n_valid = p.key_in ? a.offs[a.T_kv] : 0;
  const int64_t base = (int64_t)blockIdx.x * kSortTile;
  for (int k = 0; k < kSortTile / 256; ++k) {
    int32_t key, val;
    if (sort_item(a, p, base + 256 * k + tid, n_valid, key, val))
      atomicAdd(&s_h[(key >> p.shift) & 255], 1u);
  }
  __syncthreads();
  a.sort_hist[(int64_t)tid * p.nblk + blockIdx.x] = s_h[tid];
}

// In place: hist[d][b] = the items of digit d in tiles before b; tot[d] = all.
__global__ __launch_bounds__(256) void bwd_sort_scan_kernel(BwdArgs a, SortPass p) {
  __shared__ uint32_t s_w[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t* h = a.sort_hist + (int64_t)blockIdx.x * p.nblk;
  uint32_t carry = 0;
  for (int b0 = 0; b0 < p.nblk; b0 += 256) {
    const int i = b0 + tid;
    const uint32_t v = i < p.nblk ? h[i] : 0u;
    uint32_t incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    if (lane == 63) s_w[wave] = incl;
    __syncthreads();
    uint32_t before = carry;
    for (int w = 0; w < wave; ++w) before += s_w[w];
    if (i < p.nblk) h[i] = before + incl - v;
    carry += s_w[0] + s_w[1] + s_w[2] + s_w[3];
    __syncthreads();
  }
  if (tid == 0) a.sort_tot[blockIdx.x] = carry;
}

__global__ __launch_bounds__(256) void bwd_sort_scatter_kernel(BwdArgs a, SortPass p) {
  __shared__ uint32_t s_cnt[kSortWaves][256];  // per wave: items of each digit so far
  __shared__ uint32_t s_base[256];
  __shared__ uint32_t s_w[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t n_valid = p.key_in ? a.offs[a.T_kv] : 0;
  const int64_t tile0 = (int64_t)blockIdx.x * kSortTile;
  if (p.key_in && tile0 >= n_valid) return;  // uniform
#pragma unroll
  for (int w = 0; w < kSortWaves; ++w) s_cnt[w][tid] = 0;
  {
    // digit d's first output position in this tile: all smaller digits plus
    // digit d's items in earlier tiles
    const uint32_t tot = a.sort_tot[tid];
    uint32_t incl = tot;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    if (lane == 63) s_w[wave] = incl;
    __syncthreads();
    uint32_t before = 0;
    for (int w = 0; w < wave; ++w) before += s_w[w];
    s_base[tid] = before + incl - tot + a.sort_hist[(int64_t)tid * p.nblk + blockIdx.x];
  }
  __syncthreads();
  // Wave w ranks its 1024 consecutive items 64 at a time; lanes with equal
  // digits find each other with one ballot per digit bit.
  const uint64_t below = (1ull << lane) - 1ull;
  const int64_t i0 = tile0 + (int64_t)wave * (kSortIter * 64) + lane;
  int32_t key[kSortIter], val[kSortIter];
  uint32_t rk[kSortIter];
#pragma unroll
  for (int it = 0; it < kSortIter; ++it) {
    const bool ok = sort_item(a, p, i0 + 64 * it, n_valid, key[it], val[it]);
    const uint32_t d = ok ? ((uint32_t)key[it] >> p.shift) & 255u : 0u;
    uint64_t peers = __ballot(ok);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint64_t m = __ballot((d >> b) & 1u);
      peers &= ((d >> b) & 1u) ? m : ~m;
    }
    uint32_t r = 0xffffffffu;
    if (ok) {
      const uint32_t prev = s_cnt[wave][d];
      r = ((prev + (uint32_t)__popcll(peers & below)) << 8) | d;
      if ((peers & below) == 0) s_cnt[wave][d] = prev + (uint32_t)__popcll(peers);
    }
    rk[it] = r;
  }
  __syncthreads();
  {
    uint32_t run = 0;
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) {
      const uint32_t c = s_cnt[w][tid];
      s_cnt[w][tid] = run;
      run += c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < kSortIter; ++it) {
    if (rk[it] == 0xffffffffu) continue;
    const uint32_t d = rk[it] & 255u;
    const uint32_t pos = s_base[d] + s_cnt[wave][d] + (rk[it] >> 8);
    if (pos >= (uint32_t)p.n_items) continue;  // cannot happen: a rank below all items
    if (p.key_out) p.key_out[pos] = key[it];
    p.val_out[pos] = val[it];
  }
}

// dkv_ws[r] += the sum of the rows listed for KV row r (all head parts).
// 256 threads: three rows at a time, 72 threads x 8 columns per row. The
// list entries and rows are loaded U at a time with one head part (clamped
// to the list, the extra ones not added) so that each thread keeps U loads
// in flight; the sums run in list order, head parts in order within each
// entry.
template <int DQK>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs a) {
  constexpr int CPR = DQK / 8;  // 16-byte chunks per row
  constexpr int RPI = 256 / CPR;
  constexpr int U = 8;
  __shared__ float s_acc[RPI][DQK];
  const int64_t r = blockIdx.x;
  const int32_t b = a.offs[r], e = a.offs[r + 1];
  if (b == e) return;  // uniform
  const int tid = threadIdx.x;
  const int ro = tid / CPR, ch = tid - ro * CPR;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  auto add = [&](const u32x4& v) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[2 * k] += bf16_bits_to_f32(v[k] & 0xffffu);
      acc[2 * k + 1] += bf16_bits_to_f32(v[k] >> 16);
    }
  };
  if (ro < RPI && a.nparts == 1) {  // one head part: U entries at a time
    for (int32_t p0 = b + ro; p0 < e; p0 += U * RPI) {
      int64_t c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int32_t p = p0 + u * RPI;
        c[u] = a.list[p < e ? p : e - 1];
      }
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u)  // streaming loads: each row piece is read once
        v[u] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(a.wsC + c[u] * DQK + 8 * ch));
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (p0 + u * RPI < e) add(v[u]);
    }
  } else if (ro < RPI) {  // several head parts, in order within each entry
    const int64_t part_stride = a.chunk_rows * a.Kw;
    for (int32_t p = b + ro; p < e; p += RPI) {
      const int64_t c = a.list[p];
      for (int part = 0; part < a.nparts; ++part)
        add(load16(a.wsC + (c + part * part_stride) * DQK + 8 * ch));
    }
  }
  if (ro < RPI) {
#pragma unroll
    for (int k = 0; k < 8; ++k) s_acc[ro][8 * ch + k] = acc[k];
  }
  __syncthreads();
  for (int d = tid; d < DQK; d += 256) {
    float sum = 0.0f;
#pragma unroll
    for (int k = 0; k < RPI; ++k) sum += s_acc[k][d];
    a.dkv_ws[r * DQK + d] += sum;
  }
}

__global__ __launch_bounds__(256) void bwd_fill_kernel(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

__global__ __launch_bounds__(256) void bwd_convert_kernel(const float* p, uint16_t* o,
                                                          int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) o[i] = (uint16_t)f32_to_bf16_bits(p[i]);
}

// ------------------------------------------------ KV-tile dkv (dense rows) --
// When each row selects a large share of the KV rows, dkv is computed per
// tile of 128 KV rows as a dense product over the query rows that select
// into it, instead of one dkv row per slot:
//   dkv[j] += sum over rows t, heads h of  dS[t, slot_t(j), h] q[t, h]
//                                        + P[t, slot_t(j), h] dout[t, h]
// (zero where row t selects no slot for j). bwd_map_kernel writes, per row,
// the slot that selects each KV row; bwd_merge_kernel folds repeated ids of
// a row into the lowest such slot (sums in ascending slot order), after the
// dq pass has read the per-slot values; bwd_dkv_tile_kernel accumulates one
// (64-row part, KV tile) pair in registers and writes it as an fp32 partial;
// bwd_tile_reduce_kernel adds the parts of each KV row in ascending order.
// No atomics decide any sum, so dkv is reproducible.

// Slot of each KV row for one query row (the lowest slot when an id repeats;
// -1 where none), in windows of 8192 KV rows; rows with a repeated id are
// queued for the merge.
__global__ __launch_bounds__(256) void bwd_map_kernel(BwdArgs a) {
  constexpr int W = 8192;
  __shared__ int32_t s_m[W];
  __shared__ int32_t s_dup;
  const int tid = threadIdx.x;
  const int64_t rc = blockIdx.x;
  const int64_t t = a.row0 + rc;
  const int L = row_len(a, t);
  const int32_t* ix = a.indices + t * a.ld_idx;
  if (tid == 0) s_dup = 0;
  for (int64_t w0 = 0; w0 < a.ld_map; w0 += W) {
    const int nw = (int)(a.ld_map - w0 < W ? a.ld_map - w0 : W);  // a multiple of 128
    for (int j = tid; j < nw; j += 256) s_m[j] = INT32_MAX;
    __syncthreads();
    for (int s = tid; s < L; s += 256) {
      const int32_t v = ix[s];
      if (v >= 0 && v < a.T_kv && v >= w0 && v - w0 < nw) atomicMin(&s_m[v - w0], s);
    }
    __syncthreads();
    for (int s = tid; s < L; s += 256) {
      const int32_t v = ix[s];
      if (v >= 0 && v < a.T_kv && v >= w0 && v - w0 < nw && s_m[v - w0] != s) s_dup = 1;
    }
    uint32_t* out = reinterpret_cast<uint32_t*>(a.map + rc * a.ld_map + w0);
    for (int j = 2 * tid; j < nw; j += 512) {
      const int32_t lo = s_m[j], hi = s_m[j + 1];
      out[j >> 1] = (lo == INT32_MAX ? 0xffffu : (uint32_t)lo) |
                    ((hi == INT32_MAX ? 0xffffu : (uint32_t)hi) << 16);
    }
    __syncthreads();
  }
  if (tid == 0 && s_dup) {
    const uint32_t pos = atomicAdd(a.dup_count, 1u);
    a.dup_rows[pos] = (int32_t)rc;
  }
}

// For each queued row: its (id, slot) pairs sorted (bitonic, in LDS); each
// run of one id with more than one slot is summed in ascending slot order,
// in fp32, into the run's lowest slot (P and dS, every head).
__global__ __launch_bounds__(256) void bwd_merge_kernel(BwdArgs a) {
  constexpr int NMAX = 8192;  // slots per row (k_width rounded up to 32)
  constexpr uint32_t kNone = 0xffffffffu;
  __shared__ uint32_t s_k[NMAX];
  if (blockIdx.x >= *a.dup_count) return;  // uniform
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t rc = a.dup_rows[blockIdx.x];
  const int64_t t = a.row0 + rc;
  const int L = row_len(a, t);
  const int32_t* ix = a.indices + t * a.ld_idx;
  int n2 = 64;
  while (n2 < L) n2 <<= 1;
  for (int i = tid; i < n2; i += 256) {
    uint32_t k = kNone;
    if (i < L) {
      const int32_t v = ix[i];
      if (v >= 0 && v < a.T_kv) k = ((uint32_t)v << 13) | (uint32_t)i;
    }
    s_k[i] = k;
  }
  __syncthreads();
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < n2; i += 256) {
        const int o = i ^ j;
        if (o > i) {
          const uint32_t x = s_k[i], y = s_k[o];
          if ((x > y) == ((i & k) == 0)) {
            s_k[i] = y;
            s_k[o] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  const int hp = (a.H + 31) / 32 * 32;
  uint16_t* P = a.wsP + rc * (int64_t)a.Kw * hp;
  uint16_t* D = a.wsD + rc * (int64_t)a.Kw * hp;
  for (int i = wave; i < n2; i += 4) {
    const uint32_t k = s_k[i];
    if (k == kNone) break;  // the rest are unused
    const uint32_t id = k >> 13;
    if (i > 0 && (s_k[i - 1] >> 13) == id) continue;                       // not a run start
    if (i + 1 >= n2 || s_k[i + 1] == kNone || (s_k[i + 1] >> 13) != id) continue;  // single
    const int rep = (int)(k & 8191u);
    for (int h = lane; h < hp; h += 64) {
      float sp = 0.0f, sd = 0.0f;
      for (int m = i; m < n2 && s_k[m] != kNone && (s_k[m] >> 13) == id; ++m) {
        const int s = (int)(s_k[m] & 8191u);
        sp += bf16_bits_to_f32(P[pds_off(s, h, a.Kw)]);
        sd += bf16_bits_to_f32(D[pds_off(s, h, a.Kw)]);
      }
      P[pds_off(rep, h, a.Kw)] = (uint16_t)f32_to_bf16_bits(sp);
      D[pds_off(rep, h, a.Kw)] = (uint16_t)f32_to_bf16_bits(sd);
    }
  }
}

// One (part of 64 query rows, tile of 128 KV rows) per workgroup, 4 waves.
// C[j][d] over the tile's 128 KV rows and all D_qk dims: wave w holds
// j 0..127 x d 128w .. 128w+127 (4 x 4 blocks of v_mfma_f32_32x32x16_bf16)
// plus, for D_qk = 576, j 32w .. 32w+31 x d 512..575 (2 blocks): 288 fp32
// accumulators, the 256 of the main blocks in AGPRs (the compiler's MFMA),
// the other 32 in VGPRs (the MFMA written inline), so that no accumulator
// moves between the register files inside the loop.
// Per step (one query row, 16 heads) the k = heads operands are staged in
// LDS by asynchronous copies through buffer descriptors:
//   q rows (16 heads x D_qk) and dout rows (16 x 512), each row padded to a
//   stride of 16 dwords modulo 64 banks, so that the transposed reads
//   (ds_read_b64_tr_b16: 8 rows x 64 bytes) meet each bank at most twice --
//   B operands;
//   dS and P of the slot that selects each of the 128 KV rows ([k half][j]
//   16-byte runs, zeros where none) -- A operands, one ds_read_b128 each.
// Three stages; the copies of step s + 3 and the LDS reads of the operands
// overlap the MFMAs (see the step loop). Parts are spread so that the
// tiles of one part run on one XCD (block b on XCD b % 8) and share its L2
// for q and dout.
template <int DQK, int HP>
__global__ __launch_bounds__(256, 1) void bwd_dkv_tile_kernel(BwdArgs a) {
  constexpr int HS = HP / 16;                            // steps per query row
  constexpr int RQ = DQK == 576 ? 608 : 544, RG = 544;   // LDS row strides (elements)
  constexpr int QROWB = DQK * 2, QPADB = RQ * 2, GPADB = RG * 2;
  constexpr int QIN = 16 * QPADB / 1024;                 // copies of the q block (19 or 17)
  constexpr int QREG = 19 * 1024, GREG = 17 * 1024, AOFF = QREG + GREG;
  constexpr int STAGE = AOFF + 8192;
  constexpr int NST = 3;
  constexpr int R = kBwdTileRows, BJ = kBwdTileKV;
  constexpr int NX = DQK == 576 ? 2 : 0;      // blocks of dims 512..575 per wave
  constexpr uint32_t OOB = 0x80000000u;       // past every descriptor: reads zeros
  static_assert(16 * QPADB % 1024 == 0 && QIN <= 19 && 16 * GPADB == GREG, "stage layout");
  static_assert((QPADB / 4) % 64 == 16 || (QPADB / 4) % 64 == 48, "q row stride");
  static_assert((GPADB / 4) % 64 == 16, "dout row stride");
  __shared__ __attribute__((aligned(16))) unsigned char smem[NST * STAGE];
  __shared__ __attribute__((aligned(16))) int16_t s_map[R * BJ];
  __shared__ int32_t s_rows[R];
  __shared__ int32_t s_flag[R];
  __shared__ int32_t s_nrows;

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, r32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nj = (int)(a.ld_map / BJ);
  const int64_t n = a.T_q - a.row0 < a.chunk_rows ? a.T_q - a.row0 : a.chunk_rows;
  const int np = (int)((n + R - 1) / R);
  const int item = (int)(blockIdx.x >> 3);
  const int p = 8 * (item / nj) + (int)(blockIdx.x & 7);
  const int J = item % nj;
  if (p >= np) return;  // uniform
  const int64_t rbeg = (int64_t)p * R;
  const int nr = (int)(n - rbeg < R ? n - rbeg : R);

  // the part's map rows over this tile; rows that select into it
  for (int c = tid; c < R * 16; c += 256) {
    const int r = c >> 4, ch = c & 15;
    const u32x4 v = r < nr ? load16(a.map + (rbeg + r) * a.ld_map + (int64_t)J * BJ + 8 * ch)
                           : u32x4{~0u, ~0u, ~0u, ~0u};
    *reinterpret_cast<u32x4*>(s_map + r * BJ + 8 * ch) = v;
  }
  __syncthreads();
  for (int r = wave; r < R; r += 4) {
    const uint32_t v = reinterpret_cast<const uint32_t*>(s_map + r * BJ)[lane];
    const uint64_t any = __ballot(v != 0xffffffffu);
    if (lane == 0) s_flag[r] = any != 0;
  }
  __syncthreads();
  if (wave == 0) {
    const bool f = s_flag[lane] != 0;
    const uint64_t m = __ballot(f);
    if (f) s_rows[__popcll(m & ((1ull << lane) - 1ull))] = lane;
    if (lane == 0) s_nrows = __popcll(m);
  }
  __syncthreads();
  const int nrows = s_nrows;
  const int rows_v = lane < nrows ? s_rows[lane] : 0;  // lane i: i-th selecting row
  if (tid == 0) a.part_flag[(int64_t)p * nj + J] = nrows > 0 ? 1 : 0;
  if (nrows == 0) return;  // uniform

  // this wave's nine q / dout copies of a stage: copy k = wave + 4i covers
  // 1 KiB of the padded LDS block; rel = its lane's byte offset from the
  // step's first head row in global memory (OOB for padding)
  uint32_t rel[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    const int k = wave + 4 * i;
    if (k < 19) {
      const int b = 1024 * k + 16 * lane, r = b / QPADB, cb = b - r * QPADB;
      rel[i] = (k < QIN && cb < QROWB) ? (uint32_t)(r * QROWB + cb) : OOB;
    } else {
      const int b = 1024 * (k - 19) + 16 * lane, r = b / GPADB, cb = b - r * GPADB;
      rel[i] = cb < 1024 ? (uint32_t)(r * 1024 + cb) : OOB;
    }
  }
  const uint32_t lds0 = lds_addr(smem);
  const int64_t slab = (int64_t)a.Kw * HP;  // P / dS elements per chunk row
  const int S = nrows * HS;
  // prep(s): a step's descriptors, LDS stage and this lane's dS / P offset,
  // set up a step ahead of its copies. Steps past the last get descriptors of
  // no bytes: their copies read nothing and write zeros into a free stage, so
  // every step issues the same 11 copies per wave.
  struct Copies {
    i32x4 rq, rg, rD, rP;
    uint32_t base, va;
  };
  auto prep = [&](int s) {
    Copies c;
    const bool live = s < S;
    const int ri = live ? s / HS : 0, hg = s % HS;
    const int rl = __builtin_amdgcn_readlane(rows_v, ri);
    const int slot = s_map[rl * BJ + 32 * wave + r32];
    const int64_t rc = rbeg + rl, t = a.row0 + rc;
    const int h0 = 16 * hg, hl = live && a.H - h0 > 0 ? a.H - h0 : 0;  // heads left from h0
    c.rq = buffer_rsrc_words(a.q + (t * a.H + h0) * DQK, (uint32_t)(hl * QROWB));
    c.rg = buffer_rsrc_words(a.dout + (t * a.H + h0) * 512, (uint32_t)(hl * 1024));
    c.rD = buffer_rsrc_words(a.wsD + rc * slab, live ? (uint32_t)(slab * 2) : 0u);
    c.rP = buffer_rsrc_words(a.wsP + rc * slab, live ? (uint32_t)(slab * 2) : 0u);
    c.base = lds0 + (uint32_t)((s % NST) * STAGE);
    c.va = slot >= 0 ? (uint32_t)pds_off(slot, h0 + 8 * half, a.Kw) * 2u : OOB;
    return c;
  };
  // copy i of this wave: 0..8 the q / dout copies, 9 dS, 10 P
  auto copy = [&](const Copies& c, auto ic) {
    constexpr int i = decltype(ic)::value;
    if constexpr (i < 9) {
      const int k = wave + 4 * i;
      const bool isq = k < 19;
      const i32x4 r = isq ? c.rq : c.rg;
      const uint32_t lo = isq ? 1024u * (uint32_t)k : (uint32_t)QREG + 1024u * (uint32_t)(k - 19);
      dma16_buf_imm<0>(rel[i], r, c.base + lo);
    } else if constexpr (i == 9) {
      dma16_buf_imm<0>(c.va, c.rD, c.base + (uint32_t)AOFF + 1024u * (uint32_t)wave);
    } else {
      dma16_buf_imm<0>(c.va, c.rP, c.base + (uint32_t)AOFF + 4096u + 1024u * (uint32_t)wave);
    }
  };

  const int G = lane >> 4, li = lane & 15;
  const int rsel = 8 * (G >> 1) + (li >> 2);
  const int csel = 16 * (G & 1) + 4 * (li & 3);
  f32x16 acc[4][4];
  f32x16 accx[NX > 0 ? NX : 1];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[m][b] = f32x16{};
#pragma unroll
  for (int e = 0; e < (NX > 0 ? NX : 1); ++e) accx[e] = f32x16{};

  // Each step is two halves: the dS q products (18 MFMAs for D_qk = 576)
  // on operand set X, then the P dout products (16) on set Y. Each set is
  // read from LDS while the other half multiplies: Y of step s during its
  // first half, X of step s + 1 during its second half, after the barrier in
  // the middle of step s (own copies of step s + 1 waited for; every wave's
  // reads of step s ended). The 11 copies of step s + 3 go into the stage of
  // step s between the MFMAs from that barrier to the next one: 6 in the
  // second half of step s, 5 in the first half of step s + 1.
  // X: dS of m-blocks 0..3 (0..3), dS of m-block w (4), q blocks (5..8),
  // q dims 512.. (9, 10); Y: P of m-blocks 0..3 (0..3), dout blocks (4..7).
  constexpr int NXR = 9 + NX, NYR = 8;
  auto load_x = [&](int s, u32x4* X) {
    const unsigned char* st = smem + (s % NST) * STAGE;
    const uint16_t* sq = reinterpret_cast<const uint16_t*>(st);
#pragma unroll
    for (int m = 0; m < 4; ++m)
      X[m] = *reinterpret_cast<const u32x4*>(st + AOFF + 1024 * m + 16 * lane);
    if constexpr (NX > 0)
      X[4] = *reinterpret_cast<const u32x4*>(st + AOFF + 1024 * wave + 16 * lane);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint16_t* qb = sq + rsel * RQ + 32 * (4 * wave + b) + csel;
      const u32x2 q0 = lds_read_tr16(qb), q1 = lds_read_tr16(qb + 4 * RQ);
      X[5 + b] = u32x4{q0.x, q0.y, q1.x, q1.y};
    }
#pragma unroll
    for (int e = 0; e < NX; ++e) {
      const uint16_t* qb = sq + rsel * RQ + 512 + 32 * e + csel;
      const u32x2 q0 = lds_read_tr16(qb), q1 = lds_read_tr16(qb + 4 * RQ);
      X[9 + e] = u32x4{q0.x, q0.y, q1.x, q1.y};
    }
  };
  auto load_y = [&](int s, u32x4* Y) {
    const unsigned char* st = smem + (s % NST) * STAGE;
    const uint16_t* sg = reinterpret_cast<const uint16_t*>(st + QREG);
#pragma unroll
    for (int m = 0; m < 4; ++m)
      Y[m] = *reinterpret_cast<const u32x4*>(st + AOFF + 4096 + 1024 * m + 16 * lane);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint16_t* gb = sg + rsel * RG + 32 * (4 * wave + b) + csel;
      const u32x2 g0 = lds_read_tr16(gb), g1 = lds_read_tr16(gb + 4 * RG);
      Y[4 + b] = u32x4{g0.x, g0.y, g1.x, g1.y};
    }
  };
  // first half: copies 6..10 of c after MFMAs 1, 4, 7, 10, 13
  auto mfma_x = [&](const u32x4* X, const Copies& c) {
    static_for<16 + NX>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      if constexpr (j < 16) {
        constexpr int b = j / 4, m = j % 4;
        acc[m][b] = mfma32x32x16(X[m], X[5 + b], acc[m][b]);
      } else {
        constexpr int e = j - 16;
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(accx[e]) : "v"(X[4]), "v"(X[9 + e]));
      }
      if constexpr (j % 3 == 1 && j / 3 < 5) copy(c, std::integral_constant<int, 6 + j / 3>{});
    });
  };
  // second half: copies 0..5 of c after MFMAs 0, 3, 6, 9, 12, 15
  auto mfma_y = [&](const u32x4* Y, const Copies& c) {
    static_for<16>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      constexpr int b = j / 4, m = j % 4;
      acc[m][b] = mfma32x32x16(Y[m], Y[4 + b], acc[m][b]);
      if constexpr (j % 3 == 0) copy(c, std::integral_constant<int, j / 3>{});
    });
  };
  u32x4 X[NXR], Y[NYR];
  Copies cw = prep(2);
  {
    const Copies c0 = prep(0), c1 = prep(1);
    static_for<11>([&](auto ic) { copy(c0, ic); });
    static_for<11>([&](auto ic) { copy(c1, ic); });
    static_for<6>([&](auto ic) { copy(cw, ic); });
  }
  wait_vmcnt_le<17>();  // this wave's copies of step 0 are in LDS
  __syncthreads();
  load_x(0, X);
  for (int s = 0; s < S; ++s) {
    // (scheduling barriers: the MFMAs of a half stay on their side of the
    // workgroup barrier, with the other set's reads issued ahead of them)
    const Copies cn = prep(s + 3);
    load_y(s, Y);
    mfma_x(X, cw);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt_le<11>();  // this wave's copies of step s + 1 are in LDS
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    cw = cn;
    load_x(s + 1, X);  // past the last step: unused values
    mfma_y(Y, cw);
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_vmcnt0();  // the copies issued past the last step

  if constexpr (NX > 0)  // wait states before VALU reads of the inline MFMA results
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(accx[0]), "+v"(accx[1]));
  float* out = a.part + ((int64_t)p * a.ld_map + (int64_t)J * BJ) * DQK;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        out[(int64_t)(32 * m + crow(i, half)) * DQK + 32 * (4 * wave + b) + r32] = acc[m][b][i];
  if constexpr (NX > 0) {
#pragma unroll
    for (int e = 0; e < NX; ++e)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        out[(int64_t)(32 * wave + crow(i, half)) * DQK + 512 + 32 * e + r32] = accx[e][i];
  }
}

// dkv_ws[j] += the written partials of KV row j, in ascending part order.
template <int DQK>
__global__ __launch_bounds__(256) void bwd_tile_reduce_kernel(BwdArgs a) {
  constexpr int C4 = DQK / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.T_kv * C4) return;
  const int64_t j = i / C4;
  const int c = (int)(i - j * C4);
  const int64_t n = a.T_q - a.row0 < a.chunk_rows ? a.T_q - a.row0 : a.chunk_rows;
  const int np = (int)((n + kBwdTileRows - 1) / kBwdTileRows);
  const int nj = (int)(a.ld_map / kBwdTileKV);
  const int J = (int)(j / kBwdTileKV);
  f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int p = 0; p < np; ++p) {
    if (!a.part_flag[(int64_t)p * nj + J]) continue;
    s += *reinterpret_cast<const f32x4*>(a.part + ((int64_t)p * a.ld_map + j) * DQK + 4 * c);
  }
  f32x4* d = reinterpret_cast<f32x4*>(a.dkv_ws + j * DQK + 4 * c);
  *d = *d + s;
}

template <int DQK, int NW>
hipError_t launch_bwd_nw(BwdArgs a, int64_t chunk, hipStream_t st) {
  constexpr int NWD = DQK == 576 ? 6 : 4;
  constexpr int HP = NW * 32;
  constexpr int HC = HP % 64 == 0 ? 64 : 32;
  a.nparts = HP / HC;
  a.chunk_rows = chunk;
  // Buffer-descriptor gathers take 32-bit offsets below 2^31: used whenever
  // every kv byte read lies below that.
  const int64_t span = a.T_kv > 0 ? ((a.T_kv - 1) * a.ld_kv + DQK) * 2 : 0;
  const bool buf = span < ((int64_t)1 << 31) && a.ld_kv * 2 < (1 << 24);
  a.span_kv = buf ? (uint32_t)span : 0u;
  a.row_bytes = buf ? (uint32_t)(a.ld_kv * 2) : 0u;
  for (int64_t r0 = 0; r0 < a.T_q; r0 += chunk) {
    a.row0 = r0;
    const int64_t n = a.T_q - r0 < chunk ? a.T_q - r0 : chunk;
    constexpr int NWC = NW == 3 ? 4 : NW;
    if (!a.tiles && a.T_kv > 0)  // the P / dS pass counts the slots per KV row
      hipLaunchKernelGGL(bwd_fill_kernel, dim3((unsigned)((a.T_kv + 255) / 256)), dim3(256), 0,
                         st, reinterpret_cast<float*>(a.cnt), a.T_kv);
    if (buf)
      hipLaunchKernelGGL((bwd_pds_kernel<DQK, NW, NWC, true>), dim3((unsigned)n), dim3(NWC * 64), 0,
                         st, a);
    else
      hipLaunchKernelGGL((bwd_pds_kernel<DQK, NW, NWC, false>), dim3((unsigned)n),
                         dim3(NWC * 64), 0, st, a);
    if (buf)
      hipLaunchKernelGGL((bwd_dq_ring_kernel<DQK, NW, true>), dim3((unsigned)n), dim3(NW * 128), 0,
                         st, a);
    else
      hipLaunchKernelGGL((bwd_dq_ring_kernel<DQK, NW, false>), dim3((unsigned)n), dim3(NW * 128),
                         0, st, a);
    if (a.tiles) {
      // KV-tile dkv: merge repeated ids after the dq pass has read them
      hipLaunchKernelGGL(bwd_fill_kernel, dim3(1), dim3(256), 0, st,
                         reinterpret_cast<float*>(a.dup_count), (int64_t)1);
      hipLaunchKernelGGL(bwd_map_kernel, dim3((unsigned)n), dim3(256), 0, st, a);
      hipLaunchKernelGGL(bwd_merge_kernel, dim3((unsigned)n), dim3(256), 0, st, a);
      const int64_t nj = a.ld_map / kBwdTileKV;
      const int64_t np = (n + kBwdTileRows - 1) / kBwdTileRows;
      hipLaunchKernelGGL((bwd_dkv_tile_kernel<DQK, HP>), dim3((unsigned)(8 * nj * ((np + 7) / 8))),
                         dim3(256), 0, st, a);
      const int64_t nr = a.T_kv * (DQK / 4);
      hipLaunchKernelGGL((bwd_tile_reduce_kernel<DQK>), dim3((unsigned)((nr + 255) / 256)),
                         dim3(256), 0, st, a);
      continue;
    }
    hipLaunchKernelGGL((bwd_dkv_kernel<DQK, NW, NWD>), dim3((unsigned)(n * (HP / HC))),
                       dim3(NWD * 64), 0, st, a);
    if (a.T_kv > 0) {
      hipLaunchKernelGGL(bwd_scan_kernel, dim3(1), dim3(1024), 0, st, a);
      // keys below T_kv: 8 bits a pass, the last pass writes the list
      const int bits = a.T_kv > 1 ? 32 - __builtin_clz((uint32_t)(a.T_kv - 1)) : 0;
      const int passes = bits > 8 ? (bits + 7) / 8 : 1;
      SortPass p{};
      p.n_items = n * a.Kw;
      p.nblk = (int)((p.n_items + kSortTile - 1) / kSortTile);
      for (int ps = 0; ps < passes; ++ps) {
        const bool last = ps + 1 == passes;
        p.shift = 8 * ps;
        p.key_out = last ? nullptr : a.sort_keys[ps & 1];
        p.val_out = last ? a.list : a.sort_vals[ps & 1];
        hipLaunchKernelGGL(bwd_sort_hist_kernel, dim3((unsigned)p.nblk), dim3(256), 0, st, a, p);
        hipLaunchKernelGGL(bwd_sort_scan_kernel, dim3(256), dim3(256), 0, st, a, p);
        hipLaunchKernelGGL(bwd_sort_scatter_kernel, dim3((unsigned)p.nblk), dim3(256), 0, st, a,
                           p);
        p.key_in = a.sort_keys[ps & 1];
        p.val_in = a.sort_vals[ps & 1];
      }
      hipLaunchKernelGGL((bwd_reduce_kernel<DQK>), dim3((unsigned)a.T_kv), dim3(256), 0, st, a);
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_attn_bwd(BwdArgs a, int64_t chunk, hipStream_t st) {
  const int64_t nkv = a.T_kv * a.D_qk;
  if (nkv) hipLaunchKernelGGL(bwd_fill_kernel, dim3((unsigned)((nkv + 255) / 256)), dim3(256), 0,
                              st, a.dkv_ws, nkv);
  if (a.T_q > 0) {
    const int64_t pairs = a.T_q * a.H;
    hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, st, a);
  }
  if (a.d_sink) {
    if (a.sink && a.T_q > 0)
      hipLaunchKernelGGL(bwd_sink_kernel, dim3((unsigned)a.H), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(bwd_fill_kernel, dim3(1), dim3(256), 0, st, a.d_sink, (int64_t)a.H);
  }
  hipError_t e = hipSuccess;
  if (a.T_q > 0 && a.k_width > 0) {
    const int nw = (a.H + 31) / 32;
#define DSA_BWD_CASE(DD, NN) \
    if (a.D_qk == DD && nw == NN) e = launch_bwd_nw<DD, NN>(a, chunk, st); else
    DSA_BWD_CASE(576, 1) DSA_BWD_CASE(576, 2) DSA_BWD_CASE(576, 3) DSA_BWD_CASE(576, 4)
    DSA_BWD_CASE(512, 1) DSA_BWD_CASE(512, 2) DSA_BWD_CASE(512, 3) DSA_BWD_CASE(512, 4)
    e = hipErrorInvalidValue;
#undef DSA_BWD_CASE
  } else if (a.T_q > 0) {
    // no slot at all: dq is zero
    const int64_t nq = a.T_q * a.H * a.D_qk;
    hipLaunchKernelGGL(bwd_fill_kernel, dim3((unsigned)((nq / 2 + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<float*>(a.dq), nq / 2);
  }
  if (e != hipSuccess) return e;
  if (nkv) hipLaunchKernelGGL(bwd_convert_kernel, dim3((unsigned)((nkv + 255) / 256)), dim3(256),
                              0, st, a.dkv_ws, a.dkv, nkv);
  return hipGetLastError();
}

}  // namespace dsa
