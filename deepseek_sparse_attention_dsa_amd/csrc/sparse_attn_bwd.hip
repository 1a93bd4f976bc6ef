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
//    (scale folded in) as bf16, slot-major ([row][slot][head]).
//  * bwd_dq_ring_kernel: dq = dS . K with both operands read transposed from
//    LDS (ds_read_b64_tr_b16), two waves per 32-head block splitting the
//    dims; K gathered into the same copy ring as bwd_pds_kernel.
//  * bwd_dkv_kernel: per tile, dS^T . q + P^T . dout (the query's q and dout
//    staged in LDS), each slot's row written once as bf16 (per 64-head part).
//  * bwd_count / bwd_scan: slots per KV row and the offsets of their lists;
//    bwd_sort_{hist,scan,scatter}: a stable radix sort of the chunk's valid
//    slots by KV row, giving each KV row the ascending list of the slot rows
//    written for it (no atomics decide an order, so dkv is reproducible).
//  * bwd_reduce_kernel: one workgroup per KV row sums its list (and parts) in
//    fp32 into the dkv workspace; no atomics touch the data.
//  * bwd_convert_kernel: fp32 workspace -> bf16 dkv.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {
namespace {

constexpr int kBT = 32;  // slots per tile
constexpr float kLog2eB = 1.442695040888963387f;

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
// both written as bf16 to the slot-major workspaces ([row][slot][head]);
// invalid slots and heads past H write zeros. The S chain uses the compiler's
// MFMA (its accumulator in AGPRs, q where the allocator puts it); the dP chain
// is written inline with its accumulator in VGPRs, so that the two
// accumulators and both operand sets fit the register files together, and
// the wait states the compiler would insert before VALU reads of dP are
// given after the chain.
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
  const bool comp = wave < NW;  // uniform
  const int h0 = 32 * wave;
  const int hA = h0 + r32;

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
  float lz2[16], dd[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int h = h0 + crow(i, half);
    lz2[i] = h < a.H ? a.logZ[t * a.H + h] * kLog2eB : __builtin_inff();
    dd[i] = h < a.H ? a.Dsum[t * a.H + h] : 0.0f;
  }
  const float c2 = a.scale * kLog2eB;
  uint16_t* wsP = a.wsP + rc * (int64_t)a.Kw * HP;
  uint16_t* wsD = a.wsD + rc * (int64_t)a.Kw * HP;

  int32_t id_next = id_second;
  uint32_t mask_cur = 0;
  if (n_tiles > 0) {
    const int32_t id0 = valid_id(id_first);
    mask_cur = (uint32_t)ballot(id0 >= 0);
    const CopySrc cs0 = prep_copy(smem_base, id0);
    static_for<NCOPY>([&](auto jc) { copy_one(cs0, jc); });
  }
  for (int it = 0; it < n_tiles; ++it) {
    wait_vmcnt0();
    __syncthreads();  // tile it has landed in every wave's share; tile it-1 is consumed
    uint32_t mask_next = 0;
    const bool copy_next = it + 1 < n_tiles;  // uniform
    CopySrc cs{};
    if (copy_next) {
      const int32_t idv = valid_id(id_next);
      mask_next = (uint32_t)ballot(idv >= 0);
      cs = prep_copy(smem_base + ((it + 1) & 1) * STAGE, idv);
    }
    auto copies_at = [&](auto kc) {  // copies spread over the S k-steps
      constexpr int ks = decltype(kc)::value;
      constexpr int j0 = (ks * NCOPY + KS - 1) / KS, j1 = ((ks + 1) * NCOPY + KS - 1) / KS;
      if (copy_next)
        static_for<j1 - j0>([&](auto dj) {
          copy_one(cs, std::integral_constant<int, j0 + decltype(dj)::value>{});
        });
    };
    const unsigned char* tile = smem + (it & 1) * STAGE;
    f32x16 sacc, dacc;
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
      static_for<KS>([&](auto kc) {
        constexpr int ks = decltype(kc)::value;
        const u32x4 cur = bf[ks % PF];
        if constexpr (ks + PF < KS) bf[ks % PF] = kread(ks + PF);
        sacc = mfma32x32x16(qa[ks], cur, ks == 0 ? f32x16{} : sacc);
        if constexpr (ks == 0)
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(dacc) : "v"(ga[0]), "v"(cur));
        else if constexpr (ks < KV)
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(dacc) : "v"(ga[ks]), "v"(cur));
        copies_at(kc);
      });
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(dacc));
    } else {
      static_for<KS>([&](auto kc) { copies_at(kc); });
    }
    if (copy_next) id_next = (it + 2 < n_tiles) ? load_id((it + 2) * kBT, key_row) : -1;
    if (comp) {
      const int slot = it * kBT + r32;
      const bool valid = (mask_cur >> r32) & 1u;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float pv[4], dv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g + e;
          const float p = valid ? fast_exp2(fmaf(sacc[i], c2, -lz2[i])) : 0.0f;
          pv[e] = p;
          dv[e] = a.scale * p * (dacc[i] - dd[i]);
        }
        const int64_t off = (int64_t)slot * HP + h0 + 8 * g + 4 * half;  // 4 consecutive heads
        *reinterpret_cast<u32x2*>(wsP + off) = u32x2{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])};
        *reinterpret_cast<u32x2*>(wsD + off) = u32x2{pack_bf16x2(dv[0], dv[1]), pack_bf16x2(dv[2], dv[3])};
      }
    }
    mask_cur = mask_next;
  }
}

// ---------------------------------------------------------- dq, ring --
// One workgroup per query row, waves (head block hb = w/2, dim half dh = w%2).
// dq[h][d] on 32x32x16 with k = slots: A = dS (heads x slots) and B = K
// (slots x dims), both read transposed (ds_read_b64_tr_b16). The K tiles are
// gathered into the same swizzled 2-stage ring as bwd_pds_kernel (copies of
// tile i+1 issued by the first min(2*NW, 4) waves between the MFMAs of tile
// i); each tile's dS rows ([slot][head], contiguous in the workspace) are
// loaded one tile ahead into registers and stored to a padded LDS tile.
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
  auto load_ds = [&](int tl) -> u32x4 { return load16(wsD + (int64_t)(tl * kBT + dslot) * HP + 8 * dch); };
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
// 32-dim blocks. C[s][d] on 32x32x16 with k = heads: A = dS^T / P^T
// (slot rows, heads contiguous in the workspace), B = q / dout of the chunk's
// heads read transposed from LDS ([head][dim]). (The transposed product, with
// runs of 4 dims per lane stored 8 bytes at a time, measured slower: its
// stores coalesce less than these 2-byte stores of 32 consecutive dims.)
template <int DQK, int NW, int NWD>
__global__ __launch_bounds__(NWD * 64) void bwd_dkv_kernel(BwdArgs a) {
  constexpr int HP = NW * 32;
  constexpr int HC = HP % 64 == 0 ? 64 : 32;  // heads per chunk (divides HP)
  constexpr int RQ = DQK + 8, RG = 512 + 8;
  constexpr int NBLK = DQK / 32;
  constexpr int BPW = NBLK / NWD;
  static_assert(NBLK % NWD == 0, "dim blocks split evenly over waves");
  __shared__ __attribute__((aligned(16))) uint16_t sq[HC * RQ];
  __shared__ __attribute__((aligned(16))) uint16_t sg[HC * RG];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5, r32 = lane & 31;
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

  // Per tile: wait for everything issued one tile earlier (this tile's A
  // fragments, the stores of two tiles back), then issue the stores of the
  // previous tile and the A loads of the next one, then this tile's MFMAs.
  // A fragments alternate between two register sets, so no move waits on a
  // load in flight.
  constexpr int NK = HC / 16;
  const int ntiles = (L + kBT - 1) / kBT;
  u32x4 adA[NK], apA[NK], adB[NK], apB[NK];
  auto load_a = [&](int tl, u32x4* ad, u32x4* ap) {
    const int64_t srow = (int64_t)(tl * kBT + r32) * HP + hc0 + 8 * half;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      ad[kk] = load16(wsD + srow + 16 * kk);
      ap[kk] = load16(wsP + srow + 16 * kk);
    }
  };
  // C: lane -> dim column, slot rows crow(i); the row of slot s of this head
  // part goes to wsC[part][rc][s] (bf16). pend holds the previous tile's.
  uint16_t* crow_base = a.wsC + ((int64_t)(hc0 / HC) * a.chunk_rows + rc) * a.Kw * DQK;
  uint32_t pend[BPW][16];
  int pend_tl = -1;
  auto store_pending = [&]() {
    if (pend_tl < 0) return;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int s = pend_tl * kBT + crow(i, half);
#pragma unroll
      for (int b = 0; b < BPW; ++b)
        crow_base[(int64_t)s * DQK + (wave * BPW + b) * 32 + r32] = (uint16_t)pend[b][i];
    }
  };
  auto body = [&](int tl, const u32x4* ad, const u32x4* ap, u32x4* nad, u32x4* nap) {
    wait_vmcnt0();
    store_pending();
    if (tl + 1 < ntiles) load_a(tl + 1, nad, nap);
    f32x16 acc[BPW];
#pragma unroll
    for (int b = 0; b < BPW; ++b) acc[b] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {   // 16-head k-steps
#pragma unroll
      for (int b = 0; b < BPW; ++b) {
        const int col = (wave * BPW + b) * 32;
        const uint16_t* qb = sq + (16 * kk + rsel) * RQ + col + csel;
        const u32x2 q0 = lds_read_tr16(qb);
        const u32x2 q1 = lds_read_tr16(qb + 4 * RQ);
        acc[b] = mfma32x32x16(ad[kk], u32x4{q0.x, q0.y, q1.x, q1.y}, acc[b]);
        if (col < 512) {
          const uint16_t* gb = sg + (16 * kk + rsel) * RG + col + csel;
          const u32x2 g0 = lds_read_tr16(gb);
          const u32x2 g1 = lds_read_tr16(gb + 4 * RG);
          acc[b] = mfma32x32x16(ap[kk], u32x4{g0.x, g0.y, g1.x, g1.y}, acc[b]);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < BPW; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) pend[b][i] = f32_to_bf16_bits(acc[b][i]);
    pend_tl = tl;
  };
  __syncthreads();  // q and dout staged
  if (ntiles > 0) load_a(0, adA, apA);
  for (int tl = 0; tl < ntiles;) {
    body(tl, adA, apA, adB, apB);
    if (++tl >= ntiles) break;
    body(tl, adB, apB, adA, apA);
    ++tl;
  }
  store_pending();
}

// ---------------------------------------------- sort of the slots by KV row --
__global__ __launch_bounds__(256) void bwd_count_kernel(BwdArgs a) {
  const int64_t t = a.row0 + blockIdx.x;
  const int L = row_len(a, t);
  for (int s = threadIdx.x; s < L; s += 256) {
    const int32_t v = a.indices[t * a.ld_idx + s];
    if (v >= 0 && v < a.T_kv) atomicAdd(&a.cnt[v], 1);
  }
}

// offs = exclusive prefix sum of cnt (T_kv + 1 entries).
__global__ __launch_bounds__(1024) void bwd_scan_kernel(BwdArgs a) {
  __shared__ int32_t s_w[16];
  __shared__ int32_t s_carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int64_t base = 0; base <= a.T_kv; base += 1024) {
    const int64_t i = base + tid;
    const int32_t v = i < a.T_kv ? a.cnt[i] : 0;
    int32_t incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    if (lane == 63) s_w[wave] = incl;
    __syncthreads();
    int32_t before = s_carry;
    for (int w = 0; w < wave; ++w) before += s_w[w];
    if (i <= a.T_kv) a.offs[i] = before + incl - v;
    __syncthreads();
    if (tid == 1023) s_carry = before + incl;
    __syncthreads();
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
// 256 threads: three rows at a time, 72 threads x 8 columns per row.
template <int DQK>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs a) {
  constexpr int CPR = DQK / 8;  // 16-byte chunks per row
  constexpr int RPI = 256 / CPR;
  __shared__ float s_acc[RPI][DQK];
  const int64_t r = blockIdx.x;
  const int32_t b = a.offs[r], e = a.offs[r + 1];
  if (b == e) return;  // uniform
  const int tid = threadIdx.x;
  const int ro = tid / CPR, ch = tid - ro * CPR;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (ro < RPI) {
    const int64_t part_stride = a.chunk_rows * a.Kw;
    for (int32_t p = b + ro; p < e; p += RPI) {
      const int64_t c = a.list[p];
      for (int part = 0; part < a.nparts; ++part) {
        const u32x4 v = load16(a.wsC + (c + part * part_stride) * DQK + 8 * ch);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[2 * k] += bf16_bits_to_f32(v[k] & 0xffffu);
          acc[2 * k + 1] += bf16_bits_to_f32(v[k] >> 16);
        }
      }
    }
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
    hipLaunchKernelGGL((bwd_dkv_kernel<DQK, NW, NWD>), dim3((unsigned)(n * (HP / HC))),
                       dim3(NWD * 64), 0, st, a);
    if (a.T_kv > 0) {
      hipLaunchKernelGGL(bwd_fill_kernel, dim3((unsigned)((a.T_kv + 255) / 256)), dim3(256), 0,
                         st, reinterpret_cast<float*>(a.cnt), a.T_kv);
      hipLaunchKernelGGL(bwd_count_kernel, dim3((unsigned)n), dim3(256), 0, st, a);
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
