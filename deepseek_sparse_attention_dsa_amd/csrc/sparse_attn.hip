// Sparse MQA / GQA attention forward over gathered KV rows, for gfx950.
//
// Semantics: cuDNN Frontend DSA page, section 1 "Sparse Attention Forward":
// for query row t, head h and valid slot j the score is
// scale * q[t,h,:] . kv[idx[t,j], :]; invalid (-1) and out-of-bounds slots are
// -inf; duplicates are distinct slots; topk_length clamps the valid prefix;
// the per-head sink joins only the output denominator; lse is KV-only; empty
// rows give out = 0, max_logits = -inf, lse = +inf; with D_qk = 576 the value
// rows are the first 512 KV dims. The same kernel serves the block-routed
// sparse GQA of the NeMo cudnn_qsa page (D = 256, separate K and V, one KV
// head shared by 12 query heads).
//
// Mapping: one workgroup per query row, one wave per 32 query heads, all on
// v_mfma_f32_32x32x16_bf16 (the 16x16x32 form runs at half the bf16 rate on
// gfx950).
//  * The wave's 32 heads of Q stay in VGPRs for the whole row as the B
//    operand of S^T = K_tile . Q^T; O[32 heads x D_v] accumulates in fp32
//    registers (1 wave per SIMD: 144 + 256 registers for D_qk = 576).
//  * Tiles of 32 selected KV rows are gathered with asynchronous
//    global -> LDS copies (global_load_lds_dwordx4) into a 2-stage ring: the
//    copy of tile i+1 runs while tile i is computed. Dims [16u, 16u+16) of
//    the 32 rows form 1 KiB block u of 16-byte slots; row r, half h (dims
//    16u + 8h .. +7) sits in slot 32*h + ((r + 4h + 8*(u%2)) mod 32). One
//    copy instruction fills one block, lane l always copying the same row
//    (one per block parity, so no lane looks up another lane's id). With
//    this rotation the q.k operand read of a k-step is 1 KiB in lane order,
//    and the two 16-lane groups of each half-wave of a transposed v read hit
//    disjoint LDS banks. Invalid rows copy from a zero constant, so masked
//    rows hold zeros (0 * V never meets a non-finite value).
//  * p.v reads V straight from the same row-major tile with
//    ds_read_b64_tr_b16 (4 keys x 16 dims per 16-lane group, transposed), so
//    no transposed copy of V is ever written.
//  * Softmax runs in the exp2 domain against a fixed per-head reference: the
//    max of the head's first tile with a valid key. Later logits may exceed
//    it by up to 2^64 (bf16 P and fp32 O/l keep their relative precision at
//    any scale), so O is never rescaled and the accumulators are touched by
//    MFMAs only. If some logit goes further (possible only for extreme
//    inputs), the workgroup runs the row again with the exact row max it has
//    just measured as the reference. Either way the result is the same
//    softmax; only the reference of the exp2 changes.
//  * The epilogue stages bf16 output rows through LDS so the stores are
//    contiguous 16-byte writes.
#include "dsa_device.h"
#include "dsa_launch.h"

#include <type_traits>

namespace dsa {

// Source of the copies for masked rows (one zero row of up to 1024 bf16).
__device__ const u32x4 g_zero_row[128] = {};

namespace {

constexpr int kBN = 32;          // key slots per tile
constexpr float kHeadroom = 64.0f;  // logits may exceed the reference by 2^64
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963387f;

template <int DQK, int DV, bool SHARED, int NW>
struct Cfg {
  static constexpr int NT = NW * 64;
  static constexpr int KS = DQK / 16;                       // q.k k-steps
  static constexpr int NB = DV / 32;                        // p.v column blocks
  static constexpr int K_INST = DQK / 16;                   // copy instructions for K
  static constexpr int V_INST = SHARED ? 0 : DV / 16;       // ... and for a separate V
  static constexpr int INST = K_INST + V_INST;
  static constexpr int K_PER_WAVE = K_INST / NW;            // copies per wave and tile
  static constexpr int V_PER_WAVE = V_INST / NW;
  static constexpr int STAGE_BYTES = INST * 1024;
  static_assert(K_INST % NW == 0 && V_INST % NW == 0, "copies must split evenly over waves");
  static constexpr int V_BASE = SHARED ? 0 : K_INST * 1024; // byte offset of the V slots
  static constexpr int OUT_ROW_U16 = DV + 8;                // staged output row (bf16)
  static constexpr int STAGE_OUT_WAVES =
      (2 * STAGE_BYTES) / (32 * OUT_ROW_U16 * 2) < NW ? (2 * STAGE_BYTES) / (32 * OUT_ROW_U16 * 2)
                                                      : NW;
  static_assert(STAGE_OUT_WAVES >= 1, "stage buffers too small for output staging");
  static_assert(DQK <= 1024 && DV <= 1024, "zero row covers 1024 dims");
};

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1 (compile-time i).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_impl(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<0, N>(f);
}

template <int DQK, int DV, bool SHARED, int NW>
__global__ __launch_bounds__(NW * 64, 1) void sparse_attn_kernel(AttnArgs a) {
  using C = Cfg<DQK, DV, SHARED, NW>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * C::STAGE_BYTES];
  __shared__ float s_red[NW][32];
  __shared__ int s_redo[NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;      // which 8-wide k half of an MFMA operand
  const int r32 = lane & 31;       // MFMA row / column owned by this lane
  const int64_t t = (int64_t)gridDim.x - 1 - blockIdx.x;  // long rows first
  const int h0 = wave * 32;

  const int32_t* idx_row = a.indices + t * a.ld_idx;
  int L = a.k_width;
  if (a.topk_length) {
    const int tl = a.topk_length[t];
    L = tl < 0 ? 0 : (tl > L ? L : tl);
  }
  if (a.T_kv <= 0) L = 0;
  const int n_tiles = (L + kBN - 1) / kBN;

  // Copy lanes: lane l fills slot l of every block, i.e. half h = l/32 of
  // row (l%32 - 4h - 8*(u%2)) mod 32. rowE / rowO are its rows in even / odd
  // blocks.
  const int hcp = lane >> 5;
  const int rowE = ((lane & 31) - 4 * hcp) & 31;
  const int rowO = ((lane & 31) - 4 * hcp - 8) & 31;

  // Raw index of row `row` of the tile starting at slot j0 (-1 past the
  // valid prefix). It is validated only when used, one iteration later: a
  // compare right after the load would make the compiler wait for every
  // outstanding vector-memory operation, the tile copies included.
  auto load_id = [&](int j0, int row) -> int32_t {
    const int j = j0 + row;
    int32_t raw = -1;
    if (j < L) raw = idx_row[j];
    return raw;
  };
  auto valid_id = [&](int32_t raw) -> int32_t {
    return (raw >= 0 && (int64_t)raw < a.T_kv) ? raw : -1;
  };

  // This wave's share of the asynchronous copies of one tile: wave w fills
  // K blocks [w*K_PER_WAVE, (w+1)*K_PER_WAVE) (and the same range of V
  // blocks). Copy j of the share moves one block; its offset within the row
  // goes into the instruction's immediate, which shifts the LDS address as
  // well, hence M0 = block base - offset. The copies of tile i+1 are spread
  // over the q.k MFMAs of tile i so that their issue (back-pressured by the
  // L2 -> LDS path) overlaps matrix work instead of stalling in front of it.
  const uint32_t smem_base = lds_addr(smem);
  struct CopySrc {
    const uint16_t* k0;  // even-parity block source
    const uint16_t* k1;  // odd-parity block source
    const uint16_t* v0;
    const uint16_t* v1;
    uint32_t km0, vm0;
  };
  auto prep_copy = [&](uint32_t stage, int32_t idE, int32_t idO) -> CopySrc {
    CopySrc cs;
    const int hsel = 8 * hcp;
    const uint16_t* zero = reinterpret_cast<const uint16_t*>(g_zero_row) + hsel;
    {
      const int c0 = C::K_PER_WAVE * wave;
      const uint16_t* sE = (idE >= 0 ? a.k + (int64_t)idE * a.ld_k + hsel : zero) + 16 * c0;
      const uint16_t* sO = (idO >= 0 ? a.k + (int64_t)idO * a.ld_k + hsel : zero) + 16 * c0;
      const bool flip = (c0 & 1) != 0;  // block c0 + j has parity (c0 + j) % 2
      cs.k0 = flip ? sO : sE;
      cs.k1 = flip ? sE : sO;
      cs.km0 = __builtin_amdgcn_readfirstlane(stage + 1024u * (uint32_t)c0);
    }
    cs.v0 = cs.v1 = nullptr;
    cs.vm0 = 0;
    if constexpr (!SHARED) {
      const int c0 = C::V_PER_WAVE * wave;
      const uint16_t* sE = (idE >= 0 ? a.v + (int64_t)idE * a.ld_v + hsel : zero) + 16 * c0;
      const uint16_t* sO = (idO >= 0 ? a.v + (int64_t)idO * a.ld_v + hsel : zero) + 16 * c0;
      const bool flip = (c0 & 1) != 0;
      cs.v0 = flip ? sO : sE;
      cs.v1 = flip ? sE : sO;
      cs.vm0 = __builtin_amdgcn_readfirstlane(stage + C::V_BASE + 1024u * (uint32_t)c0);
    }
    return cs;
  };
  constexpr int NCOPY = C::K_PER_WAVE + C::V_PER_WAVE;
  auto copy_one = [&](const CopySrc& cs, auto jc) {
    constexpr int J = decltype(jc)::value;
    if constexpr (J < C::K_PER_WAVE) {
      dma16_imm<32 * J>((J & 1) ? cs.k1 : cs.k0, cs.km0 + 992u * J);
    } else {
      constexpr int U = J - C::K_PER_WAVE;
      dma16_imm<32 * U>((U & 1) ? cs.v1 : cs.v0, cs.vm0 + 992u * U);
    }
  };
  auto copy_all = [&](const CopySrc& cs) {
    static_for<NCOPY>([&](auto jc) { copy_one(cs, jc); });
  };

  // Q fragments (B operand): lane -> head h0 + r32, dims 16*ks + 8*half .. +7.
  u32x4 qf[C::KS];
  {
    const int head = h0 + r32;
    const uint16_t* qrow = a.q + (t * a.H + head) * (int64_t)DQK + 8 * half;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      qf[ks] = (head < a.H) ? load16(qrow + 16 * ks) : u32x4{0u, 0u, 0u, 0u};
  }

  f32x16 o[C::NB];
  float m_ref = -__builtin_inff();   // exp2 reference (log2 units) of head r32
  float m_true = -__builtin_inff();  // true running max of head r32
  float l_run = 0.f;                 // partial sum of exp2(x - m_ref), this lane's keys

  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
      // Some logit exceeded its reference by more than the headroom: run
      // the row again with the exact max (measured in pass 0) as reference.
      bool redo = false;
#pragma unroll
      for (int w = 0; w < NW; ++w) redo |= s_redo[w] != 0;
      if (!redo) break;
      m_ref = m_true;
    }
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[nb][i] = 0.f;
    l_run = 0.f;
    bool overflow = false;

    int32_t idE_next = -1, idO_next = -1;
    uint32_t mask_cur = 0;
    if (n_tiles > 0) {
      const int32_t idE = valid_id(load_id(0, rowE));
      const int32_t idO = valid_id(load_id(0, rowO));
      mask_cur = (uint32_t)ballot(idE >= 0);  // lanes 0..31 hold rows 0..31
      if (pass == 1) __syncthreads();  // pass 0's last tile is consumed by every wave
      copy_all(prep_copy(smem_base, idE, idO));
      if (n_tiles > 1) {
        idE_next = load_id(kBN, rowE);
        idO_next = load_id(kBN, rowO);
      }
    }

    for (int it = 0; it < n_tiles; ++it) {
      wait_vmcnt0();
      __syncthreads();  // every wave's copies of tile it have landed; tile it-1 is consumed
      uint32_t mask_next = 0;
      const bool copy_next = it + 1 < n_tiles;  // uniform over the workgroup
      CopySrc cs{};
      if (copy_next) {
        const int32_t idE = valid_id(idE_next);
        const int32_t idO = valid_id(idO_next);
        mask_next = (uint32_t)ballot(idE >= 0);
        cs = prep_copy(smem_base + ((it + 1) & 1) * C::STAGE_BYTES, idE, idO);
      }
      const unsigned char* tile = smem + (it & 1) * C::STAGE_BYTES;

      // ---- S^T = K_tile . Q^T: lane holds head r32, keys 8*(i/4)+4*half+(i%4) ----
      // Two accumulators (even / odd k-steps) keep consecutive MFMAs independent.
      f32x16 sc, sc1;
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = sc1[i] = 0.f;
      {
        // Operand reads run PF k-steps ahead of the MFMAs that use them.
        // lane reads row r32, half `half` of block ks: slot
        // 32*half + ((r32 + 4*half + 8*(ks%2)) mod 32)
        const unsigned char* kE = tile + (32 * half + ((r32 + 4 * half) & 31)) * 16;
        const unsigned char* kO = tile + (32 * half + ((r32 + 4 * half + 8) & 31)) * 16;
        auto kread = [&](int ks) -> u32x4 {
          return *reinterpret_cast<const u32x4*>(((ks & 1) ? kO : kE) + ks * 1024);
        };
        constexpr int PF = 4;
        u32x4 af[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) af[i] = kread(i);
        static_for<C::KS>([&](auto kc) {
          constexpr int ks = decltype(kc)::value;
          const u32x4 cur = af[ks % PF];
          if constexpr (ks + PF < C::KS) af[ks % PF] = kread(ks + PF);
          if constexpr (ks & 1)
            sc1 = mfma32x32x16(cur, qf[ks], sc1);
          else
            sc = mfma32x32x16(cur, qf[ks], sc);
          // copies j with floor(j * KS / NCOPY) == ks go out at this k-step
          constexpr int j0 = (ks * NCOPY + C::KS - 1) / C::KS;
          constexpr int j1 = ((ks + 1) * NCOPY + C::KS - 1) / C::KS;
          if (copy_next) {
            static_for<j1 - j0>([&](auto dj) {
              copy_one(cs, std::integral_constant<int, j0 + decltype(dj)::value>{});
            });
          }
        });
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[i] += sc1[i];
      }
      if (copy_next) {
        idE_next = (it + 2 < n_tiles) ? load_id((it + 2) * kBN, rowE) : -1;
        idO_next = (it + 2 < n_tiles) ? load_id((it + 2) * kBN, rowO) : -1;
      }

      // ---- softmax weights against the fixed reference, exp2 domain ----
      float x[16];
      float mloc = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i >> 2) + 4 * half + (i & 3);
        const bool ok = (mask_cur >> key) & 1u;
        x[i] = ok ? sc[i] * a.scale_log2 : -__builtin_inff();
        mloc = fmaxf(mloc, x[i]);
      }
      mloc = fmaxf(mloc, shfl_xor_f(mloc, 32));
      m_true = fmaxf(m_true, mloc);
      if (m_ref == -__builtin_inff()) m_ref = mloc;  // first tile with a valid key
      overflow |= mloc > m_ref + kHeadroom;
      const bool live = (m_ref > -__builtin_inff()) && !overflow;
      float p[16];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = fast_exp2(x[i] - m_ref);  // masked keys: exp2(-inf) = 0
        p[i] = live ? p[i] : 0.f;
        psum += p[i];
      }
      l_run += psum;

      // ---- O += P . V ----
      u32x4 pa[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        pa[st][0] = pack_bf16x2(p[8 * st + 0], p[8 * st + 1]);
        pa[st][1] = pack_bf16x2(p[8 * st + 2], p[8 * st + 3]);
        pa[st][2] = pack_bf16x2(p[8 * st + 4], p[8 * st + 5]);
        pa[st][3] = pack_bf16x2(p[8 * st + 6], p[8 * st + 7]);
      }
      {
        // Transposed reads: 16-lane group g reads keys 16*st + 4*(g/2) (+8),
        // dims 32*nb + 16*(g%2); lane i of the group points at key + i/4,
        // dim + 4*(i%4).
        // Row key, dim d lives in block u = d/16 at slot
        // 32*h + ((key + 4h + 8*(u%2)) mod 32), h = (d%16)/8, byte 2*(d%8).
        // Group g reads block 2*nb + g%2, so u%2 = g%2; its lane li reads
        // key + li/4 with dims + 4*(li%4), i.e. h = (li%4)/2, byte 8*(li%2).
        const int g = lane >> 4, li = lane & 15;
        const int vh = (li & 3) >> 1;
        auto vslot = [&](int key) -> int {
          return 32 * vh + ((key + (li >> 2) + 4 * vh + 8 * (g & 1)) & 31);
        };
        // The four transposed reads of column block nb+1 are issued before
        // the two MFMAs of block nb.
        // slot offsets of the 4 key groups used by a column block (st, lo/hi)
        const unsigned char* vb0 = tile + C::V_BASE + (g & 1) * 1024 + 8 * (li & 1);
        const int s00 = vslot(4 * (g >> 1)) * 16, s01 = vslot(8 + 4 * (g >> 1)) * 16;
        const int s10 = vslot(16 + 4 * (g >> 1)) * 16, s11 = vslot(24 + 4 * (g >> 1)) * 16;
        auto vread = [&](int nb, u32x4* vb) {
          const unsigned char* p0 = vb0 + nb * 2048;
          const u32x2 a0 = lds_read_tr16(p0 + s00);
          const u32x2 a1 = lds_read_tr16(p0 + s01);
          const u32x2 b0 = lds_read_tr16(p0 + s10);
          const u32x2 b1 = lds_read_tr16(p0 + s11);
          vb[0] = u32x4{a0.x, a0.y, a1.x, a1.y};
          vb[1] = u32x4{b0.x, b0.y, b1.x, b1.y};
        };
        // Column blocks go in pairs so that consecutive MFMAs never
        // accumulate into the same block; the next pair's reads are issued
        // before the current pair's MFMAs.
        static_assert(C::NB % 2 == 0, "column blocks are processed in pairs");
        u32x4 vcur[4], vnxt[4];
        vread(0, vcur);
        vread(1, vcur + 2);
#pragma unroll
        for (int nb = 0; nb < C::NB; nb += 2) {
          if (nb + 2 < C::NB) {
            vread(nb + 2, vnxt);
            vread(nb + 3, vnxt + 2);
          }
          o[nb] = mfma32x32x16(pa[0], vcur[0], o[nb]);
          o[nb + 1] = mfma32x32x16(pa[0], vcur[2], o[nb + 1]);
          o[nb] = mfma32x32x16(pa[1], vcur[1], o[nb]);
          o[nb + 1] = mfma32x32x16(pa[1], vcur[3], o[nb + 1]);
#pragma unroll
          for (int i = 0; i < 4; ++i) vcur[i] = vnxt[i];
        }
      }
      mask_cur = mask_next;
    }
    if (pass == 0) {
      const bool any = ballot(overflow) != 0;
      if (lane == 0) s_redo[wave] = any ? 1 : 0;
      __syncthreads();
    }
  }

  // ---- epilogue ----
  const float l_tot = l_run + shfl_xor_f(l_run, 32);
  const int head = h0 + r32;
  const bool empty = !(m_ref > -__builtin_inff());
  float inv = 0.f;
  if (!empty) {
    float denom = l_tot;
    if (a.sink && head < a.H) denom += fast_exp2(a.sink[head] * kLog2e - m_ref);
    inv = 1.0f / denom;
  }
  if (half == 0 && head < a.H) {
    a.lse[t * a.H + head] = empty ? __builtin_inff() : (m_ref + fast_log2(l_tot)) * kLn2;
    if (a.max_logits) a.max_logits[t * a.H + head] = empty ? -__builtin_inff() : m_true * kLn2;
  }
  if (lane < 32) s_red[wave][lane] = inv;
  __builtin_amdgcn_s_waitcnt(0xc07f);
  float iv[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(&s_red[wave][8 * j + 4 * half]);
#pragma unroll
    for (int q = 0; q < 4; ++q) iv[4 * j + q] = v[q];
  }

  // Stage bf16 rows [32 heads][DV] in LDS, then store contiguous 16-B chunks.
  constexpr int ROUNDS = (NW + C::STAGE_OUT_WAVES - 1) / C::STAGE_OUT_WAVES;
  constexpr int CH = DV / 8;
  uint16_t* out_stage = reinterpret_cast<uint16_t*>(smem) +
                        (wave % C::STAGE_OUT_WAVES) * 32 * C::OUT_ROW_U16;
#pragma unroll
  for (int round = 0; round < ROUNDS; ++round) {
    const bool mine = wave / C::STAGE_OUT_WAVES == round;
    __syncthreads();
    if (mine) {
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int hr = 8 * (i >> 2) + 4 * half + (i & 3);
          out_stage[hr * C::OUT_ROW_U16 + 32 * nb + r32] =
              __builtin_bit_cast(uint16_t, (__bf16)(o[nb][i] * iv[i]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
    if (mine) {
      for (int c = lane; c < 32 * CH; c += 64) {
        const int hr = c / CH;
        const int cc = c - hr * CH;
        const int hh = h0 + hr;
        if (hh < a.H) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(out_stage + hr * C::OUT_ROW_U16 + 8 * cc);
          *reinterpret_cast<u32x4*>(a.out + (t * a.H + hh) * (int64_t)DV + 8 * cc) = v;
        }
      }
    }
  }
}

template <int DQK, int DV, bool SHARED>
hipError_t launch_cfg(const AttnArgs& a, hipStream_t st) {
  const int nw = (a.H + 31) / 32;
  dim3 grid((unsigned)a.T_q);
  switch (nw) {
    case 1:
      hipLaunchKernelGGL((sparse_attn_kernel<DQK, DV, SHARED, 1>), grid, dim3(64), 0, st, a);
      break;
    case 2:
      hipLaunchKernelGGL((sparse_attn_kernel<DQK, DV, SHARED, 2>), grid, dim3(128), 0, st, a);
      break;
    case 3:
    case 4:
      hipLaunchKernelGGL((sparse_attn_kernel<DQK, DV, SHARED, 4>), grid, dim3(256), 0, st, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_attn(const AttnArgs& a, int D_qk, int D_v, hipStream_t st) {
  if (a.T_q == 0) return hipSuccess;
  const bool shared = (a.v == a.k && a.ld_v == a.ld_k);
  if (D_qk == 576 && D_v == 512 && shared) return launch_cfg<576, 512, true>(a, st);
  if (D_qk == 512 && D_v == 512 && shared) return launch_cfg<512, 512, true>(a, st);
  if (D_qk == 256 && D_v == 256 && shared) return launch_cfg<256, 256, true>(a, st);
  if (D_qk == 256 && D_v == 256 && !shared) return launch_cfg<256, 256, false>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace dsa
