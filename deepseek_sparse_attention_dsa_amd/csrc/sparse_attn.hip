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
//    operand of S^T = K_tile . Q^T (one accumulator chain); O[32 heads x D_v]
//    accumulates in fp32 registers (1 wave per SIMD: 144 + 256 registers for
//    D_qk = 576).
//  * Tiles of 32 selected KV rows are gathered with asynchronous
//    global -> LDS copies (global_load_lds_dwordx4) into a 2-stage ring: the
//    copies of tile i+1 are interleaved with the q.k MFMAs of tile i (during
//    p.v they would compete with the transposed V reads for LDS). Rows
//    8g .. 8g+7 (row group g) and dims 64s .. 64s+63 (segment s) of a tile
//    form the 1 KiB block 4s + g: one copy instruction moves it as eight whole
//    128-byte row segments, consecutive lanes taking consecutive 16-byte
//    chunks of one row (8 cache-line requests, where 32 rows x 32 bytes would
//    need 32; the gather runs about 1.5x faster that way, and only runs of
//    consecutive lanes coalesce). Inside the block, the
//    16-byte chunk c (dims 64s + 8c .. +7) of row 8g + r sits in slot
//    8r + (c ^ f(r, g)) with f = 4*((r>>1)&1) + (r>>2) + 2*(g&1). Under this
//    swizzle a q.k operand read (16 lanes: rows 16m .. 16m+15, one chunk) and
//    a transposed v read (16 or 32 lanes: 4 rows x 2 or 4 chunks) touch
//    every LDS bank at most once. Invalid rows copy from a zero constant, so
//    masked rows hold zeros (0 * V never meets a non-finite value).
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
constexpr int kCopyStart = 0;
constexpr int kCopyTail = 32;
constexpr int kPvGroup = 4;      // column blocks per k-step group of the P.V MFMAs
constexpr float kHeadroom = 64.0f;  // logits may exceed the reference by 2^64
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963387f;

template <int DQK, int DV, bool SHARED, int NW>
struct Cfg {
  static constexpr int NT = NW * 64;
  static constexpr int KS = DQK / 16;                       // q.k k-steps
  static constexpr int NB = DV / 32;                        // p.v column blocks
  static constexpr int K_SEG = DQK / 64;                    // 64-dim segments of a K row
  static constexpr int V_SEG = SHARED ? 0 : DV / 64;        // ... of a separate V row
  static constexpr int K_INST = 4 * K_SEG;                  // copy instructions (1 KiB blocks) for K
  static constexpr int V_INST = 4 * V_SEG;                  // ... and for a separate V
  static constexpr int GPW = 4 / NW;                        // row groups copied per wave
  static constexpr int INST = K_INST + V_INST;
  static constexpr int K_PER_WAVE = K_INST / NW;            // copies per wave and tile
  static constexpr int V_PER_WAVE = V_INST / NW;
  static constexpr int STAGE_BYTES = INST * 1024;
  static_assert(NW == 1 || NW == 2 || NW == 4, "row groups split evenly over waves");
  static_assert(DQK % 64 == 0 && DV % 64 == 0, "rows are copied in 64-dim segments");
  static constexpr int V_BASE = SHARED ? 0 : K_INST * 1024; // byte offset of the V slots
  static constexpr int OUT_ROW_U16 = DV + 8;                // staged output row (bf16)
  static constexpr int STAGE_OUT_WAVES =
      (2 * STAGE_BYTES) / (32 * OUT_ROW_U16 * 2) < NW ? (2 * STAGE_BYTES) / (32 * OUT_ROW_U16 * 2)
                                                      : NW;
  static_assert(STAGE_OUT_WAVES >= 1, "stage buffers too small for output staging");
  static_assert(DQK <= 1024 && DV <= 1024, "zero row covers 1024 dims");
};


template <int DQK, int DV, bool SHARED, int NW, bool BUF>
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

  // Every lane tracks the id of tile row lane % 32 (the key mask needs all
  // 32). As a copy lane, lane l fills slot l of a block: row 8g + (l >> 3),
  // chunk (l & 7) ^ f(l >> 3, g).
  const int key_row = lane & 31;
  const int crow = lane >> 3;
  auto swz = [](int r, int g) -> int { return 4 * ((r >> 1) & 1) + (r >> 2) + 2 * (g & 1); };

  // Raw index of row `row` of the tile starting at slot j0 (-1 past the
  // row's k_width slots; the valid prefix L is applied when the id is
  // validated, so that these loads need not wait for topk_length). It is
  // validated only when used, one iteration later: a compare right after the
  // load would make the compiler wait for every outstanding vector-memory
  // operation, the tile copies included.
  auto load_id = [&](int j0, int row) -> int32_t {
    const int j = j0 + row;
    int32_t raw = -1;
    if (j < a.k_width) raw = idx_row[j];
    return raw;
  };
  // raw: the id of slot j; -1 unless j is inside the valid prefix and the id
  // inside [0, T_kv)
  auto valid_id = [&](int32_t raw, int j) -> int32_t {
    return (j < L && raw >= 0 && (int64_t)raw < a.T_kv) ? raw : -1;
  };

  // This wave's share of the asynchronous copies of one tile: wave w copies
  // row groups g = GPW*w + gi (gi < GPW) of every segment. Copy j of the
  // share moves block (g = GPW*w + j % GPW, s = j / GPW) of K, then the
  // same for a separate V. The segment offset 128*s goes into the
  // instruction's immediate, which shifts the LDS address as well, hence
  // M0 = block base - 128*s.
  const uint32_t smem_base = lds_addr(smem);
  // Copy sources. BUF: 32-bit byte offsets into buffer descriptors over K
  // and V (rows of at most 2^31 bytes in all); a masked row gets an offset
  // past the descriptor's range, which the hardware reads as zeros. Else
  // 64-bit addresses, with masked rows read from a zero constant.
  struct CopySrc {
    const uint16_t* k[BUF ? 1 : C::GPW];  // per row group: this lane's row + chunk
    const uint16_t* v[(BUF || SHARED) ? 1 : C::GPW];
    uint32_t ko[BUF ? C::GPW : 1];
    uint32_t vo[(BUF && !SHARED) ? C::GPW : 1];
    uint32_t m0;                // stage + first block of this wave's groups
  };
  i32x4 rsrc_k{}, rsrc_v{};
  if constexpr (BUF) {
    rsrc_k = buffer_rsrc_words(a.k, a.span_k);
    if constexpr (!SHARED) rsrc_v = buffer_rsrc_words(a.v, a.span_v);
  }
  constexpr uint32_t kPastRange = 0x80000000u;  // > every descriptor range, no wrap
  // idv: validated id of tile row lane % 32 (-1: zero row).
  auto prep_copy = [&](uint32_t stage, int32_t idv) -> CopySrc {
    CopySrc cs;
    int32_t idg[C::GPW];
#pragma unroll
    for (int gi = 0; gi < C::GPW; ++gi)
      idg[gi] = __shfl(idv, 8 * (C::GPW * wave + gi) + crow, kWave);  // all shuffles first
#pragma unroll
    for (int gi = 0; gi < C::GPW; ++gi) {
      const int g = C::GPW * wave + gi;
      const int chunk = (lane & 7) ^ swz(crow, g);
      const bool ok = idg[gi] >= 0;
      if constexpr (BUF) {
        // ids < 2^24 and row strides < 2^24 bytes here (the host checks the
        // span), so one 24-bit multiply-add forms the offset
        // (the multiply-add on every lane and a select, not a branch)
        const uint32_t idu = (uint32_t)idg[gi];
        const uint32_t ko = __umul24(idu, a.row_bytes_k) + 16u * chunk;
        cs.ko[gi] = ok ? ko : kPastRange;
        if constexpr (!SHARED) {
          const uint32_t vo = __umul24(idu, a.row_bytes_v) + 16u * chunk;
          cs.vo[gi] = ok ? vo : kPastRange;
        }
      } else {
        const uint16_t* zero = reinterpret_cast<const uint16_t*>(g_zero_row);
        const uint64_t row = ok ? (uint64_t)(uint32_t)idg[gi] : 0ull;
        cs.k[gi] = (ok ? a.k : zero) + row * (uint64_t)a.ld_k + 8 * chunk;
        if constexpr (!SHARED) cs.v[gi] = (ok ? a.v : zero) + row * (uint64_t)a.ld_v + 8 * chunk;
      }
    }
    cs.m0 = __builtin_amdgcn_readfirstlane(stage + 1024u * (uint32_t)(C::GPW * wave));
    return cs;
  };
  constexpr int NCOPY = C::K_PER_WAVE + C::V_PER_WAVE;
  static_assert(C::K_PER_WAVE == C::GPW * C::K_SEG && C::V_PER_WAVE == C::GPW * C::V_SEG,
                "copy shares");
  auto copy_one = [&](const CopySrc& cs, auto jc) {
    constexpr int J = decltype(jc)::value;
    if constexpr (J < C::K_PER_WAVE) {
      constexpr int GI = J % C::GPW, S = J / C::GPW;
      const uint32_t m0 = cs.m0 + (uint32_t)(1024 * (4 * S + GI) - 128 * S);
      if constexpr (BUF) dma16_buf_imm<128 * S>(cs.ko[GI], rsrc_k, m0);
      else dma16_imm<128 * S>(cs.k[GI], m0);
    } else {
      constexpr int U = J - C::K_PER_WAVE;
      constexpr int GI = U % C::GPW, S = U / C::GPW;
      const uint32_t m0 = cs.m0 + (uint32_t)(C::V_BASE + 1024 * (4 * S + GI) - 128 * S);
      if constexpr (BUF) dma16_buf_imm<128 * S>(cs.vo[GI], rsrc_v, m0);
      else dma16_imm<128 * S>(cs.v[GI], m0);
    }
  };
  auto copy_all = [&](const CopySrc& cs) {
    static_for<NCOPY>([&](auto jc) { copy_one(cs, jc); });
  };
  // The q.k MFMA of one k-step with copy J issued around it: the MFMA sits
  // between the M0 write and the copy, so it is the wait state the copy's M0
  // read needs (copy_one pays an s_nop for it). FIRST: the chain's first
  // MFMA (no accumulator input).
  auto mfma_with_copy = [&](f32x16& acc, const u32x4& ka, const u32x4& qb, const CopySrc& cs,
                            auto jc, auto firstc) {
    constexpr int J = decltype(jc)::value;
    constexpr bool FIRST = decltype(firstc)::value;
    constexpr bool IS_K = J < C::K_PER_WAVE;
    constexpr int U = IS_K ? J : J - C::K_PER_WAVE;
    constexpr int GI = U % C::GPW, S = U / C::GPW;
    constexpr int IMM = 128 * S;
    const uint32_t m0 =
        cs.m0 + (uint32_t)((IS_K ? 0 : C::V_BASE) + 1024 * (4 * S + GI) - 128 * S);
    if constexpr (BUF) {
      uint32_t voff;
      i32x4 rs;
      if constexpr (IS_K) {
        voff = cs.ko[GI];
        rs = rsrc_k;
      } else {
        voff = cs.vo[GI];
        rs = rsrc_v;
      }
      if constexpr (FIRST)
        asm volatile(
            "s_mov_b32 m0, %3\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0\n\t"
            "buffer_load_dwordx4 %4, %5, 0 offen offset:%6 lds"
            : "=v"(acc)
            : "v"(ka), "v"(qb), "s"(m0), "v"(voff), "s"(rs), "i"(IMM)
            : "memory");
      else
        asm volatile(
            "s_mov_b32 m0, %3\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
            "buffer_load_dwordx4 %4, %5, 0 offen offset:%6 lds"
            : "+v"(acc)
            : "v"(ka), "v"(qb), "s"(m0), "v"(voff), "s"(rs), "i"(IMM)
            : "memory");
    } else {
      const uint16_t* gp;
      if constexpr (IS_K) gp = cs.k[GI];
      else gp = cs.v[GI];
      if constexpr (FIRST)
        asm volatile(
            "s_mov_b32 m0, %3\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0\n\t"
            "global_load_lds_dwordx4 %4, off offset:%5"
            : "=v"(acc)
            : "v"(ka), "v"(qb), "s"(m0), "v"(gp), "i"(IMM)
            : "memory");
      else
        asm volatile(
            "s_mov_b32 m0, %3\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
            "global_load_lds_dwordx4 %4, off offset:%5"
            : "+v"(acc)
            : "v"(ka), "v"(qb), "s"(m0), "v"(gp), "i"(IMM)
            : "memory");
    }
  };

  // The first two tiles' ids are loaded before Q (and together with
  // topk_length), so that the first copies can be issued while the Q loads
  // are still in flight.
  const int32_t id_first = load_id(0, key_row);
  const int32_t id_second = load_id(kBN, key_row);

  // Q fragments (B operand): lane -> head h0 + r32, dims 16*ks + 8*half .. +7.
  u32x4 qf[C::KS];
  {
    // Unconditional loads (lanes past the last head read the last head's
    // row, then zero it), so that the compiler's wait for the ids above
    // counts every Q load as issued after them.
    const int head = h0 + r32;
    const int hq = head < a.H ? head : a.H - 1;
    const uint16_t* qrow = a.q + (t * a.H + hq) * (int64_t)DQK + 8 * half;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[ks] = load16(qrow + 16 * ks);
    if (h0 + 32 > a.H) {  // uniform: a partial head block
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        if (head >= a.H) qf[ks] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  // The head's sink logit, loaded now so that its latency is not paid after
  // the last tile.
  const float sink_logit =
      (a.sink && h0 + r32 < a.H) ? a.sink[h0 + r32] : -__builtin_inff();

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

    int32_t id_next = -1;
    uint32_t mask_cur = 0;
    if (n_tiles > 0) {
      const int32_t id0 = valid_id(id_first, key_row);
      mask_cur = (uint32_t)ballot(id0 >= 0);  // lanes 0..31 hold rows 0..31
      if (pass == 1) __syncthreads();  // pass 0's last tile is consumed by every wave
      copy_all(prep_copy(smem_base, id0));
      id_next = id_second;
    }

    for (int it = 0; it < n_tiles; ++it) {
      wait_vmcnt0();
      __syncthreads();  // every wave's copies of tile it have landed; tile it-1 is consumed
      const bool copy_next = it + 1 < n_tiles;  // uniform over the workgroup
      // The copies of tile it+1 go out unconditionally: after the last tile
      // every slot is past the valid prefix, so they fill the free stage
      // with zeros (out-of-range offsets, or the zero row) and no branch per
      // copy is needed. They are waited for before the LDS is reused.
      const int32_t idv = valid_id(id_next, (it + 1) * kBN + key_row);
      const uint32_t mask_next = (uint32_t)ballot(idv >= 0);
      const CopySrc cs = prep_copy(smem_base + ((it + 1) & 1) * C::STAGE_BYTES, idv);
      const unsigned char* tile = smem + (it & 1) * C::STAGE_BYTES;
      constexpr int S0 = kCopyStart;
      constexpr int S1 =
          C::KS + 2 * C::NB - kCopyTail > C::KS ? C::KS + 2 * C::NB - kCopyTail : C::KS;
      constexpr int NSLOT = S1 - S0;
      // copies [j0, j1) of the share go out at slot sl (the q.k k-steps, then
      // the p.v MFMAs): the copies spread evenly over slots S0 .. S1-1
      auto slot_first = [](int slot) constexpr -> int {
        const int sl = slot - S0;
        return sl < 0 ? 0 : sl < NSLOT ? (sl * NCOPY + NSLOT - 1) / NSLOT : NCOPY;
      };
      auto copies_at_slot = [&](auto slotc, auto skipc) {
        constexpr int slot = decltype(slotc)::value;
        constexpr int SKIP = decltype(skipc)::value;  // leading copies already issued
        constexpr int j0 = slot_first(slot) + SKIP, j1 = slot_first(slot + 1);
        static_for<(j1 > j0 ? j1 - j0 : 0)>([&](auto dj) {
          copy_one(cs, std::integral_constant<int, j0 + decltype(dj)::value>{});
        });
      };

      // ---- S^T = K_tile . Q^T: lane holds head r32, keys 8*(i/4)+4*half+(i%4) ----
      // One accumulator chain (dependent MFMAs of one shape issue back to
      // back; a second chain would cost 16 registers and 16 adds per tile).
      // The chain is written as inline MFMAs so that S accumulates in VGPRs:
      // the compiler keeps every MFMA result of this kernel in AGPRs, which
      // O fills completely, and would otherwise move S and one O block
      // between the two files every tile. The wait states that the compiler
      // inserts after its own MFMAs are given explicitly after the chain
      // (the softmax reads S with VALU instructions).
      f32x16 sc;
      {
        // Operand reads run PF k-steps ahead of the MFMAs that use them.
        // k-step ks: the lane reads row r32 (group g = r32/8, r = r32%8),
        // chunk c = 2*(ks%4) + half of segment ks/4, at slot 8r + (c ^ f);
        // c ^ f = 2*((ks%4) ^ (f>>1)) + (half ^ (f&1)).
        const int kg = r32 >> 3, kr = r32 & 7;
        const int kf = swz(kr, kg);
        const unsigned char* kbase = tile + kg * 1024 + kr * 128 + 16 * (half ^ (kf & 1));
        const unsigned char* kq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) kq[q] = kbase + 32 * (q ^ (kf >> 1));
        auto kread = [&](int ks) -> u32x4 {
          return *reinterpret_cast<const u32x4*>(kq[ks & 3] + (ks >> 2) * 4096);
        };
        constexpr int PF = 4;
        u32x4 af[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) af[i] = kread(i);
        static_for<C::KS>([&](auto kc) {
          constexpr int ks = decltype(kc)::value;
          const u32x4 cur = af[ks % PF];
          if constexpr (ks + PF < C::KS) af[ks % PF] = kread(ks + PF);
          constexpr int jf = slot_first(ks);
          constexpr bool with_copy = slot_first(ks + 1) > jf;
          if constexpr (with_copy) {
            // the slot's first copy around the MFMA, any others after it
            mfma_with_copy(sc, cur, qf[ks], cs, std::integral_constant<int, jf>{},
                           std::bool_constant<ks == 0>{});
            copies_at_slot(std::integral_constant<int, ks>{}, std::integral_constant<int, 1>{});
          } else if constexpr (ks == 0) {
            asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(sc) : "v"(cur), "v"(qf[ks]));
          } else {
            asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(sc) : "v"(cur), "v"(qf[ks]));
          }
        });
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(sc));
      }

      if (copy_next) id_next = (it + 2 < n_tiles) ? load_id((it + 2) * kBN, key_row) : -1;

      // ---- softmax weights against the fixed reference, exp2 domain ----
      // Tiles whose 32 slots are all valid (the usual case inside a compact
      // prefix) skip the mask; otherwise masked scores become -inf once, so
      // the max ignores them and their weights come out as exp2(-inf) = 0.
      // Scale and reference fold into one FMA (scale > 0, so the raw max
      // scales to the scaled max). Until some key of the row is valid the
      // reference is -inf and every score of the tile is -inf: any finite
      // offset then gives zero weights. Once a pass has overflowed, its
      // results are discarded and the row is run again, so no select guards
      // the weights against it.
      const bool full = mask_cur == 0xFFFFFFFFu;  // uniform
      if (!full) {
        const uint32_t mh = mask_cur >> (4 * half);  // key 8*(i/4) + 4*half + i%4
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (!((mh >> (8 * (i >> 2) + (i & 3))) & 1u)) sc[i] = -__builtin_inff();
      }
      // The scaled max of the head's 32 scores: the lane's 16 (IEEE maximum,
      // v_maximum3_f32: no NaN quieting of each operand), then the half-wave
      // exchange.
      auto max_of = [&](float m, int i0, int i1) -> float {
#pragma unroll
        for (int i = i0; i < i1; ++i) m = __builtin_elementwise_maximum(m, sc[i]);
        return m;
      };
      // The reference is the max of the first tile with a valid key, so that
      // tile takes its max before the weights. Every tile finishes its max
      // (for max_logits and the headroom check) in the shadow of the first
      // P.V MFMAs; for the reference tile that repeats the same value.
      const bool set_ref = ballot(m_ref == -__builtin_inff()) != 0;  // uniform
      // the lane's max over sc[0..7] now (they become weights first), over
      // all 16 before sc[8..15] become weights
      const float m_lo = max_of(sc[0], 1, 8);
      float m_lo_hi;
      if (set_ref) {
        m_lo_hi = max_of(m_lo, 8, 16);
        const float m = halfwave_max(m_lo_hi) * a.scale_log2;
        if (m_ref == -__builtin_inff()) m_ref = m;
      }
      const float neg_ref = m_ref == -__builtin_inff() ? 0.f : -m_ref;
      float mloc;
      // ---- O += P . V ----
      u32x4 pa[2];
      float psum = 0.f;
      {
        // Transposed reads: for column block nb and key half st, 16-lane
        // group G reads keys 16*st + 8*b + 4*(G/2) .. +3 (b = 0, 1), dims
        // 32*nb + 16*(G%2) .. +15; its lane li points at key + li/4, dims
        // + 4*(li%4). Key 8g + r (g = 2*st + b, r = 4*(G/2) + li/4) and
        // chunk c = 4*(nb%2) + 2*(G%2) + (li%4)/2 of segment nb/2 sit at slot
        // 8r + (c ^ f(r, g)), where
        //   c ^ f = 4*((nb%2) ^ (li/8)) + 2*((G%2) ^ b) + (((li/2)%2) ^ (G/2)).
        const int G = lane >> 4, li = lane & 15;
        const int vr = 4 * (G >> 1) + (li >> 2);
        const unsigned char* vbase =
            tile + C::V_BASE + vr * 128 + 16 * (((li >> 1) & 1) ^ (G >> 1)) + 8 * (li & 1);
        const unsigned char* va[2][2];  // [nb % 2][b]
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int b = 0; b < 2; ++b)
            va[pp][b] = vbase + 1024 * b + 16 * (4 * (pp ^ (li >> 3)) + 2 * ((G & 1) ^ b));
        // The MFMAs run in groups of kPvGroup column blocks: k-step 0 of the
        // group's blocks, then their k-step 1 (MFMA f accumulates block
        // nb = kPvGroup*(f / (2*kPvGroup)) + f % kPvGroup over key half
        // st = (f / kPvGroup) % 2), so the first kPvGroup MFMAs need only the
        // k-step 0 weights and the k-step 1 weights are computed while they
        // run; consecutive MFMAs never accumulate into the same block. (A
        // longer first group would leave more time for them but spills
        // registers.) Its V fragment is read VPF MFMAs ahead.
        auto vfrag = [&](int f) -> u32x4 {
          const int nb = (f / (2 * kPvGroup)) * kPvGroup + f % kPvGroup,
                    st = (f / kPvGroup) % 2;
          const int so = (nb >> 1) * 4096 + st * 2048;
          const u32x2 x0 = lds_read_tr16(va[nb & 1][0] + so);
          const u32x2 x1 = lds_read_tr16(va[nb & 1][1] + so);
          return u32x4{x0.x, x0.y, x1.x, x1.y};
        };
        static_assert(C::NB % kPvGroup == 0, "column blocks come in whole groups");
        constexpr int VPF = 4;
        u32x4 vq[VPF];
#pragma unroll
        for (int i = 0; i < VPF; ++i) vq[i] = vfrag(i);
        __builtin_amdgcn_sched_barrier(0);  // the first V reads go out before the weights
        // Weights of k-step 0 of the P.V product (keys 0..15: sc[0..7]) first;
        // those of k-step 1 (sc[8..15]) are computed under the k-step 0 MFMAs.
        {
          float p[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) p[i] = fast_exp2(fmaf(sc[i], a.scale_log2, neg_ref));
#pragma unroll
          for (int i = 0; i < 8; ++i) psum += p[i];
          pa[0] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                        pack_bf16x2(p[6], p[7])};
        }
        static_for<2 * C::NB>([&](auto fc) {
          constexpr int f = decltype(fc)::value;
          constexpr int nb = (f / (2 * kPvGroup)) * kPvGroup + f % kPvGroup,
                        st = (f / kPvGroup) % 2;
          const u32x4 cur = vq[f % VPF];
          if constexpr (f + VPF < 2 * C::NB) vq[f % VPF] = vfrag(f + VPF);
          o[nb] = mfma32x32x16(pa[st], cur, o[nb]);
          copies_at_slot(std::integral_constant<int, C::KS + f>{}, std::integral_constant<int, 0>{});
          // VALU work in the shadow of this MFMA: the k-step 1 weights (two
          // per MFMA) before MFMA kPvGroup needs them, then the tile max and
          // the weight sum.
          if constexpr (f == 0) m_lo_hi = max_of(m_lo, 8, 16);
          if constexpr (f < kPvGroup) {
            constexpr int i0 = 8 + f * 8 / kPvGroup, i1 = 8 + (f + 1) * 8 / kPvGroup;
#pragma unroll
            for (int i = i0; i < i1; ++i) sc[i] = fast_exp2(fmaf(sc[i], a.scale_log2, neg_ref));
            if constexpr (f == kPvGroup - 1)
              pa[1] = u32x4{pack_bf16x2(sc[8], sc[9]), pack_bf16x2(sc[10], sc[11]),
                            pack_bf16x2(sc[12], sc[13]), pack_bf16x2(sc[14], sc[15])};
          } else if constexpr (f == kPvGroup) {
            mloc = halfwave_max(m_lo_hi) * a.scale_log2;
          } else if constexpr (f == kPvGroup + 1) {
#pragma unroll
            for (int i = 8; i < 16; ++i) psum += sc[i];
          }
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      m_true = __builtin_elementwise_maximum(m_true, mloc);
      overflow |= mloc > m_ref + kHeadroom;
      l_run += psum;
      mask_cur = mask_next;
    }
    // the last tile's zero-filling copies land before any LDS reuse (the
    // next pass's copies, the output staging after the next barrier)
    wait_vmcnt0();
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
    if (a.sink && head < a.H) denom += fast_exp2(sink_logit * kLog2e - m_ref);
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
      // Lane chunk c = lane + 64 * j: head row c / CH, 16-byte chunk c % CH.
      constexpr int PER_LANE = 32 * CH / 64;
      static_assert((32 * CH) % 64 == 0 && PER_LANE % 8 == 0, "store batches");
      if (h0 + 32 <= a.H) {  // uniform: a whole head block, stores in batches of 8
        uint16_t* orow = a.out + (t * a.H + h0) * (int64_t)DV;
#pragma unroll
        for (int j0 = 0; j0 < PER_LANE; j0 += 8) {
          u32x4 v[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int c = lane + 64 * (j0 + j);
            v[j] = *reinterpret_cast<const u32x4*>(out_stage + (c / CH) * C::OUT_ROW_U16 +
                                                   8 * (c % CH));
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int c = lane + 64 * (j0 + j);
            *reinterpret_cast<u32x4*>(orow + (c / CH) * DV + 8 * (c % CH)) = v[j];
          }
        }
      } else {
        for (int c = lane; c < 32 * CH; c += 64) {
          const int hr = c / CH;
          const int cc = c - hr * CH;
          const int hh = h0 + hr;
          if (hh < a.H) {
            const u32x4 v =
                *reinterpret_cast<const u32x4*>(out_stage + hr * C::OUT_ROW_U16 + 8 * cc);
            *reinterpret_cast<u32x4*>(a.out + (t * a.H + hh) * (int64_t)DV + 8 * cc) = v;
          }
        }
      }
    }
  }
}

template <int DQK, int DV, bool SHARED, bool BUF>
hipError_t launch_nw(const AttnArgs& a, hipStream_t st) {
  const int nw = (a.H + 31) / 32;
  dim3 grid((unsigned)a.T_q);
  switch (nw) {
    case 1:
      hipLaunchKernelGGL((sparse_attn_kernel<DQK, DV, SHARED, 1, BUF>), grid, dim3(64), 0, st, a);
      break;
    case 2:
      hipLaunchKernelGGL((sparse_attn_kernel<DQK, DV, SHARED, 2, BUF>), grid, dim3(128), 0, st, a);
      break;
    case 3:
    case 4:
      hipLaunchKernelGGL((sparse_attn_kernel<DQK, DV, SHARED, 4, BUF>), grid, dim3(256), 0, st, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Bytes from a row-major matrix's first element to the end of its last row's
// first `dims` elements (0 without rows).
int64_t row_span(int64_t rows, int64_t ld, int dims) {
  return rows > 0 ? ((rows - 1) * ld + dims) * 2 : 0;
}

template <int DQK, int DV, bool SHARED>
hipError_t launch_cfg(AttnArgs a, hipStream_t st) {
  // Buffer-descriptor copies take 32-bit offsets below kPastRange (2^31):
  // used whenever every K and V byte the kernel reads lies below it.
  const int64_t sk = row_span(a.T_kv, a.ld_k, DQK);
  const int64_t sv = SHARED ? 0 : row_span(a.T_kv, a.ld_v, DV);
  const int64_t lim = (int64_t)1 << 31;
  if (sk < lim && sv < lim && a.ld_k * 2 < (1 << 24) && a.ld_v * 2 < (1 << 24)) {
    a.span_k = (uint32_t)sk;
    a.span_v = (uint32_t)sv;
    a.row_bytes_k = (uint32_t)(a.ld_k * 2);
    a.row_bytes_v = (uint32_t)(a.ld_v * 2);
    return launch_nw<DQK, DV, SHARED, true>(a, st);
  }
  return launch_nw<DQK, DV, SHARED, false>(a, st);
}

}  // namespace

hipError_t launch_sparse_attn(const AttnArgs& a, int D_qk, int D_v, hipStream_t st) {
  if (a.T_q == 0) return hipSuccess;
  const bool shared = (a.v == a.k && a.ld_v == a.ld_k);
  if (D_qk == 576 && D_v == 512 && shared) return launch_cfg<576, 512, true>(a, st);
  if (D_qk == 512 && D_v == 512 && shared) return launch_cfg<512, 512, true>(a, st);
  if (D_qk == 256 && D_v == 256 && shared) return launch_cfg<256, 256, true>(a, st);
  if (D_qk == 256 && D_v == 256 && !shared) {
    // at most 16 heads: the one-wave-per-row kernel of sparse_gqa.hip
    if (a.H <= 16) {
      const hipError_t e = launch_sparse_gqa(a, st);
      if (e != hipErrorInvalidValue) return e;
    }
    return launch_cfg<256, 256, false>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace dsa
