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
//    copy of tile i+1 runs while tile i is computed. A tile is stored as
//    16-byte slots, slot 64*u + 2*r + h holding row r, dims 16*u + 8*h .. +7:
//    one copy instruction moves dims [16u, 16u+16) of all 32 rows, lane l
//    always copies row l/2 (so no lane ever looks up another row's id), the
//    q.k operand read of a k-step is one contiguous 1 KiB block and the
//    transposed v reads touch 4 rows x 32 contiguous bytes: no bank
//    conflicts. Invalid rows copy from a zero constant, so masked rows hold
//    zeros (0 * V never meets a non-finite value).
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

// Bits 0, 2, 4, ... of x packed into bits 0, 1, 2, ...
__device__ __forceinline__ uint32_t even_bits(uint64_t x) {
  x &= 0x5555555555555555ull;
  x = (x | (x >> 1)) & 0x3333333333333333ull;
  x = (x | (x >> 2)) & 0x0F0F0F0F0F0F0F0Full;
  x = (x | (x >> 4)) & 0x00FF00FF00FF00FFull;
  x = (x | (x >> 8)) & 0x0000FFFF0000FFFFull;
  x = (x | (x >> 16)) & 0x00000000FFFFFFFFull;
  return (uint32_t)x;
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

  // Raw index of tile row (lane / 2) for the tile starting at slot j0 (-1
  // past the valid prefix). It is validated only when used, one iteration
  // later: a compare right after the load would make the compiler wait for
  // every outstanding vector-memory operation, the tile copies included.
  auto load_id = [&](int j0) -> int32_t {
    const int j = j0 + (lane >> 1);
    int32_t raw = -1;
    if (j < L) raw = idx_row[j];
    return raw;
  };
  auto valid_id = [&](int32_t raw) -> int32_t {
    return (raw >= 0 && (int64_t)raw < a.T_kv) ? raw : -1;
  };

  // Issue this wave's share of the asynchronous copies of one tile: copy c
  // moves dims [16c, 16c + 16) of the 32 rows, lane l taking row l/2, dims
  // 16c + 8*(l%2) .. +7. Wave w issues copies [w*PER_WAVE, (w+1)*PER_WAVE);
  // each copy's offset within the row goes into the instruction's immediate
  // (which shifts the LDS address as well, hence M0 = slot base - offset).
  const uint32_t smem_base = lds_addr(smem);
  auto issue_tile = [&](uint32_t stage, int32_t id) {
    const int hsel = 8 * (lane & 1);
    const uint16_t* zero = reinterpret_cast<const uint16_t*>(g_zero_row) + hsel;
    {
      const uint16_t* src = (id >= 0 ? a.k + (int64_t)id * a.ld_k + hsel : zero) +
                            16 * C::K_PER_WAVE * wave;
      const uint32_t m0 =
          __builtin_amdgcn_readfirstlane(stage + 1024u * (uint32_t)(C::K_PER_WAVE * wave));
      static_for<C::K_PER_WAVE>([&](auto u) {
        dma16_imm<32 * decltype(u)::value>(src, m0 + 992u * decltype(u)::value);
      });
    }
    if constexpr (!SHARED) {
      const uint16_t* src = (id >= 0 ? a.v + (int64_t)id * a.ld_v + hsel : zero) +
                            16 * C::V_PER_WAVE * wave;
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(
          stage + C::V_BASE + 1024u * (uint32_t)(C::V_PER_WAVE * wave));
      static_for<C::V_PER_WAVE>([&](auto u) {
        dma16_imm<32 * decltype(u)::value>(src, m0 + 992u * decltype(u)::value);
      });
    }
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

    int32_t id_next = -1;
    uint32_t mask_cur = 0;
    if (n_tiles > 0) {
      const int32_t id0 = valid_id(load_id(0));
      mask_cur = even_bits(ballot(id0 >= 0));
      if (pass == 1) __syncthreads();  // pass 0's last tile is consumed by every wave
      issue_tile(smem_base, id0);
      if (n_tiles > 1) id_next = load_id(kBN);
    }

    for (int it = 0; it < n_tiles; ++it) {
      wait_vmcnt0();
      __syncthreads();  // every wave's copies of tile it have landed; tile it-1 is consumed
      uint32_t mask_next = 0;
      if (it + 1 < n_tiles) {
        const int32_t idn = valid_id(id_next);
        mask_next = even_bits(ballot(idn >= 0));
        issue_tile(smem_base + ((it + 1) & 1) * C::STAGE_BYTES, idn);
        id_next = (it + 2 < n_tiles) ? load_id((it + 2) * kBN) : -1;
      }
      const unsigned char* tile = smem + (it & 1) * C::STAGE_BYTES;

      // ---- S^T = K_tile . Q^T: lane holds head r32, keys 8*(i/4)+4*half+(i%4) ----
      f32x16 sc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = 0.f;
      {
        const unsigned char* krow = tile + (2 * r32 + half) * 16;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const u32x4 af = *reinterpret_cast<const u32x4*>(krow + ks * 1024);
          sc = mfma32x32x16(af, qf[ks], sc);
          // keep the operand reads a few steps ahead, not all hoisted
          if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
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
        p[i] = live ? fast_exp2(x[i] - m_ref) : 0.f;
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
        // In slot terms: row key, dim d lives at slot 64*(d/16) + 2*key +
        // (d%16)/8, byte 2*(d%8).
        const int g = lane >> 4, li = lane & 15;
        const unsigned char* vbase = tile + C::V_BASE + (g & 1) * 1024 +
                                     (2 * (4 * (g >> 1) + (li >> 2)) + ((li & 3) >> 1)) * 16 +
                                     8 * (li & 1);
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const unsigned char* p0 = vbase + nb * 2048 + st * 512;
            const u32x2 lo = lds_read_tr16(p0);
            const u32x2 hi = lds_read_tr16(p0 + 256);
            o[nb] = mfma32x32x16(pa[st], u32x4{lo.x, lo.y, hi.x, hi.y}, o[nb]);
          }
          if ((nb & 1) == 1) __builtin_amdgcn_sched_barrier(0);
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
              (uint16_t)f32_to_bf16_bits(o[nb][i] * iv[i]);
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
