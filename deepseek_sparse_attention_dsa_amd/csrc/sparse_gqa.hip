// Block-routed sparse GQA forward (D_qk = D_v = 256, separate K and V, at
// most 16 query heads on one KV head), for gfx950.
//
// Semantics: those of sparse_attn_kernel (cuDNN Frontend DSA page, section 1
// "Sparse Attention Forward"; the NeMo cudnn_qsa page's
// cudnn_sparse_gqa_attention for this form): for query row t, head h and
// valid slot j the score is scale * q[t,h,:] . k[idx[t,j], :]; invalid (-1)
// and out-of-range slots are -inf; duplicates are distinct slots;
// topk_length clamps the valid prefix; the per-head sink joins only the
// output denominator; lse is KV-only; an empty row gives out = 0,
// max_logits = -inf, lse = +inf.
//
// Mapping: one wave (one workgroup) per query row, 16-slot tiles, heads on
// the 16 columns of the MFMAs (12 of 16 used by the workload this serves,
// where a 32-head MFMA would use 12 of 32).
//  * S^T = K . Q^T on v_mfma_f32_16x16x32_bf16: lane l supplies key row l%16
//    of the tile and k values 8*(l/16) .. +7 of each 32-wide k-step; k-step
//    ks of lane group g = l/16 takes dims 32*ks + 8*g .. +7 (a permutation
//    of the 256 dims; Q uses the same one). Two accumulator chains (even and
//    odd k-steps).
//  * K and V rows are gathered with asynchronous global -> LDS copies (one
//    1 KB block = 8 key rows x 64 dims per copy, whole 128-byte row
//    segments: consecutive lanes take consecutive 16-byte chunks of a row,
//    which the address unit handles several lanes at a time; loads straight
//    into the MFMA operand layout put a different row in every lane and kept
//    the address unit busy about 40 cycles per 1 KB). The K tile (8 KB) is
//    read into registers as soon as it lands, so one buffer serves it; V
//    (the P.V B operand, keys along k) is read during P.V, from a 2-stage
//    ring of 8 KB tiles.
//  * The S^T output (lane l: head l%16, keys 4*(l/16) .. +3) is exactly the
//    A operand of P.V on v_mfma_f32_16x16x16_bf16 (heads x keys) for the
//    same lane: no exchange.
//  * V is read with ds_read_b64_tr_b16 (4 keys x 16 dims per 16-lane group,
//    transposed). Inside a V block, 32-byte piece q of row r is stored at
//    piece q ^ ((r >> 1) & 3); inside a K block, 16-byte chunk c of row r of
//    key group kg at position c ^ (4*kg + (r >> 1)). Either way the rows of
//    one read (eight 32-byte pieces, or sixteen 16-byte chunks) fall on
//    distinct LDS banks.
//  * Softmax in the exp2 domain against a fixed per-head reference (the max
//    of the first tile with a valid key), O never rescaled; a logit more
//    than 2^64 above the reference makes the row run again with its exact
//    max as the reference, which gives the same softmax.
// 24 KB of LDS and few registers per row put six rows on a CU (at least one
// wave per SIMD, two on half of them), so that one row's memory waits and
// VALU work overlap another's MFMAs; the general kernel's 64 KB per row left
// two of four SIMDs idle.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {
namespace {

constexpr int kGT = 16;           // slots per tile
constexpr int kGD = 256;          // head dim of q, k and v
constexpr int kGStage = kGT * kGD * 2;  // bytes of one K or V tile (8 KB)
constexpr float kGHeadroom = 64.0f;
constexpr float kGLn2 = 0.693147180559945309f;
constexpr float kGLog2e = 1.442695040888963387f;
constexpr uint32_t kGPastRange = 0x80000000u;  // past every descriptor range

// One v_mfma_f32_16x16x16_bf16: D[16x16] = A[16x16] * B[16x16] + C; lane l
// supplies A row l%16 and B column l%16 over k = 4*(l/16) .. +3 and
// receives D column l%16, rows 4*(l/16) .. +3.
__device__ __forceinline__ f32x4 mfma16x16x16(const u32x2& a, const u32x2& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                  __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
void sparse_gqa_kernel(AttnArgs a) {
  // V stages 0 and 1, then the K buffer (24 KB; the epilogue reuses it for
  // the output rows and the normalisers)
  __shared__ __attribute__((aligned(1024))) unsigned char smem[3 * kGStage];
  float* const s_inv = reinterpret_cast<float*>(smem + kGStage);

  const int lane = threadIdx.x;
  const int hl = lane & 15;   // head (S^T column, P.V A row); key row of the tile
  const int g = lane >> 4;    // k group of the MFMA operands
  const int64_t t = (int64_t)gridDim.x - 1 - blockIdx.x;

  const int32_t* idx_row = a.indices + t * a.ld_idx;
  int L = a.k_width;
  if (a.topk_length) {
    const int tl = a.topk_length[t];
    L = tl < 0 ? 0 : (tl > L ? L : tl);
  }
  if (a.T_kv <= 0) L = 0;
  const int n_tiles = (L + kGT - 1) / kGT;

  // Lane l tracks slot l % 16 of a tile. The raw id is validated one tile
  // after its load (a compare right after a load would wait for every
  // outstanding load, the copies included).
  auto load_id = [&](int j0) -> int32_t {
    const int j = j0 + hl;
    return j < a.k_width ? idx_row[j] : -1;
  };
  auto valid_id = [&](int32_t raw, int j) -> int32_t {
    return (j < L && raw >= 0 && (int64_t)raw < a.T_kv) ? raw : -1;
  };

  const i32x4 rk = buffer_rsrc_words(a.k, a.span_k);
  const i32x4 rv = buffer_rsrc_words(a.v, a.span_v);
  const uint32_t smem_base = lds_addr(smem);
  const uint32_t kbuf = smem_base + 2 * kGStage;

  // K copies of one tile into the K buffer: block (segment s, key group kg)
  // at byte 1024 * (2s + kg); lane p of a copy fills slot p = 8r + pos with
  // chunk (pos ^ (4kg + (r >> 1))) of key row 8kg + r.
  auto copy_k = [&](int32_t idv) {
    const int r = lane >> 3;
#pragma unroll
    for (int kg = 0; kg < 2; ++kg) {
      const int32_t id = __shfl(idv, 8 * kg + r, kWave);
      const uint32_t chunk = (uint32_t)((lane & 7) ^ (4 * kg + (r >> 1)));
      const uint32_t koff = id >= 0 ? __umul24((uint32_t)id, a.row_bytes_k) + 16u * chunk
                                    : kGPastRange;
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(kbuf + 1024u * kg);
      dma16_buf_imm<0>(koff, rk, m0);
      dma16_buf_imm<128>(koff, rk, m0 + 2048u - 128u);
      dma16_buf_imm<256>(koff, rk, m0 + 4096u - 256u);
      dma16_buf_imm<384>(koff, rk, m0 + 6144u - 384u);
    }
  };
  // K fragments of the tile in the K buffer: k-step ks: key row hl, dims
  // 32ks + 8g .. +7 = chunk c = 4ks + g of segment c / 8.
  u32x4 kf[8];
  const unsigned char* const kb = smem + 2 * kGStage;
  const int kkg = hl >> 3, kr = hl & 7;
  const unsigned char* const krow = kb + 1024 * kkg + 128 * kr;
  const int ksw = 4 * kkg + (kr >> 1);
  auto read_k = [&]() {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int c = 4 * ks + g;
      kf[ks] = *reinterpret_cast<const u32x4*>(krow + 2048 * (c >> 3) + 16 * ((c & 7) ^ ksw));
    }
  };
  // V copies of one tile into stage `stage`: block (segment s, key group kg)
  // at byte 1024 * (2s + kg); lane p of a copy fills slot p = 8r + pos with
  // chunk (pos ^ 2*((r >> 1) & 3)) of key row 8kg + r.
  auto copy_v = [&](int32_t idv, uint32_t stage) {
    const int r = lane >> 3;
    const uint32_t chunk = (uint32_t)((lane & 7) ^ (2 * ((r >> 1) & 3)));
#pragma unroll
    for (int kg = 0; kg < 2; ++kg) {
      const int32_t id = __shfl(idv, 8 * kg + r, kWave);
      const uint32_t voff = id >= 0 ? __umul24((uint32_t)id, a.row_bytes_v) + 16u * chunk
                                    : kGPastRange;
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(stage + 1024u * kg);
      dma16_buf_imm<0>(voff, rv, m0);
      dma16_buf_imm<128>(voff, rv, m0 + 2048u - 128u);
      dma16_buf_imm<256>(voff, rv, m0 + 4096u - 256u);
      dma16_buf_imm<384>(voff, rv, m0 + 6144u - 384u);
    }
  };

  // Q fragments (B operand of S^T): head hl, dims 32ks + 8g .. +7.
  u32x4 qf[8];
  {
    const int hq = hl < a.H ? hl : a.H - 1;
    const uint16_t* qrow = a.q + (t * a.H + hq) * (int64_t)kGD + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = load16(qrow + 32 * ks);
    if (hl >= a.H) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qf[ks] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  const float sink_logit = (a.sink && hl < a.H) ? a.sink[hl] : -__builtin_inff();

  // P.V transposed reads: for dim block nb (16 dims) lane (g, li = hl) points
  // at key row 4g + li/4, dims 16nb + 4(li%4) .. +3: block (nb/4, kg), row
  // r, piece (nb%4) ^ ((r >> 1) & 3), chunk half (li%4)/2, byte 8*(li%2).
  const int vkey = 4 * g + (hl >> 2);
  const int vr = vkey & 7;
  const uint32_t vbase =
      (uint32_t)(1024 * (vkey >> 3) + 128 * vr + 16 * ((hl & 3) >> 1) + 8 * (hl & 1));
  const int vsw = (vr >> 1) & 3;
  auto vread = [&](const unsigned char* stage_ptr, int nb) -> u32x2 {
    return lds_read_tr16(stage_ptr + vbase + 2048 * (nb >> 2) + 32 * ((nb & 3) ^ vsw));
  };

  f32x4 o[16];
  float m_ref = -__builtin_inff();   // exp2 reference of head hl (log2 units)
  float m_lane = -__builtin_inff();  // the lane's running max (scaled, log2 units)
  float l_lane = 0.f;                // the lane's sum of exp2(x - m_ref)

  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
      // some logit exceeded the reference by more than the headroom: run
      // the row again with its exact max as the reference
      float m = __builtin_elementwise_maximum(m_lane, shfl_xor_f(m_lane, 16));
      m = __builtin_elementwise_maximum(m, shfl_xor_f(m, 32));
      m_ref = m;
    }
#pragma unroll
    for (int nb = 0; nb < 16; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    l_lane = 0.f;
    bool overflow = false;

    int32_t id_next = -1;
    uint32_t mask_cur = 0;
    if (n_tiles > 0) {
      const int32_t id0 = valid_id(load_id(0), hl);
      mask_cur = (uint32_t)ballot(id0 >= 0) & 0xFFFFu;
      copy_k(id0);
      copy_v(id0, smem_base);
      id_next = load_id(kGT);
    }

    for (int it = 0; it < n_tiles; ++it) {
      // Everything the previous step issued has landed: this tile's K and V
      // rows and the next tile's ids. K goes to registers at once, which
      // frees its buffer for the next tile's copies.
      wait_vmcnt0();
      read_k();
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the K buffer is free
      const unsigned char* stage_ptr = smem + (it & 1) * kGStage;
      // ---- S^T = K . Q^T (even and odd k-steps in two chains) ----
      f32x4 s0 = mfma16x16x32(kf[0], qf[0], f32x4{0.f, 0.f, 0.f, 0.f});
      f32x4 s1 = mfma16x16x32(kf[1], qf[1], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int ks = 2; ks < 8; ks += 2) {
        s0 = mfma16x16x32(kf[ks], qf[ks], s0);
        s1 = mfma16x16x32(kf[ks + 1], qf[ks + 1], s1);
      }
      // ---- the next tile's K loads and V copies, then the ids after it ----
      const bool has_next = it + 1 < n_tiles;  // uniform
      uint32_t mask_next = 0;
      if (has_next) {
        const int32_t idv = valid_id(id_next, (it + 1) * kGT + hl);
        mask_next = (uint32_t)ballot(idv >= 0) & 0xFFFFu;
        copy_k(idv);
        copy_v(idv, smem_base + ((it + 1) & 1) * kGStage);
      }
      id_next = load_id((it + 2) * kGT);

      // ---- softmax weights against the fixed reference ----
      // s0[i] + s1[i]: key 4g + i, head hl
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = (mask_cur >> (4 * g + i)) & 1u;
        x[i] = ok ? (s0[i] + s1[i]) * a.scale_log2 : -__builtin_inff();
      }
      float mt = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[0], x[1]),
                                               __builtin_elementwise_maximum(x[2], x[3]));
      if (ballot(m_ref == -__builtin_inff()) != 0) {  // uniform: no reference yet
        float m = __builtin_elementwise_maximum(mt, shfl_xor_f(mt, 16));
        m = __builtin_elementwise_maximum(m, shfl_xor_f(m, 32));
        m_ref = m;  // -inf while no key of the row was valid
      }
      m_lane = __builtin_elementwise_maximum(m_lane, mt);
      overflow |= mt > m_ref + kGHeadroom;
      const float neg_ref = m_ref == -__builtin_inff() ? 0.f : -m_ref;
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = fast_exp2(x[i] + neg_ref);
        l_lane += p[i];
      }
      const u32x2 pa{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};

      // ---- O += P . V (this tile's V rows landed at the wait above) ----
#pragma unroll
      for (int nb = 0; nb < 16; ++nb) o[nb] = mfma16x16x16(pa, vread(stage_ptr, nb), o[nb]);
      mask_cur = mask_next;
    }
    wait_vmcnt0();
    if (ballot(overflow) == 0) break;  // (pass 1 never overflows: its reference is the max)
  }

  // ---- epilogue ----
  float l_h = l_lane + shfl_xor_f(l_lane, 16);
  l_h += shfl_xor_f(l_h, 32);
  float m_h = __builtin_elementwise_maximum(m_lane, shfl_xor_f(m_lane, 16));
  m_h = __builtin_elementwise_maximum(m_h, shfl_xor_f(m_h, 32));
  const bool empty = !(m_ref > -__builtin_inff());
  float inv = 0.f;
  if (!empty) {
    float denom = l_h;
    if (a.sink && hl < a.H) denom += fast_exp2(sink_logit * kGLog2e - m_ref);
    inv = 1.0f / denom;
  }
  if (g == 0 && hl < a.H) {
    a.lse[t * a.H + hl] = empty ? __builtin_inff() : (m_ref + fast_log2(l_h)) * kGLn2;
    if (a.max_logits) a.max_logits[t * a.H + hl] = empty ? -__builtin_inff() : m_h * kGLn2;
  }
  if (g == 0) s_inv[hl] = inv;
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  float iv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) iv[i] = s_inv[4 * g + i];
  // Stage bf16 rows [16 heads][256 dims] (8 KB) in stage 0, then store
  // contiguous 16-byte chunks of the H real heads. o[nb][i]: head 4g + i,
  // dim 16nb + hl.
  uint16_t* stg = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
  for (int nb = 0; nb < 16; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      stg[(4 * g + i) * kGD + 16 * nb + hl] = (uint16_t)f32_to_bf16_bits(o[nb][i] * iv[i]);
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  uint16_t* out_row = a.out + t * a.H * (int64_t)kGD;
  const int n_chunks = a.H * (kGD / 8);  // 16-byte chunks of the row's output
  for (int c = lane; c < n_chunks; c += 64)
    *reinterpret_cast<u32x4*>(out_row + 8 * c) = *reinterpret_cast<const u32x4*>(stg + 8 * c);
}

}  // namespace

// The GQA form this kernel serves, with K and V spans below 2^31 bytes and
// row strides below 2^24 bytes; anything else returns hipErrorInvalidValue
// (the caller then takes the general kernel).
hipError_t launch_sparse_gqa(AttnArgs a, hipStream_t st) {
  if (a.H < 1 || a.H > 16) return hipErrorInvalidValue;
  auto span = [](int64_t rows, int64_t ld, int dims) -> int64_t {
    return rows > 0 ? ((rows - 1) * ld + dims) * 2 : 0;
  };
  const int64_t sk = span(a.T_kv, a.ld_k, kGD), sv = span(a.T_kv, a.ld_v, kGD);
  const int64_t lim = (int64_t)1 << 31;
  if (!(sk < lim && sv < lim && a.ld_k * 2 < (1 << 24) && a.ld_v * 2 < (1 << 24)))
    return hipErrorInvalidValue;
  a.span_k = (uint32_t)sk;
  a.span_v = (uint32_t)sv;
  a.row_bytes_k = (uint32_t)(a.ld_k * 2);
  a.row_bytes_v = (uint32_t)(a.ld_v * 2);
  if (a.T_q == 0) return hipSuccess;
  hipLaunchKernelGGL(sparse_gqa_kernel, dim3((unsigned)a.T_q), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa
