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
// Mapping (one workgroup per query row, one wave per 16 query heads):
//  * Q of the wave's 16 heads stays in VGPRs for the whole row as the B
//    operand of S^T = K_tile . Q^T on v_mfma_f32_16x16x32_bf16, so every lane
//    ends up holding one head's logits for 8 of the 32 keys of a tile.
//  * Each 32-slot tile of gathered KV rows is loaded once per workgroup with
//    16-byte global loads (consecutive lanes read consecutive 16 B of a row)
//    and stored to LDS twice: row-major for q.k, and transposed (dim-major,
//    4 keys per 8-byte write) so that the p.v B operand is two 8-byte LDS
//    reads per lane.
//  * Online softmax in the exp2 domain; the lane's 8 probabilities are
//    exactly its A operand for O += P . V (the key order inside the
//    contraction is permuted identically on both operands).
//  * O[16 heads x D_v] accumulates in fp32 VGPRs; the epilogue applies the
//    sink, writes lse / max_logits, and stages bf16 rows through LDS so the
//    output store is contiguous.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {
namespace {

constexpr int kBN = 32;  // key slots per tile

__device__ __forceinline__ uint32_t half_of(const u32x4& d, int e) {
  const uint32_t w = d[e >> 1];
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

template <int DQK, int DV, bool SHARED, int NW>
__global__ __launch_bounds__(NW * 64, 2) void sparse_attn_kernel(AttnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int KS = DQK / 32;             // q.k MFMA k-steps
  constexpr int NB = DV / 16;              // p.v MFMA column blocks
  constexpr int KROW = DQK / 2 + 4;        // u32 per K row in LDS (16 B pad)
  constexpr int VROW = (kBN + 4) / 2;      // u32 per V^T row in LDS (8 B pad)
  constexpr int NCH = DQK / 8;             // 16-byte chunks per K row
  constexpr int NVCH = DV / 8;             // 16-byte chunks per V row
  constexpr int K_U32 = kBN * KROW;
  constexpr int V_U32 = DV * VROW;
  constexpr int OUT_ROW = DV / 2 + 4;      // u32 per staged output row
  constexpr int TILE_U32 = K_U32 + V_U32;
  constexpr int WAVE_STAGE_U32 = 16 * OUT_ROW;
  // Waves that stage their output rows at the same time (the tile buffer is
  // reused for staging, so large workgroups stage in rounds).
  constexpr int STAGE_WAVES = (TILE_U32 / WAVE_STAGE_U32) < NW ? (TILE_U32 / WAVE_STAGE_U32) : NW;
  static_assert(STAGE_WAVES >= 1, "tile buffer smaller than one wave's output rows");
  constexpr int LDS_U32 = TILE_U32;
  __shared__ uint32_t lds[LDS_U32];
  __shared__ int32_t s_ids[2][kBN];

  uint32_t* ktile = lds;
  uint32_t* vtile = lds + K_U32;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;       // lane group 0..3
  const int c16 = lane & 15;     // position inside the 16-wide MFMA block
  const int64_t t = blockIdx.x;
  const int h0 = wave * 16;

  const int32_t* idx_row = a.indices + t * a.ld_idx;
  int L = a.k_width;
  if (a.topk_length) {
    int tl = a.topk_length[t];
    L = tl < 0 ? 0 : (tl > L ? L : tl);
  }
  auto slot_id = [&](int slot) -> int32_t {
    if (slot >= L) return -1;
    const int32_t id = idx_row[slot];
    return (id >= 0 && (int64_t)id < a.T_kv) ? id : -1;
  };

  // Q fragments: lane -> head h0 + c16, dims 32*ks + 8*g .. +7.
  u32x4 qf[KS];
  {
    const int head = h0 + c16;
    const uint16_t* qrow = a.q + (t * a.H + head) * (int64_t)DQK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = (head < a.H) ? load16(qrow + 32 * ks) : u32x4{0u, 0u, 0u, 0u};
  }

  f32x4 o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();  // running max (log2 units) of head c16
  float l_run = 0.f;                // this lane's partial sum of exp2

  if (tid < kBN) s_ids[0][tid] = slot_id(tid);
  __syncthreads();

  const int n_tiles = (L + kBN - 1) / kBN;
  for (int it = 0; it < n_tiles; ++it) {
    const int j0 = it * kBN;
    const int32_t* ids = s_ids[it & 1];

    // ---- gather the tile's KV rows into LDS ----
    for (int item = tid; item < (kBN / 4) * NCH; item += NT) {
      const int kg = item / NCH;
      const int dc = item - kg * NCH;
      u32x4 d[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int32_t id = ids[4 * kg + i];
        d[i] = id >= 0 ? load16(a.k + (int64_t)id * a.ld_k + 8 * dc) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4*>(&ktile[(4 * kg + i) * KROW + 4 * dc]) = d[i];
      if (SHARED && dc < NVCH) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          u32x2 w;
          w.x = half_of(d[0], e) | (half_of(d[1], e) << 16);
          w.y = half_of(d[2], e) | (half_of(d[3], e) << 16);
          *reinterpret_cast<u32x2*>(&vtile[(8 * dc + e) * VROW + 2 * kg]) = w;
        }
      }
    }
    if (!SHARED) {
      for (int item = tid; item < (kBN / 4) * NVCH; item += NT) {
        const int kg = item / NVCH;
        const int dc = item - kg * NVCH;
        u32x4 d[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int32_t id = ids[4 * kg + i];
          d[i] = id >= 0 ? load16(a.v + (int64_t)id * a.ld_v + 8 * dc) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          u32x2 w;
          w.x = half_of(d[0], e) | (half_of(d[1], e) << 16);
          w.y = half_of(d[2], e) | (half_of(d[3], e) << 16);
          *reinterpret_cast<u32x2*>(&vtile[(8 * dc + e) * VROW + 2 * kg]) = w;
        }
      }
    }
    __syncthreads();
    if (tid < kBN) s_ids[(it + 1) & 1][tid] = slot_id(j0 + kBN + tid);

    // ---- S^T = K_tile . Q^T : lane holds head c16, keys 16*mb + 4*g + i ----
    f32x4 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint32_t* krow = ktile + (16 * mb + c16) * KROW + 4 * g;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 af = *reinterpret_cast<const u32x4*>(krow + 16 * ks);
        acc = mfma16x16x32(af, qf[ks], acc);
      }
      s[mb] = acc;
    }

    // ---- online softmax (log2 domain) ----
    float x[8];
    float mt = -__builtin_inff();
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = ids[16 * mb + 4 * g + i] >= 0;
        const float v = ok ? s[mb][i] * a.scale_log2 : -__builtin_inff();
        x[4 * mb + i] = v;
        mt = fmaxf(mt, v);
      }
    }
    mt = fmaxf(mt, shfl_xor_f(mt, 16));
    mt = fmaxf(mt, shfl_xor_f(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    // Everything still masked for this head: keep the state unchanged.
    const bool live = m_new > -__builtin_inff();
    const float alpha = live ? fast_exp2(m_run - m_new) : 1.0f;
    float p[8];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = live ? fast_exp2(x[i] - m_new) : 0.f;
      psum += p[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;

    // Rescale O: lane holds heads 4*g + i of the wave's group.
    float al[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[nb][i] *= al[i];
    }

    // ---- O += P . V ----
    u32x4 pa;
    pa[0] = pack_bf16x2(p[0], p[1]);
    pa[1] = pack_bf16x2(p[2], p[3]);
    pa[2] = pack_bf16x2(p[4], p[5]);
    pa[3] = pack_bf16x2(p[6], p[7]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint32_t* vrow = vtile + (16 * nb + c16) * VROW + 2 * g;
      const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 8);
      const u32x4 vb = u32x4{lo.x, lo.y, hi.x, hi.y};
      o[nb] = mfma16x16x32(pa, vb, o[nb]);
    }
    __syncthreads();
  }

  // ---- epilogue ----
  float l_tot = l_run;
  l_tot += shfl_xor_f(l_tot, 16);
  l_tot += shfl_xor_f(l_tot, 32);
  const int head = h0 + c16;
  const bool empty = !(m_run > -__builtin_inff());
  constexpr float kLn2 = 0.693147180559945309f;
  constexpr float kLog2e = 1.442695040888963387f;
  float inv = 0.f;
  if (!empty) {
    float denom = l_tot;
    if (a.sink && head < a.H) denom += fast_exp2(a.sink[head] * kLog2e - m_run);
    inv = 1.0f / denom;
  }
  if (g == 0 && head < a.H) {
    a.lse[t * a.H + head] = empty ? __builtin_inff() : (m_run + fast_log2(l_tot)) * kLn2;
    if (a.max_logits) a.max_logits[t * a.H + head] = empty ? -__builtin_inff() : m_run * kLn2;
  }
  float iv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) iv[i] = __shfl(inv, 4 * g + i, 64);

  // Stage the wave's 16 x DV bf16 rows in LDS, then store contiguous rows.
  constexpr int CH_PER_ROW = DV / 8;  // 16-byte chunks per output row
#pragma unroll
  for (int round = 0; round < (NW + STAGE_WAVES - 1) / STAGE_WAVES; ++round) {
    const bool mine = wave / STAGE_WAVES == round;
    uint32_t* stage = lds + (wave % STAGE_WAVES) * WAVE_STAGE_U32;
    uint16_t* stage16 = reinterpret_cast<uint16_t*>(stage);
    if (round > 0) __syncthreads();
    if (mine) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          stage16[(4 * g + i) * (2 * OUT_ROW) + 16 * nb + c16] =
              (uint16_t)f32_to_bf16_bits(o[nb][i] * iv[i]);
      }
    }
    __syncthreads();
    if (mine) {
      for (int c = lane; c < 16 * CH_PER_ROW; c += 64) {
        const int hr = c / CH_PER_ROW;
        const int cc = c - hr * CH_PER_ROW;
        const int hh = h0 + hr;
        if (hh < a.H) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(&stage[hr * OUT_ROW + 4 * cc]);
          *reinterpret_cast<u32x4*>(a.out + (t * a.H + hh) * (int64_t)DV + 8 * cc) = v;
        }
      }
    }
  }
}

template <int DQK, int DV, bool SHARED>
hipError_t launch_cfg(const AttnArgs& a, hipStream_t st) {
  const int nw = (a.H + 15) / 16;
  dim3 grid((unsigned)a.T_q);
  if (nw <= 1) {
    hipLaunchKernelGGL((sparse_attn_kernel<DQK, DV, SHARED, 1>), grid, dim3(64), 0, st, a);
  } else if (nw <= 2) {
    hipLaunchKernelGGL((sparse_attn_kernel<DQK, DV, SHARED, 2>), grid, dim3(128), 0, st, a);
  } else if (nw <= 4) {
    hipLaunchKernelGGL((sparse_attn_kernel<DQK, DV, SHARED, 4>), grid, dim3(256), 0, st, a);
  } else if (nw <= 8) {
    hipLaunchKernelGGL((sparse_attn_kernel<DQK, DV, SHARED, 8>), grid, dim3(512), 0, st, a);
  } else {
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
