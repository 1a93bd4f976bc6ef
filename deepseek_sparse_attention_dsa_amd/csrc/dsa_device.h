// Device-side helpers shared by the gfx950 DSA kernels (internal header).
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 -> packed bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// One v_mfma_f32_16x16x32_bf16: D[16x16] = A[16x32] * B[32x16] + C.
// Lane l supplies A row (l % 16) and B column (l % 16), each over the eight
// k values 8*(l/16) .. 8*(l/16)+7, and receives D column (l % 16), rows
// 4*(l/16) .. 4*(l/16)+3.
__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// One v_mfma_f32_32x32x16_bf16: D[32x32] = A[32x16] * B[16x32] + C.
// Lane l supplies A row (l % 32) and B column (l % 32), each over the eight
// k values 8*(l/32) .. 8*(l/32)+7, and receives D column (l % 32), rows
// 8*(i/4) + 4*(l/32) + (i%4) for its 16 values i.
__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// One v_mfma_f32_32x32x64_f8f6f4 on FP8 E4M3 (OCP) operands:
// D[32x32] = A[32x64] * B[64x32] + C, fp32 accumulation. Lane l supplies A
// row (l % 32) and B column (l % 32); byte j of its 32 covers
// k = 32*(j/16) + 16*(l/32) + (j%16). D has the mfma32x32x16 layout. The
// unscaled instruction is the scaled builtin with constant zero scales.
__device__ __forceinline__ f32x16 mfma32x32x64_fp8(const i32x8& a, const i32x8& b,
                                                   const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The block-scaled form (v_mfma_scale_f32_32x32x64_f8f6f4): byte 0 of sa is
// the E8M0 scale of A row (l % 32) over k block l/32 (k = 32*(l/32) .. +31),
// byte 0 of sb the scale of B column (l % 32) over the same k block; every
// product of a block is multiplied by 2^(sa-127) * 2^(sb-127).
__device__ __forceinline__ f32x16 mfma32x32x64_mxfp8(const i32x8& a, int sa, const i32x8& b,
                                                     int sb, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// ds_read_b64_tr_b16: inside each group of 16 lanes, lane i receives 16-bit
// element (i % 4) of the 8-byte reads of source lanes i/4, 4 + i/4, 8 + i/4
// and 12 + i/4. With source lane j pointing at row r0 + j/4, column
// c0 + 4*(j%4) of a row-major bf16 matrix, lane i gets column c0 + i of rows
// r0 .. r0+3: a 4 x 16 block read transposed.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* lds_ptr) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(lds_ptr));
  return __builtin_bit_cast(u32x2, r);
}

// Asynchronous 16-byte global -> LDS copy (global_load_lds_dwordx4): lane l's
// 16 bytes land at LDS byte address lds_base + 16 * l, lds_base being
// wave-uniform. Issued through inline asm so that the compiler does not
// insert its own (blanket) waits for it: the caller waits with
// wait_vmcnt0() before reading the data. The s_nop is the wait state an SALU
// write of M0 needs before an instruction that reads M0 as an LDS address.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds_base)
               : "memory");
}

// Same copy with an immediate byte offset IMM (0 <= IMM < 4096). The offset
// applies to both addresses: global gptr + IMM -> LDS lds_base + IMM + 16*l.
template <int IMM>
__device__ __forceinline__ void dma16_imm(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%2"
               :
               : "v"(gptr), "s"(lds_base), "i"(IMM)
               : "memory");
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Calls f(std::integral_constant<int, i>{}) for i = 0 .. N-1 (compile-time i).
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

// Raw buffer descriptor words (gfx9: 32-bit data, stride 0, range checked)
// over `bytes` bytes at `base`; base and bytes must be wave-uniform.
__device__ __forceinline__ i32x4 buffer_rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// Asynchronous 16-byte-per-lane copy through a buffer descriptor:
// bytes voff + IMM .. +15 of the buffer -> LDS lds_base + IMM + 16*l (the
// same addressing as dma16_imm, measured on the device). Lanes whose range
// falls outside the descriptor write zeros (also measured).
template <int IMM>
__device__ __forceinline__ void dma16_buf_imm(uint32_t voff, i32x4 rsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen offset:%3 lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds_base), "i"(IMM)
               : "memory");
}

// s_waitcnt vmcnt(0) through the builtin, so that the compiler's own wait
// tracking also knows that every earlier vector-memory load has completed.
__device__ __forceinline__ void wait_vmcnt0() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt = 0, expcnt and lgkmcnt unconstrained
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)p;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }

// Sum over the two half-waves in one VALU exchange (v_permlane32_swap):
// lane l < 32 gets a[l] + a[l + 32], lane l >= 32 gets b[l - 32] + b[l].
__device__ __forceinline__ float halfwave_sums(float a, float b) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
// max(v[l], v[l ^ 32]) in every lane, through one v_permlane32_swap (IEEE
// maximum: a NaN operand gives NaN).
__device__ __forceinline__ float halfwave_max(float v) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __builtin_elementwise_maximum(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ int shfl_xor_i(int v, int m) { return __shfl_xor(v, m, kWave); }

// Wave-wide inclusive scan / reductions on DPP lane moves (no LDS round
// trips): row_shr 1, 2, 4, 8 inside each 16-lane row, then row_bcast 15 and
// row_bcast 31 carry the row totals upwards (GFX9 DPP controls).
template <typename Op>
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t v, Op op, uint32_t ident) {
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x111, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x112, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x114, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x118, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x142, 0xa, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x143, 0xc, 0xf, false));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = wave_incl_scan_dpp(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; }, 0u);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = wave_incl_scan_dpp(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; }, 0xffffffffu);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v = wave_incl_scan_dpp(v, [](uint32_t a, uint32_t b) { return a + b; }, 0u);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  const uint32_t s = wave_incl_scan_dpp(
      __float_as_uint(v),
      [](uint32_t a, uint32_t b) { return __float_as_uint(__uint_as_float(a) + __uint_as_float(b)); },
      0u);
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)s, 63));
}

// Number of set bits of `mask` in lanes strictly below the calling lane.
__device__ __forceinline__ uint32_t popc_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Raw buffer descriptor (word 3 = 0x00020000 on gfx9: 32-bit data, stride 0)
// of `bytes` bytes at `base`, which must be the same in every lane of the
// wave: it is taken from the first active lane. The hardware range check
// drops stores at byte offsets >= bytes and reads such loads as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  const uint64_t pu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(p >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)pu, 0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
}

__device__ __forceinline__ void buffer_store_f32(float v, __amdgpu_buffer_rsrc_t rsrc,
                                                 uint32_t byte_off) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(v), rsrc, (int)byte_off, 0, 0);
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace dsa
