// Measurement aids (libdsa_peaks.so): the dense MFMA rate and the HBM copy
// rate this device sustains, so that each kernel's roofline fraction can be
// read against what the chip actually delivers as well as against its
// published peaks. Nothing here is part of the attention path.
//
// - MFMA loop: every wave runs independent accumulator chains of one MFMA
//   form over register operands (no memory traffic in the loop), four waves
//   per SIMD, and stores one value per lane at the end so that nothing is
//   optimised away.
// - Copy: a grid-stride 16-byte vector copy; bytes moved = 2 x the buffer size.
// - Read: the same loop without the stores (one value per thread at the end).
#include "dsa_device.h"
#include "dsa_peaks.h"

namespace {

using dsa::f32x16;
using dsa::i32x8;
using dsa::u32x4;

constexpr int kChains = 4;      // independent accumulator chains per wave
constexpr int kThreads = 256;   // four waves per workgroup

__device__ __forceinline__ uint32_t seed_word(uint32_t i) {
  // small nonzero operands (bf16 pairs / FP8 bytes of moderate magnitude)
  return 0x3c003c00u ^ ((i * 2654435761u) & 0x00ff00ffu);
}

template <int KIND>
__global__ __launch_bounds__(kThreads) void mfma_loop_kernel(int64_t iters, float* sink) {
  const uint32_t tid = blockIdx.x * kThreads + threadIdx.x;
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.0f;
  if constexpr (KIND == DSA_PEAK_BF16) {
    const u32x4 a = {seed_word(tid), seed_word(tid + 1), seed_word(tid + 2), seed_word(tid + 3)};
    const u32x4 b = {seed_word(tid + 4), seed_word(tid + 5), seed_word(tid + 6),
                     seed_word(tid + 7)};
#pragma unroll 1
    for (int64_t it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = dsa::mfma32x32x16(a, b, acc[c]);
  } else {
    i32x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (int)(seed_word(tid + i) & 0x37373737u);
      b[i] = (int)(seed_word(tid + 8 + i) & 0x37373737u);
    }
#pragma unroll 1
    for (int64_t it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kChains; ++c) {
        if constexpr (KIND == DSA_PEAK_FP8)
          acc[c] = dsa::mfma32x32x64_fp8(a, b, acc[c]);
        else
          acc[c] = dsa::mfma32x32x64_mxfp8(a, 127, b, 127, acc[c]);
      }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  sink[tid] = s;
}

// Streaming loads and stores (nontemporal: the data is touched once). On
// MI355X one 16-byte copy per thread and trip, or two loads per trip for
// the read, at four workgroups per CU measured fastest among 1-8 loads in
// flight per thread and 1-64 workgroups per CU.
__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                        uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t x = 0u;
  for (; i + stride < n16; i += 2 * stride) {
    const u32x4 v0 = __builtin_nontemporal_load(src + i);
    const u32x4 v1 = __builtin_nontemporal_load(src + i + stride);
    x ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
  }
  if (i < n16) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = x;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0u; }

}  // namespace

extern "C" {

int dsa_peak_threads_per_block(void) { return kThreads; }

double dsa_peak_mfma_flop(int32_t kind, int64_t iters, int32_t n_blocks) {
  if (iters < 1 || n_blocks < 1) return -1.0;
  double per;  // FLOP of one MFMA
  switch (kind) {
    case DSA_PEAK_BF16: per = 2.0 * 32 * 32 * 16; break;
    case DSA_PEAK_FP8:
    case DSA_PEAK_MXFP8: per = 2.0 * 32 * 32 * 64; break;
    default: return -1.0;
  }
  return per * kChains * (double)iters * (kThreads / 64) * (double)n_blocks;
}

int dsa_peak_mfma(int32_t kind, int64_t iters, int32_t n_blocks, float* sink, void* stream) {
  if (iters < 1 || n_blocks < 1 || sink == nullptr || !aligned16(sink)) return 1;
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid((unsigned)n_blocks), block(kThreads);
  switch (kind) {
    case DSA_PEAK_BF16:
      hipLaunchKernelGGL(mfma_loop_kernel<DSA_PEAK_BF16>, grid, block, 0, st, iters, sink);
      break;
    case DSA_PEAK_FP8:
      hipLaunchKernelGGL(mfma_loop_kernel<DSA_PEAK_FP8>, grid, block, 0, st, iters, sink);
      break;
    case DSA_PEAK_MXFP8:
      hipLaunchKernelGGL(mfma_loop_kernel<DSA_PEAK_MXFP8>, grid, block, 0, st, iters, sink);
      break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int dsa_peak_copy(const void* src, void* dst, int64_t bytes, int32_t n_blocks, void* stream) {
  if (bytes < 16 || bytes % 16 != 0 || n_blocks < 1 || src == nullptr || dst == nullptr ||
      !aligned16(src) || !aligned16(dst))
    return 1;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)n_blocks), dim3(kThreads), 0,
                     (hipStream_t)stream, (const u32x4*)src, (u32x4*)dst, bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int dsa_peak_read(const void* src, int64_t bytes, int32_t n_blocks, uint32_t* sink, void* stream) {
  if (bytes < 16 || bytes % 16 != 0 || n_blocks < 1 || src == nullptr || sink == nullptr ||
      !aligned16(src))
    return 1;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)n_blocks), dim3(kThreads), 0,
                     (hipStream_t)stream, (const u32x4*)src, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
