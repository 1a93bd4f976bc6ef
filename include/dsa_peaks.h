/*
 * dsa_peaks.h - measurement aids of libdsa_peaks.so (gfx950).
 *
 * Not part of the attention path: three probes that measure what this device
 * sustains - the dense MFMA rate of one MFMA form and the HBM copy and read
 * rates - so that a kernel's achieved rate can be set against them as well as
 * against the chip's published peaks. The caller times the launches (events
 * on `stream`) and divides the work these functions define by that time.
 *
 * Conventions: device pointers, `stream` a hipStream_t (NULL: the null
 * stream). Launches are asynchronous. Return 0 on success, 1 for invalid
 * arguments (nothing launched), 2 when the launch itself fails.
 */
#ifndef DSA_PEAKS_H
#define DSA_PEAKS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* MFMA forms of the loop probe. */
#define DSA_PEAK_BF16 0  /* v_mfma_f32_32x32x16_bf16: 32768 FLOP each */
#define DSA_PEAK_FP8 1   /* v_mfma_scale_f32_32x32x64_f8f6f4, E4M3, unit scales: 131072 FLOP */
#define DSA_PEAK_MXFP8 2 /* the same with E8M0 block scales applied: 131072 FLOP */

/* Threads per workgroup of every probe (four waves). */
int dsa_peak_threads_per_block(void);

/*
 * dsa_peak_mfma_flop - FLOP that dsa_peak_mfma performs for these arguments
 * (each wave: 4 accumulator chains x iters MFMAs of the form); -1 for an
 * unknown kind, iters < 1 or n_blocks < 1.
 */
double dsa_peak_mfma_flop(int32_t kind, int64_t iters, int32_t n_blocks);

/*
 * dsa_peak_mfma - n_blocks workgroups run the MFMA loop on register operands.
 *   sink  device float [n_blocks * dsa_peak_threads_per_block()], 16-byte
 *         aligned: one value per thread, written at the end (contents
 *         meaningless; they only keep the loop alive)
 */
int dsa_peak_mfma(int32_t kind, int64_t iters, int32_t n_blocks, float* sink, void* stream);

/*
 * dsa_peak_copy - dst[0, bytes) = src[0, bytes) with streaming (nontemporal)
 * 16-byte loads and stores over a grid of n_blocks workgroups (grid-stride). bytes a positive
 * multiple of 16; src and dst 16-byte aligned and not overlapping. HBM bytes
 * moved: 2 * bytes.
 */
int dsa_peak_copy(const void* src, void* dst, int64_t bytes, int32_t n_blocks, void* stream);

/*
 * dsa_peak_read - reads src[0, bytes) with streaming 16-byte loads (grid-stride)
 * and writes one word per thread to sink (device uint32
 * [n_blocks * dsa_peak_threads_per_block()]). HBM bytes read: bytes.
 */
int dsa_peak_read(const void* src, int64_t bytes, int32_t n_blocks, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_PEAKS_H */
