// Internal host-side launchers behind the C ABI (one per kernel family).
// Arguments are assumed validated by the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

hipError_t launch_packed_metadata(const int32_t* cu, int32_t n_seq, int64_t T, int32_t* row_starts,
                                  int32_t* seq_lens, hipStream_t st);

hipError_t launch_ratio_metadata(const int32_t* cu_q, const int32_t* cu_k, const int32_t* offsets,
                                 int32_t n_seq, int64_t T_q, int32_t ratio, int32_t* row_starts,
                                 int32_t* seq_lens, hipStream_t st);

// T_kv: rows of k (key loads are clamped into [0, T_kv)).
hipError_t launch_indexer(const void* q, const void* k, const void* w, int w_dtype,
                          const int32_t* row_starts, const int32_t* seq_lens, int64_t T_kv, int H,
                          int D, int64_t row_begin, int64_t n_rows, float* scores, int64_t ld,
                          hipStream_t st);

// FP8 indexer: mx selects E8M0 block scales (true) or fp32 per-token descales.
hipError_t launch_indexer_fp8(const void* q, const void* qs, const void* k, const void* ks,
                              bool mx, const void* w, int w_dtype, const int32_t* rs,
                              const int32_t* sl, int64_t T_kv, int H, int64_t row_begin,
                              int64_t n_rows, float* scores, int64_t ld, hipStream_t st);

struct FusedArgs;

// Combined indexer + top-k (rows of at most 4096 columns): bf16 or FP8 inputs.
hipError_t launch_indexer_topk(const void* q, const void* k, const void* w, int w_dtype,
                               const int32_t* rs, const int32_t* sl, int64_t T_kv, int H, int D,
                               int64_t row_begin, int64_t n_rows, int64_t n_cols,
                               const FusedArgs& fa, hipStream_t st);
hipError_t launch_indexer_topk_fp8(const void* q, const void* qs, const void* k, const void* ks,
                                   bool mx, const void* w, int w_dtype, const int32_t* rs,
                                   const int32_t* sl, int64_t T_kv, int H, int64_t row_begin,
                                   int64_t n_rows, int64_t n_cols, const FusedArgs& fa,
                                   hipStream_t st);

// Caller-owned buffer of the combined indexer + top-k for rows longer than
// the on-chip path takes (DSA page section 4: candidates per row, then a
// stage-2 select). Stage 1 (the indexer pass) appends each row's candidates;
// stage 2 selects from them; rows whose list cannot hold their top k are
// queued and redone by the rescue pass from recomputed dense scores.
constexpr int64_t kCandCap = 8192;   // candidates kept per row
constexpr int kCandSpillRows = 256;  // dense rows of the rescue pass (one per workgroup)
struct CandArgs {
  uint32_t* cand;      // [n_rows, kCandCap] (score bits, local column)
  int64_t cap;         // kCandCap
  int32_t* count;      // [n_rows] candidates found (also past cap)
  int32_t* queue;      // [n_rows] rows queued for the rescue
  uint32_t* n_queued;  // their number
  float* spill;        // [n_spill, spill_ld] rescue score rows
  int64_t spill_ld;
  int n_spill;
};

// Stage 1: the indexer pass appending candidates (bf16 inputs).
hipError_t launch_indexer_cand(const void* q, const void* k, const void* w, int w_dtype,
                               const int32_t* rs, const int32_t* sl, int64_t T_kv, int H, int D,
                               int64_t row_begin, int64_t n_rows, int64_t n_cols, int top_k,
                               const CandArgs& ca, hipStream_t st);
// Stage 2 (seq_lens and row_starts start at the first row).
hipError_t launch_topk_cand(const int32_t* seq_lens, const int32_t* row_starts, int64_t n_rows,
                            int64_t n_cols, int k, int32_t* indices, int64_t ld_idx,
                            int32_t* topk_length, float* logits, float* softmax, float* lse,
                            const CandArgs& ca, hipStream_t st);
// Rescue of the queued rows.
hipError_t launch_indexer_rescue(const void* q, const void* k, const void* w, int w_dtype,
                                 const int32_t* rs, const int32_t* sl, int64_t T_kv, int H, int D,
                                 int64_t row_begin, int64_t n_rows, int64_t n_cols,
                                 const FusedArgs& fa, const CandArgs& ca, hipStream_t st);
// The same two passes for FP8 (E4M3) inputs (mx: E8M0 block scales, else
// fp32 per-token descales); stage 2 is launch_topk_cand.
hipError_t launch_indexer_cand_fp8(const void* q, const void* qs, const void* k, const void* ks,
                                   bool mx, const void* w, int w_dtype, const int32_t* rs,
                                   const int32_t* sl, int64_t T_kv, int H, int64_t row_begin,
                                   int64_t n_rows, int64_t n_cols, int top_k, const CandArgs& ca,
                                   hipStream_t st);
hipError_t launch_indexer_rescue_fp8(const void* q, const void* qs, const void* k, const void* ks,
                                     bool mx, const void* w, int w_dtype, const int32_t* rs,
                                     const int32_t* sl, int64_t T_kv, int H, int64_t row_begin,
                                     int64_t n_rows, int64_t n_cols, const FusedArgs& fa,
                                     const CandArgs& ca, hipStream_t st);

hipError_t launch_topk(const float* scores, int64_t ld, int64_t n_rows, int64_t n_cols,
                       const int32_t* seq_lens, const int32_t* row_starts, int k, int32_t* indices,
                       int64_t ld_idx, int32_t* topk_length, float* values, hipStream_t st);

struct AttnArgs {
  const uint16_t* q;
  int64_t T_q;
  int H;
  const uint16_t* k;
  int64_t T_kv;
  int64_t ld_k;
  const uint16_t* v;  // never null here: the ABI layer substitutes k for shared KV
  int64_t ld_v;
  const int32_t* indices;
  int64_t ld_idx;
  int k_width;
  const int32_t* topk_length;
  const float* sink;
  float scale_log2;  // softmax_scale * log2(e)
  uint16_t* out;
  float* lse;
  float* max_logits;
  // Filled by the launcher: byte extents of K and V as read through buffer
  // descriptors, and their row strides in bytes.
  uint32_t span_k, span_v;
  uint32_t row_bytes_k, row_bytes_v;
};

hipError_t launch_sparse_attn(const AttnArgs& a, int D_qk, int D_v, hipStream_t st);
// The block-routed GQA form (D_qk = D_v = 256, separate V, H <= 16, K and V
// spans below 2^31 bytes); hipErrorInvalidValue for anything else.
hipError_t launch_sparse_gqa(AttnArgs a, hipStream_t st);

// Sparse attention backward (shared latent KV, D_v = 512).
struct BwdArgs {
  const uint16_t* q;        // [T_q, H, D_qk]
  const uint16_t* kv;       // [T_kv, ld_kv]
  int64_t T_q, T_kv, ld_kv;
  int H, D_qk, D_v;
  const int32_t* indices;   // [T_q, ld_idx]
  int64_t ld_idx;
  int k_width;
  const int32_t* topk_length;
  const float* sink;        // [H] or null
  float scale;
  const uint16_t* out;      // [T_q, H, D_v]
  const uint16_t* dout;     // [T_q, H, D_v]
  const float* lse;         // [T_q, H]
  float* logZ;              // workspace [T_q, H]
  float* Dsum;              // workspace [T_q, H]
  uint16_t* wsP;            // workspace [chunk, Kw, 32*ceil(H/32)] bf16
  uint16_t* wsD;            // same
  uint16_t* wsC;            // workspace [nparts, chunk, Kw, D_qk] bf16: dkv row per slot
  int32_t* cnt;             // workspace [T_kv]: slots per KV row (chunk)
  int32_t* offs;            // workspace [T_kv + 1]: list offsets
  int32_t* list;            // workspace [chunk * Kw]: slot rows grouped by KV row
  int32_t* sort_keys[2];    // workspace [chunk * Kw] each: radix sort keys between passes
  int32_t* sort_vals[2];    // same, slot numbers
  uint32_t* sort_hist;      // workspace [256, ceil(chunk * Kw / 4096)]
  uint32_t* sort_tot;       // workspace [256]
  int nparts;               // head parts of the dkv pass (64 heads each)
  int64_t chunk_rows;       // rows of the P / dS / C buffers
  int Kw;                   // k_width rounded up to 32
  uint16_t* dq;             // [T_q, H, D_qk] bf16
  float* dkv_ws;            // workspace [T_kv, D_qk] fp32
  uint16_t* dkv;            // [T_kv, D_qk] bf16
  float* d_sink;            // [H] or null
  int64_t row0;             // first row of the current chunk
  uint32_t span_kv;         // launcher: bytes of kv read through a buffer descriptor
  uint32_t row_bytes;       // launcher: ld_kv * 2
  // KV-tile dkv (dense selections, see bwd_uses_kv_tiles): per chunk row the
  // slot of each KV row ([chunk, ld_map] int16, -1: none), fp32 partial sums
  // per (row part, KV tile) and whether each was written, rows with repeated
  // ids (their slots are merged before the tile pass).
  bool tiles;
  int16_t* map;             // workspace [chunk, ld_map]
  int64_t ld_map;           // T_kv rounded up to the KV tile
  float* part;              // workspace [n_parts, ld_map, D_qk]
  int32_t* part_flag;       // workspace [n_parts, ld_map / tile]
  uint32_t* dup_count;      // workspace [1]
  int32_t* dup_rows;        // workspace [chunk]
};

// Whether the backward takes the KV-tile dkv (dense selections: at least one
// key in eight selected per row, up to 32768 KV rows and 8192 slots); the
// workspace layout follows the same rule.
constexpr int kBwdTileKV = 128;    // KV rows per tile
constexpr int kBwdTileRows = 64;   // query rows per part
inline bool bwd_uses_kv_tiles(int64_t T_kv, int32_t k_width) {
  const int64_t kw = ((int64_t)k_width + 31) / 32 * 32;
  return T_kv > 0 && T_kv <= 32768 && k_width > 0 && kw <= 8192 && 8 * (int64_t)k_width >= T_kv;
}

hipError_t launch_sparse_attn_bwd(BwdArgs a, int64_t chunk, hipStream_t st);

}  // namespace dsa
