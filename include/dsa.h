/*
 * dsa.h - C ABI of the MI355X (gfx950) DeepSeek Sparse Attention forward path.
 *
 * Stream-ordered calls covering the forward hot path of DSA and the sparse
 * attention backward:
 *   dsa_packed_metadata  per-token document start and causal length (THD)
 *   dsa_ratio_causal_metadata  the same for the ratio-causal mask with query
 *                        causal offsets (compressed keys, split queries)
 *   dsa_indexer_fwd      lightning-indexer scores  sum_h W_h * ReLU(q_h . k)
 *   dsa_indexer_fwd_fp8  the same scores from FP8 (E4M3) Q and K with
 *                        per-token descales or per-32 E8M0 block scales
 *   dsa_topk             per-row top-K select, ascending global indices, -1 pad
 *                        (dsa_topk_workspace_bytes: its workspace query, 0)
 *   dsa_indexer_topk_fused  indexer scores + top-K (+ logits, softmax, LSE)
 *                        without dense scores: kept on chip for rows of up
 *                        to 4096 columns, reduced to per-row candidates in a
 *                        caller-owned buffer for longer rows
 *                        (dsa_indexer_topk_cand_buffer_size: its size query)
 *   dsa_sparse_attn_fwd  sparse MQA/GQA attention over the selected KV rows
 *   dsa_sparse_attn_bwd  its gradients (dq, dkv, d_sink) for shared latent KV
 *                        (dsa_sparse_attn_bwd_workspace_bytes: its workspace
 *                        query; dsa_sparse_attn_bwd_kv_tiles: which dkv
 *                        scheme a shape takes; dsa_sparse_attn_bwd_noalloc:
 *                        the same without a caller workspace, for callers
 *                        that cannot allocate)
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers marked "device" are device pointers on the current HIP device.
 *   The caller owns every buffer (inputs and outputs). The library never
 *   allocates, frees or synchronises inside these calls; work is enqueued on
 *   `stream` (a hipStream_t passed as void*; NULL = the legacy default stream)
 *   and the call returns before it runs.
 * - Arguments are validated on the host before anything is launched. On a bad
 *   argument the call returns a non-OK status, launches nothing, and
 *   dsa_last_error() describes the problem. Values that live in device memory
 *   (cu_seqlens monotonicity, index ranges) are not checked on the host; the
 *   kernels treat out-of-range indices as invalid slots instead.
 * - Status codes: DSA_ERR_TYPE for an unknown dtype enum, DSA_ERR_VALUE for a
 *   shape, size, pointer, alignment or scale that is out of contract,
 *   DSA_ERR_RUNTIME when no gfx950 device is current or a launch fails.
 * - bf16 means IEEE-754 binary32 truncated to its upper 16 bits (bfloat16).
 *
 * Source of the semantics: the cuDNN Frontend page "DeepSeek Sparse Attention
 * (DSA)" (sections 1, 3, 4 and 5) and the NeMo AutoModel API pages for
 * nemo_automodel...glm_moe_dsa.kernels.cudnn_dsa (cudnn_indexer_topk,
 * cudnn_sparse_attention, prepare_cudnn_dsa_packed_metadata) and
 * nemo_automodel...qwen3_8_flash_next.cudnn_qsa (cudnn_sparse_gqa_attention).
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_TYPE = 1,    /* bad dtype enum                                  */
  DSA_ERR_VALUE = 2,   /* bad shape / size / pointer / alignment / scale  */
  DSA_ERR_RUNTIME = 3  /* no gfx950 device current, or a launch failed    */
} dsa_status;

typedef enum { DSA_BF16 = 0, DSA_F32 = 1 } dsa_dtype;

/* Scale forms of FP8 indexer inputs (DSA page section 3, "Precision paths"). */
typedef enum {
  DSA_FP8_PER_TOKEN = 0, /* fp32 descales: q [T, H_idx], k [T_kv]            */
  DSA_MXFP8 = 1          /* E8M0 bytes per 32 elements: q [T, H_idx, D/32],
                            k [T_kv, D/32]                                  */
} dsa_fp8_scaling;

/* Message for the last non-OK status returned on the calling thread
 * (thread-local, valid until the next call on that thread). Never NULL. */
const char* dsa_last_error(void);

/* ABI version of this header (bumped on any signature change). */
#define DSA_ABI_VERSION 10
int dsa_abi_version(void);

/* Limits enforced by the host checks. */
#define DSA_MAX_TOPK 2048           /* top_k <= 2048 (DSA page, section 5)  */
#define DSA_TOPK_MAX_COLS 65536     /* longest score row dsa_topk selects on */
#define DSA_MAX_HEADS 128           /* attention query heads per call        */
#define DSA_FUSED_MAX_COLS 4096     /* longest row dsa_indexer_topk_fused keeps
                                       on chip (longer rows: candidate buffer) */
/* Device scratch of dsa_sparse_attn_bwd_noalloc (bytes, per device). */
#define DSA_NOALLOC_SCRATCH_BYTES (256ll * 1024 * 1024)

/* Input precision of dsa_indexer_topk_fused. */
typedef enum {
  DSA_INDEXER_BF16 = 0,  /* bf16 q_idx / k_idx, no scales (dsa_indexer_fwd)  */
  DSA_INDEXER_FP8 = 1,   /* E4M3 with per-token fp32 descales                */
  DSA_INDEXER_MXFP8 = 2  /* E4M3 with E8M0 scales per 32 elements            */
} dsa_indexer_precision;

/*
 * dsa_packed_metadata - step a0.
 * For compact packed THD sequences (cudnn_dsa page,
 * prepare_cudnn_dsa_packed_metadata: per-query starts and real causal
 * lengths; causality restarts at each document):
 *   row_starts[t] = cu_seqlens[d], seq_lens[t] = t - cu_seqlens[d] + 1
 * where d is the document holding token t (cu_seqlens[d] <= t < cu_seqlens[d+1]).
 *   cu_seqlens  device int32 [n_seq + 1], cu_seqlens[0] = 0, non-decreasing,
 *               cu_seqlens[n_seq] = T (not checked on the host)
 *   row_starts, seq_lens  device int32 [T] outputs
 * Errors: n_seq < 1, T < 0 or T > INT32_MAX, a NULL pointer with T > 0.
 * T = 0 is a no-op.
 */
int dsa_packed_metadata(const int32_t* cu_seqlens, int32_t n_seq, int64_t T,
                        int32_t* row_starts, int32_t* seq_lens, void* stream);

/*
 * dsa_ratio_causal_metadata - step a0 for the ratio-causal mask.
 * DSA page section 3 ("Indexer Forward"): THD segment b stores its queries at
 * rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) and its compressed keys at rows
 * [cu_seqlens_k[b], cu_seqlens_k[b+1]); the keys are a compressed prefix that
 * starts at compressed column 0. Local query row i of segment b
 * (t = cu_seqlens_q[b] + i) may score local key column j only when
 *   j < clamp(floor((q_causal_offsets[b] + i + 1) / ratio), 0,
 *             cu_seqlens_k[b+1] - cu_seqlens_k[b])
 * so this writes
 *   row_starts[t] = cu_seqlens_k[b], seq_lens[t] = that bound.
 * q_causal_offsets[b] is the global, uncompressed token position of segment
 * b's first query (its place in the causal timeline, not where it is
 * stored); NULL means 0 for every segment. The outputs feed dsa_indexer_fwd
 * and dsa_topk as they are. ratio 1, no offsets and cu_seqlens_k ==
 * cu_seqlens_q give exactly dsa_packed_metadata's result.
 *   cu_seqlens_q, cu_seqlens_k  device int32 [n_seq + 1], starting at 0,
 *               non-decreasing, cu_seqlens_q[n_seq] = T_q (not checked on
 *               the host; a row past cu_seqlens_q[n_seq] is given the last
 *               segment)
 *   q_causal_offsets  device int32 [n_seq] or NULL
 *   ratio       >= 1 (tokens per compressed key)
 *   row_starts, seq_lens  device int32 [T_q] outputs
 * Errors: n_seq < 1, T_q < 0 or T_q > INT32_MAX, ratio < 1, a NULL pointer
 * (other than q_causal_offsets) with T_q > 0. T_q = 0 is a no-op.
 */
int dsa_ratio_causal_metadata(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              const int32_t* q_causal_offsets, int32_t n_seq, int64_t T_q,
                              int32_t ratio, int32_t* row_starts, int32_t* seq_lens,
                              void* stream);

/*
 * dsa_indexer_fwd - step a1, lightning-indexer scores.
 * DSA page section 3: for query row t and local key column j < seq_lens[t]
 * (the causal mask from dsa_packed_metadata, or the ratio-causal mask with
 * query causal offsets from dsa_ratio_causal_metadata),
 *   scores[t - row_begin, j] = sum_h W[t, h] * max(0, sum_d q_idx[t, h, d] * k_idx[row_starts[t] + j, d])
 * The indexer key has a single head shared by all H_idx query heads. No
 * scaling is applied inside: W already carries any 1/sqrt(H) and 1/sqrt(D)
 * factors (cudnn_dsa page, cudnn_indexer_topk, head_weights).
 *   q_idx       device bf16 [T, H_idx, D_idx], contiguous
 *   k_idx       device bf16 [T_kv, D_idx], contiguous
 *   w           device [T, H_idx], dtype w_dtype (DSA_BF16 or DSA_F32),
 *               aligned to its element size (any storage offset works)
 *   row_starts, seq_lens  device int32 [T] (from either metadata call)
 *   T, H_idx, D_idx       H_idx in [1, 64], D_idx in {64, 128}
 *   T_kv        rows of k_idx; key rows outside [0, T_kv) are never read
 *               (row_starts[t] + seq_lens[t] <= T_kv is the caller's
 *               contract; T_kv = 0 writes nothing)
 *   row_begin, n_rows     rows [row_begin, row_begin + n_rows) of T; the
 *                         caller chunks rows to bound the score buffer
 *   scores      device fp32 [n_rows, ld_scores] output, 16-byte aligned,
 *               ld_scores % 4 == 0. Only columns j < min(seq_lens[t],
 *               ld_scores) are written; later columns are left untouched, so
 *               ld_scores must be at least the longest causal length of the
 *               chunk for every key to be scored.
 * fp32 accumulation of bf16 products (MFMA), fp32 epilogue.
 */
int dsa_indexer_fwd(const void* q_idx, const void* k_idx, const void* w, int32_t w_dtype,
                    const int32_t* row_starts, const int32_t* seq_lens, int64_t T, int64_t T_kv,
                    int32_t H_idx, int32_t D_idx, int64_t row_begin, int64_t n_rows,
                    float* scores, int64_t ld_scores, void* stream);

/*
 * dsa_indexer_fwd_fp8 - step a1 from FP8 inputs.
 * DSA page section 3, "Precision paths": Q and K are FP8 E4M3 (the OCP
 * encoding: bias 7, no infinities, S.1111.111 = NaN, max 448) with either
 *   DSA_FP8_PER_TOKEN: fp32 descales q_scale [T, H_idx] (one per token and
 *     head) and k_scale [T_kv] (one per key token), real values being
 *     E4M3 value * descale; descales must be >= 0;
 *   DSA_MXFP8: E8M0 scale bytes (2^(byte - 127)) q_scale [T, H_idx, D_idx/32]
 *     and k_scale [T_kv, D_idx/32], one per 32 consecutive elements of the
 *     head dim; real values being E4M3 value * 2^(byte - 127).
 * The scores are dsa_indexer_fwd's definition on those real values, with the
 * same row, column, mask and buffer conventions:
 *   scores[t - row_begin, j] = sum_h W[t, h] * max(0, Q[t, h, :] . K[row_starts[t] + j, :])
 *   q8          device uint8 E4M3 [T, H_idx, D_idx], 16-byte aligned
 *   k8          device uint8 E4M3 [T_kv, D_idx], 16-byte aligned
 *   q_scale, k_scale  device, layout by `scaling`; k_scale 4-byte aligned
 *   w, w_dtype  device [T, H_idx], DSA_BF16 or DSA_F32 (W as in
 *               dsa_indexer_fwd; a caller may pre-multiply the query
 *               descales into fp32 W and pass unit q descales)
 *   D_idx       128 (the section's head-dim constraint); H_idx in [1, 64]
 *   other arguments as for dsa_indexer_fwd.
 * E4M3 products are exact; the MFMA sums them in fp32 (per 32-element block
 * for MXFP8), then the epilogue is fp32. NaN codes give unspecified scores.
 * Errors: as dsa_indexer_fwd, plus DSA_ERR_VALUE for an unknown scaling or
 * D_idx != 128.
 */
int dsa_indexer_fwd_fp8(const void* q8, const void* q_scale, const void* k8, const void* k_scale,
                        int32_t scaling, const void* w, int32_t w_dtype,
                        const int32_t* row_starts, const int32_t* seq_lens, int64_t T,
                        int64_t T_kv, int32_t H_idx, int32_t D_idx, int64_t row_begin,
                        int64_t n_rows, float* scores, int64_t ld_scores, void* stream);

/*
 * dsa_topk - steps a2 + a3, radix top-K with per-row length, compaction and
 * local -> global conversion.
 * DSA page section 5 (radix top-K over input_values (n_rows, num_cols) with a
 * per-row effective length) and section 4 (deterministic tie-break: exact
 * ties at the K-th boundary go to the smallest column); cudnn_dsa page
 * (global coordinates, ascending valid prefix, -1 suffix).
 * For row r with n = clamp(seq_lens[r], 0, n_cols):
 *   n <= k : the selection is every column 0..n-1;
 *   n >  k : the k largest of scores[r, 0..n-1], ties to the lower column;
 *            -0.0 and +0.0 are equal values.
 *   indices[r, 0..m-1] = row_starts[r] + selected columns in ascending order
 *   (plain column ids when row_starts is NULL), indices[r, m..k-1] = -1,
 *   m = min(n, k); topk_length[r] = m; values[r, i] = the selected score
 *   (-inf in padded slots).
 *   scores      device fp32 [n_rows, ld_scores], 16-byte aligned, ld % 4 == 0
 *   n_cols      1..DSA_TOPK_MAX_COLS, n_cols <= ld_scores
 *   seq_lens    device int32 [n_rows]
 *   row_starts  device int32 [n_rows] or NULL
 *   k           1..DSA_MAX_TOPK
 *   indices     device int32 [n_rows, ld_indices] output, ld_indices >= k
 *   topk_length device int32 [n_rows] output or NULL
 *   values      device fp32 [n_rows, ld_indices] output or NULL
 * Scores must not be NaN (NaN order is unspecified).
 */
int dsa_topk(const float* scores, int64_t ld_scores, int64_t n_rows, int64_t n_cols,
             const int32_t* seq_lens, const int32_t* row_starts, int32_t k,
             int32_t* indices, int64_t ld_indices, int32_t* topk_length, float* values,
             void* stream);

/*
 * dsa_topk_workspace_bytes - device workspace dsa_topk needs for these sizes.
 * The DSA page (section 4) has callers own every buffer, sizing them with a
 * query before the call. dsa_topk keeps each row's working set on chip
 * (registers and LDS) and takes no workspace argument, so this returns 0 for
 * every size dsa_topk accepts (0 <= n_rows <= INT32_MAX, 1 <= n_cols <=
 * DSA_TOPK_MAX_COLS, 1 <= k <= DSA_MAX_TOPK) and -1 for sizes it rejects.
 */
int64_t dsa_topk_workspace_bytes(int64_t n_rows, int64_t n_cols, int32_t k);

/*
 * dsa_indexer_topk_fused - steps a1 + a2 + a3 in one launch.
 * DSA page section 4 (combined indexer forward + top-K: indices, logits and
 * the softmax over the selected scores with its LSE, without dense scores;
 * section 6 defines that softmax) with the selection and output form of
 * dsa_topk. For query rows t in [row_begin, row_begin + n_rows), row
 * r = t - row_begin of the outputs:
 *   scores of row t: dsa_indexer_fwd's definition over local columns
 *     j < n = clamp(seq_lens[t], 0, n_cols), from bf16 inputs
 *     (DSA_INDEXER_BF16; q_scale and k_scale unused) or from FP8 inputs
 *     with the scales of dsa_indexer_fwd_fp8 (DSA_INDEXER_FP8: per-token,
 *     DSA_INDEXER_MXFP8: block-scaled);
 *   indices[r, :], topk_length[r]: dsa_topk on those scores (k largest,
 *     ties to the lower column, ascending, + row_starts[t], -1 suffix);
 *   logits[r, i]  = the selected score, -inf in padded slots   (or NULL)
 *   softmax[r, i] = exp(logits[r, i] - lse[r]), 0 in padded slots (or NULL)
 *   lse[r]        = ln sum_i exp(logits[r, i]) over the selected slots,
 *                   +inf for a row with no slot                 (or NULL)
 * A row whose seq_lens exceeds n_cols is treated as n_cols long (as dsa_topk
 * does). No dense score matrix is written:
 * - n_cols <= DSA_FUSED_MAX_COLS: each row's scores stay in the CU's local
 *   memory and are selected there, in one launch; cand_buffer is unused
 *   (may be NULL).
 * - DSA_FUSED_MAX_COLS < n_cols <= DSA_TOPK_MAX_COLS (any precision): the
 *   DSA page's candidate scheme (section 4: a caller-owned candidate buffer,
 *   then a stage-2 select). The indexer pass appends, for each row, the
 *   columns whose score reaches a lower bound sampled from the row, as
 *   (score key, column) pairs; a second launch selects the top k from them;
 *   a third redoes exactly, from recomputed scores, any row whose candidates
 *   could not hold its top k (rare; correct for every input, slower). The
 *   result is the same as on the short-row path: dsa_topk of
 *   dsa_indexer_fwd's scores, bit for bit.
 *   cand_buffer  device float [cand_floats], 16-byte aligned, caller-owned
 *                scratch of at least dsa_indexer_topk_cand_buffer_size(
 *                n_rows, n_cols, k) floats; its contents on entry do not
 *                matter and are overwritten. Calls that overlap in time must
 *                not share one buffer.
 *   q_idx, k_idx, w, w_dtype, row_starts, seq_lens, T, T_kv, H_idx, D_idx,
 *   row_begin, n_rows: as dsa_indexer_fwd (bf16) or dsa_indexer_fwd_fp8
 *   k           1..DSA_MAX_TOPK
 *   indices     device int32 [n_rows, ld_indices], ld_indices >= k; logits
 *               and softmax use the same row stride
 *   topk_length device int32 [n_rows] or NULL
 * With T_kv = 0 every row is empty (k_idx and k_scale may then be NULL).
 * Errors: those of dsa_indexer_fwd / dsa_indexer_fwd_fp8 and dsa_topk,
 * DSA_ERR_VALUE for an unknown precision, n_cols outside
 * [1, DSA_TOPK_MAX_COLS], or a missing, misaligned or too small cand_buffer
 * when n_cols > DSA_FUSED_MAX_COLS.
 */
int dsa_indexer_topk_fused(const void* q_idx, const void* q_scale, const void* k_idx,
                           const void* k_scale, int32_t precision, const void* w,
                           int32_t w_dtype, const int32_t* row_starts, const int32_t* seq_lens,
                           int64_t T, int64_t T_kv, int32_t H_idx, int32_t D_idx,
                           int64_t row_begin, int64_t n_rows, int64_t n_cols, int32_t k,
                           int32_t* indices, int64_t ld_indices, int32_t* topk_length,
                           float* logits, float* softmax, float* lse, float* cand_buffer,
                           int64_t cand_floats, void* stream);

/*
 * dsa_indexer_topk_cand_buffer_size - floats of the candidate buffer that
 * dsa_indexer_topk_fused needs for these sizes (the DSA page, section 4,
 * sizes its candidate buffer with such a query, in floats). 0 when
 * n_cols <= DSA_FUSED_MAX_COLS or n_rows = 0 (no buffer is used), -1 for
 * sizes the call rejects (n_rows outside [0, INT32_MAX], n_cols outside
 * [1, DSA_TOPK_MAX_COLS], k outside [1, DSA_MAX_TOPK]). The size grows
 * linearly with n_rows (8192 (score, column) pairs per row, plus up to 256
 * rows of n_cols floats for the rescue); callers may split long row ranges
 * with row_begin / n_rows to bound it.
 */
int64_t dsa_indexer_topk_cand_buffer_size(int64_t n_rows, int64_t n_cols, int32_t k);

/*
 * dsa_sparse_attn_fwd - steps a4 / a5, sparse attention forward.
 * DSA page section 1: for query row t, head h and slot j < L_t, where
 * L_t = clamp(topk_length[t], 0, k_width) (k_width when topk_length is NULL),
 * slot j is valid iff 0 <= indices[t, j] < T_kv; invalid slots have score
 * -inf, duplicates stay distinct slots. With s_j = scale * q[t,h,:D_qk] . K[idx_j,:D_qk]:
 *   max_logits[t,h] = max_j s_j
 *   lse[t,h]        = ln sum_j exp(s_j)          (KV-only, excludes the sink)
 *   out[t,h,:]      = sum_j exp(s_j) V[idx_j,:D_v] / (sum_j exp(s_j) + exp(sink_h))
 * The sink is a per-head fp32 logit in scaled units that enters only the
 * output denominator (attn_sink NULL == -inf). A row with no valid slot gets
 * out = 0, max_logits = -inf, lse = +inf.
 *   q          device bf16 [T_q, H, D_qk], contiguous; H in [1, DSA_MAX_HEADS]
 *   k          device bf16 [T_kv, ld_k] key rows (shared latent KV for MLA)
 *   v          device bf16 [T_kv, ld_v] value rows, or NULL: V = k[:, :D_v]
 *              (D_qk = 576 uses the first 512 KV dims as V; section 1)
 *   (D_qk, D_v) in {(576, 512), (512, 512), (256, 256)}
 *   indices    device int32 [T_q, ld_indices], global KV row ids, -1 invalid
 *              (may be NULL when k_width = 0)
 *   k_width    0..ld_indices slots per row (0: every row is empty)
 *   topk_length device int32 [T_q] or NULL (compact prefix lengths)
 *   attn_sink  device fp32 [H] or NULL
 *   softmax_scale finite, > 0 (callers default it to 1/sqrt(D_qk))
 *   out        device bf16 [T_q, H, D_v] output
 *   lse        device fp32 [T_q, H] output (natural log)
 *   max_logits device fp32 [T_q, H] output or NULL
 * k, v, q, out need 16-byte alignment; ld_k, ld_v multiples of 8 elements.
 * Softmax in fp32 (exp2 domain), bf16 MFMA for q.k and p.v, fp32 accumulation,
 * output rounded to bf16 (round to nearest even).
 */
int dsa_sparse_attn_fwd(const void* q, int64_t T_q, int32_t H, int32_t D_qk,
                        const void* k, int64_t T_kv, int64_t ld_k,
                        const void* v, int64_t ld_v, int32_t D_v,
                        const int32_t* indices, int64_t ld_indices, int32_t k_width,
                        const int32_t* topk_length, const float* attn_sink,
                        float softmax_scale, void* out, float* lse, float* max_logits,
                        void* stream);

/*
 * dsa_sparse_attn_bwd_workspace_bytes - device workspace dsa_sparse_attn_bwd
 * uses for these sizes: fp32 statistics [T_q, H] x 2, an fp32 dkv
 * accumulator [T_kv, D_qk], per-KV-row counts and offsets [T_kv], and per
 * query row of a chunk its bf16 P and dS plus the buffers of its dkv scheme,
 * for chunks of up to 4 GiB (min(T_q, rows that fit) rows at a time):
 *  - KV tiles, when every row may select at least one key in eight
 *    (8 * k_width >= T_kv, T_kv <= 32768, k_width rounded up to 32 <= 8192):
 *    an int16 slot map per row over T_kv rounded up to 128, and per part of
 *    64 query rows an fp32 partial [T_kv rounded up to 128, D_qk] and its
 *    tile flags;
 *  - per-slot rows otherwise: the bf16 dkv rows of its slots, its slot list
 *    and the slot sort's key / value buffers.
 * Returns -1 for sizes out of contract.
 */
int64_t dsa_sparse_attn_bwd_workspace_bytes(int64_t T_q, int32_t H, int64_t T_kv, int32_t D_qk,
                                            int32_t k_width);

/*
 * dsa_sparse_attn_bwd_kv_tiles - which dkv scheme dsa_sparse_attn_bwd takes
 * for T_kv KV rows and k_width slots per row: 1 for KV tiles (8 * k_width >=
 * T_kv, 0 < T_kv <= 32768, 0 < k_width rounded up to 32 <= 8192), 0 for
 * per-slot rows (the rule of dsa_sparse_attn_bwd_workspace_bytes). Needs no
 * device; -1 for T_kv or k_width below 0.
 */
int dsa_sparse_attn_bwd_kv_tiles(int64_t T_kv, int32_t k_width);

/*
 * dsa_sparse_attn_bwd - gradients of dsa_sparse_attn_fwd for shared latent
 * KV (V = kv[:, :D_v]).
 * DSA page section 2 ("Sparse Attention Backward", the gradient of section
 * 1's forward): given the forward's out and KV-only lse and the gradient
 * dout of a loss with respect to out, for query row t, head h and valid slot
 * j (the validity rules of dsa_sparse_attn_fwd), with
 * P_j = exp(s_j) / (sum_i exp(s_i) + exp(sink_h)), D = dout . out,
 * dS_j = P_j (dout . v_j - D):
 *   dq[t, h, :]        = scale sum_j dS_j kv[idx_j, :D_qk]
 *   dkv[r, :]          = sum over slots with idx_j = r of scale dS_j q[t, h, :]
 *                        (+ P_j dout[t, h, :] on the first D_v columns)
 *   d_sink[h]          = -sum_t P_sink(t, h) D(t, h),
 *                        P_sink = exp(sink_h) / (sum_i exp(s_i) + exp(sink_h))
 * Duplicate slots contribute separately. P comes from the given lse
 * (log of the denominator = log(exp(lse) + exp(sink))), D from the given
 * out; an empty row (lse = +inf) contributes nothing.
 *   q, kv, indices, ld_indices, k_width, topk_length, attn_sink,
 *   softmax_scale: as dsa_sparse_attn_fwd; (D_qk, D_v) in {(576, 512),
 *   (512, 512)}, v is kv[:, :512]; H in [1, DSA_MAX_HEADS]
 *   out, dout   device bf16 [T_q, H, D_v], contiguous, 16-byte aligned
 *   lse         device fp32 [T_q, H]
 *   dq          device bf16 [T_q, H, D_qk] output
 *   dkv         device bf16 [T_kv, D_qk] output (contiguous)
 *   d_sink      device fp32 [H] output or NULL (0 when attn_sink is NULL)
 *   workspace   device memory, 256-byte aligned, owned by the caller, of
 *               workspace_bytes bytes: at least what one query row needs
 *               (fixed statistics plus one row of the chunk buffers);
 *               dsa_sparse_attn_bwd_workspace_bytes gives a size that holds
 *               up to 4 GiB of chunk buffers, and a larger workspace
 *               processes more query rows per pass
 * bf16 MFMA products with fp32 accumulation; P and dS are rounded to bf16
 * before the dq and dkv products. dkv by one of two schemes (the rule of
 * dsa_sparse_attn_bwd_workspace_bytes):
 *  - KV tiles: per tile of 128 KV rows and part of 64 query rows, dS^T q +
 *    P^T dout over the part's rows and heads as one fp32 product (zeros
 *    where a row selects no slot for a KV row; a row's repeated ids first
 *    merged into its lowest slot, summed in ascending slot order and rounded
 *    to bf16), the parts then added in ascending order;
 *  - per-slot rows: each slot's dkv row (summed over the heads) rounded to
 *    bf16, then summed per KV row in fp32 in ascending (row, slot) order
 *    (a stable sort).
 * No atomics decide an order: equal inputs and workspace sizes give
 * identical bits. d_sink is summed in a fixed order.
 * Errors: the checks of dsa_sparse_attn_fwd, DSA_ERR_VALUE for D_v != 512,
 * a separate V, or a workspace too small for one row.
 */
int dsa_sparse_attn_bwd(const void* q, int64_t T_q, int32_t H, int32_t D_qk, const void* kv,
                        int64_t T_kv, int64_t ld_kv, int32_t D_v, const int32_t* indices,
                        int64_t ld_indices, int32_t k_width, const int32_t* topk_length,
                        const float* attn_sink, float softmax_scale, const void* out,
                        const void* dout, const float* lse, void* dq, void* dkv, float* d_sink,
                        void* workspace, int64_t workspace_bytes, void* stream);

/*
 * dsa_sparse_attn_bwd_noalloc - dsa_sparse_attn_bwd for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops,
 * harnesses that forbid allocation): the same gradients from the same
 * kernels, with the workspace replaced by a scratch array that the library
 * keeps in device memory, DSA_NOALLOC_SCRATCH_BYTES per device, held from the
 * first call on a device until the process ends. The call allocates and
 * frees nothing.
 *   Arguments: as dsa_sparse_attn_bwd, without workspace / workspace_bytes.
 *   Results: bit for bit those of dsa_sparse_attn_bwd given a workspace of
 *   DSA_NOALLOC_SCRATCH_BYTES bytes (the workspace size sets the chunks of
 *   query rows, and with them the order of the dkv sums).
 *   Sizes: the scratch must hold the fixed buffers plus one query row's
 *   (dsa_sparse_attn_bwd_workspace_bytes with T_q = 1 and the same other
 *   sizes, plus the [T_q, H] statistics); larger sizes return DSA_ERR_VALUE
 *   with nothing launched.
 *   Concurrency: every call on a device uses that device's one scratch
 *   array, which keeps the previous call's contents (each call clears what
 *   it needs zeroed). Calls that overlap on one device (other streams, other
 *   threads) race on it; order them on one stream.
 * Errors: those of dsa_sparse_attn_bwd; DSA_ERR_RUNTIME if the scratch's
 * device address cannot be obtained.
 */
int dsa_sparse_attn_bwd_noalloc(const void* q, int64_t T_q, int32_t H, int32_t D_qk,
                                const void* kv, int64_t T_kv, int64_t ld_kv, int32_t D_v,
                                const int32_t* indices, int64_t ld_indices, int32_t k_width,
                                const int32_t* topk_length, const float* attn_sink,
                                float softmax_scale, const void* out, const void* dout,
                                const float* lse, void* dq, void* dkv, float* d_sink,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
