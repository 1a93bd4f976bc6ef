// C ABI of the DSA forward path: host-side validation, device check, launch.
// Every argument check runs before any HIP call, so a bad call returns its
// status without touching the runtime. Nothing here allocates or synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "dsa.h"
#include "dsa_launch.h"
#include "dsa_select.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// 1 = gfx950, 0 = other arch, cached per device ordinal.
constexpr int kMaxDev = 64;
int g_arch_ok[kMaxDev];
std::once_flag g_arch_once[kMaxDev];

int check_device(const char* fn) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDev)
    return fail(DSA_ERR_RUNTIME, "%s: no HIP device is current (%s)", fn, hipGetErrorString(e));
  std::call_once(g_arch_once[dev], [dev]() {
    hipDeviceProp_t prop;
    g_arch_ok[dev] = 0;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess)
      g_arch_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
  });
  if (!g_arch_ok[dev])
    return fail(DSA_ERR_RUNTIME, "%s: device %d is not a gfx950 (MI355X) GPU", fn, dev);
  return DSA_OK;
}

// Scratch of dsa_sparse_attn_bwd_noalloc, for callers that cannot allocate.
// One copy per device, at its own address, held until the process ends; every
// call on a device shares it. In host code `scratch` names a host-side stand-in,
// never the device memory: its device address is looked up once per device
// (with that device current) and only that address is passed to kernels.
__device__ __align__(256) unsigned char scratch[DSA_NOALLOC_SCRATCH_BYTES];
void* g_scratch_ptr[kMaxDev];
char g_scratch_err[kMaxDev][128];
std::once_flag g_scratch_once[kMaxDev];

// Device address of `scratch` on device `dev` (current), or NULL if the
// lookup failed (the reason is in g_scratch_err[dev]).
void* noalloc_scratch(int dev) {
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr || (uintptr_t)p % 256 != 0) {
      snprintf(g_scratch_err[dev], sizeof(g_scratch_err[dev]), "hipGetSymbolAddress: %s",
               e != hipSuccess ? hipGetErrorString(e) : "bad address");
      g_scratch_ptr[dev] = nullptr;
    } else {
      g_scratch_ptr[dev] = p;
    }
  });
  return g_scratch_ptr[dev];
}

int launched(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(DSA_ERR_RUNTIME, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return DSA_OK;
}

}  // namespace

extern "C" {

const char* dsa_last_error(void) { return g_err; }

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

int dsa_packed_metadata(const int32_t* cu_seqlens, int32_t n_seq, int64_t T, int32_t* row_starts,
                        int32_t* seq_lens, void* stream) {
  const char* fn = "dsa_packed_metadata";
  REQUIRE(n_seq >= 1, DSA_ERR_VALUE, "%s: n_seq must be >= 1 (got %d)", fn, n_seq);
  REQUIRE(T >= 0 && T <= INT32_MAX, DSA_ERR_VALUE, "%s: T must be in [0, 2^31-1] (got %lld)", fn,
          (long long)T);
  if (T == 0) return DSA_OK;
  REQUIRE(cu_seqlens && row_starts && seq_lens, DSA_ERR_VALUE, "%s: NULL pointer argument", fn);
  if (int rc = check_device(fn)) return rc;
  return launched(fn, dsa::launch_packed_metadata(cu_seqlens, n_seq, T, row_starts, seq_lens,
                                                  (hipStream_t)stream));
}

int dsa_ratio_causal_metadata(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              const int32_t* q_causal_offsets, int32_t n_seq, int64_t T_q,
                              int32_t ratio, int32_t* row_starts, int32_t* seq_lens,
                              void* stream) {
  const char* fn = "dsa_ratio_causal_metadata";
  REQUIRE(n_seq >= 1, DSA_ERR_VALUE, "%s: n_seq must be >= 1 (got %d)", fn, n_seq);
  REQUIRE(T_q >= 0 && T_q <= INT32_MAX, DSA_ERR_VALUE, "%s: T_q must be in [0, 2^31-1] (got %lld)",
          fn, (long long)T_q);
  REQUIRE(ratio >= 1, DSA_ERR_VALUE, "%s: ratio must be >= 1 (got %d)", fn, ratio);
  if (T_q == 0) return DSA_OK;
  REQUIRE(cu_seqlens_q && cu_seqlens_k && row_starts && seq_lens, DSA_ERR_VALUE,
          "%s: NULL pointer argument", fn);
  if (int rc = check_device(fn)) return rc;
  return launched(fn, dsa::launch_ratio_metadata(cu_seqlens_q, cu_seqlens_k, q_causal_offsets,
                                                 n_seq, T_q, ratio, row_starts, seq_lens,
                                                 (hipStream_t)stream));
}

int dsa_indexer_fwd(const void* q_idx, const void* k_idx, const void* w, int32_t w_dtype,
                    const int32_t* row_starts, const int32_t* seq_lens, int64_t T, int64_t T_kv,
                    int32_t H_idx, int32_t D_idx, int64_t row_begin, int64_t n_rows,
                    float* scores, int64_t ld_scores, void* stream) {
  const char* fn = "dsa_indexer_fwd";
  REQUIRE(w_dtype == DSA_BF16 || w_dtype == DSA_F32, DSA_ERR_TYPE,
          "%s: w_dtype must be DSA_BF16 or DSA_F32 (got %d)", fn, w_dtype);
  REQUIRE(H_idx >= 1 && H_idx <= 64, DSA_ERR_VALUE, "%s: H_idx must be in [1, 64] (got %d)", fn,
          H_idx);
  REQUIRE(D_idx == 64 || D_idx == 128, DSA_ERR_VALUE, "%s: D_idx must be 64 or 128 (got %d)", fn,
          D_idx);
  REQUIRE(T >= 0 && T <= INT32_MAX, DSA_ERR_VALUE, "%s: T must be in [0, 2^31-1]", fn);
  REQUIRE(T_kv >= 0 && T_kv <= INT32_MAX, DSA_ERR_VALUE, "%s: T_kv must be in [0, 2^31-1]", fn);
  REQUIRE(row_begin >= 0 && n_rows >= 0 && row_begin + n_rows <= T, DSA_ERR_VALUE,
          "%s: rows [%lld, %lld) outside [0, T=%lld)", fn, (long long)row_begin,
          (long long)(row_begin + n_rows), (long long)T);
  REQUIRE(ld_scores >= 4 && ld_scores % 4 == 0, DSA_ERR_VALUE,
          "%s: ld_scores must be a positive multiple of 4 (got %lld)", fn, (long long)ld_scores);
  if (n_rows == 0 || T_kv == 0) return DSA_OK;
  REQUIRE(q_idx && k_idx && w && row_starts && seq_lens && scores, DSA_ERR_VALUE,
          "%s: NULL pointer argument", fn);
  REQUIRE(aligned(q_idx, 16) && aligned(k_idx, 16) && aligned(scores, 16), DSA_ERR_VALUE,
          "%s: q_idx, k_idx and scores must be 16-byte aligned", fn);
  REQUIRE(aligned(w, w_dtype == DSA_F32 ? 4 : 2), DSA_ERR_VALUE, "%s: w misaligned", fn);
  REQUIRE(n_rows <= (int64_t)8 * INT32_MAX, DSA_ERR_VALUE, "%s: too many rows", fn);
  if (int rc = check_device(fn)) return rc;
  return launched(fn, dsa::launch_indexer(q_idx, k_idx, w, w_dtype, row_starts, seq_lens, T_kv,
                                          H_idx, D_idx, row_begin, n_rows, scores, ld_scores,
                                          (hipStream_t)stream));
}

int dsa_indexer_fwd_fp8(const void* q8, const void* q_scale, const void* k8, const void* k_scale,
                        int32_t scaling, const void* w, int32_t w_dtype,
                        const int32_t* row_starts, const int32_t* seq_lens, int64_t T,
                        int64_t T_kv, int32_t H_idx, int32_t D_idx, int64_t row_begin,
                        int64_t n_rows, float* scores, int64_t ld_scores, void* stream) {
  const char* fn = "dsa_indexer_fwd_fp8";
  REQUIRE(w_dtype == DSA_BF16 || w_dtype == DSA_F32, DSA_ERR_TYPE,
          "%s: w_dtype must be DSA_BF16 or DSA_F32 (got %d)", fn, w_dtype);
  REQUIRE(scaling == DSA_FP8_PER_TOKEN || scaling == DSA_MXFP8, DSA_ERR_VALUE,
          "%s: scaling must be DSA_FP8_PER_TOKEN or DSA_MXFP8 (got %d)", fn, scaling);
  REQUIRE(H_idx >= 1 && H_idx <= 64, DSA_ERR_VALUE, "%s: H_idx must be in [1, 64] (got %d)", fn,
          H_idx);
  REQUIRE(D_idx == 128, DSA_ERR_VALUE, "%s: D_idx must be 128 (got %d)", fn, D_idx);
  REQUIRE(T >= 0 && T <= INT32_MAX, DSA_ERR_VALUE, "%s: T must be in [0, 2^31-1]", fn);
  REQUIRE(T_kv >= 0 && T_kv <= INT32_MAX, DSA_ERR_VALUE, "%s: T_kv must be in [0, 2^31-1]", fn);
  REQUIRE(row_begin >= 0 && n_rows >= 0 && row_begin + n_rows <= T, DSA_ERR_VALUE,
          "%s: rows [%lld, %lld) outside [0, T=%lld)", fn, (long long)row_begin,
          (long long)(row_begin + n_rows), (long long)T);
  REQUIRE(ld_scores >= 4 && ld_scores % 4 == 0, DSA_ERR_VALUE,
          "%s: ld_scores must be a positive multiple of 4 (got %lld)", fn, (long long)ld_scores);
  if (n_rows == 0 || T_kv == 0) return DSA_OK;
  REQUIRE(q8 && q_scale && k8 && k_scale && w && row_starts && seq_lens && scores, DSA_ERR_VALUE,
          "%s: NULL pointer argument", fn);
  REQUIRE(aligned(q8, 16) && aligned(k8, 16) && aligned(scores, 16), DSA_ERR_VALUE,
          "%s: q8, k8 and scores must be 16-byte aligned", fn);
  REQUIRE(aligned(k_scale, 4) && (scaling == DSA_MXFP8 || aligned(q_scale, 4)), DSA_ERR_VALUE,
          "%s: scale tensors misaligned", fn);
  REQUIRE(aligned(w, w_dtype == DSA_F32 ? 4 : 2), DSA_ERR_VALUE, "%s: w misaligned", fn);
  if (int rc = check_device(fn)) return rc;
  return launched(fn, dsa::launch_indexer_fp8(q8, q_scale, k8, k_scale, scaling == DSA_MXFP8, w,
                                              w_dtype, row_starts, seq_lens, T_kv, H_idx,
                                              row_begin, n_rows, scores, ld_scores,
                                              (hipStream_t)stream));
}

// Layout of the candidate buffer of the combined path for long rows, in
// 4-byte words: the queue length, the per-row counts and the queue, the
// rescue's dense rows, then the candidate lists (16-byte aligned).
struct CandLayout {
  int64_t count, queue, spill, spill_ld, n_spill, cand, total;
};
static CandLayout cand_layout(int64_t n_rows, int64_t n_cols) {
  CandLayout L;
  auto up4 = [](int64_t x) { return (x + 3) / 4 * 4; };
  L.count = 4;
  L.queue = L.count + up4(n_rows);
  L.spill = L.queue + up4(n_rows);
  L.spill_ld = up4(n_cols);
  L.n_spill = std::min<int64_t>(dsa::kCandSpillRows, n_rows);
  L.cand = L.spill + L.n_spill * L.spill_ld;
  L.total = L.cand + n_rows * dsa::kCandCap * 2;
  return L;
}

int64_t dsa_indexer_topk_cand_buffer_size(int64_t n_rows, int64_t n_cols, int32_t k) {
  if (n_rows < 0 || n_rows > INT32_MAX || n_cols < 1 || n_cols > DSA_TOPK_MAX_COLS || k < 1 ||
      k > DSA_MAX_TOPK)
    return -1;
  if (n_cols <= DSA_FUSED_MAX_COLS || n_rows == 0) return 0;
  return cand_layout(n_rows, n_cols).total;
}

int dsa_indexer_topk_fused(const void* q_idx, const void* q_scale, const void* k_idx,
                           const void* k_scale, int32_t precision, const void* w,
                           int32_t w_dtype, const int32_t* row_starts, const int32_t* seq_lens,
                           int64_t T, int64_t T_kv, int32_t H_idx, int32_t D_idx,
                           int64_t row_begin, int64_t n_rows, int64_t n_cols, int32_t k,
                           int32_t* indices, int64_t ld_indices, int32_t* topk_length,
                           float* logits, float* softmax, float* lse, float* cand_buffer,
                           int64_t cand_floats, void* stream) {
  const char* fn = "dsa_indexer_topk_fused";
  REQUIRE(w_dtype == DSA_BF16 || w_dtype == DSA_F32, DSA_ERR_TYPE,
          "%s: w_dtype must be DSA_BF16 or DSA_F32 (got %d)", fn, w_dtype);
  REQUIRE(precision == DSA_INDEXER_BF16 || precision == DSA_INDEXER_FP8 ||
              precision == DSA_INDEXER_MXFP8,
          DSA_ERR_VALUE, "%s: unknown precision %d", fn, precision);
  const bool fp8 = precision != DSA_INDEXER_BF16;
  REQUIRE(H_idx >= 1 && H_idx <= 64, DSA_ERR_VALUE, "%s: H_idx must be in [1, 64] (got %d)", fn,
          H_idx);
  REQUIRE(D_idx == 128 || (!fp8 && D_idx == 64), DSA_ERR_VALUE,
          "%s: D_idx must be 128 (or 64 for bf16 inputs; got %d)", fn, D_idx);
  REQUIRE(T >= 0 && T <= INT32_MAX, DSA_ERR_VALUE, "%s: T must be in [0, 2^31-1]", fn);
  REQUIRE(T_kv >= 0 && T_kv <= INT32_MAX, DSA_ERR_VALUE, "%s: T_kv must be in [0, 2^31-1]", fn);
  REQUIRE(row_begin >= 0 && n_rows >= 0 && row_begin + n_rows <= T, DSA_ERR_VALUE,
          "%s: rows [%lld, %lld) outside [0, T=%lld)", fn, (long long)row_begin,
          (long long)(row_begin + n_rows), (long long)T);
  REQUIRE(n_cols >= 1 && n_cols <= DSA_TOPK_MAX_COLS, DSA_ERR_VALUE,
          "%s: n_cols must be in [1, %d] (got %lld)", fn, DSA_TOPK_MAX_COLS, (long long)n_cols);
  REQUIRE(k >= 1 && k <= DSA_MAX_TOPK, DSA_ERR_VALUE, "%s: k must be in [1, %d] (got %d)", fn,
          DSA_MAX_TOPK, k);
  REQUIRE(ld_indices >= k, DSA_ERR_VALUE, "%s: ld_indices (%lld) < k (%d)", fn,
          (long long)ld_indices, k);
  const bool long_rows = n_cols > DSA_FUSED_MAX_COLS;
  if (n_rows == 0) return DSA_OK;
  if (long_rows) {
    const int64_t need = dsa_indexer_topk_cand_buffer_size(n_rows, n_cols, k);
    REQUIRE(cand_buffer && cand_floats >= need, DSA_ERR_VALUE,
            "%s: n_cols = %lld needs a candidate buffer of %lld floats "
            "(dsa_indexer_topk_cand_buffer_size; got %lld)",
            fn, (long long)n_cols, (long long)need, (long long)cand_floats);
    REQUIRE(aligned(cand_buffer, 16), DSA_ERR_VALUE, "%s: cand_buffer must be 16-byte aligned",
            fn);
  }
  REQUIRE(q_idx && (k_idx || T_kv == 0) && w && row_starts && seq_lens && indices &&
              (!fp8 || (q_scale && (k_scale || T_kv == 0))),
          DSA_ERR_VALUE, "%s: NULL pointer argument", fn);
  REQUIRE(aligned(q_idx, 16) && aligned(k_idx, 16), DSA_ERR_VALUE,
          "%s: q_idx and k_idx must be 16-byte aligned", fn);
  REQUIRE(!fp8 || (aligned(k_scale, 4) && (precision == DSA_INDEXER_MXFP8 || aligned(q_scale, 4))),
          DSA_ERR_VALUE, "%s: scale tensors misaligned", fn);
  REQUIRE(aligned(w, w_dtype == DSA_F32 ? 4 : 2), DSA_ERR_VALUE, "%s: w misaligned", fn);
  if (int rc = check_device(fn)) return rc;
  // (T_kv = 0: every row is empty; the kernels then load no key.)
  dsa::FusedArgs fa{k, indices, ld_indices, topk_length, logits, softmax, lse};
  if (long_rows) {
    // Stage 1 (indexer pass appending candidates), stage 2 (select from the
    // candidates; rows they cannot serve are queued), rescue (queued rows).
    const CandLayout L = cand_layout(n_rows, n_cols);
    uint32_t* buf = reinterpret_cast<uint32_t*>(cand_buffer);
    dsa::CandArgs ca{buf + L.cand,
                     dsa::kCandCap,
                     reinterpret_cast<int32_t*>(buf + L.count),
                     reinterpret_cast<int32_t*>(buf + L.queue),
                     buf,
                     cand_buffer + L.spill,
                     L.spill_ld,
                     (int)L.n_spill};
    hipStream_t st = (hipStream_t)stream;
    const bool mx = precision == DSA_INDEXER_MXFP8;
    if (int rc = launched(fn, fp8 ? dsa::launch_indexer_cand_fp8(q_idx, q_scale, k_idx, k_scale,
                                                                mx, w, w_dtype, row_starts,
                                                                seq_lens, T_kv, H_idx, row_begin,
                                                                n_rows, n_cols, k, ca, st)
                                  : dsa::launch_indexer_cand(q_idx, k_idx, w, w_dtype, row_starts,
                                                             seq_lens, T_kv, H_idx, D_idx,
                                                             row_begin, n_rows, n_cols, k, ca,
                                                             st)))
      return rc;
    const int64_t n_eff = T_kv > 0 ? n_cols : 0;
    if (int rc = launched(fn, dsa::launch_topk_cand(seq_lens + row_begin, row_starts + row_begin,
                                                    n_rows, n_eff, k, indices, ld_indices,
                                                    topk_length, logits, softmax, lse, ca, st)))
      return rc;
    if (fp8)
      return launched(fn, dsa::launch_indexer_rescue_fp8(q_idx, q_scale, k_idx, k_scale, mx, w,
                                                         w_dtype, row_starts, seq_lens, T_kv,
                                                         H_idx, row_begin, n_rows, n_cols, fa,
                                                         ca, st));
    return launched(fn, dsa::launch_indexer_rescue(q_idx, k_idx, w, w_dtype, row_starts, seq_lens,
                                                   T_kv, H_idx, D_idx, row_begin, n_rows, n_cols,
                                                   fa, ca, st));
  }
  if (fp8)
    return launched(fn, dsa::launch_indexer_topk_fp8(q_idx, q_scale, k_idx, k_scale,
                                                     precision == DSA_INDEXER_MXFP8, w, w_dtype,
                                                     row_starts, seq_lens, T_kv, H_idx, row_begin,
                                                     n_rows, n_cols, fa, (hipStream_t)stream));
  return launched(fn, dsa::launch_indexer_topk(q_idx, k_idx, w, w_dtype, row_starts, seq_lens,
                                               T_kv, H_idx, D_idx, row_begin, n_rows, n_cols, fa,
                                               (hipStream_t)stream));
}

int64_t dsa_topk_workspace_bytes(int64_t n_rows, int64_t n_cols, int32_t k) {
  // Every row's working set stays in registers and LDS: no device workspace.
  if (n_rows < 0 || n_rows > INT32_MAX || n_cols < 1 || n_cols > DSA_TOPK_MAX_COLS || k < 1 ||
      k > DSA_MAX_TOPK)
    return -1;
  return 0;
}

int dsa_topk(const float* scores, int64_t ld_scores, int64_t n_rows, int64_t n_cols,
             const int32_t* seq_lens, const int32_t* row_starts, int32_t k, int32_t* indices,
             int64_t ld_indices, int32_t* topk_length, float* values, void* stream) {
  const char* fn = "dsa_topk";
  REQUIRE(k >= 1 && k <= DSA_MAX_TOPK, DSA_ERR_VALUE, "%s: k must be in [1, %d] (got %d)", fn,
          DSA_MAX_TOPK, k);
  REQUIRE(n_cols >= 1 && n_cols <= DSA_TOPK_MAX_COLS, DSA_ERR_VALUE,
          "%s: n_cols must be in [1, %d] (got %lld)", fn, DSA_TOPK_MAX_COLS, (long long)n_cols);
  REQUIRE(ld_scores >= n_cols && ld_scores % 4 == 0, DSA_ERR_VALUE,
          "%s: ld_scores must be >= n_cols and a multiple of 4 (got %lld)", fn,
          (long long)ld_scores);
  REQUIRE(ld_indices >= k, DSA_ERR_VALUE, "%s: ld_indices (%lld) < k (%d)", fn,
          (long long)ld_indices, k);
  REQUIRE(n_rows >= 0 && n_rows <= INT32_MAX, DSA_ERR_VALUE, "%s: n_rows out of range", fn);
  if (n_rows == 0) return DSA_OK;
  REQUIRE(scores && seq_lens && indices, DSA_ERR_VALUE, "%s: NULL pointer argument", fn);
  REQUIRE(aligned(scores, 16), DSA_ERR_VALUE, "%s: scores must be 16-byte aligned", fn);
  if (int rc = check_device(fn)) return rc;
  return launched(fn, dsa::launch_topk(scores, ld_scores, n_rows, n_cols, seq_lens, row_starts, k,
                                       indices, ld_indices, topk_length, values,
                                       (hipStream_t)stream));
}

int dsa_sparse_attn_fwd(const void* q, int64_t T_q, int32_t H, int32_t D_qk, const void* k,
                        int64_t T_kv, int64_t ld_k, const void* v, int64_t ld_v, int32_t D_v,
                        const int32_t* indices, int64_t ld_indices, int32_t k_width,
                        const int32_t* topk_length, const float* attn_sink, float softmax_scale,
                        void* out, float* lse, float* max_logits, void* stream) {
  const char* fn = "dsa_sparse_attn_fwd";
  REQUIRE(H >= 1 && H <= DSA_MAX_HEADS, DSA_ERR_VALUE, "%s: H must be in [1, %d] (got %d)", fn,
          DSA_MAX_HEADS, H);
  const bool dims_ok = (D_qk == 576 && D_v == 512) || (D_qk == 512 && D_v == 512) ||
                       (D_qk == 256 && D_v == 256);
  REQUIRE(dims_ok, DSA_ERR_VALUE,
          "%s: (D_qk, D_v) must be (576, 512), (512, 512) or (256, 256) (got (%d, %d))", fn, D_qk,
          D_v);
  REQUIRE(!(D_qk == 576 && v != nullptr), DSA_ERR_VALUE,
          "%s: D_qk = 576 is shared latent KV; pass v = NULL (V = kv[:, :512])", fn);
  REQUIRE(v == nullptr || v == k || D_qk == 256, DSA_ERR_VALUE,
          "%s: a separate V tensor is supported for D_qk = D_v = 256 only", fn);
  REQUIRE(T_q >= 0 && T_q <= INT32_MAX, DSA_ERR_VALUE, "%s: T_q out of range", fn);
  REQUIRE(T_kv >= 0 && T_kv <= INT32_MAX, DSA_ERR_VALUE, "%s: T_kv out of range", fn);
  REQUIRE(ld_k >= D_qk && ld_k % 8 == 0, DSA_ERR_VALUE,
          "%s: ld_k must be >= D_qk and a multiple of 8 (got %lld)", fn, (long long)ld_k);
  if (v) {
    REQUIRE(ld_v >= D_v && ld_v % 8 == 0, DSA_ERR_VALUE,
            "%s: ld_v must be >= D_v and a multiple of 8 (got %lld)", fn, (long long)ld_v);
  }
  REQUIRE(ld_indices >= 1 && k_width >= 0 && k_width <= ld_indices, DSA_ERR_VALUE,
          "%s: need 0 <= k_width <= ld_indices (got %d, %lld)", fn, k_width,
          (long long)ld_indices);
  REQUIRE(isfinite(softmax_scale) && softmax_scale > 0.0f, DSA_ERR_VALUE,
          "%s: softmax_scale must be finite and > 0", fn);
  if (T_q == 0) return DSA_OK;
  REQUIRE(q && (indices || k_width == 0) && out && lse && (k || T_kv == 0), DSA_ERR_VALUE,
          "%s: NULL pointer argument", fn);
  REQUIRE(aligned(q, 16) && aligned(out, 16) && aligned(k, 16) && aligned(v, 16), DSA_ERR_VALUE,
          "%s: q, k, v and out must be 16-byte aligned", fn);
  if (int rc = check_device(fn)) return rc;
  dsa::AttnArgs a;
  a.q = (const uint16_t*)q;
  a.T_q = T_q;
  a.H = H;
  a.k = (const uint16_t*)k;
  a.T_kv = k ? T_kv : 0;
  a.ld_k = ld_k;
  a.v = v ? (const uint16_t*)v : (const uint16_t*)k;
  a.ld_v = v ? ld_v : ld_k;
  a.indices = indices;
  a.ld_idx = ld_indices;
  a.k_width = k_width;
  a.topk_length = topk_length;
  a.sink = attn_sink;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.out = (uint16_t*)out;
  a.lse = lse;
  a.max_logits = max_logits;
  return launched(fn, dsa::launch_sparse_attn(a, D_qk, D_v, (hipStream_t)stream));
}

static int64_t up256(int64_t x) { return (x + 255) / 256 * 256; }

// Statistics [T_q, H] x 2, the fp32 dkv accumulator, and the sort arrays.
static int64_t bwd_fixed_bytes(int64_t T_q, int32_t H, int64_t T_kv, int32_t D_qk) {
  return up256(T_q * H * 4) * 2 + up256(T_kv * D_qk * 4) + up256(T_kv * 4) +
         up256((T_kv + 1) * 4) + up256(256 * 4);
}

// Per query row of a chunk: P and dS (bf16 [Kw, HP]) and then either
//  * (per-slot dkv) the dkv rows of its slots (bf16 [parts, Kw, D_qk]) and,
//    per slot, its entry of the sorted slot list and the radix sort's two key
//    / value buffers; plus the sort's digit histograms, 256 per 4096 slots;
//  * (KV-tile dkv) its slot map (int16 [ld_map]) and queue entry; plus per
//    part of 64 rows an fp32 partial [ld_map, D_qk] and its tile flags.
struct BwdShape {
  bool tiles;
  int64_t p, c, l, kw, ld_map, d_qk;
};
static BwdShape bwd_shape(int64_t T_kv, int32_t H, int32_t k_width, int32_t D_qk) {
  const int64_t hp = (H + 31) / 32 * 32, kw = ((int64_t)k_width + 31) / 32 * 32;
  const int64_t parts = hp % 64 == 0 ? hp / 64 : hp / 32;
  const bool tiles = dsa::bwd_uses_kv_tiles(T_kv, k_width);
  const int64_t ld_map = (T_kv + dsa::kBwdTileKV - 1) / dsa::kBwdTileKV * dsa::kBwdTileKV;
  return BwdShape{tiles, kw * hp * 2, parts * kw * D_qk * 2, kw * 4, kw, ld_map, D_qk};
}
static int64_t bwd_hist_bytes(const BwdShape& r, int64_t rows) {
  return (rows * r.kw + 4095) / 4096 * 256 * 4;
}
static int64_t bwd_chunk_bytes(const BwdShape& r, int64_t rows) {
  if (r.tiles) {
    const int64_t np = (rows + dsa::kBwdTileRows - 1) / dsa::kBwdTileRows;
    return 2 * up256(rows * r.p) + up256(rows * r.ld_map * 2) +
           up256(np * r.ld_map * r.d_qk * 4) + up256(np * (r.ld_map / dsa::kBwdTileKV) * 4) +
           up256(4) + up256(rows * 4);
  }
  return 2 * up256(rows * r.p) + up256(rows * r.c) + 5 * up256(rows * r.l) +
         up256(bwd_hist_bytes(r, rows));
}
// The most rows (at least 1, at most T_q) whose chunk buffers take at most
// `budget` bytes (the buffers grow with the rows).
static int64_t bwd_fit_rows(const BwdShape& r, int64_t T_q, int64_t budget) {
  int64_t lo = 1, hi = T_q > 1 ? T_q : 1;
  if (r.kw > 0 && hi > INT32_MAX / r.kw) hi = INT32_MAX / r.kw;  // slot numbers are int32
  if (bwd_chunk_bytes(r, hi) <= budget) return hi;
  while (hi - lo > 1) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (bwd_chunk_bytes(r, mid) <= budget) lo = mid; else hi = mid;
  }
  return lo;
}

int64_t dsa_sparse_attn_bwd_workspace_bytes(int64_t T_q, int32_t H, int64_t T_kv, int32_t D_qk,
                                            int32_t k_width) {
  if (T_q < 0 || T_q > INT32_MAX || H < 1 || H > DSA_MAX_HEADS || T_kv < 0 || T_kv > INT32_MAX ||
      (D_qk != 576 && D_qk != 512) || k_width < 0)
    return -1;
  const BwdShape row = bwd_shape(T_kv, H, k_width, D_qk);
  const int64_t rows = bwd_fit_rows(row, T_q, (int64_t)1 << 32);  // chunk buffers within 4 GiB
  return bwd_fixed_bytes(T_q, H, T_kv, D_qk) + bwd_chunk_bytes(row, rows);
}

int dsa_sparse_attn_bwd_kv_tiles(int64_t T_kv, int32_t k_width) {
  if (T_kv < 0 || k_width < 0) return -1;
  return dsa::bwd_uses_kv_tiles(T_kv, k_width) ? 1 : 0;
}

// The backward of both entry points. `noalloc`: the workspace is the no-alloc
// scratch of the current device (its size is a fixed maximum, so a size
// beyond it is reported as such and nothing is launched).
static int bwd_run(const char* fn, const void* q, int64_t T_q, int32_t H, int32_t D_qk,
                   const void* kv, int64_t T_kv, int64_t ld_kv, int32_t D_v,
                   const int32_t* indices, int64_t ld_indices, int32_t k_width,
                   const int32_t* topk_length, const float* attn_sink, float softmax_scale,
                   const void* out, const void* dout, const float* lse, void* dq, void* dkv,
                   float* d_sink, void* workspace, int64_t workspace_bytes, bool noalloc,
                   void* stream);

int dsa_sparse_attn_bwd(const void* q, int64_t T_q, int32_t H, int32_t D_qk, const void* kv,
                        int64_t T_kv, int64_t ld_kv, int32_t D_v, const int32_t* indices,
                        int64_t ld_indices, int32_t k_width, const int32_t* topk_length,
                        const float* attn_sink, float softmax_scale, const void* out,
                        const void* dout, const float* lse, void* dq, void* dkv, float* d_sink,
                        void* workspace, int64_t workspace_bytes, void* stream) {
  return bwd_run("dsa_sparse_attn_bwd", q, T_q, H, D_qk, kv, T_kv, ld_kv, D_v, indices,
                 ld_indices, k_width, topk_length, attn_sink, softmax_scale, out, dout, lse, dq,
                 dkv, d_sink, workspace, workspace_bytes, false, stream);
}

int dsa_sparse_attn_bwd_noalloc(const void* q, int64_t T_q, int32_t H, int32_t D_qk,
                                const void* kv, int64_t T_kv, int64_t ld_kv, int32_t D_v,
                                const int32_t* indices, int64_t ld_indices, int32_t k_width,
                                const int32_t* topk_length, const float* attn_sink,
                                float softmax_scale, const void* out, const void* dout,
                                const float* lse, void* dq, void* dkv, float* d_sink,
                                void* stream) {
  return bwd_run("dsa_sparse_attn_bwd_noalloc", q, T_q, H, D_qk, kv, T_kv, ld_kv, D_v, indices,
                 ld_indices, k_width, topk_length, attn_sink, softmax_scale, out, dout, lse, dq,
                 dkv, d_sink, nullptr, DSA_NOALLOC_SCRATCH_BYTES, true, stream);
}

static int bwd_run(const char* fn, const void* q, int64_t T_q, int32_t H, int32_t D_qk,
                   const void* kv, int64_t T_kv, int64_t ld_kv, int32_t D_v,
                   const int32_t* indices, int64_t ld_indices, int32_t k_width,
                   const int32_t* topk_length, const float* attn_sink, float softmax_scale,
                   const void* out, const void* dout, const float* lse, void* dq, void* dkv,
                   float* d_sink, void* workspace, int64_t workspace_bytes, bool noalloc,
                   void* stream) {
  REQUIRE(H >= 1 && H <= DSA_MAX_HEADS, DSA_ERR_VALUE, "%s: H must be in [1, %d] (got %d)", fn,
          DSA_MAX_HEADS, H);
  REQUIRE((D_qk == 576 || D_qk == 512) && D_v == 512, DSA_ERR_VALUE,
          "%s: (D_qk, D_v) must be (576, 512) or (512, 512) (got (%d, %d))", fn, D_qk, D_v);
  REQUIRE(T_q >= 0 && T_q <= INT32_MAX, DSA_ERR_VALUE, "%s: T_q out of range", fn);
  REQUIRE(T_kv >= 0 && T_kv <= INT32_MAX, DSA_ERR_VALUE, "%s: T_kv out of range", fn);
  REQUIRE(ld_kv >= D_qk && ld_kv % 8 == 0, DSA_ERR_VALUE,
          "%s: ld_kv must be >= D_qk and a multiple of 8 (got %lld)", fn, (long long)ld_kv);
  REQUIRE(ld_indices >= 1 && k_width >= 0 && k_width <= ld_indices, DSA_ERR_VALUE,
          "%s: need 0 <= k_width <= ld_indices (got %d, %lld)", fn, k_width,
          (long long)ld_indices);
  REQUIRE(isfinite(softmax_scale) && softmax_scale > 0.0f, DSA_ERR_VALUE,
          "%s: softmax_scale must be finite and > 0", fn);
  REQUIRE((q && out && dout && lse && dq) || T_q == 0, DSA_ERR_VALUE, "%s: NULL pointer argument",
          fn);
  REQUIRE((kv && dkv) || T_kv == 0, DSA_ERR_VALUE, "%s: NULL kv or dkv", fn);
  REQUIRE(indices || k_width == 0 || T_q == 0, DSA_ERR_VALUE, "%s: NULL indices", fn);
  REQUIRE(aligned(q, 16) && aligned(kv, 16) && aligned(out, 16) && aligned(dout, 16) &&
              aligned(dq, 16) && aligned(dkv, 16) && aligned(workspace, 256),
          DSA_ERR_VALUE, "%s: q, kv, out, dout, dq, dkv need 16-byte and workspace 256-byte "
          "alignment", fn);
  const int64_t fixed = bwd_fixed_bytes(T_q, H, T_kv, D_qk);
  const BwdShape row = bwd_shape(T_kv, H, k_width, D_qk);
  if (noalloc) {
    REQUIRE(fixed + bwd_chunk_bytes(row, 1) <= workspace_bytes, DSA_ERR_VALUE,
            "%s: these sizes need %lld bytes of scratch for one query row, more than the "
            "%lld-byte no-alloc scratch (use dsa_sparse_attn_bwd with a workspace)", fn,
            (long long)(fixed + bwd_chunk_bytes(row, 1)), (long long)workspace_bytes);
  } else {
    REQUIRE(workspace && workspace_bytes >= fixed + bwd_chunk_bytes(row, 1), DSA_ERR_VALUE,
            "%s: workspace of %lld bytes is below the %lld bytes one row needs", fn,
            (long long)workspace_bytes, (long long)(fixed + bwd_chunk_bytes(row, 1)));
  }
  if (T_q == 0 && T_kv == 0 && !d_sink) return DSA_OK;
  if (int rc = check_device(fn)) return rc;
  if (noalloc) {
    int dev = -1;
    (void)hipGetDevice(&dev);  // valid: check_device has just succeeded
    workspace = noalloc_scratch(dev);
    if (!workspace)
      return fail(DSA_ERR_RUNTIME, "%s: the no-alloc scratch of device %d has no address (%s)",
                  fn, dev, g_scratch_err[dev]);
  }
  unsigned char* w = (unsigned char*)workspace;
  dsa::BwdArgs a{};
  a.q = (const uint16_t*)q;
  a.kv = (const uint16_t*)kv;
  a.T_q = T_q;
  a.T_kv = kv ? T_kv : 0;
  a.ld_kv = ld_kv;
  a.H = H;
  a.D_qk = D_qk;
  a.D_v = D_v;
  a.indices = indices;
  a.ld_idx = ld_indices;
  a.k_width = indices ? k_width : 0;
  a.topk_length = topk_length;
  a.sink = attn_sink;
  a.scale = softmax_scale;
  a.out = (const uint16_t*)out;
  a.dout = (const uint16_t*)dout;
  a.lse = lse;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    unsigned char* p = w + off;
    off += up256(bytes);
    return p;
  };
  a.logZ = (float*)take(T_q * H * 4);
  a.Dsum = (float*)take(T_q * H * 4);
  a.dkv_ws = (float*)take(T_kv * D_qk * 4);
  a.cnt = (int32_t*)take(T_kv * 4);
  a.offs = (int32_t*)take((T_kv + 1) * 4);
  a.sort_tot = (uint32_t*)take(256 * 4);
  // the largest chunk of rows whose buffers fit the rest of the workspace
  const int64_t chunk = bwd_fit_rows(row, T_q, workspace_bytes - fixed);
  a.wsP = (uint16_t*)take(chunk * row.p);
  a.wsD = (uint16_t*)take(chunk * row.p);
  a.tiles = row.tiles;
  if (row.tiles) {
    const int64_t np = (chunk + dsa::kBwdTileRows - 1) / dsa::kBwdTileRows;
    a.ld_map = row.ld_map;
    a.map = (int16_t*)take(chunk * row.ld_map * 2);
    a.part = (float*)take(np * row.ld_map * D_qk * 4);
    a.part_flag = (int32_t*)take(np * (row.ld_map / dsa::kBwdTileKV) * 4);
    a.dup_count = (uint32_t*)take(4);
    a.dup_rows = (int32_t*)take(chunk * 4);
  } else {
    a.wsC = (uint16_t*)take(chunk * row.c);
    a.list = (int32_t*)take(chunk * row.l);
    for (int k = 0; k < 2; ++k) {
      a.sort_keys[k] = (int32_t*)take(chunk * row.l);
      a.sort_vals[k] = (int32_t*)take(chunk * row.l);
    }
    a.sort_hist = (uint32_t*)take(bwd_hist_bytes(row, chunk));
  }
  a.Kw = (k_width + 31) / 32 * 32;
  a.dq = (uint16_t*)dq;
  a.dkv = (uint16_t*)dkv;
  a.d_sink = d_sink;
  return launched(fn, dsa::launch_sparse_attn_bwd(a, chunk, (hipStream_t)stream));
}

}  // extern "C"
