"""CPU fp64 oracle for the DeepSeek Sparse Attention forward hot path.

TEST INFRASTRUCTURE ONLY. This module is the reference the HIP kernels are
checked against. Only the test suite, the smoke check and the bench's CPU
baseline leg may import it; the product path never calls it and shares no code
with it (no kernels, headers, helpers, tables or constants).

Every function is written from the definitions on the pages:

* "DeepSeek Sparse Attention (DSA)", cuDNN Frontend OSS API docs
  (docs.nvidia.com/cudnn/fe-oss-apis/dsa): section 1 "Sparse Attention
  Forward" (slot semantics, sink, LSE, empty rows, topk_length clamp, D_qk=576
  with V = first 512 dims), section 3 "Indexer Forward (score-only)" (score
  formula, ratio-causal mask, and the FP8 / MXFP8 input precisions), section
  4 "Combined Indexer Forward + Top-K"
  (deterministic tie-break toward the smallest index) and section 5
  "Indexer Top-K" (per-row effective length, top_k <= 2048).
* "nemo_automodel...glm_moe_dsa.kernels.cudnn_dsa" API page:
  prepare_cudnn_dsa_packed_metadata (per-query starts and causal lengths of
  packed THD sequences), _topk_wrapper_chunked (scores [T, S_max] with causal
  lengths [T]), cudnn_indexer_topk / cudnn_sparse_attention (global indices,
  ascending valid prefix, -1 suffix).

Arithmetic is float64 throughout; bf16 inputs are widened exactly from their
bit patterns. Plain loops over rows, with a library matmul as the only
primitive, so each step can be read against the definition.

Readings where the pages are silent (each is listed with its reason in the
repository's design notes): indexer scores carry no internal scaling (the
caller pre-scales W); K has a single head shared by all indexer heads; masked
score columns are -inf; -0.0 and +0.0 are equal values and tie; selected
indices are emitted in ascending order; the sink is a per-head logit in scaled
units that enters only the output denominator; LSE is the natural log over
key slots only; empty rows give out=0, lse=+inf, max_logits=-inf.
"""

from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------------------
# Input widening
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact bf16 -> float64: a bf16 value is the top 16 bits of an fp32."""
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Step a0: packed-THD metadata
# ---------------------------------------------------------------------------

def packed_metadata(cu_seqlens, T: int):
    """Per-token document start and causal length for compact packed THD.

    cudnn_dsa page, prepare_cudnn_dsa_packed_metadata: cu_seqlens are the
    cumulative real-token lengths [n_seq+1]; each query gets the start of its
    sequence and its real causal length (causality restarts per document).
    Returns (row_starts, seq_lens) as int64 arrays of length T.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    starts = np.zeros(T, dtype=np.int64)
    seq_lens = np.zeros(T, dtype=np.int64)
    for d in range(len(cu) - 1):
        for t in range(int(cu[d]), int(cu[d + 1])):
            starts[t] = cu[d]
            seq_lens[t] = t - cu[d] + 1
    return starts, seq_lens


def ratio_causal_metadata(cu_seqlens_q, cu_seqlens_k, T_q: int, ratio: int = 1,
                          q_causal_offsets=None):
    """Per-query key-segment start and visible key count, ratio-causal mask.

    DSA page section 3 ("Indexer Forward"): for THD segment b, local query row
    q_local may score local key column j only when
        j < clamp((q_causal_offsets[b] + q_local + 1) // ratio, 0, seqlen_k_b),
    where q_causal_offsets[b] is the global, uncompressed token position of the
    segment's first query (zero for every segment when omitted) -- not its
    storage offset -- and the key columns of segment b are a compressed prefix
    starting at compressed column 0. cu_seqlens_q locates where segment b's
    queries are stored, cu_seqlens_k where its keys are stored; seqlen_k_b is
    cu_seqlens_k[b+1] - cu_seqlens_k[b]. `//` is floor division.

    Returns (row_starts, seq_lens) as int64 arrays of length T_q: row_starts[t]
    = cu_seqlens_k[b] (key row of local column 0), seq_lens[t] = the count
    above. With ratio 1, no offsets and cu_seqlens_k == cu_seqlens_q this is
    packed_metadata.
    """
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    n_seq = len(cq) - 1
    off = (np.zeros(n_seq, dtype=np.int64) if q_causal_offsets is None
           else np.asarray(q_causal_offsets, dtype=np.int64))
    starts = np.zeros(T_q, dtype=np.int64)
    seq_lens = np.zeros(T_q, dtype=np.int64)
    for b in range(n_seq):
        seqlen_k = int(ck[b + 1] - ck[b])
        for t in range(int(cq[b]), int(cq[b + 1])):
            q_local = t - int(cq[b])
            visible = (int(off[b]) + q_local + 1) // ratio
            starts[t] = ck[b]
            seq_lens[t] = min(max(visible, 0), seqlen_k)
    return starts, seq_lens


# ---------------------------------------------------------------------------
# Step a1: lightning-indexer scores
# ---------------------------------------------------------------------------

def indexer_scores(q_idx, k_idx, w, row_starts, seq_lens, rows, width=None):
    """Dense indexer scores for the given query rows, local key columns.

    DSA page section 3: S[q, k] = sum_h ReLU(Q_h . K^T) * W_h with a
    ratio-causal mask; with ratio 1 and no causal offsets the valid columns of
    local row q are k < q + 1 within its segment (packed_metadata), in general
    the counts of ratio_causal_metadata. The indexer K has one head
    (H_kv = 1), so every head h uses the same key row. Column j of row t is key
    start(t) + j (cudnn_dsa page, _topk_wrapper_chunked: scores [T, S_max] with
    causal lengths [T]); columns j >= seq_len(t) are -inf.

    q_idx [T, H, D], k_idx [T_kv, D], w [T, H] are float64. Returns float64
    [len(rows), width].
    """
    rows = np.asarray(rows, dtype=np.int64)
    if width is None:
        width = int(max(seq_lens[rows].max(), 1)) if len(rows) else 1
    out = np.full((len(rows), width), NEG_INF)
    for r, t in enumerate(rows):
        s = int(row_starts[t])
        n = int(seq_lens[t])
        keys = k_idx[s:s + n]                       # [n, D]
        logits = q_idx[t] @ keys.T                  # [H, n]   Q_h . K^T
        out[r, :n] = w[t] @ np.maximum(logits, 0.0)  # sum_h W_h * ReLU(.)
    return out


# ---------------------------------------------------------------------------
# Step a1 in FP8: E4M3 inputs with per-token or per-block (MX) scales
# ---------------------------------------------------------------------------

def decode_e4m3(codes) -> np.ndarray:
    """FP8 E4M3 bytes -> float64 (the OCP "E4M3FN" encoding the DSA page's FP8
    paths use): sign bit, 4 exponent bits with bias 7, 3 mantissa bits. An
    exponent field of 0 is subnormal, m/8 * 2^-6; S.1111.111 is NaN; there are
    no infinities, so the largest magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c >> 7 == 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def decode_e8m0(codes) -> np.ndarray:
    """E8M0 scale bytes -> float64: the power of two 2^(code - 127); 255 is NaN."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def indexer_scores_fp8(q8, q_scale, k8, k_scale, w, row_starts, seq_lens, rows, width=None):
    """Indexer scores of the FP8 path with per-token descales (DSA page,
    section 3, precision "fp8" on SM90).

    Q and K are E4M3 bytes; q_scale [T, H] and k_scale [T_kv] are fp32 descales
    (one per token and head for Q, one per token for the single-head K). The
    real inputs are the decoded values times their descale; the score is then
    the section's definition on them (indexer_scores).
    q8 [T, H, D] and k8 [T_kv, D] uint8, q_scale/k_scale/w float64.
    """
    q = decode_e4m3(q8) * np.asarray(q_scale, dtype=np.float64)[..., None]
    k = decode_e4m3(k8) * np.asarray(k_scale, dtype=np.float64)[:, None]
    return indexer_scores(q, k, w, row_starts, seq_lens, rows, width)


def indexer_scores_mxfp8(q8, q_sf, k8, k_sf, w, row_starts, seq_lens, rows, width=None,
                         block=32):
    """Indexer scores of the block-scaled FP8 path (DSA page, section 3,
    precision "mxfp8": E4M3 values with E8M0 scales, one per 32 consecutive
    elements along the head dimension).

    q8 [T, H, D], k8 [T_kv, D] uint8; q_sf [T, H, D/32], k_sf [T_kv, D/32]
    uint8 E8M0. Element d of a row is decoded(d) * scale[d // 32]; the score
    is then the section's definition on those values (indexer_scores).
    """
    q = decode_e4m3(q8) * np.repeat(decode_e8m0(q_sf), block, axis=-1)
    k = decode_e4m3(k8) * np.repeat(decode_e8m0(k_sf), block, axis=-1)
    return indexer_scores(q, k, w, row_starts, seq_lens, rows, width)


# ---------------------------------------------------------------------------
# Steps a2 + a3: per-row top-K select, compaction, local -> global
# ---------------------------------------------------------------------------

def topk_row(x, n: int, k: int) -> np.ndarray:
    """Selected local columns of one row, ascending.

    DSA page section 5: top-K over the first n = seq_len columns of the row.
    Section 4 (deterministic=True): exact-value ties at the K-th boundary go to
    the smallest local index. Rows with n <= K keep all n columns.
    """
    x = np.asarray(x, dtype=np.float64)[:n]
    if n <= k:
        return np.arange(n, dtype=np.int64)
    theta = np.partition(x, n - k)[n - k]          # K-th largest value
    above = np.nonzero(x > theta)[0]
    equal = np.nonzero(x == theta)[0]              # ascending column order
    chosen = np.concatenate([above, equal[: k - len(above)]])
    return np.sort(chosen)


def topk(scores, seq_lens, k: int, row_starts=None, n_cols=None):
    """Top-K indices in canonical compact form.

    cudnn_dsa page (cudnn_indexer_topk, _compact_and_sort_indices): int32
    indices in global packed coordinates (row start + local column), an
    ascending valid prefix and a -1 suffix, plus valid lengths
    min(seq_len, K). seq_lens are clamped to [0, n_cols]. With row_starts None
    the local column ids are returned.
    """
    scores = np.asarray(scores)
    n_rows = scores.shape[0]
    n_cols = scores.shape[1] if n_cols is None else n_cols
    idx = np.full((n_rows, k), -1, dtype=np.int64)
    length = np.zeros(n_rows, dtype=np.int64)
    for r in range(n_rows):
        n = int(min(max(int(seq_lens[r]), 0), n_cols))
        sel = topk_row(scores[r], n, k)
        base = 0 if row_starts is None else int(row_starts[r])
        idx[r, : len(sel)] = sel + base
        length[r] = len(sel)
    return idx.astype(np.int32), length.astype(np.int32)


def topk_softmax(scores, seq_lens, k: int, row_starts=None, n_cols=None):
    """Top-K with its logits, softmax and log-sum-exp: the outputs of the
    combined indexer + top-K path.

    DSA page section 4 (indices, logits of the selected slots, softmax over
    them, LSE; padded slots -1 / -inf) with the selected set and slot order of
    topk(); section 6 defines the softmax: predict[i] = softmax_i of the
    indexer score at the selected index i. lse is the natural log of the sum
    of exp(logit) over the selected slots; softmax = exp(logit - lse),
    0 in padded slots; a row with no selected slot has lse = +inf (the
    pages' empty-row convention for LSE).
    Returns (indices int32, lengths int32, logits, softmax, lse) with float64
    values.
    """
    scores = np.asarray(scores, dtype=np.float64)
    idx, length = topk(scores, seq_lens, k, row_starts=row_starts, n_cols=n_cols)
    n_rows = scores.shape[0]
    logits = np.full((n_rows, k), NEG_INF)
    soft = np.zeros((n_rows, k))
    lse = np.full(n_rows, np.inf)
    for r in range(n_rows):
        m = int(length[r])
        if m == 0:
            continue
        base = 0 if row_starts is None else int(row_starts[r])
        v = scores[r, idx[r, :m].astype(np.int64) - base]
        top = v.max()
        lse[r] = top + np.log(np.exp(v - top).sum())
        logits[r, :m] = v
        soft[r, :m] = np.exp(v - lse[r])
    return idx, length, logits, soft, lse


# ---------------------------------------------------------------------------
# Steps a4 / a5: sparse attention forward
# ---------------------------------------------------------------------------

def sparse_attention(q, k, v, indices, topk_length, sink, scale, d_v=None, rows=None):
    """Sparse MQA attention forward over selected key rows.

    DSA page section 1: for query row t, head h and valid slot j the score is
    scale * dot(q[t, h, :], kv[idx[t, j], :]); invalid (-1) and out-of-bounds
    ids have score -inf and duplicates stay distinct slots; topk_length is
    clamped to [0, K] and slots at or beyond it are invalid. The sink adds
    exp(sink_h) to the output denominator only; lse is KV-only (natural log,
    excludes the sink); empty rows give out = 0, max_logits = -inf, lse = +inf.
    For D_qk = 576 the values are the first 512 dims of the shared KV row
    (v is None, d_v = 512); the block-routed GQA page passes a separate V.

    q [Tq, H, Dqk], k [Tkv, Dqk], v [Tkv, Dv] or None, all float64.
    Returns (out [n, H, Dv], lse [n, H], max_logits [n, H]) for the rows.
    """
    Tq, H, _ = q.shape
    Tkv = k.shape[0]
    if v is None:
        v = k[:, :d_v]
    Dv = v.shape[1]
    kw = indices.shape[1]
    rows = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), H, Dv))
    lse = np.full((len(rows), H), np.inf)
    mx = np.full((len(rows), H), NEG_INF)
    for r, t in enumerate(rows):
        L = kw if topk_length is None else min(max(int(topk_length[t]), 0), kw)
        ids = np.asarray(indices[t, :L], dtype=np.int64)
        ids = ids[(ids >= 0) & (ids < Tkv)]
        if len(ids) == 0:
            continue
        s = scale * (q[t] @ k[ids].T)               # [H, n] scaled logits
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        l = e.sum(axis=1)
        denom = l.copy()
        if sink is not None:
            denom = denom + np.exp(np.asarray(sink, dtype=np.float64) - m)
        out[r] = (e @ v[ids]) / denom[:, None]
        lse[r] = m + np.log(l)
        mx[r] = m
    return out, lse, mx


def sparse_attention_backward(q, kv, indices, topk_length, sink, scale, dout, d_v, rows=None):
    """Gradients of the sparse attention forward (shared latent KV: K = kv,
    V = kv[:, :d_v]).

    DSA page section 2 ("Sparse Attention Backward"): for the loss whose
    gradient with respect to out is dout, returns dq [T_q, H, D_qk],
    dkv [T_kv, D_qk] and d_sink [H]. Derived from section 1's forward: with
    P_j = exp(s_j) / (sum_i exp(s_i) + exp(sink)) over the valid slots j of a
    row and out = sum_j P_j v_j,
        dP_j = dout . v_j,  D = sum_j P_j dP_j (= dout . out),
        dS_j = P_j (dP_j - D),  dq = scale sum_j dS_j k_j,
        dk_j += scale dS_j q,  dv_j += P_j dout,
        d_sink += -P_sink D with P_sink = exp(sink) / (sum_i exp(s_i) + exp(sink)).
    Duplicate slots contribute separately; dkv = dk with dv added to its
    first d_v columns. Every quantity is recomputed from the inputs in
    float64 (no forward output is trusted). Inputs float64; rows defaults to
    every query row (dq rows outside `rows` are left zero).
    """
    Tq, H, Dqk = q.shape
    Tkv = kv.shape[0]
    kw = indices.shape[1]
    v = kv[:, :d_v]
    rows = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
    dq = np.zeros_like(q)
    dkv = np.zeros((Tkv, Dqk))
    d_sink = np.zeros(H)
    sk = None if sink is None else np.asarray(sink, dtype=np.float64)
    for t in rows:
        L = kw if topk_length is None else min(max(int(topk_length[t]), 0), kw)
        ids = np.asarray(indices[t, :L], dtype=np.int64)
        ids = ids[(ids >= 0) & (ids < Tkv)]
        if len(ids) == 0:
            continue
        s = scale * (q[t] @ kv[ids].T)                       # [H, n]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        if sk is not None:
            z = z + np.exp(sk[:, None] - m)
        P = e / z                                              # [H, n]
        out = P @ v[ids]                                       # [H, d_v]
        dP = dout[t] @ v[ids].T                                # [H, n]
        D = (dout[t] * out).sum(axis=1, keepdims=True)         # [H, 1]
        dS = P * (dP - D)
        dq[t] = scale * (dS @ kv[ids])
        np.add.at(dkv, ids, scale * (dS.T @ q[t]))             # dk
        np.add.at(dkv[:, :d_v], ids, P.T @ dout[t])            # dv (shared columns)
        if sk is not None:
            p_sink = np.exp(sk - m[:, 0]) / z[:, 0]
            d_sink += -p_sink * D[:, 0]
    return dq, dkv, d_sink

