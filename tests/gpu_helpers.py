"""Shared helpers of the GPU parity tests (host-side conversion and checks)."""

import sys

import numpy as np
import torch

from oracle import dsa_oracle as O
from workloads import bf16_to_numpy_bits

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of a bf16 / fp32 / int device tensor."""
    if t.dtype == torch.bfloat16:
        return O.bf16_bits_to_f64(bf16_to_numpy_bits(t))
    return t.detach().cpu().numpy().astype(np.float64)


def i64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.int64)


def check_indexer(gpu_scores: torch.Tensor, wl, rows, row_starts, seq_lens, rel=1e-4):
    """GPU score rows (row i of gpu_scores is query row rows[i]) vs the oracle.

    Checks the stated tolerance, max-abs <= 1e-2 * ||score||_inf over the valid
    columns of each row, and a tighter internal gate `rel`.
    """
    rows = np.asarray(rows, dtype=np.int64)
    sel = torch.as_tensor(rows, device=wl.q_idx.device)
    q = f64(wl.q_idx[sel])
    w = f64(wl.w[sel])
    k = f64(wl.k_idx)
    st = np.asarray(row_starts, dtype=np.int64)[rows]
    sl = np.asarray(seq_lens, dtype=np.int64)[rows]
    ref = O.indexer_scores(q, k, w, st, sl, np.arange(len(rows)), width=max(int(sl.max()), 1))
    got = gpu_scores.detach().cpu().numpy().astype(np.float64)
    worst = 0.0
    for i in range(len(rows)):
        n = int(sl[i])
        if n == 0:
            continue
        r = ref[i, :n]
        scale = max(np.abs(r).max(), 1e-30)
        err = np.abs(got[i, :n] - r).max() / scale
        worst = max(worst, err)
        assert err <= 1e-2, (int(rows[i]), err)
        assert err <= rel, (int(rows[i]), err)
    return worst


def check_attention(out, lse, mx, q, kv, v, indices, topk_length, sink, scale, d_v, rows,
                    atol_out=1e-2, rel_row=2e-2, atol_lse=1e-3):
    """GPU attention outputs (full [T_q, ...] tensors) at `rows` vs the oracle."""
    rows_t = torch.as_tensor(rows, device=q.device)
    qn = f64(q[rows_t])
    kn = f64(kv)
    vn = None if v is None else f64(v)
    idx = i64(indices[rows_t])
    tl = None if topk_length is None else i64(topk_length[rows_t])
    sk = None if sink is None else f64(sink)
    ref_o, ref_l, ref_m = O.sparse_attention(qn, kn, vn, idx, tl, sk, scale, d_v=d_v)
    go = f64(out[rows_t])
    gl = f64(lse[rows_t])
    empty = np.isinf(ref_l)
    assert np.array_equal(np.isinf(gl) & (gl > 0), empty), "empty-row lse must be +inf"
    d_out = np.abs(go - ref_o)
    assert d_out.max() <= atol_out, d_out.max()
    row_scale = np.abs(ref_o).max(axis=2, keepdims=True)
    rel = (d_out.max(axis=2, keepdims=True) / np.maximum(row_scale, 1e-30))
    rel = np.where(row_scale > 0, rel, d_out.max(axis=2, keepdims=True))
    assert rel.max() <= rel_row, rel.max()
    fin = ~empty
    if fin.any():
        assert np.abs(gl[fin] - ref_l[fin]).max() <= atol_lse, np.abs(gl[fin] - ref_l[fin]).max()
    if mx is not None:
        gm = f64(mx[rows_t])
        assert np.all(gm[empty] == -np.inf)
        if fin.any():
            assert np.abs(gm[fin] - ref_m[fin]).max() <= 1e-3
    assert np.all(go[np.broadcast_to(empty[:, :, None], go.shape)] == 0)
    return d_out.max(), rel.max()
