"""Parity of the combined indexer + top-K path for rows longer than 4096
columns (dsa_indexer_topk_fused with a candidate buffer), from bf16 or FP8
indexer inputs.

The indexer pass of that path computes every score with the standalone
indexer's arithmetic, so its selection is compared bit-exactly with the
oracle's top-K on the standalone kernel's scores (dsa_indexer_fwd), its logits
equal those scores exactly, and softmax / LSE are within 1e-5 of the oracle's
(fp64 on the same logits) plus 4 float32 ulps of the row's |LSE|: the kernels
form exp(logit - lse) from float32 values, whose rounding alone is that large
when scores reach the hundreds, as some inputs here make them. Inputs whose candidate lists cannot hold the top k
exercise the rescue pass: a few very high scores at the start of each
document (the first of the tiles the lower bound is sampled from sees them,
so the bound overshoots the k-th largest score and too few columns pass) and
scores that are all equal (every column passes, more than a list holds). The
first word of the candidate buffer counts the rows the rescue redid.
"""

import numpy as np
import pytest
import torch

import deepseek_sparse_attention_dsa_amd as dsa
from gpu_helpers import DEV, i64, say
from oracle import dsa_oracle as O
from workloads import make_custom, quantize_fp8

pytestmark = pytest.mark.gpu

CAP = 8192  # candidates a row's list holds


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    dsa.load_library()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _run(q, k_idx, w, rs, sl, k, n_cols, row_begin=0, n_rows=None, values=True, **kw):
    n_rows = q.shape[0] - row_begin if n_rows is None else n_rows
    need = dsa.dsa_indexer_topk_cand_buffer_size(n_rows, n_cols, k)
    buf = torch.empty((need,), dtype=torch.float32, device=DEV)
    res = dsa.dsa_indexer_topk_fused(q, k_idx, w, rs, sl, k, n_cols, row_begin=row_begin,
                                     n_rows=n_rows, return_logits=values, return_softmax=values,
                                     return_lse=values, cand_buffer=buf, **kw)
    torch.cuda.synchronize()
    rescued = int(buf[:1].view(torch.int32).item())
    return res, rescued


def _quantize(q, k_idx, scaling):
    """FP8 inputs of the call for q / k_idx ("per_token" or "mx"), or None."""
    if scaling is None:
        return q, k_idx, {}
    block = 32 if scaling == "mx" else None
    q8, qs = quantize_fp8(q, block)
    k8, ks = quantize_fp8(k_idx, block)
    mode = dsa.DSA_MXFP8 if scaling == "mx" else dsa.DSA_FP8_PER_TOKEN
    return q8, k8, dict(q_scale=qs, k_scale=ks, fp8_scaling=mode)


def _scores(q, k_idx, w, rs, sl, fp8, **kw):
    """The standalone indexer's scores for the same inputs."""
    if fp8:
        return dsa.dsa_indexer_fwd_fp8(q, fp8["q_scale"], k_idx, fp8["k_scale"], w, rs, sl,
                                       scaling=fp8["fp8_scaling"], **kw)
    return dsa.dsa_indexer_fwd(q, k_idx, w, rs, sl, **kw)


def _compare(res, sc, seq_lens, row_starts, k, n_cols, rows=None):
    """res rows `rows` (all when None) against the oracle on score rows sc
    (row i of sc belongs to output row rows[i])."""
    idx, tl, logits, soft, lse = res
    rows = np.arange(idx.shape[0]) if rows is None else np.asarray(rows)
    sel = torch.as_tensor(rows, device=idx.device)
    s64 = sc.cpu().numpy().astype(np.float64)
    ref_idx, ref_len, ref_logit, ref_soft, ref_lse = O.topk_softmax(
        s64, i64(seq_lens)[rows], k, row_starts=i64(row_starts)[rows], n_cols=n_cols)
    gi = i64(idx[sel])
    bad = np.nonzero(np.any(gi != ref_idx, axis=1))[0]
    assert len(bad) == 0, (rows[bad[:5]], gi[bad[:1], :8], ref_idx[bad[:1], :8])
    assert np.array_equal(i64(tl[sel]), ref_len)
    if logits is not None:
        gl = logits[sel].cpu().numpy().astype(np.float64)
        assert np.array_equal(gl, ref_logit), "logits must be the selected scores"
        empty = np.isinf(ref_lse)
        tol = 1e-5 + 4 * 2.0 ** -23 * np.where(empty, 0.0, np.abs(ref_lse))  # per row
        gs = soft[sel].cpu().numpy().astype(np.float64)
        err = np.abs(gs - ref_soft).max(axis=1)
        assert np.all(err <= tol), (err.max(), rows[np.argmax(err - tol)])
        gz = lse[sel].cpu().numpy().astype(np.float64)
        assert np.array_equal(np.isinf(gz) & (gz > 0), empty)
        err = np.abs(gz[~empty] - ref_lse[~empty])
        assert np.all(err <= tol[~empty]), err.max(initial=0.0)


def _workload(doc_lens, H, D, wdt, k, seed):
    wl = make_custom(doc_lens, H=1, D_qk=64, D_v=64, H_idx=H, D_idx=D, topk=k, seed=seed,
                     device=DEV)
    w = wl.w if wdt == torch.bfloat16 else wl.w.float()
    return wl, w


@pytest.mark.parametrize("doc_lens,H,D,wdt,k,fp8", [
    ([12288], 64, 128, torch.bfloat16, 2048, None),
    ([9000, 700, 5200], 64, 128, torch.float32, 512, None),
    ([6000, 4500], 32, 64, torch.bfloat16, 100, None),
    ([10000], 17, 64, torch.float32, 1, None),
    ([8193, 3], 33, 128, torch.bfloat16, 2047, None),
    # FP8 inputs (D = 128): E8M0 block scales and fp32 per-token descales
    ([12288], 64, 128, torch.bfloat16, 2048, "mx"),
    ([12288], 64, 128, torch.bfloat16, 2048, "per_token"),
    ([9000, 700, 5200], 64, 128, torch.float32, 512, "mx"),
    ([8193, 3], 33, 128, torch.bfloat16, 2047, "per_token"),
    ([10000], 17, 128, torch.float32, 1, "mx"),
    ([6000, 4500], 8, 128, torch.bfloat16, 100, "per_token"),
])
def test_cand_random_scores(doc_lens, H, D, wdt, k, fp8):
    say("cand path", doc_lens, H, D, wdt, k, fp8)
    wl, w = _workload(doc_lens, H, D, wdt, k, seed=sum(doc_lens) + H)
    q, k_idx, kw = _quantize(wl.q_idx, wl.k_idx, fp8)
    rs, sl = dsa.dsa_packed_metadata(wl.cu_seqlens, wl.T)
    n_cols = max(doc_lens)
    res, rescued = _run(q, k_idx, w, rs, sl, k, n_cols, **kw)
    sc = _scores(q, k_idx, w, rs, sl, kw, width=n_cols)
    torch.cuda.synchronize()
    _compare(res, sc, sl, rs, k, n_cols)
    assert rescued == 0, "random scores leave no row to the rescue pass"


HOT = 256  # leading keys of each document with very high scores


def _hot_prefix(doc_lens, H, D, seed, flat=False):
    """Indexer inputs with positive q and w whose first HOT keys of each
    document score far above the rest (rising with the position), the other
    keys being N(0, 1/D); flat=True makes every key row the same positive
    vector instead (all scores of a row equal)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    T = sum(doc_lens)
    q = (torch.rand((T, H, D), generator=g) + 0.1).to(torch.bfloat16)
    w = (torch.rand((T, H), generator=g) + 0.1).to(torch.bfloat16)
    v = torch.rand((D,), generator=g) + 0.5
    pos = torch.cat([torch.arange(L, dtype=torch.float32) for L in doc_lens])
    if flat:
        k_idx = v[None, :].expand(T, D) / D
    else:
        k_idx = torch.randn((T, D), generator=g) / D ** 0.5
        hot = pos < HOT
        k_idx[hot] = (4.0 + pos[hot, None] / HOT) * v[None, :] / D ** 0.5
    cu = torch.tensor(np.concatenate([[0], np.cumsum(doc_lens)]).astype(np.int32))
    return q.to(DEV), k_idx.to(torch.bfloat16).to(DEV), w.to(DEV), cu.to(DEV)


# all_long: whether every row longer than a list is rescued. With a hot
# prefix the first sample tile holds 128 of the hot keys; when the bound's
# sample rank is below that, the bound lands among the hot scores and fewer
# than k columns pass (k = 2048: the bound lands among the ordinary scores
# near the k-th largest, and only part of the rows come short).
@pytest.mark.parametrize("doc_lens,H,D,k,flat,all_long,fp8", [
    ([10000], 64, 128, 2048, False, False, None),  # lower bound too high for some rows
    ([9000], 8, 64, 64, True, True, None),         # all scores equal: the lists overflow
    ([8500, 9300], 64, 128, 300, False, True, None),
    ([9100], 20, 64, 200, False, True, None),
    ([10000], 64, 128, 2048, False, False, "mx"),
    ([9000], 8, 128, 64, True, True, "per_token"),
    ([9000], 8, 128, 64, True, True, "mx"),
    ([8500, 9300], 64, 128, 300, False, True, "per_token"),
    ([9100], 20, 128, 200, False, True, "mx"),
])
def test_cand_rescue(doc_lens, H, D, k, flat, all_long, fp8):
    say("cand rescue", doc_lens, H, D, k, flat, fp8)
    q, k_idx, w, cu = _hot_prefix(doc_lens, H, D, seed=sum(doc_lens) + k, flat=flat)
    q, k_idx, kw = _quantize(q, k_idx, fp8)
    T = sum(doc_lens)
    rs, sl = dsa.dsa_packed_metadata(cu, T)
    n_cols = max(doc_lens)
    res, rescued = _run(q, k_idx, w, rs, sl, k, n_cols, **kw)
    sc = _scores(q, k_idx, w, rs, sl, kw, width=n_cols)
    torch.cuda.synchronize()
    _compare(res, sc, sl, rs, k, n_cols)
    # rows no longer than a list take every column and are never rescued
    long_rows = int(sum(max(0, L - CAP) for L in doc_lens))
    assert 0 < rescued <= long_rows and (rescued == long_rows or not all_long), (rescued,
                                                                              long_rows)
    if flat:  # every score ties: the lowest k columns of each row
        idx = res[0]
        n = torch.clamp(sl, max=k).long()
        ar = torch.arange(k, device=DEV)[None, :]
        want = torch.where(ar < n[:, None], rs.long()[:, None] + ar, -1)
        assert torch.equal(idx.long(), want)


def test_cand_mixed_rescue_and_stage2():
    """One document with random scores next to one with a hot prefix: the
    stage-2 select and the rescue serve rows of the same call."""
    say("cand mixed")
    wl, _ = _workload([9500], 64, 128, torch.bfloat16, 700, seed=77)
    q2, k2, w2, _ = _hot_prefix([8800], 64, 128, seed=78)
    q = torch.cat([wl.q_idx, q2])
    k_idx = torch.cat([wl.k_idx, k2])
    w = torch.cat([wl.w, w2])
    cu = torch.tensor([0, 9500, 18300], dtype=torch.int32, device=DEV)
    rs, sl = dsa.dsa_packed_metadata(cu, 18300)
    res, rescued = _run(q, k_idx, w, rs, sl, 700, 9500)
    sc = dsa.dsa_indexer_fwd(q, k_idx, w, rs, sl, width=9500)
    torch.cuda.synchronize()
    _compare(res, sc, sl, rs, 700, 9500)
    assert rescued == 8800 - CAP, rescued


def test_cand_window_index_only_and_empty_keys():
    """A row window, index-only outputs (the 16-byte staged stores) into rows
    wider than k, a column cap below the rows' lengths, and no keys at all."""
    say("cand window")
    wl, w = _workload([11000], 64, 128, torch.bfloat16, 1024, seed=79)
    rs, sl = dsa.dsa_packed_metadata(wl.cu_seqlens, wl.T)
    r0, n, k, n_cols = 2100, 8000, 1024, 9999
    idx = torch.full((n, k + 4), 7, dtype=torch.int32, device=DEV)
    need = dsa.dsa_indexer_topk_cand_buffer_size(n, n_cols, k)
    buf = torch.empty((need,), dtype=torch.float32, device=DEV)
    res = dsa.dsa_indexer_topk_fused(wl.q_idx, wl.k_idx, w, rs, sl, k, n_cols, row_begin=r0,
                                     n_rows=n, indices=idx[:, :k], cand_buffer=buf)
    sc = dsa.dsa_indexer_fwd(wl.q_idx, wl.k_idx, w, rs, sl, row_begin=r0, n_rows=n,
                             width=n_cols)
    torch.cuda.synchronize()
    _compare(res, sc, torch.clamp(sl[r0:r0 + n], max=n_cols), rs[r0:r0 + n], k, n_cols)
    assert torch.all(idx[:, k:] == 7), "columns past k of the index rows stay untouched"
    # no keys: every row is empty
    res, rescued = _run(wl.q_idx[:300], wl.k_idx[:0], w[:300], rs[:300], sl[:300], 64, 5000)
    idx, tl, lg, so, lse = res
    assert torch.all(idx == -1) and torch.all(tl == 0) and rescued == 0
    assert torch.all(lg == -float("inf")) and torch.all(so == 0) and torch.all(lse == float("inf"))


def _long_rows(T, k):
    rng = np.random.default_rng(5)
    rows = {0, 1, k - 2, k - 1, k, k + 1, 4095, 4096, CAP - 1, CAP, CAP + 1, 16383, 16384,
            32767, 32768, T - 2, T - 1}
    rows |= set(int(x) for x in rng.integers(0, T, size=64 - len(rows)))
    return sorted(r for r in rows if 0 <= r < T)


@pytest.mark.parametrize("fp8", [None, "mx", "per_token"])
def test_cand_long_context_sampled(fp8):
    """One 65536-token sequence, indexer 64 x 128, top-2048, all rows in one
    call (bf16 inputs, or their FP8 quantisation): sampled rows (the
    selection regimes' edges and random ones) against the oracle on each
    row's standalone scores."""
    T, k = 65536, 2048
    say("cand long context", T, fp8)
    wl = make_custom([T], H=1, D_qk=64, D_v=64, H_idx=64, D_idx=128, topk=k, seed=1003,
                     device=DEV)
    q, k_idx, kw = _quantize(wl.q_idx, wl.k_idx, fp8)
    rs, sl = dsa.dsa_packed_metadata(wl.cu_seqlens, T)
    res, rescued = _run(q, k_idx, wl.w, rs, sl, k, T, **kw)
    rows = _long_rows(T, k)
    sc = torch.empty((len(rows), T), dtype=torch.float32, device=DEV)
    for i, r in enumerate(rows):
        _scores(q, k_idx, wl.w, rs, sl, kw, row_begin=r, n_rows=1, scores=sc[i:i + 1])
    torch.cuda.synchronize()
    _compare(res, sc, sl, rs, k, T, rows=rows)
    assert rescued == 0
    # every row: a full valid prefix of ascending ids inside the row's range
    idx, tl = res[0], res[1]
    assert torch.equal(tl, torch.clamp(sl, max=k))
    valid = idx >= 0
    assert torch.equal(valid.sum(1).int(), tl)
    assert torch.all(idx[:, 1:][valid[:, 1:]] > idx[:, :-1][valid[:, 1:]])
    assert torch.all(idx.max(1).values < rs + sl)
