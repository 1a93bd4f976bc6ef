"""Pins of the CPU oracle against things other than itself.

Each pin checks the oracle against a hand-derived fixture (tests/golden), a
brute-force evaluation, a textbook/library routine it must reduce to in a
special case, or a closed form. Together they are meant to catch a dropped
term, a wrong sign or index, or a transposed operand anywhere in the oracle.
These run on the CPU only.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _num(x):
    if isinstance(x, str):
        return float(x)
    return x


def _docs_meta(doc_lens):
    cu = np.concatenate([[0], np.cumsum(doc_lens)]).astype(np.int64)
    return cu, O.packed_metadata(cu, int(cu[-1]))


# ---------------------------------------------------------------- metadata --

def test_metadata_golden():
    g = _load("metadata_cu_0_3_7.json")
    st, sl = O.packed_metadata(g["cu_seqlens"], g["cu_seqlens"][-1])
    assert st.tolist() == g["row_starts"]
    assert sl.tolist() == g["seq_lens"]


def test_metadata_matches_searchsorted():
    rng = np.random.default_rng(0)
    doc_lens = rng.integers(1, 40, size=9)
    cu, (st, sl) = _docs_meta(doc_lens)
    t = np.arange(cu[-1])
    d = np.searchsorted(cu, t, side="right") - 1
    assert np.array_equal(st, cu[d])
    assert np.array_equal(sl, t - cu[d] + 1)


def test_metadata_empty_documents():
    # zero-length documents contribute no rows and do not shift the others
    st, sl = O.packed_metadata([0, 2, 2, 5], 5)
    assert st.tolist() == [0, 0, 2, 2, 2]
    assert sl.tolist() == [1, 2, 1, 2, 3]


# ----------------------------------------------------------------- indexer --

def test_indexer_golden():
    g = _load("indexer_small.json")
    q = np.array(g["q_idx"], dtype=np.float64)
    k = np.array(g["k_idx"], dtype=np.float64)
    w = np.array(g["w"], dtype=np.float64)
    for case in g["cases"]:
        st, sl = O.packed_metadata(case["cu_seqlens"], q.shape[0])
        exp = np.array([[_num(x) for x in row] for row in case["scores"]])
        got = O.indexer_scores(q, k, w, st, sl, np.arange(q.shape[0]), width=exp.shape[1])
        assert np.array_equal(np.isinf(got), np.isinf(exp))
        np.testing.assert_allclose(got[np.isfinite(exp)], exp[np.isfinite(exp)], rtol=0, atol=1e-15)


def _indexer_brute(q, k, w, cu):
    T, H, D = q.shape
    S = np.full((T, T), -np.inf)
    for d in range(len(cu) - 1):
        a, b = int(cu[d]), int(cu[d + 1])
        for t in range(a, b):
            for key in range(a, t + 1):
                tot = 0.0
                for h in range(H):
                    dot = 0.0
                    for e in range(D):
                        dot += q[t, h, e] * k[key, e]
                    tot += w[t, h] * max(dot, 0.0)
                S[t, key - a] = tot
    return S


def test_indexer_bruteforce_multidoc():
    rng = np.random.default_rng(1)
    doc_lens = [5, 1, 17, 9]
    cu, (st, sl) = _docs_meta(doc_lens)
    T, H, D = int(cu[-1]), 4, 6
    q = rng.standard_normal((T, H, D))
    k = rng.standard_normal((T, D))
    w = rng.standard_normal((T, H))
    got = O.indexer_scores(q, k, w, st, sl, np.arange(T), width=T)
    exp = _indexer_brute(q, k, w, cu)
    assert np.array_equal(np.isinf(got), np.isinf(exp))
    fin = np.isfinite(exp)
    np.testing.assert_allclose(got[fin], exp[fin], rtol=1e-12, atol=1e-12)


def test_indexer_single_head_is_masked_relu_matmul():
    # H = 1, W = 1: the score is ReLU(q k^T) on the causal lower triangle.
    rng = np.random.default_rng(2)
    T, D = 37, 8
    q = rng.standard_normal((T, 1, D))
    k = rng.standard_normal((T, D))
    w = np.ones((T, 1))
    st, sl = O.packed_metadata([0, T], T)
    got = O.indexer_scores(q, k, w, st, sl, np.arange(T), width=T)
    full = np.maximum(q[:, 0, :] @ k.T, 0.0)
    exp = np.where(np.tril(np.ones((T, T), dtype=bool)), full, -np.inf)
    np.testing.assert_array_equal(np.isinf(got), np.isinf(exp))
    np.testing.assert_allclose(got[np.isfinite(exp)], exp[np.isfinite(exp)], rtol=1e-13, atol=1e-13)


def test_indexer_nonnegative_inputs_reduce_to_gemv():
    # q, k >= 0 elementwise: ReLU is inactive, so S = (sum_h W_h q_h) . k^T.
    rng = np.random.default_rng(3)
    T, H, D = 29, 5, 7
    q = np.abs(rng.standard_normal((T, H, D)))
    k = np.abs(rng.standard_normal((T, D)))
    w = rng.standard_normal((T, H))
    st, sl = O.packed_metadata([0, T], T)
    got = O.indexer_scores(q, k, w, st, sl, np.arange(T), width=T)
    qw = np.einsum("th,thd->td", w, q)
    for t in range(T):
        np.testing.assert_allclose(got[t, : t + 1], k[: t + 1] @ qw[t], rtol=1e-12, atol=1e-12)


def test_indexer_mask_invariant():
    rng = np.random.default_rng(4)
    doc_lens = [3, 11, 1, 6]
    cu, (st, sl) = _docs_meta(doc_lens)
    T = int(cu[-1])
    q = rng.standard_normal((T, 3, 4))
    k = rng.standard_normal((T, 4))
    w = rng.standard_normal((T, 3))
    got = O.indexer_scores(q, k, w, st, sl, np.arange(T), width=T)
    for t in range(T):
        assert np.isfinite(got[t]).sum() == sl[t]
        assert np.all(np.isfinite(got[t, : sl[t]]))
    # no score depends on a key of another document: perturbing other docs' keys
    k2 = k.copy()
    k2[: cu[1]] += 10.0
    got2 = O.indexer_scores(q, k2, w, st, sl, np.arange(T), width=T)
    assert np.array_equal(got[cu[1]:], got2[cu[1]:])


# ------------------------------------------------------- ratio-causal mask --

def _visible_columns(g, seqlen_k, ratio):
    """Compressed key columns a query at global token position g may see.

    Column c stands for the tokens c*ratio .. c*ratio + ratio - 1 (the keys
    are a compressed prefix from column 0); it is visible once every one of
    those tokens is at or before g. Enumerated token by token.
    """
    return [c for c in range(seqlen_k)
            if all(tok <= g for tok in range(c * ratio, (c + 1) * ratio))]


def _random_segments(rng, n_seq):
    q_lens = rng.integers(0, 14, size=n_seq)
    k_lens = rng.integers(0, 10, size=n_seq)
    cq = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    ck = np.concatenate([[0], np.cumsum(k_lens)]).astype(np.int64)
    return cq, ck


def test_ratio_causal_metadata_matches_token_enumeration():
    rng = np.random.default_rng(40)
    for trial in range(60):
        n_seq = int(rng.integers(1, 5))
        cq, ck = _random_segments(rng, n_seq)
        ratio = int(rng.integers(1, 6))
        off = rng.integers(-9, 26, size=n_seq) if trial % 3 else None
        T = int(cq[-1])
        st, sl = O.ratio_causal_metadata(cq, ck, T, ratio, off)
        for b in range(n_seq):
            for t in range(int(cq[b]), int(cq[b + 1])):
                g = (0 if off is None else int(off[b])) + t - int(cq[b])
                vis = _visible_columns(g, int(ck[b + 1] - ck[b]), ratio)
                assert vis == list(range(len(vis)))  # a prefix of the columns
                assert sl[t] == len(vis), (trial, b, t)
                assert st[t] == ck[b]


def test_ratio_causal_metadata_reduces_to_packed_metadata():
    # ratio 1, no offsets, keys stored like queries: the plain causal mask
    cu = np.array([0, 4, 4, 13, 20])
    st, sl = O.ratio_causal_metadata(cu, cu, 20)
    st0, sl0 = O.packed_metadata(cu, 20)
    assert np.array_equal(st, st0) and np.array_equal(sl, sl0)


def test_ratio_causal_clamps():
    # offsets before the timeline start see nothing until (g + 1) // ratio > 0;
    # rows past the compressed prefix see the whole prefix
    st, sl = O.ratio_causal_metadata([0, 6, 12], [0, 3, 5], 12, ratio=2,
                                     q_causal_offsets=[-4, 40])
    assert sl.tolist() == [0, 0, 0, 0, 0, 1] + [2] * 6
    assert st.tolist() == [0] * 6 + [3] * 6


@pytest.mark.parametrize("ratio", [1, 4])
def test_query_offsets_split_equals_whole_sequence(ratio):
    # One sequence of L tokens scored whole, and again with its queries split
    # into three stored segments whose offsets are their global positions: each
    # split row must get the same mask and the same scores as in the whole run.
    rng = np.random.default_rng(41)
    L, H, D = 23, 3, 5
    Lk = L // ratio + 1
    q = rng.standard_normal((L, H, D))
    k = rng.standard_normal((Lk, D))
    w = rng.standard_normal((L, H))
    st, sl = O.ratio_causal_metadata([0, L], [0, Lk], L, ratio)
    whole = O.indexer_scores(q, k, w, st, sl, np.arange(L), width=Lk)
    cuts = [0, 7, 15, L]
    k_rep = np.concatenate([k, k, k])                  # each segment stores the prefix
    ck = [0, Lk, 2 * Lk, 3 * Lk]
    st2, sl2 = O.ratio_causal_metadata(cuts, ck, L, ratio, q_causal_offsets=cuts[:3])
    split = O.indexer_scores(q, k_rep, w, st2, sl2, np.arange(L), width=Lk)
    assert np.array_equal(sl2, sl)
    assert np.array_equal(np.isinf(split), np.isinf(whole))
    fin = np.isfinite(whole)
    np.testing.assert_allclose(split[fin], whole[fin], rtol=0, atol=0)


def test_indexer_ratio_causal_bruteforce():
    rng = np.random.default_rng(42)
    cq = np.array([0, 9, 9, 20])
    ck = np.array([0, 4, 6, 9])
    off = [3, 0, 14]
    ratio = 3
    T, H, D = 20, 3, 4
    q = rng.standard_normal((T, H, D))
    k = rng.standard_normal((9, D))
    w = rng.standard_normal((T, H))
    st, sl = O.ratio_causal_metadata(cq, ck, T, ratio, off)
    got = O.indexer_scores(q, k, w, st, sl, np.arange(T), width=6)
    exp = np.full((T, 6), -np.inf)
    for b in range(3):
        for t in range(cq[b], cq[b + 1]):
            for c in _visible_columns(off[b] + t - cq[b], int(ck[b + 1] - ck[b]), ratio):
                tot = 0.0
                for h in range(H):
                    dot = sum(q[t, h, e] * k[ck[b] + c, e] for e in range(D))
                    tot += w[t, h] * max(dot, 0.0)
                exp[t, c] = tot
    assert np.array_equal(np.isinf(got), np.isinf(exp))
    fin = np.isfinite(exp)
    np.testing.assert_allclose(got[fin], exp[fin], rtol=1e-12, atol=1e-12)


def _ratio_mutant(cq, ck, T, ratio, off, mistake):
    """A deliberately wrong copy of the ratio-causal count."""
    sl = np.zeros(T, dtype=np.int64)
    for b in range(len(cq) - 1):
        for t in range(cq[b], cq[b + 1]):
            ql = t - cq[b]
            o = cq[b] if mistake == "storage_offset" else off[b]
            if mistake == "no_plus_one":
                v = (o + ql) // ratio
            elif mistake == "ceil":
                v = -((-(o + ql + 1)) // ratio)
            else:
                v = (o + ql + 1) // ratio
            hi = 10 ** 9 if mistake == "no_upper_clamp" else ck[b + 1] - ck[b]
            sl[t] = min(max(v, 0), hi)
    return sl


def test_planted_ratio_causal_mistakes_fail_their_pins():
    cq, ck, off, ratio = [0, 10, 22], [0, 2, 4], [5, 1], 4
    _, sl = O.ratio_causal_metadata(cq, ck, 22, ratio, off)
    enum = [len(_visible_columns(off[b] + t - cq[b], ck[b + 1] - ck[b], ratio))
            for b in range(2) for t in range(cq[b], cq[b + 1])]
    assert sl.tolist() == enum
    for mistake in ("no_plus_one", "ceil", "storage_offset", "no_upper_clamp"):
        assert _ratio_mutant(cq, ck, 22, ratio, off, mistake).tolist() != enum, mistake


# ---------------------------------------------------------------- FP8 input --

def test_decode_e4m3_matches_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.decode_e4m3(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref)) and np.isnan(got).sum() == 2
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))
    # hand-derived values of the encoding
    assert O.decode_e4m3([0x38, 0x7E, 0x01, 0x08, 0xC0])[:].tolist() == [1.0, 448.0, 2.0 ** -9,
                                                                         2.0 ** -6, -2.0]


def test_decode_e8m0_matches_torch_float8_e8m0fnu():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = O.decode_e8m0(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref)) and np.isnan(got).sum() == 1
    assert np.array_equal(got[:255], ref[:255])
    assert O.decode_e8m0([127, 128, 0]).tolist() == [1.0, 2.0, 2.0 ** -127]


def _e4m3_bytes(x32):
    """Round float32 values to E4M3 bytes with torch's cast (nearest-even)."""
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def _quant_err(x, scale):
    """Rigorous bound of |dequant(quant(x)) - x| for E4M3 with descale `scale`:
    half a unit in the last place, 2^-4 relative for normals, 2^-10 * scale in
    the subnormal range."""
    return np.maximum(np.abs(x) * 2.0 ** -4, scale * 2.0 ** -10)


def _fp8_case(rng, T, H, D, spread):
    """Real-valued indexer inputs whose magnitudes vary over tokens, heads and
    32-element blocks by factors up to e^spread."""
    q = rng.standard_normal((T, H, D)) * np.exp(spread * rng.standard_normal((T, H, 1)))
    k = rng.standard_normal((T, D)) * np.exp(spread * rng.standard_normal((T, 1)))
    blk = np.repeat(np.exp(spread * rng.standard_normal(D // 32)), 32)
    return q * blk, k * blk[::-1], rng.standard_normal((T, H))


def _score_bound(q, k, w, eq, ek, st, sl):
    T = q.shape[0]
    bound = np.zeros((T, T))
    for t in range(T):
        n, s0 = int(sl[t]), int(st[t])
        kk, ee = np.abs(k[s0:s0 + n]), ek[s0:s0 + n]
        per = (eq[t] @ (kk + ee).T) + (np.abs(q[t]) @ ee.T)   # [H, n]
        bound[t, :n] = np.abs(w[t]) @ per
    return bound


def _fp8_per_token(q, k):
    qs = np.abs(q).max(axis=2) / 448.0
    ks = np.abs(k).max(axis=1) / 448.0
    q8 = _e4m3_bytes(q / qs[..., None])
    k8 = _e4m3_bytes(k / ks[:, None])
    return q8, qs, k8, ks


def _fp8_per_block(q, k):
    def sf(x):
        amax = np.abs(x.reshape(*x.shape[:-1], -1, 32)).max(axis=-1)
        e = np.ceil(np.log2(amax / 448.0)).astype(np.int64)        # 2^e >= amax / 448
        return (e + 127).astype(np.uint8), np.repeat(np.exp2(e.astype(np.float64)), 32, axis=-1)
    q_sf, qs = sf(q)
    k_sf, ks = sf(k)
    return _e4m3_bytes(q / qs), q_sf, qs, _e4m3_bytes(k / ks), k_sf, ks


def test_fp8_indexer_within_quantisation_bound():
    rng = np.random.default_rng(50)
    T, H, D = 24, 5, 64
    q, k, w = _fp8_case(rng, T, H, D, 1.5)
    st, sl = O.packed_metadata([0, 9, T], T)
    exact = O.indexer_scores(q, k, w, st, sl, np.arange(T), width=T)
    q8, qs, k8, ks = _fp8_per_token(q, k)
    got = O.indexer_scores_fp8(q8, qs, k8, ks, w, st, sl, np.arange(T), width=T)
    bound = _score_bound(q, k, w, _quant_err(q, qs[..., None]), _quant_err(k, ks[:, None]), st, sl)
    fin = np.isfinite(exact)
    assert np.array_equal(np.isfinite(got), fin)
    assert np.all(np.abs(got[fin] - exact[fin]) <= bound[fin] * (1 + 1e-9))
    # the bound is informative: the scores move by less than 10% of their scale
    assert np.abs(got[fin] - exact[fin]).max() < 0.1 * np.abs(exact[fin]).max()


def test_mxfp8_indexer_within_quantisation_bound():
    rng = np.random.default_rng(51)
    T, H, D = 20, 4, 128
    q, k, w = _fp8_case(rng, T, H, D, 2.0)
    st, sl = O.packed_metadata([0, 20], T)
    exact = O.indexer_scores(q, k, w, st, sl, np.arange(T), width=T)
    q8, q_sf, qs, k8, k_sf, ks = _fp8_per_block(q, k)
    got = O.indexer_scores_mxfp8(q8, q_sf, k8, k_sf, w, st, sl, np.arange(T), width=T)
    bound = _score_bound(q, k, w, _quant_err(q, qs), _quant_err(k, ks), st, sl)
    fin = np.isfinite(exact)
    assert np.all(np.abs(got[fin] - exact[fin]) <= bound[fin] * (1 + 1e-9))
    assert np.abs(got[fin] - exact[fin]).max() < 0.1 * np.abs(exact[fin]).max()


def test_fp8_scale_transfer_invariance():
    # moving a power of two from a key's descale into every query descale
    # changes no score (both enter the same product)
    rng = np.random.default_rng(52)
    T, H, D = 16, 3, 32
    q8 = rng.integers(0, 256, (T, H, D)).astype(np.uint8)
    k8 = rng.integers(0, 256, (T, D)).astype(np.uint8)
    q8[(q8 & 0x7F) == 0x7F] = 0x11                             # no NaN codes
    k8[(k8 & 0x7F) == 0x7F] = 0x22
    qs = np.exp(rng.standard_normal((T, H)))
    ks = np.exp(rng.standard_normal(T))
    w = rng.standard_normal((T, H))
    st, sl = O.packed_metadata([0, T], T)
    a = O.indexer_scores_fp8(q8, qs, k8, ks, w, st, sl, np.arange(T))
    b = O.indexer_scores_fp8(q8, qs * 4.0, k8, ks / 4.0, w, st, sl, np.arange(T))
    fin = np.isfinite(a)
    np.testing.assert_allclose(b[fin], a[fin], rtol=1e-13, atol=1e-300)


def test_planted_fp8_mistakes_fail_the_bound():
    rng = np.random.default_rng(53)
    T, H, D = 24, 5, 64
    q, k, w = _fp8_case(rng, T, H, D, 1.5)
    st, sl = O.packed_metadata([0, T], T)
    exact = O.indexer_scores(q, k, w, st, sl, np.arange(T), width=T)
    fin = np.isfinite(exact)
    q8, qs, k8, ks = _fp8_per_token(q, k)
    bound = _score_bound(q, k, w, _quant_err(q, qs[..., None]), _quant_err(k, ks[:, None]), st, sl)
    qd, kd = O.decode_e4m3(q8), O.decode_e4m3(k8)
    mutants = {
        "key descales of other keys": (qd * qs[..., None], kd * ks[::-1, None]),
        "descale divided": (qd / qs[..., None], kd / ks[:, None]),
        "head descale of head 0": (qd * qs[:, :1, None], kd * ks[:, None]),
    }
    for name, (qm, km) in mutants.items():
        bad = O.indexer_scores(qm, km, w, st, sl, np.arange(T), width=T)
        assert np.any(np.abs(bad[fin] - exact[fin]) > bound[fin]), name
    # MX: the block scale of element d taken as d % (D/32) instead of d // 32
    T, H, D = 12, 3, 128
    q, k, w = _fp8_case(rng, T, H, D, 2.0)
    st, sl = O.packed_metadata([0, T], T)
    exact = O.indexer_scores(q, k, w, st, sl, np.arange(T), width=T)
    fin = np.isfinite(exact)
    q8, q_sf, qs, k8, k_sf, ks = _fp8_per_block(q, k)
    bound = _score_bound(q, k, w, _quant_err(q, qs), _quant_err(k, ks), st, sl)
    inter = lambda c: np.tile(O.decode_e8m0(c), 32)  # noqa: E731
    bad = O.indexer_scores(O.decode_e4m3(q8) * inter(q_sf), O.decode_e4m3(k8) * inter(k_sf), w,
                           st, sl, np.arange(T), width=T)
    assert np.any(np.abs(bad[fin] - exact[fin]) > bound[fin])


# ------------------------------------------------------------------- top-K --

def test_topk_golden_ties_and_signed_zero():
    g = _load("topk_ties.json")
    row = np.array(g["row"], dtype=np.float64)
    assert math.copysign(1.0, row[3]) < 0  # the fixture really holds -0.0
    for c in g["cases"]:
        idx, ln = O.topk(row[None, :], [c["seq_len"]], c["k"])
        assert idx[0].tolist() == c["indices"], c
        assert ln[0] == min(c["seq_len"], c["k"])


def _topk_brute(x, n, k):
    # full stable sort by (value descending, index ascending)
    order = sorted(range(n), key=lambda j: (-float(x[j]), j))
    return sorted(order[: min(n, k)])


@pytest.mark.parametrize("levels", [None, 2, 3, 5])
def test_topk_bruteforce_sort(levels):
    rng = np.random.default_rng(10 + (levels or 0))
    for trial in range(300):
        n_cols = int(rng.integers(1, 40))
        x = rng.standard_normal(n_cols)
        if levels is not None:
            x = np.round(x * levels / 2) / levels  # many exact ties, incl. 0
            zeros = x == 0
            x[zeros & (rng.random(n_cols) < 0.5)] = -0.0
        n = int(rng.integers(0, n_cols + 1))
        k = int(rng.integers(1, 12))
        idx, ln = O.topk(x[None, :], [n], k)
        exp = _topk_brute(x, n, k)
        assert idx[0, : len(exp)].tolist() == exp
        assert np.all(idx[0, len(exp):] == -1)
        assert ln[0] == len(exp)


def test_topk_closed_forms():
    n, k = 50, 16
    # all-equal row: the first K columns
    idx, _ = O.topk(np.full((1, n), 0.25), [n], k)
    assert idx[0].tolist() == list(range(k))
    # strictly increasing row: the last K columns
    idx, _ = O.topk(np.arange(n, dtype=np.float64)[None, :], [n], k)
    assert idx[0].tolist() == list(range(n - k, n))
    # strictly decreasing row: the first K columns
    idx, _ = O.topk(-np.arange(n, dtype=np.float64)[None, :], [n], k)
    assert idx[0].tolist() == list(range(k))
    # seq_len <= K: every causal column, then -1
    idx, ln = O.topk(np.random.default_rng(0).standard_normal((1, n)), [9], k)
    assert idx[0].tolist() == list(range(9)) + [-1] * (k - 9) and ln[0] == 9
    # global coordinates: row start added, padding stays -1
    idx, _ = O.topk(np.full((1, n), 1.0), [3], 4, row_starts=[100])
    assert idx[0].tolist() == [100, 101, 102, -1]
    # seq_len beyond the row width is clamped to the width
    idx, ln = O.topk(np.arange(6, dtype=np.float64)[None, :], [99], 8)
    assert idx[0].tolist() == [0, 1, 2, 3, 4, 5, -1, -1] and ln[0] == 6


def test_topk_invariants_random():
    rng = np.random.default_rng(5)
    n_rows, n_cols, k = 40, 300, 37
    x = np.round(rng.standard_normal((n_rows, n_cols)) * 8) / 8
    sl = rng.integers(0, n_cols + 1, size=n_rows)
    idx, ln = O.topk(x, sl, k)
    for r in range(n_rows):
        n = sl[r]
        sel = idx[r, : ln[r]]
        assert ln[r] == min(n, k)
        assert np.all(np.diff(sel) > 0) and np.all(sel >= 0) and np.all(sel < max(n, 1))
        if n > k:
            mask = np.zeros(n, dtype=bool)
            mask[sel] = True
            lo, hi = x[r, :n][mask].min(), x[r, :n][~mask].max()
            assert lo >= hi
            # tie rule: unselected columns equal to the threshold lie after
            # every selected column of that value
            tie_sel = np.nonzero(mask & (x[r, :n] == lo))[0]
            tie_uns = np.nonzero(~mask & (x[r, :n] == lo))[0]
            if len(tie_uns):
                assert tie_sel.max() < tie_uns.min()


# ------------------------------------------------- top-K softmax and LSE --

def test_topk_softmax_matches_scipy_and_indexer_recompute():
    from scipy.special import logsumexp, softmax
    rng = np.random.default_rng(60)
    T, H, D, K = 40, 3, 5, 7
    q = rng.standard_normal((T, H, D))
    k = rng.standard_normal((T, D))
    w = rng.standard_normal((T, H))
    cu = np.array([0, 13, 13, 40])
    st, sl = O.packed_metadata(cu, T)
    sc = O.indexer_scores(q, k, w, st, sl, np.arange(T), width=T)
    idx, ln, logits, soft, lse = O.topk_softmax(sc, sl, K, row_starts=st, n_cols=T)
    for t in range(T):
        m = int(ln[t])
        sel = idx[t, :m].astype(np.int64)
        # section 6: softmax of the indexer score recomputed at the selected keys
        rec = np.array([w[t] @ np.maximum(q[t] @ k[j], 0.0) for j in sel])
        np.testing.assert_allclose(logits[t, :m], rec, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(soft[t, :m], softmax(rec), rtol=1e-12, atol=1e-15)
        assert abs(lse[t] - logsumexp(rec)) < 1e-12
        assert np.all(logits[t, m:] == -np.inf) and np.all(soft[t, m:] == 0.0)
        assert abs(soft[t, :m].sum() - 1.0) < 1e-12


def test_topk_softmax_closed_forms():
    # equal logits: softmax 1/m and lse = v + ln m; one column: softmax 1, lse = v;
    # an empty row: lse = +inf, no slot
    x = np.array([[2.5] * 6, [-1.0, 0, 0, 0, 0, 0], [9.0] * 6])
    idx, ln, logits, soft, lse = O.topk_softmax(x, [6, 1, 0], 4)
    np.testing.assert_allclose(soft[0], 0.25)
    assert abs(lse[0] - (2.5 + math.log(4))) < 1e-14
    assert soft[1].tolist() == [1.0, 0, 0, 0] and lse[1] == -1.0
    assert ln[2] == 0 and lse[2] == np.inf and np.all(idx[2] == -1)


def test_planted_topk_softmax_mistakes_fail():
    # Normalising over the whole row instead of the selected slots, or an LSE
    # that drops its max term, break the pins above (softmax sums to 1 over
    # the selected slots; lse equals scipy's logsumexp of the selected logits).
    from scipy.special import logsumexp
    rng = np.random.default_rng(61)
    lens = [30, 12, 9]
    x = rng.standard_normal((3, 30)) * 0.5  # mass outside the top-8 stays large
    idx, ln, logits, soft, lse = O.topk_softmax(x, lens, 8)
    for r in range(3):
        m = int(ln[r])
        v = logits[r, :m]
        assert abs(lse[r] - logsumexp(v)) < 1e-12
        whole = logsumexp(x[r, :lens[r]])
        assert abs(np.exp(v - whole).sum() - 1.0) > 1e-3        # row-normalised: not 1
        no_max = np.log(np.exp(v - v.max()).sum())
        assert abs(no_max - logsumexp(v)) > 1e-3                 # max term dropped


# --------------------------------------------------------------- attention --

def test_attention_golden():
    g = _load("attention_two_keys.json")
    q = np.array(g["q"], dtype=np.float64)
    k = np.array(g["k"], dtype=np.float64)
    v = np.array(g["v"], dtype=np.float64)
    for c in g["cases"]:
        idx = np.array([c["indices"]], dtype=np.int64)
        tl = None if c["topk_length"] is None else np.array([c["topk_length"]])
        sink = None if c["sink"] is None else np.array([c["sink"]])
        out, lse, mx = O.sparse_attention(q, k, v, idx, tl, sink, g["scale"])
        np.testing.assert_allclose(out[0, 0], c["out"], rtol=0, atol=1e-14)
        assert lse[0, 0] == pytest.approx(_num(c["lse"]), abs=1e-14) or (
            np.isinf(_num(c["lse"])) and lse[0, 0] == _num(c["lse"]))
        assert mx[0, 0] == pytest.approx(_num(c["max_logits"]), abs=1e-14) or (
            np.isinf(_num(c["max_logits"])) and mx[0, 0] == _num(c["max_logits"]))


def _sdpa(q, k, v, scale, mask):
    """torch's scaled_dot_product_attention in float64 on the CPU."""
    tq = torch.from_numpy(np.ascontiguousarray(q))
    tk = torch.from_numpy(np.ascontiguousarray(k))
    tv = torch.from_numpy(np.ascontiguousarray(v))
    tm = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask))
    return torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=tm, scale=scale).numpy()


def _causal_full_indices(T, width):
    idx = np.full((T, width), -1, dtype=np.int64)
    for t in range(T):
        idx[t, : t + 1] = np.arange(t + 1)
    return idx


@pytest.mark.parametrize("shared", [True, False])
def test_attention_dense_identity_sdpa(shared):
    # Top-K covering every causal key and no sink == dense causal attention.
    rng = np.random.default_rng(20)
    T, H, Dqk, Dv = 23, 3, 12, 8
    q = rng.standard_normal((T, H, Dqk))
    kv = rng.standard_normal((T, Dqk))
    v = None if shared else rng.standard_normal((T, Dv))
    scale = 0.37
    idx = _causal_full_indices(T, T + 5)
    out, lse, _ = O.sparse_attention(q, kv, v, idx, None, None, scale, d_v=Dv)
    vv = kv[:, :Dv] if shared else v
    causal = np.where(np.tril(np.ones((T, T), dtype=bool)), 0.0, -np.inf)
    ref = _sdpa(q.transpose(1, 0, 2), np.broadcast_to(kv, (H, T, Dqk)),
                np.broadcast_to(vv, (H, T, Dv)), scale, causal)
    np.testing.assert_allclose(out, ref.transpose(1, 0, 2), rtol=1e-12, atol=1e-13)
    # LSE through a probe key: logit 0, value = one-hot in an extra value dim.
    # Its attention weight is 1 / (1 + exp(lse)).
    kp = np.concatenate([kv, np.zeros((1, Dqk))])
    vp = np.zeros((T + 1, Dv + 1))
    vp[:T, :Dv] = vv
    vp[T, Dv] = 1.0
    maskp = np.concatenate([causal, np.zeros((T, 1))], axis=1)
    refp = _sdpa(q.transpose(1, 0, 2), np.broadcast_to(kp, (H, T + 1, Dqk)),
                 np.broadcast_to(vp, (H, T + 1, Dv + 1)), scale, maskp)
    wprobe = refp[:, :, Dv].T
    np.testing.assert_allclose(lse, np.log(1.0 / wprobe - 1.0), rtol=1e-10, atol=1e-10)


def test_attention_sink_as_extra_key_sdpa():
    # The sink equals one more key with per-head logit sink_h and a zero value.
    rng = np.random.default_rng(21)
    T, H, D = 17, 4, 10
    q = rng.standard_normal((T, H, D))
    kv = rng.standard_normal((T, D))
    sink = rng.standard_normal(H) * 2
    scale = 0.5
    idx = _causal_full_indices(T, T)
    out, lse, mx = O.sparse_attention(q, kv, None, idx, None, sink, scale, d_v=D)
    causal = np.where(np.tril(np.ones((T, T), dtype=bool)), 0.0, -np.inf)
    kp = np.concatenate([kv, np.zeros((1, D))])
    vp = np.concatenate([kv, np.zeros((1, D))])
    mask = np.zeros((H, T, T + 1))
    mask[:, :, :T] = causal
    mask[:, :, T] = sink[:, None]
    ref = _sdpa(q.transpose(1, 0, 2), np.broadcast_to(kp, (H, T + 1, D)),
                np.broadcast_to(vp, (H, T + 1, D)), scale, mask)
    np.testing.assert_allclose(out, ref.transpose(1, 0, 2), rtol=1e-12, atol=1e-13)
    # the sink does not enter lse or max_logits
    _, lse0, mx0 = O.sparse_attention(q, kv, None, idx, None, None, scale, d_v=D)
    np.testing.assert_array_equal(lse, lse0)
    np.testing.assert_array_equal(mx, mx0)


def test_attention_duplicate_slot_is_log2_bias_sdpa():
    rng = np.random.default_rng(22)
    Tkv, H, D = 9, 2, 6
    q = rng.standard_normal((1, H, D))
    kv = rng.standard_normal((Tkv, D))
    idx = np.array([[0, 3, 3, 7, 8]])
    out, _, _ = O.sparse_attention(q, kv, None, idx, None, None, 0.8, d_v=D)
    keys = np.array([0, 3, 7, 8])
    mask = np.zeros((1, len(keys)))
    mask[0, 1] = math.log(2.0)
    ref = _sdpa(q.transpose(1, 0, 2), np.broadcast_to(kv[keys], (H, 4, D)),
                np.broadcast_to(kv[keys], (H, 4, D)), 0.8, mask)
    np.testing.assert_allclose(out[0], ref[:, 0, :], rtol=1e-12, atol=1e-13)


def test_attention_closed_forms():
    rng = np.random.default_rng(23)
    Tkv, H, Dqk, Dv, W = 30, 3, 16, 12, 11
    kv = rng.standard_normal((Tkv, Dqk))
    idx = rng.integers(0, Tkv, size=(1, W))
    # V all ones: every output is 1 without a sink
    v1 = np.ones((Tkv, Dv))
    q = rng.standard_normal((1, H, Dqk))
    out, _, _ = O.sparse_attention(q, kv, v1, idx, None, None, 0.3)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-14)
    # q = 0: lse = ln(n), out = mean of the selected V rows
    v = rng.standard_normal((Tkv, Dv))
    out, lse, mx = O.sparse_attention(np.zeros((1, H, Dqk)), kv, v, idx, None, None, 0.3)
    np.testing.assert_allclose(lse, math.log(W), rtol=0, atol=1e-14)
    np.testing.assert_allclose(out[0], np.broadcast_to(v[idx[0]].mean(0), (H, Dv)), atol=1e-14)
    np.testing.assert_array_equal(mx, 0.0)
    # a single valid slot: out = that V row, lse = max = its scaled logit
    one = np.array([[-1, 5, -1, 99]])
    out, lse, mx = O.sparse_attention(q, kv, v, one, None, None, 0.3)
    np.testing.assert_allclose(out[0], np.broadcast_to(v[5], (H, Dv)), atol=1e-14)
    s = 0.3 * np.array([sum(q[0, h, d] * kv[5, d] for d in range(Dqk)) for h in range(H)])
    np.testing.assert_allclose(lse[0], s, atol=1e-13)
    np.testing.assert_allclose(mx[0], s, atol=1e-13)
    # sink closed form: out_sink = out / (1 + exp(sink - lse))
    sink = rng.standard_normal(H)
    o0, l0, _ = O.sparse_attention(q, kv, v, idx, None, None, 0.3)
    o1, l1, _ = O.sparse_attention(q, kv, v, idx, None, sink, 0.3)
    np.testing.assert_allclose(o1, o0 / (1.0 + np.exp(sink[None, :] - l0))[:, :, None], rtol=1e-12)
    np.testing.assert_array_equal(l0, l1)


def test_attention_permutation_and_invalid_slots():
    rng = np.random.default_rng(24)
    Tkv, H, D = 40, 2, 9
    q = rng.standard_normal((1, H, D))
    kv = rng.standard_normal((Tkv, D))
    base = np.array([[3, 17, 5, 39, 0]])
    o0, l0, m0 = O.sparse_attention(q, kv, None, base, None, None, 0.6, d_v=D)
    perm = np.array([[39, 0, 5, 3, 17]])
    o1, l1, m1 = O.sparse_attention(q, kv, None, perm, None, None, 0.6, d_v=D)
    np.testing.assert_allclose(o1, o0, rtol=1e-13)
    np.testing.assert_allclose(l1, l0, rtol=1e-13)
    # -1, negative and out-of-range ids, and slots past topk_length are removed
    noisy = np.array([[3, -1, 17, 40, 5, -7, 39, 1000, 0, 22, 11]])
    o2, l2, m2 = O.sparse_attention(q, kv, None, noisy, np.array([9]), None, 0.6, d_v=D)
    np.testing.assert_allclose(o2, o0, rtol=1e-13)
    np.testing.assert_allclose(l2, l0, rtol=1e-13)
    np.testing.assert_array_equal(m2, m0)


def test_oracle_detects_planted_mistakes():
    """The pins above must fail for typical slips; plant a few on the CPU."""
    rng = np.random.default_rng(30)
    T, H, D = 12, 3, 5
    q = rng.standard_normal((T, H, D))
    k = rng.standard_normal((T, D))
    w = rng.standard_normal((T, H))
    cu = np.array([0, 5, 12])
    st, sl = O.packed_metadata(cu, T)
    good = O.indexer_scores(q, k, w, st, sl, np.arange(T), width=T)
    brute = _indexer_brute(q, k, w, cu)
    fin = np.isfinite(brute)
    # a dropped ReLU, a sign flip of W, the ReLU applied after the head sum
    # and the weights of the wrong query row all differ from brute force
    no_relu = np.full_like(good, -np.inf)
    flip = np.full_like(good, -np.inf)
    relu_late = np.full_like(good, -np.inf)
    wrong_row = np.full_like(good, -np.inf)
    for t in range(T):
        n, s0 = sl[t], st[t]
        qk = q[t] @ k[s0:s0 + n].T  # [H, n]
        no_relu[t, :n] = w[t] @ qk
        flip[t, :n] = -(w[t] @ np.maximum(qk, 0))
        relu_late[t, :n] = np.maximum(w[t] @ qk, 0)
        wrong_row[t, :n] = w[(t + 1) % T] @ np.maximum(qk, 0)
    assert np.allclose(good[fin], brute[fin])
    for mutant in (no_relu, flip, relu_late, wrong_row):
        assert not np.allclose(mutant[fin], brute[fin])


def _attn_mutant(q, kv, idx, sink, scale, d_v, mistake):
    """A deliberately wrong copy of the attention definition (fp64 loops)."""
    T, H, _ = q.shape
    out = np.zeros((T, H, d_v))
    lse = np.zeros((T, H))
    for t in range(T):
        sel = [j for j in idx[t] if 0 <= j < kv.shape[0]]
        kk = kv[sel]
        for h in range(H):
            if mistake == "transposed":
                s = scale * (kk[:, : q.shape[2]] @ q[t].T)[:, (h + 1) % H]
            else:
                s = (1.0 if mistake == "no_scale" else scale) * (kk @ q[t, h])
            m = s.max()
            e = np.exp(s - m)
            den = e.sum() + (np.exp(sink[h] - m) if sink is not None else 0.0)
            out[t, h] = (e @ kk[:, :d_v]) / den
            lse[t, h] = m + np.log(den if mistake == "sink_in_lse" else e.sum())
    return out, lse


def test_planted_topk_and_attention_mistakes_fail_their_pins():
    """Typical slips in the top-K and attention definitions fail the pins above."""
    rng = np.random.default_rng(31)
    # top-K: ties to the higher column, or one column too few, disagree with
    # the brute-force stable sort on a tie-heavy row.
    x = np.round(rng.standard_normal(40) * 1.5) / 1.5
    n, k = 35, 9
    x[n - 1] = 10.0  # the row's last valid column is selected
    exp = _topk_brute(x, n, k)
    assert O.topk(x[None, :], [n], k)[0][0, :k].tolist() == exp
    high_tie = sorted(sorted(range(n), key=lambda j: (-float(x[j]), -j))[:k])
    short = sorted(sorted(range(n - 1), key=lambda j: (-float(x[j]), j))[:k])
    assert high_tie != exp
    assert short != exp
    # attention: a missing scale, the sink inside the LSE, or a transposed
    # head/key operand disagree with the dense-identity pin (SDPA).
    T, H, D = 9, 3, 6
    q = rng.standard_normal((T, H, D))
    kv = rng.standard_normal((T, D))
    sink = rng.standard_normal(H)
    scale = 0.41
    idx = _causal_full_indices(T, T)
    causal = np.where(np.tril(np.ones((T, T), dtype=bool)), 0.0, -np.inf)
    ref = _sdpa(q.transpose(1, 0, 2), np.broadcast_to(kv, (H, T, D)),
                np.broadcast_to(kv, (H, T, D)), scale, causal).transpose(1, 0, 2)
    good_o, good_l, _ = O.sparse_attention(q, kv, None, idx, None, None, scale, d_v=D)
    np.testing.assert_allclose(good_o, ref, rtol=1e-12, atol=1e-13)
    for mistake in ("no_scale", "transposed"):
        o, _ = _attn_mutant(q, kv, idx, None, scale, D, mistake)
        assert not np.allclose(o, ref, atol=1e-6), mistake
    # sink in the LSE: breaks the closed form lse(sink) == lse(no sink)
    _, l_mut = _attn_mutant(q, kv, idx, sink, scale, D, "sink_in_lse")
    _, l_ok, _ = O.sparse_attention(q, kv, None, idx, None, sink, scale, d_v=D)
    np.testing.assert_allclose(l_ok, good_l, rtol=1e-12)
    assert not np.allclose(l_mut, good_l, atol=1e-6)


# ------------------------------------------------------ attention backward --

def _bwd_case(rng, T=7, H=3, D=6, dv=4, K=5, dup=True):
    q = rng.standard_normal((T, H, D))
    kv = rng.standard_normal((T, D))
    idx = np.full((T, K), -1, dtype=np.int64)
    for t in range(T):
        c = rng.permutation(t + 1)[: min(K, t + 1)]
        idx[t, : len(c)] = c
    if dup:
        idx[T - 1, -1] = idx[T - 1, 0]  # a duplicated slot
        idx[2, -1] = T + 5              # an out-of-range id: invalid slot
    tl = np.array([min(K, t + 1) for t in range(T)])
    tl[T - 1] = K
    tl[2] = K
    sink = rng.standard_normal(H)
    dout = rng.standard_normal((T, H, dv))
    return q, kv, idx, tl, sink, dout


def _loss(q, kv, idx, tl, sink, scale, dout, dv):
    out, _, _ = O.sparse_attention(q, kv, None, idx, tl, sink, scale, d_v=dv)
    return float((out * dout).sum())


def test_attention_backward_finite_differences():
    rng = np.random.default_rng(70)
    q, kv, idx, tl, sink, dout = _bwd_case(rng)
    scale, dv = 0.37, 4
    dq, dkv, ds = O.sparse_attention_backward(q, kv, idx, tl, sink, scale, dout, dv)
    h = 1e-6
    for arr, grad in ((q, dq), (kv, dkv), (sink, ds)):
        flat, gflat = arr.reshape(-1), grad.reshape(-1)
        for i in rng.choice(flat.size, size=min(12, flat.size), replace=False):
            old = flat[i]
            flat[i] = old + h
            up = _loss(q, kv, idx, tl, sink, scale, dout, dv)
            flat[i] = old - h
            dn = _loss(q, kv, idx, tl, sink, scale, dout, dv)
            flat[i] = old
            assert abs((up - dn) / (2 * h) - gflat[i]) < 1e-7 * max(1.0, abs(gflat[i])), i


def _dense_torch_grads(q, kv, sink, scale, dout, dv):
    """Dense causal attention with a sink written in torch (fp64, CPU), its
    gradients by autograd."""
    T, H, D = q.shape
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(kv, requires_grad=True)
    st = torch.tensor(sink, requires_grad=True)
    logits = scale * torch.einsum("thd,sd->ths", qt, kt)
    causal = torch.tril(torch.ones(T, T, dtype=torch.bool))
    logits = logits.masked_fill(~causal[:, None, :], float("-inf"))
    full = torch.cat([logits, st[None, :, None].expand(T, H, 1)], dim=2)
    w = torch.softmax(full, dim=2)[:, :, :T]
    out = torch.einsum("ths,sd->thd", w, kt[:, :dv])
    (out * torch.tensor(dout)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), st.grad.numpy()


def test_attention_backward_matches_autograd_of_dense_attention():
    rng = np.random.default_rng(71)
    T, H, D, dv = 9, 4, 8, 6
    q = rng.standard_normal((T, H, D))
    kv = rng.standard_normal((T, D))
    sink = rng.standard_normal(H)
    dout = rng.standard_normal((T, H, dv))
    scale = 0.29
    idx = _causal_full_indices(T, T)
    dq, dkv, ds = O.sparse_attention_backward(q, kv, idx, None, sink, scale, dout, dv)
    rq, rk, rs = _dense_torch_grads(q, kv, sink, scale, dout, dv)
    np.testing.assert_allclose(dq, rq, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dkv, rk, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ds, rs, rtol=1e-10, atol=1e-12)


def test_planted_backward_mistakes_fail_autograd():
    rng = np.random.default_rng(72)
    T, H, D, dv = 6, 2, 5, 3
    q = rng.standard_normal((T, H, D))
    kv = rng.standard_normal((T, D))
    sink = rng.standard_normal(H)
    dout = rng.standard_normal((T, H, dv))
    scale = 0.5
    idx = _causal_full_indices(T, T)
    rq, rk, rs = _dense_torch_grads(q, kv, sink, scale, dout, dv)
    # mistakes written as edits of the definition: no -D term, sink sign,
    # dv left out of the shared columns
    def mutant(kind):
        dq = np.zeros_like(q); dkv = np.zeros((T, D)); dsk = np.zeros(H)
        for t in range(T):
            ids = np.arange(t + 1)
            s = scale * (q[t] @ kv[ids].T)
            z = np.exp(s).sum(1, keepdims=True) + np.exp(sink)[:, None]
            P = np.exp(s) / z
            out = P @ kv[ids, :dv]
            dP = dout[t] @ kv[ids, :dv].T
            Dd = 0.0 if kind == "no_D" else (dout[t] * out).sum(1, keepdims=True)
            dS = P * (dP - Dd)
            dq[t] = scale * dS @ kv[ids]
            dkv[ids] += scale * dS.T @ q[t]
            if kind != "no_dv":
                dkv[ids, :dv] += P.T @ dout[t]
            psink = np.exp(sink) / z[:, 0]
            dsk += (1 if kind == "sink_sign" else -1) * psink * (dout[t] * out).sum(1)
        return dq, dkv, dsk
    for kind in ("no_D", "sink_sign", "no_dv"):
        dq, dkv, dsk = mutant(kind)
        assert not (np.allclose(dq, rq) and np.allclose(dkv, rk) and np.allclose(dsk, rs)), kind

