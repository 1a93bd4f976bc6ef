"""Parity of the ratio-causal mask with query causal offsets (HIP vs oracle).

DSA page section 3: keys are a compressed prefix (one key per `ratio`
tokens) and each THD segment's queries carry their global token position.
Metadata is bit-exact; indexer scores are within 1e-2 * ||row||_inf (and the
tighter 1e-4 internal gate); top-K is bit-exact against the oracle run on the
GPU's own fp32 scores.
"""

import numpy as np
import pytest
import torch

import deepseek_sparse_attention_dsa_amd as dsa
from gpu_helpers import DEV, check_indexer, i64, say
from oracle import dsa_oracle as O
from workloads import make_split

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    dsa.load_library()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _meta(wl):
    return dsa.dsa_ratio_causal_metadata(wl.cu_seqlens_q, wl.cu_seqlens_k, wl.T_q, wl.ratio,
                                         wl.q_causal_offsets)


def _ref_meta(wl):
    off = None if wl.q_causal_offsets is None else i64(wl.q_causal_offsets)
    return O.ratio_causal_metadata(i64(wl.cu_seqlens_q), i64(wl.cu_seqlens_k), wl.T_q, wl.ratio,
                                   off)


# (q_lens, k_lens, offsets, ratio)
META_CASES = [
    ([300], [300], None, 1),
    ([257, 0, 190], [70, 5, 48], [0, 3, 2000], 4),
    ([129, 64, 7], [40, 33, 0], [-17, 60, 5], 3),
    ([1, 2, 3], [1, 1, 1], [0, 0, -1], 2),
    ([8192], [65536], [57344], 1),       # last rank of an 8-way split of T = 65536
    ([8192], [16384], [57344], 4),
]


@pytest.mark.parametrize("case", range(len(META_CASES)))
def test_ratio_metadata(case):
    q_lens, k_lens, off, ratio = META_CASES[case]
    say("ratio metadata", q_lens, k_lens, off, ratio)
    wl = make_split(q_lens, k_lens, off, ratio, H_idx=1, D_idx=64, seed=case, device=DEV)
    rs, sl = _meta(wl)
    st_ref, sl_ref = _ref_meta(wl)
    assert np.array_equal(i64(rs), st_ref) and np.array_equal(i64(sl), sl_ref)


def test_ratio_metadata_equals_packed_metadata():
    say("ratio metadata vs packed")
    cu = torch.tensor([0, 5, 5, 900, 1000], dtype=torch.int32, device=DEV)
    a = dsa.dsa_ratio_causal_metadata(cu, cu, 1000)
    b = dsa.dsa_packed_metadata(cu, 1000)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# (q_lens, k_lens, offsets, ratio, H_idx, D_idx)
IDX_CASES = [
    ([257, 0, 190], [70, 5, 48], [0, 3, 2000], 4, 64, 128),
    ([129, 64, 7], [40, 33, 0], [-17, 60, 5], 3, 17, 64),
    ([300, 200], [300, 200], [0, 100], 1, 64, 128),
    ([500], [130], [20], 4, 64, 128),
    ([65, 1], [1, 300], [0, 999], 1, 33, 128),
]


@pytest.mark.parametrize("case", range(len(IDX_CASES)))
def test_indexer_ratio_causal(case):
    q_lens, k_lens, off, ratio, H, D = IDX_CASES[case]
    say("indexer ratio-causal", q_lens, k_lens, off, ratio, H, D)
    wl = make_split(q_lens, k_lens, off, ratio, H_idx=H, D_idx=D, seed=20 + case, device=DEV)
    rs, sl = _meta(wl)
    width = max(max(k_lens), 1)
    ld = (width + 3) // 4 * 4 + 4
    buf = torch.full((wl.T_q, ld), float("nan"), device=DEV)
    dsa.dsa_indexer_fwd(wl.q_idx, wl.k_idx, wl.w, rs, sl, scores=buf)
    torch.cuda.synchronize()
    err = check_indexer(buf, wl, np.arange(wl.T_q), i64(rs), i64(sl))
    say("  worst rel err", err)
    g = buf.cpu().numpy()
    sln = i64(sl)
    for t in range(wl.T_q):
        assert np.all(np.isnan(g[t, sln[t]:])), "columns past the mask must stay untouched"


# (q_lens, k_lens, offsets, ratio, K)
CHAIN_CASES = [
    ([700, 300], [180, 80], [40, 1000], 4, 64),
    ([1500], [1500], [2600], 1, 1024),
    ([3000, 40], [2600, 10], [7000, 0], 3, 2048),
]


@pytest.mark.parametrize("case", range(len(CHAIN_CASES)))
def test_indexer_topk_ratio_chain(case):
    q_lens, k_lens, off, ratio, K = CHAIN_CASES[case]
    say("indexer+topk ratio-causal", q_lens, k_lens, off, ratio, K)
    wl = make_split(q_lens, k_lens, off, ratio, seed=40 + case, device=DEV)
    width = max(k_lens)
    idx, tl = dsa.indexer_topk(wl.q_idx, wl.k_idx, wl.w, wl.cu_seqlens_q, K,
                               cu_seqlens_k=wl.cu_seqlens_k, ratio=ratio,
                               q_causal_offsets=wl.q_causal_offsets, max_seqlen=width)
    rs, sl = _meta(wl)
    sc = dsa.dsa_indexer_fwd(wl.q_idx, wl.k_idx, wl.w, rs, sl, width=width)
    torch.cuda.synchronize()
    check_indexer(sc, wl, np.arange(wl.T_q), i64(rs), i64(sl))
    ref_idx, ref_len = O.topk(sc.cpu().numpy().astype(np.float64), i64(sl), K,
                              row_starts=i64(rs), n_cols=width)
    assert np.array_equal(i64(tl), ref_len)
    bad = np.nonzero(np.any(i64(idx) != ref_idx, axis=1))[0]
    assert len(bad) == 0, bad[:5]


@pytest.mark.parametrize("ratio", [1, 4])
def test_last_rank_of_eight_way_split(ratio):
    """One GPU's share of T = 65536 split 8 ways by query rows: the last 8192
    rows at causal offset 57344 against every (compressed) key."""
    T, Tq, K = 65536, 8192, 2048
    Tk = T // ratio
    say("rank share", Tq, Tk, ratio)
    wl = make_split([Tq], [Tk], [T - Tq], ratio, seed=60 + ratio, device=DEV)
    idx, tl = dsa.indexer_topk(wl.q_idx, wl.k_idx, wl.w, wl.cu_seqlens_q, K,
                               cu_seqlens_k=wl.cu_seqlens_k, ratio=ratio,
                               q_causal_offsets=wl.q_causal_offsets, max_seqlen=Tk)
    rs, sl = _meta(wl)
    torch.cuda.synchronize()
    st_ref, sl_ref = _ref_meta(wl)
    assert np.array_equal(i64(rs), st_ref) and np.array_equal(i64(sl), sl_ref)
    assert np.array_equal(i64(tl), np.minimum(sl_ref, K))
    rng = np.random.default_rng(ratio)
    rows = sorted(set([0, 1, 2, 3, 4095, Tq - 2, Tq - 1] + rng.integers(0, Tq, 3).tolist()))
    gi = i64(idx)
    for r in rows:
        sc = dsa.dsa_indexer_fwd(wl.q_idx, wl.k_idx, wl.w, rs, sl, row_begin=int(r), n_rows=1,
                                 width=Tk)
        torch.cuda.synchronize()
        check_indexer(sc, wl, [r], i64(rs), i64(sl))
        ref_idx, _ = O.topk(sc.cpu().numpy().astype(np.float64), sl_ref[r:r + 1], K,
                            row_starts=st_ref[r:r + 1], n_cols=Tk)
        assert np.array_equal(gi[r], ref_idx[0]), r


@pytest.mark.parametrize("ratio,scaling", [(1, "mx"), (4, "per_token")])
def test_last_rank_fp8_candidate_path(ratio, scaling):
    """The same rank share from FP8 indexer inputs: indexer_topk takes the
    combined candidate path for these long rows; sampled rows against the
    oracle's top-K on the standalone FP8 scores."""
    from workloads import quantize_fp8
    T, Tq, K = 65536, 8192, 2048
    Tk = T // ratio
    say("rank share fp8", Tq, Tk, ratio, scaling)
    wl = make_split([Tq], [Tk], [T - Tq], ratio, seed=70 + ratio, device=DEV)
    block = 32 if scaling == "mx" else None
    q8, qs = quantize_fp8(wl.q_idx, block)
    k8, ks = quantize_fp8(wl.k_idx, block)
    mode = dsa.DSA_MXFP8 if scaling == "mx" else dsa.DSA_FP8_PER_TOKEN
    idx, tl = dsa.indexer_topk(q8, k8, wl.w, wl.cu_seqlens_q, K, cu_seqlens_k=wl.cu_seqlens_k,
                               ratio=ratio, q_causal_offsets=wl.q_causal_offsets, max_seqlen=Tk,
                               q_scale=qs, k_scale=ks, fp8_scaling=mode)
    rs, sl = _meta(wl)
    torch.cuda.synchronize()
    st_ref, sl_ref = _ref_meta(wl)
    assert np.array_equal(i64(tl), np.minimum(sl_ref, K))
    rng = np.random.default_rng(10 + ratio)
    rows = sorted(set([0, 1, 2047, 2048, 4095, Tq - 2, Tq - 1] + rng.integers(0, Tq, 5).tolist()))
    gi = i64(idx)
    for r in rows:
        sc = dsa.dsa_indexer_fwd_fp8(q8, qs, k8, ks, wl.w, rs, sl, scaling=mode, row_begin=int(r),
                                     n_rows=1, width=Tk)
        torch.cuda.synchronize()
        ref_idx, _ = O.topk(sc.cpu().numpy().astype(np.float64), sl_ref[r:r + 1], K,
                            row_starts=st_ref[r:r + 1], n_cols=Tk)
        assert np.array_equal(gi[r], ref_idx[0]), r


@pytest.mark.parametrize("cfg", [6, 7])
def test_split_config_sampled(cfg):
    """The split-query / compressed-key workloads as the bench runs them:
    chained indexer + top-K, then attention over the selected global rows."""
    from workloads import CONFIGS, make_config
    from gpu_helpers import check_attention
    say("config", cfg)
    wl = make_config(cfg, device=DEV)
    width = max(CONFIGS[cfg]["k_lens"])
    K = wl.topk
    idx, tl = dsa.indexer_topk(wl.q_idx, wl.k_idx, wl.w, wl.cu_seqlens_q, K,
                               cu_seqlens_k=wl.cu_seqlens_k, ratio=wl.ratio,
                               q_causal_offsets=wl.q_causal_offsets, max_seqlen=width)
    out, lse, mx = dsa.dsa_sparse_attn_fwd(wl.q, wl.kv, idx, topk_length=tl, attn_sink=wl.sink,
                                           softmax_scale=wl.scale)
    rs, sl = _meta(wl)
    torch.cuda.synchronize()
    st_ref, sl_ref = _ref_meta(wl)
    assert np.array_equal(i64(rs), st_ref) and np.array_equal(i64(sl), sl_ref)
    T = wl.T_q
    rows = np.array(sorted({0, 1, 2, 3, 5, T // 2, T - 2, T - 1}))
    gi = i64(idx)
    for r in rows:
        sc = dsa.dsa_indexer_fwd(wl.q_idx, wl.k_idx, wl.w, rs, sl, row_begin=int(r), n_rows=1,
                                 width=width)
        torch.cuda.synchronize()
        check_indexer(sc, wl, [r], i64(rs), i64(sl))
        ref_idx, _ = O.topk(sc.cpu().numpy().astype(np.float64), sl_ref[r:r + 1], K,
                            row_starts=st_ref[r:r + 1], n_cols=width)
        assert np.array_equal(gi[r], ref_idx[0]), r
    check_attention(out, lse, mx, wl.q, wl.kv, None, idx, tl, wl.sink, wl.scale, wl.D_v, rows)
    # whole-tensor properties at full size
    tln = i64(tl)
    assert np.array_equal(tln, np.minimum(sl_ref, K))
    valid = gi >= 0
    assert np.array_equal(valid.sum(1), tln)
    assert np.all(np.where(valid, gi < (st_ref + sl_ref)[:, None], True))
    assert np.all(np.diff(np.where(valid, gi, np.iinfo(np.int32).max), axis=1) >= 0)
    fin = tln > 0
    assert torch.isfinite(lse[torch.as_tensor(fin, device=DEV)]).all()
