"""Parity of the FP8 indexer (E4M3 with per-token descales or MXFP8 block
scales) through the C ABI against the CPU oracle on the same bytes.

Scores are within the indexer tolerance 1e-2 * ||row||_inf and an internal
1e-3 gate (the FP8 MFMA sums its exact E4M3 products at a precision of about
1e-4 of their absolute sum; the observed worst is below 1e-4 of the row
maximum); top-K on the GPU's FP8 scores is bit-exact against the oracle.
"""

import numpy as np
import pytest
import torch

import deepseek_sparse_attention_dsa_amd as dsa
from gpu_helpers import DEV, f64, i64, say
from oracle import dsa_oracle as O
from workloads import make_config, make_custom, make_split, quantize_fp8

pytestmark = pytest.mark.gpu

GATE = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    dsa.load_library()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _quant(q_idx, k_idx, scaling):
    block = 32 if scaling == dsa.DSA_MXFP8 else None
    q8, qs = quantize_fp8(q_idx, block)
    k8, ks = quantize_fp8(k_idx, block)
    return q8, qs, k8, ks


def _check(gpu_scores, q8, qs, k8, ks, w, rows, row_starts, seq_lens, scaling):
    rows = np.asarray(rows, dtype=np.int64)
    sel = torch.as_tensor(rows, device=q8.device)
    st = np.asarray(row_starts, dtype=np.int64)[rows]
    sl = np.asarray(seq_lens, dtype=np.int64)[rows]
    width = max(int(sl.max()), 1)
    fn = O.indexer_scores_fp8 if scaling == dsa.DSA_FP8_PER_TOKEN else O.indexer_scores_mxfp8
    ref = fn(i64(q8[sel]), f64(qs[sel]) if qs.dtype != torch.uint8 else i64(qs[sel]),
             i64(k8), f64(ks) if ks.dtype != torch.uint8 else i64(ks), f64(w[sel]), st, sl,
             np.arange(len(rows)), width=width)
    got = gpu_scores.detach().cpu().numpy().astype(np.float64)
    worst = 0.0
    for i in range(len(rows)):
        n = int(sl[i])
        if n == 0:
            continue
        scale = max(np.abs(ref[i, :n]).max(), 1e-30)
        err = np.abs(got[i, :n] - ref[i, :n]).max() / scale
        worst = max(worst, err)
        assert err <= 1e-2, (int(rows[i]), err)
        assert err <= GATE, (int(rows[i]), err)
    return worst


SCALINGS = [dsa.DSA_FP8_PER_TOKEN, dsa.DSA_MXFP8]


@pytest.mark.parametrize("scaling", SCALINGS, ids=["per_token", "mx"])
@pytest.mark.parametrize("doc_lens,H,wdt", [
    ([256], 64, torch.bfloat16),
    ([1, 70, 5, 130, 64], 64, torch.bfloat16),
    ([200, 9], 3, torch.float32),
    ([77, 300], 17, torch.float32),
    ([513], 32, torch.bfloat16),
    ([129], 33, torch.bfloat16),
])
def test_fp8_indexer_small(doc_lens, H, wdt, scaling):
    say("fp8 indexer", doc_lens, H, wdt, scaling)
    wl = make_custom(doc_lens, H=1, D_qk=256, D_v=256, H_idx=H, D_idx=128, seed=71, device=DEV)
    w = wl.w.float() if wdt == torch.float32 else wl.w
    q8, qs, k8, ks = _quant(wl.q_idx, wl.k_idx, scaling)
    rs, sl = dsa.dsa_packed_metadata(wl.cu_seqlens, wl.T)
    ld = (max(doc_lens) + 3) // 4 * 4 + 4
    buf = torch.full((wl.T, ld), float("nan"), device=DEV)
    dsa.dsa_indexer_fwd_fp8(q8, qs, k8, ks, w, rs, sl, scaling=scaling, scores=buf)
    torch.cuda.synchronize()
    err = _check(buf, q8, qs, k8, ks, w, np.arange(wl.T), i64(rs), i64(sl), scaling)
    say("  worst rel err", err)
    g = buf.cpu().numpy()
    sln = i64(sl)
    for t in range(wl.T):
        assert np.all(np.isnan(g[t, sln[t]:])), "columns past the mask must stay untouched"


@pytest.mark.parametrize("scaling", SCALINGS, ids=["per_token", "mx"])
def test_fp8_indexer_extreme_scales(scaling):
    """Rows and 32-blocks whose magnitudes differ by up to 2^20, and a zero row."""
    say("fp8 extreme scales", scaling)
    g = torch.Generator(device=DEV).manual_seed(5)
    T, H = 200, 64
    q = torch.randn((T, H, 128), generator=g, device=DEV)
    k = torch.randn((T, 128), generator=g, device=DEV)
    q = q * torch.exp2(torch.randint(-10, 11, (T, H, 1), generator=g, device=DEV).float())
    k = k * torch.exp2(torch.randint(-10, 11, (T, 1), generator=g, device=DEV).float())
    k = k * torch.exp2(torch.randint(-6, 7, (1, 4), generator=g, device=DEV).float()
                       ).repeat_interleave(32, dim=1)
    k[17] = 0.0
    w = torch.randn((T, H), generator=g, device=DEV).to(torch.bfloat16)
    q8, qs, k8, ks = _quant(q, k, scaling)
    cu = torch.tensor([0, T], dtype=torch.int32, device=DEV)
    rs, sl = dsa.dsa_packed_metadata(cu, T)
    sc = dsa.dsa_indexer_fwd_fp8(q8, qs, k8, ks, w, rs, sl, scaling=scaling, width=T)
    torch.cuda.synchronize()
    _check(sc, q8, qs, k8, ks, w, np.arange(T), i64(rs), i64(sl), scaling)


@pytest.mark.parametrize("scaling", SCALINGS, ids=["per_token", "mx"])
def test_fp8_indexer_ratio_causal(scaling):
    say("fp8 ratio-causal", scaling)
    wl = make_split([257, 0, 190], [70, 5, 48], [0, 3, 2000], 4, seed=73, device=DEV)
    q8, qs, k8, ks = _quant(wl.q_idx, wl.k_idx, scaling)
    rs, sl = dsa.dsa_ratio_causal_metadata(wl.cu_seqlens_q, wl.cu_seqlens_k, wl.T_q, wl.ratio,
                                           wl.q_causal_offsets)
    sc = dsa.dsa_indexer_fwd_fp8(q8, qs, k8, ks, wl.w, rs, sl, scaling=scaling, width=70)
    torch.cuda.synchronize()
    _check(sc, q8, qs, k8, ks, wl.w, np.arange(wl.T_q), i64(rs), i64(sl), scaling)


@pytest.mark.parametrize("scaling", SCALINGS, ids=["per_token", "mx"])
@pytest.mark.parametrize("cfg", [2, 4])
def test_fp8_indexer_topk_config(cfg, scaling):
    """The FP8 chain at the full sizes of the named workloads, on sampled rows."""
    say("fp8 chain config", cfg, scaling)
    wl = make_config(cfg, device=DEV)
    q8, qs, k8, ks = _quant(wl.q_idx, wl.k_idx, scaling)
    T, K = wl.T, wl.topk
    idx, tl = dsa.indexer_topk(q8, k8, wl.w, wl.cu_seqlens, K, max_seqlen=T, q_scale=qs,
                               k_scale=ks, fp8_scaling=scaling)
    rs, sl = dsa.dsa_packed_metadata(wl.cu_seqlens, T)
    torch.cuda.synchronize()
    rows = [0, 1, 2047, 2048, 2049, T // 2, T - 1]
    gi = i64(idx)
    for r in rows:
        sc = dsa.dsa_indexer_fwd_fp8(q8, qs, k8, ks, wl.w, rs, sl, scaling=scaling, row_begin=r,
                                     n_rows=1, width=T)
        torch.cuda.synchronize()
        _check(sc, q8, qs, k8, ks, wl.w, [r], i64(rs), i64(sl), scaling)
        ref_idx, ref_len = O.topk(sc.cpu().numpy().astype(np.float64), i64(sl)[[r]], K,
                                  row_starts=i64(rs)[[r]], n_cols=T)
        assert np.array_equal(gi[r], ref_idx[0]) and i64(tl)[r] == ref_len[0], r
    assert np.array_equal(i64(tl), np.minimum(np.arange(T) + 1, K))
