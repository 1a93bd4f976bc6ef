"""Parity of the combined indexer + top-K launch (dsa_indexer_topk_fused).

The combined kernels compute every score with the same arithmetic as the
standalone indexer kernels, so their selection is compared bit-exactly with
the oracle's top-K on the standalone kernels' scores, their logits equal those
scores exactly, and softmax / LSE are within 1e-5 of the oracle's (fp64 on
the same logits).
"""

import numpy as np
import pytest
import torch

import deepseek_sparse_attention_dsa_amd as dsa
from gpu_helpers import DEV, i64, say
from oracle import dsa_oracle as O
from workloads import make_config, make_custom, make_split, quantize_fp8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    dsa.load_library()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _compare(fused, scores, seq_lens, row_starts, k, n_cols):
    idx, tl, logits, soft, lse = fused
    sc = scores.cpu().numpy().astype(np.float64)
    ref_idx, ref_len, ref_logit, ref_soft, ref_lse = O.topk_softmax(
        sc, i64(seq_lens), k, row_starts=i64(row_starts), n_cols=n_cols)
    gi = i64(idx)
    bad = np.nonzero(np.any(gi != ref_idx, axis=1))[0]
    assert len(bad) == 0, (bad[:5], gi[bad[:1]], ref_idx[bad[:1]])
    assert np.array_equal(i64(tl), ref_len)
    if logits is not None:
        gl = logits.cpu().numpy().astype(np.float64)
        assert np.array_equal(gl, ref_logit), "logits must be the selected scores"
    if soft is not None:
        gs = soft.cpu().numpy().astype(np.float64)
        assert np.abs(gs - ref_soft).max() <= 1e-5, np.abs(gs - ref_soft).max()
    if lse is not None:
        gz = lse.cpu().numpy().astype(np.float64)
        empty = np.isinf(ref_lse)
        assert np.array_equal(np.isinf(gz) & (gz > 0), empty)
        assert np.abs(gz[~empty] - ref_lse[~empty]).max(initial=0.0) <= 1e-5


def _fused(wl_q, wl_k, w, rs, sl, k, n_cols, **kw):
    return dsa.dsa_indexer_topk_fused(wl_q, wl_k, w, rs, sl, k, n_cols, return_logits=True,
                                      return_softmax=True, return_lse=True, **kw)


@pytest.mark.parametrize("doc_lens,H,D,wdt,k", [
    ([256], 4, 64, torch.bfloat16, 64),
    ([1, 70, 5, 130, 64], 64, 128, torch.bfloat16, 7),
    ([200, 9], 3, 128, torch.float32, 64),
    ([77, 300], 17, 64, torch.float32, 1),
    ([513, 1000], 64, 128, torch.bfloat16, 2048),
    ([4096], 64, 128, torch.bfloat16, 2048),
    ([2500, 1596], 33, 128, torch.bfloat16, 100),
])
def test_fused_bf16(doc_lens, H, D, wdt, k):
    say("fused bf16", doc_lens, H, D, wdt, k)
    wl = make_custom(doc_lens, H=1, D_qk=256, D_v=256, H_idx=H, D_idx=D, seed=91, device=DEV)
    w = wl.w.float() if wdt == torch.float32 else wl.w
    rs, sl = dsa.dsa_packed_metadata(wl.cu_seqlens, wl.T)
    n_cols = max(doc_lens)
    fused = _fused(wl.q_idx, wl.k_idx, w, rs, sl, k, n_cols)
    sc = dsa.dsa_indexer_fwd(wl.q_idx, wl.k_idx, w, rs, sl, width=n_cols)
    torch.cuda.synchronize()
    _compare(fused, sc, sl, rs, k, n_cols)


@pytest.mark.parametrize("scaling", [dsa.DSA_FP8_PER_TOKEN, dsa.DSA_MXFP8], ids=["per_token", "mx"])
@pytest.mark.parametrize("doc_lens,H,k", [([1, 70, 5, 130, 64], 64, 7), ([4096], 64, 2048),
                                          ([777, 300], 17, 64)])
def test_fused_fp8(doc_lens, H, k, scaling):
    say("fused fp8", doc_lens, H, k, scaling)
    wl = make_custom(doc_lens, H=1, D_qk=256, D_v=256, H_idx=H, D_idx=128, seed=92, device=DEV)
    block = 32 if scaling == dsa.DSA_MXFP8 else None
    q8, qs = quantize_fp8(wl.q_idx, block)
    k8, ks = quantize_fp8(wl.k_idx, block)
    rs, sl = dsa.dsa_packed_metadata(wl.cu_seqlens, wl.T)
    n_cols = max(doc_lens)
    fused = _fused(q8, k8, wl.w, rs, sl, k, n_cols, q_scale=qs, k_scale=ks, fp8_scaling=scaling)
    sc = dsa.dsa_indexer_fwd_fp8(q8, qs, k8, ks, wl.w, rs, sl, scaling=scaling, width=n_cols)
    torch.cuda.synchronize()
    _compare(fused, sc, sl, rs, k, n_cols)


def test_fused_ratio_causal_and_chunks():
    say("fused ratio-causal")
    wl = make_split([700, 300, 9], [180, 80, 0], [40, 1000, 3], 4, seed=93, device=DEV)
    rs, sl = dsa.dsa_ratio_causal_metadata(wl.cu_seqlens_q, wl.cu_seqlens_k, wl.T_q, wl.ratio,
                                           wl.q_causal_offsets)
    k = 64
    n_cols = 180
    r0, n = 311, 600
    idx = torch.full((n, k + 3), 7, dtype=torch.int32, device=DEV)
    fused = dsa.dsa_indexer_topk_fused(wl.q_idx, wl.k_idx, wl.w, rs, sl, k, n_cols, row_begin=r0,
                                       n_rows=n, indices=idx[:, :k], return_logits=True,
                                       return_softmax=True, return_lse=True)
    sc = dsa.dsa_indexer_fwd(wl.q_idx, wl.k_idx, wl.w, rs, sl, row_begin=r0, n_rows=n,
                             width=n_cols)
    torch.cuda.synchronize()
    _compare(fused, sc, sl[r0:r0 + n], rs[r0:r0 + n], k, n_cols)
    assert torch.all(idx[:, k:] == 7), "columns past k of the index rows stay untouched"


def test_fused_column_cap_and_empty_keys():
    say("fused n_cols cap, T_kv = 0")
    wl = make_custom([900], H=1, D_qk=256, D_v=256, H_idx=64, D_idx=128, seed=94, device=DEV)
    rs, sl = dsa.dsa_packed_metadata(wl.cu_seqlens, wl.T)
    k, cap = 50, 333  # rows longer than 333 columns are taken as 333 long
    fused = _fused(wl.q_idx, wl.k_idx, wl.w, rs, sl, k, cap)
    sc = dsa.dsa_indexer_fwd(wl.q_idx, wl.k_idx, wl.w, rs, sl, width=900)
    torch.cuda.synchronize()
    _compare(fused, sc[:, :336], torch.clamp(sl, max=cap), rs, k, cap)
    # no keys at all: every row is empty
    empty_k = wl.k_idx[:0]
    idx, tl, lg, so, lse = _fused(wl.q_idx, empty_k, wl.w, rs, sl, k, 100)
    torch.cuda.synchronize()
    assert torch.all(idx == -1) and torch.all(tl == 0)
    assert torch.all(lg == -float("inf")) and torch.all(so == 0) and torch.all(lse == float("inf"))


@pytest.mark.parametrize("cfg", [1, 2, 8])
def test_fused_chain_matches_two_kernel_path(cfg):
    """indexer_topk at full workload size: the combined launch and the
    score-chunk path give identical selections."""
    say("fused chain config", cfg)
    wl = make_config(cfg, device=DEV)
    fp8 = wl.extra.get("fp8")
    kw = {}
    q, kk = wl.q_idx, wl.k_idx
    if fp8:
        q, kk = fp8["q8"], fp8["k8"]
        kw = dict(q_scale=fp8["q_scale"], k_scale=fp8["k_scale"],
                  fp8_scaling=dsa.DSA_MXFP8 if fp8["scaling"] == "mx" else dsa.DSA_FP8_PER_TOKEN)
    a = dsa.indexer_topk(q, kk, wl.w, wl.cu_seqlens, wl.topk, max_seqlen=max(wl.doc_lens),
                         fused=True, return_softmax=True, **kw)
    b = dsa.indexer_topk(q, kk, wl.w, wl.cu_seqlens, wl.topk, max_seqlen=max(wl.doc_lens),
                         fused=False, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    soft = a[3]
    sums = soft.double().sum(1)
    assert torch.allclose(sums[a[1] > 0], torch.ones_like(sums[a[1] > 0]), atol=1e-4)
