"""Parity of the batched block-routed GQA entry (sparse_gqa_attention) through
the C ABI against the CPU oracle: the layout of NeMo-QSA
`cudnn_sparse_gqa_attention` (query [B, S, H_q, 256], key / value [B, S, H_kv,
256], one route set per token shared by the KV heads, ids local to the batch
row), with the pages' head layouts (24, 2) and (12, 1): every (batch row, KV
head) group is compared with the oracle's attention over that group's query
heads, key and value rows. Tolerances are those of the other attention
parity tests (1e-2 absolute, 2e-2 of each row's largest output).
"""

import numpy as np
import pytest
import torch

import deepseek_sparse_attention_dsa_amd as dsa
from gpu_helpers import DEV, f64, say
from oracle import dsa_oracle as O
from workloads import qsa_routes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    dsa.load_library()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _inputs(B, S, H_q, H_kv, width, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = (torch.randn((B, S, H_q, 256), generator=g) / 16).to(torch.bfloat16)
    k = (torch.randn((B, S, H_kv, 256), generator=g) / 16).to(torch.bfloat16)
    v = (torch.randn((B, S, H_kv, 256), generator=g) / 16).to(torch.bfloat16)
    rng = np.random.default_rng(seed)
    ids = np.stack([qsa_routes([S], width, rng) for _ in range(B)])  # [B, S, width]
    return q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(ids).to(DEV)


def _compare(out, q, k, v, ids, scale):
    B, S, H_q, _ = q.shape
    H_kv = k.shape[2]
    G = H_q // H_kv
    o = f64(out)
    for b in range(B):
        idx = ids[b].cpu().numpy().astype(np.int64)
        for g in range(H_kv):
            ref, _, _ = O.sparse_attention(f64(q[b, :, G * g:G * (g + 1)]), f64(k[b, :, g]),
                                           f64(v[b, :, g]), idx, None, None, scale, d_v=256)
            got = o[b, :, G * g:G * (g + 1)]
            d = np.abs(got - ref)
            assert d.max() <= 1e-2, (b, g, d.max())
            row = np.abs(ref).max(axis=2, keepdims=True)
            rel = np.where(row > 0, d.max(axis=2, keepdims=True) / np.maximum(row, 1e-30),
                           d.max(axis=2, keepdims=True))
            assert rel.max() <= 2e-2, (b, g, rel.max())


@pytest.mark.parametrize("B,S,H_q,H_kv,width", [(2, 300, 24, 2, 64), (3, 257, 12, 1, 128)])
def test_batched_gqa_head_groups(B, S, H_q, H_kv, width):
    say("batched gqa", B, S, H_q, H_kv, width)
    q, k, v, ids = _inputs(B, S, H_q, H_kv, width, seed=B * 100 + H_q)
    out = dsa.sparse_gqa_attention(q, k, v, ids)
    torch.cuda.synchronize()
    assert out.shape == (B, S, H_q, 256) and out.dtype == torch.bfloat16
    _compare(out, q, k, v, ids, 1 / 16)


def test_batched_gqa_strided_int64_ids_and_scale():
    """Strided query / key views, int64 ids with out-of-range entries (including
    one that an int32 cast alone would wrap into range), an explicit scale;
    then the same call with int32 ids gives the same output bits."""
    say("batched gqa strided int64")
    B, S, H_q, H_kv, width = 2, 200, 24, 2, 32
    q, k, v, ids = _inputs(B, S, H_q, H_kv, width, seed=7)
    ids64 = ids.to(torch.int64)
    ids64[0, 5, 0] = S + 3
    ids64[1, 9, 1] = (1 << 32) + 4  # int32 narrowing alone would make this id 4
    ids64[1, 9, 2] = -7
    qs = q.transpose(2, 1).contiguous().transpose(2, 1)  # same values, strided view
    assert not qs.is_contiguous()
    out = dsa.sparse_gqa_attention(qs, k, v, ids64, softmax_scale=0.05)
    ref_ids = ids64.clone()
    ref_ids[(ref_ids < 0) | (ref_ids >= S)] = -1
    ids32 = ref_ids.to(torch.int32)
    out32 = dsa.sparse_gqa_attention(q, k, v, ids32, softmax_scale=0.05)
    torch.cuda.synchronize()
    assert torch.equal(out, out32)
    _compare(out, q, k, v, ids32, 0.05)
