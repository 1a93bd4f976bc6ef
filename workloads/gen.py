"""Seeded synthetic workloads for the DSA forward path.

Shapes and value distributions follow the five workloads the pages' kernels are
sized for: GLM-style sparse MLA (576-dim latent+rope queries over one shared
576-dim KV row, 512-dim values) with a 64-head x 128-dim lightning indexer and
K = 2048, and the 12-head x 256-dim block-routed sparse GQA of the Qwen3 QSA
page. Every tensor is N(0, 1)/sqrt(last dim) in fp32, rounded to bf16 (RNE),
except the sink (N(0, 1) fp32) and the QSA tensors (N(0, 1)/16).

Tensors are drawn with a torch Generator on the requested device in a fixed
order: q, kv (or k, v), q_idx, k_idx, w, sink. Document lengths and QSA routes
come from a numpy Generator seeded from the same seed (drawn first, since the
token count depends on them). Nothing here evaluates the method.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

# Workloads, in the order the bench and parity tests refer to them.
CONFIGS = {
    1: dict(name="tiny_T256", doc_lens=[256], H=16, D_qk=576, D_v=512, shared_kv=True,
            H_idx=4, D_idx=64, topk=64, scale=1.0 / math.sqrt(576), sink=True),
    2: dict(name="single_T4096", doc_lens=[4096], H=64, D_qk=576, D_v=512, shared_kv=True,
            H_idx=64, D_idx=128, topk=2048, scale=1.0 / math.sqrt(576), sink=True),
    3: dict(name="packed8_U512_4096_H128", doc_lens=None, n_docs=8, doc_len_range=(512, 4096),
            H=128, D_qk=576, D_v=512, shared_kv=True,
            H_idx=64, D_idx=128, topk=2048, scale=1.0 / math.sqrt(576), sink=True),
    4: dict(name="long_T65536", doc_lens=[65536], H=64, D_qk=576, D_v=512, shared_kv=True,
            H_idx=64, D_idx=128, topk=2048, scale=1.0 / math.sqrt(576), sink=True),
    5: dict(name="qsa_B4x8192_H12_D256", doc_lens=[8192] * 4, H=12, D_qk=256, D_v=256,
            shared_kv=False, H_idx=0, D_idx=0, topk=512, scale=1.0 / 16.0, sink=False,
            qsa=True, value_std=1.0 / 16.0),
    # One GPU's share of T = 65536 split 8 ways by query rows: the last 8192
    # rows (global offset 57344) against all 65536 keys (ratio-causal mask
    # with query causal offsets, ratio 1).
    6: dict(name="cp8_last_rank_T65536", split=True, q_lens=[8192], k_lens=[65536],
            offsets=[57344], ratio=1, H=64, D_qk=576, D_v=512, H_idx=64, D_idx=128, topk=2048),
    # Compressed keys: T = 65536 queries over 16384 keys, one key per 4 tokens,
    # top-512 (the DSA page's ratio-4 indexer example).
    7: dict(name="ratio4_T65536_K512", split=True, q_lens=[65536], k_lens=[16384],
            offsets=None, ratio=4, H=64, D_qk=576, D_v=512, H_idx=64, D_idx=128, topk=512),
    # Workloads 2 and 4 with FP8 indexer inputs (same seeds and bf16 values,
    # quantised by quantize_fp8): E8M0 block scales, or fp32 per-token descales.
    8: dict(name="single_T4096_mxfp8", base=2, indexer_fp8="mx"),
    9: dict(name="long_T65536_mxfp8", base=4, indexer_fp8="mx"),
    10: dict(name="long_T65536_fp8_per_token", base=4, indexer_fp8="per_token"),
}


@dataclass
class Workload:
    name: str
    T: int
    doc_lens: List[int]
    cu_seqlens: torch.Tensor          # int32 [n_docs+1]
    H: int
    D_qk: int
    D_v: int
    shared_kv: bool
    q: torch.Tensor                   # bf16 [T, H, D_qk]
    kv: torch.Tensor                  # bf16 [T, D_qk]  (K rows; V = kv[:, :D_v] when shared)
    v: Optional[torch.Tensor]         # bf16 [T, D_v] when K/V are separate
    H_idx: int
    D_idx: int
    q_idx: Optional[torch.Tensor]     # bf16 [T, H_idx, D_idx]
    k_idx: Optional[torch.Tensor]     # bf16 [T, D_idx]
    w: Optional[torch.Tensor]         # bf16 [T, H_idx]
    sink: Optional[torch.Tensor]      # fp32 [H]
    topk: int
    scale: float
    routes: Optional[torch.Tensor] = None   # int32 [T, W] (block-routed GQA only)
    seed: int = 0
    stress: bool = False
    extra: dict = field(default_factory=dict)


def bf16_to_numpy_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 bit patterns as a numpy uint16 array (host copy)."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _randn(gen, shape, std, device):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return (x * std).to(torch.bfloat16)


def qsa_routes(doc_lens: List[int], width: int, rng: np.random.Generator,
               max_blocks: Optional[int] = None) -> np.ndarray:
    """Four-token block routes for block-routed sparse GQA.

    For the token at position p of a document, the row holds up to
    (width/4 - 1) distinct complete causal blocks chosen uniformly without
    replacement from blocks 0..p//4-1 (ascending, four ids each), then the
    causal tail group [4*(p//4) .. p] padded with -1 to four slots, then -1
    groups up to `width`. Ids are packed coordinates (document origin + local).
    """
    assert width % 4 == 0 and width >= 4
    groups = width // 4
    max_blocks = groups - 1 if max_blocks is None else max_blocks
    T = int(sum(doc_lens))
    out = np.full((T, width), -1, dtype=np.int32)
    origin = 0
    for L in doc_lens:
        for c0 in range(0, L, 1024):
            p = np.arange(c0, min(L, c0 + 1024))
            nb = p // 4
            m = np.minimum(nb, max_blocks)
            nmax = int(nb.max()) if len(nb) else 0
            if nmax > 0:
                keys = rng.random((len(p), nmax))
                keys[np.arange(nmax)[None, :] >= nb[:, None]] = np.inf
                order = np.argsort(keys, axis=1, kind="stable")
            for r, pos in enumerate(p):
                row = out[origin + pos]
                mm = int(m[r])
                if mm > 0:
                    blocks = np.sort(order[r, :mm])
                    ids = (blocks[:, None] * 4 + np.arange(4)[None, :]).reshape(-1)
                    row[: 4 * mm] = origin + ids
                tail = np.arange(4 * nb[r], pos + 1)
                row[4 * mm: 4 * mm + len(tail)] = origin + tail
        origin += L
    return out


def make_custom(doc_lens, H, D_qk, D_v, shared_kv=True, H_idx=4, D_idx=64, topk=64,
                scale=None, sink=True, seed=0, device="cpu", routes_width=None,
                stress=False, value_std=None, name="custom"):
    """Build a workload of any shape with the same recipe as the named configs."""
    doc_lens = [int(x) for x in doc_lens]
    T = int(sum(doc_lens))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(doc_lens)]).astype(np.int32))
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    std_qk = value_std if value_std is not None else 1.0 / math.sqrt(D_qk)
    std_v = value_std if value_std is not None else 1.0 / math.sqrt(D_v)
    scale = (1.0 / math.sqrt(D_qk)) if scale is None else float(scale)
    q = _randn(gen, (T, H, D_qk), std_qk, device)
    kv = _randn(gen, (T, D_qk), std_qk, device)
    v = None if shared_kv else _randn(gen, (T, D_v), std_v, device)
    q_idx = k_idx = w = None
    if H_idx > 0:
        q_idx = _randn(gen, (T, H_idx, D_idx), 1.0 / math.sqrt(D_idx), device)
        k_idx = _randn(gen, (T, D_idx), 1.0 / math.sqrt(D_idx), device)
        w = _randn(gen, (T, H_idx), 1.0 / math.sqrt(H_idx), device)
    sk = None
    if sink:
        sk = torch.randn((H,), generator=gen, device=device, dtype=torch.float32)
    if stress:
        # Scaled attention logits with std ~4 instead of ~1/D (softmax far from
        # uniform), and sinks of the same order as the log-sum-exp.
        fac = 4.0 / (scale * math.sqrt(D_qk) * std_qk * std_qk)
        q = (q.float() * fac).to(torch.bfloat16)
        if sk is not None:
            sk = sk * 2.0 + 4.0 * math.sqrt(2.0 * math.log(max(topk, 2)))
    routes = None
    if routes_width is not None:
        rng = np.random.default_rng(int(seed) + 7)
        routes = torch.from_numpy(qsa_routes(doc_lens, routes_width, rng)).to(device)
    return Workload(name=name, T=T, doc_lens=doc_lens, cu_seqlens=cu.to(device), H=H,
                    D_qk=D_qk, D_v=D_v, shared_kv=shared_kv, q=q, kv=kv, v=v, H_idx=H_idx,
                    D_idx=D_idx, q_idx=q_idx, k_idx=k_idx, w=w, sink=sk, topk=topk,
                    scale=scale, routes=routes, seed=int(seed), stress=stress)


def config_doc_lens(i: int, seed=None) -> List[int]:
    """Document lengths of a named packed workload (drawn before any tensor)."""
    c = CONFIGS[i]
    seed = 1000 + i if seed is None else int(seed)
    if c.get("doc_lens") is None:
        lo, hi = c["doc_len_range"]
        rng = np.random.default_rng(seed)
        return [int(x) for x in rng.integers(lo, hi, size=c["n_docs"], endpoint=True)]
    return list(c["doc_lens"])


def make_config(i: int, device="cpu", seed=None, stress=False):
    """One of the named workloads (a Workload, or a SplitWorkload for the
    split-query / compressed-key ones); seed defaults to 1000 + i."""
    c = dict(CONFIGS[i])
    if c.get("indexer_fp8"):
        wl = make_config(c["base"], device=device, seed=seed, stress=stress)
        wl.name = c["name"] + ("_stress" if stress else "")
        block = 32 if c["indexer_fp8"] == "mx" else None
        q8, qs = quantize_fp8(wl.q_idx, block)
        k8, ks = quantize_fp8(wl.k_idx, block)
        wl.extra["fp8"] = dict(scaling=c["indexer_fp8"], q8=q8, q_scale=qs, k8=k8, k_scale=ks)
        return wl
    seed = 1000 + i if seed is None else int(seed)
    if c.get("split"):
        assert not stress
        return make_split(c["q_lens"], c["k_lens"], c["offsets"], c["ratio"], H_idx=c["H_idx"],
                          D_idx=c["D_idx"], H=c["H"], D_qk=c["D_qk"], D_v=c["D_v"],
                          topk=c["topk"], seed=seed, device=device, name=c["name"])
    doc_lens = config_doc_lens(i, seed)
    wl = make_custom(doc_lens, c["H"], c["D_qk"], c["D_v"], shared_kv=c["shared_kv"],
                     H_idx=c["H_idx"], D_idx=c["D_idx"], topk=c["topk"], scale=c["scale"],
                     sink=c["sink"], seed=seed, device=device,
                     routes_width=c["topk"] if c.get("qsa") else None, stress=stress,
                     value_std=c.get("value_std"), name=c["name"] + ("_stress" if stress else ""))
    return wl


@dataclass
class SplitWorkload:
    """Queries and keys stored as THD segments of their own (ratio-causal mask).

    Segment b stores q_lens[b] query rows and k_lens[b] (compressed) key rows;
    offsets[b] is the global token position of its first query.
    """
    name: str
    T_q: int
    T_kv: int
    cu_seqlens_q: torch.Tensor        # int32 [n_seq+1]
    cu_seqlens_k: torch.Tensor        # int32 [n_seq+1]
    q_causal_offsets: Optional[torch.Tensor]  # int32 [n_seq] or None
    ratio: int
    H: int
    D_qk: int
    D_v: int
    q: Optional[torch.Tensor]         # bf16 [T_q, H, D_qk]
    kv: Optional[torch.Tensor]        # bf16 [T_kv, D_qk], V = kv[:, :D_v]
    H_idx: int
    D_idx: int
    q_idx: torch.Tensor               # bf16 [T_q, H_idx, D_idx]
    k_idx: torch.Tensor               # bf16 [T_kv, D_idx]
    w: torch.Tensor                   # bf16 [T_q, H_idx]
    sink: Optional[torch.Tensor]      # fp32 [H]
    topk: int
    scale: float
    seed: int = 0
    v: Optional[torch.Tensor] = None  # values are always kv[:, :D_v] here
    extra: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return self.T_q


def make_split(q_lens, k_lens, offsets, ratio, H_idx=64, D_idx=128, H=0, D_qk=576, D_v=512,
               topk=2048, seed=0, device="cpu", name="split"):
    """Split-query / compressed-key workload with the named configs' recipe.

    Draw order: q and kv (when H > 0), q_idx, k_idx, w, sink.
    """
    q_lens = [int(x) for x in q_lens]
    k_lens = [int(x) for x in k_lens]
    assert len(q_lens) == len(k_lens)
    T_q, T_kv = int(sum(q_lens)), int(sum(k_lens))
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32))
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum(k_lens)]).astype(np.int32))
    off = None if offsets is None else torch.tensor(np.asarray(offsets, dtype=np.int32))
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    q = kv = sk = None
    if H > 0:
        q = _randn(gen, (T_q, H, D_qk), 1.0 / math.sqrt(D_qk), device)
        kv = _randn(gen, (T_kv, D_qk), 1.0 / math.sqrt(D_qk), device)
    q_idx = _randn(gen, (T_q, H_idx, D_idx), 1.0 / math.sqrt(D_idx), device)
    k_idx = _randn(gen, (T_kv, D_idx), 1.0 / math.sqrt(D_idx), device)
    w = _randn(gen, (T_q, H_idx), 1.0 / math.sqrt(H_idx), device)
    if H > 0:
        sk = torch.randn((H,), generator=gen, device=device, dtype=torch.float32)
    return SplitWorkload(name=name, T_q=T_q, T_kv=T_kv, cu_seqlens_q=cu_q.to(device),
                         cu_seqlens_k=cu_k.to(device),
                         q_causal_offsets=None if off is None else off.to(device), ratio=int(ratio),
                         H=H, D_qk=D_qk, D_v=D_v, q=q, kv=kv, H_idx=H_idx, D_idx=D_idx,
                         q_idx=q_idx, k_idx=k_idx, w=w, sink=sk, topk=int(topk),
                         scale=1.0 / math.sqrt(D_qk), seed=int(seed))


def quantize_fp8(x: torch.Tensor, block: Optional[int] = None):
    """E4M3 bytes and scales of x (bf16/fp32 [..., D]) through torch's float8 casts.

    block None: one fp32 descale per row of the last dim, amax / 448 (1.0 for
    an all-zero row). block 32: one E8M0 byte per 32 elements, the smallest
    power of two 2^e >= amax / 448 (code e + 127). Returns (uint8 codes,
    scales): scales fp32 [...] or uint8 [..., D / block].
    """
    xf = x.float()
    if block is None:
        amax = xf.abs().amax(dim=-1)
        scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        q = (xf / scale[..., None]).to(torch.float8_e4m3fn).view(torch.uint8)
        return q, scale
    xb = xf.reshape(*xf.shape[:-1], -1, block)
    amax = xb.abs().amax(dim=-1)
    e = torch.ceil(torch.log2(torch.clamp(amax / 448.0, min=2.0 ** -127))).clamp(-127, 127)
    q = (xb / torch.exp2(e)[..., None]).to(torch.float8_e4m3fn).view(torch.uint8)
    return q.reshape(x.shape), (e + 127).to(torch.uint8)
