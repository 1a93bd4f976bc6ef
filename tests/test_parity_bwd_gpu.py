"""Parity of the sparse attention backward (dsa_sparse_attn_bwd) with the CPU
oracle's gradients (fp64, recomputed from the inputs).

The GPU path takes the forward kernel's own bf16 out and fp32 lse, rounds P
and dS to bf16 before the dq / dkv products and writes bf16 gradients, so
each gradient is compared with max-abs error <= 2e-2 * ||ref||_inf and a
relative Frobenius error <= 1e-2; d_sink (fp32, fixed-order sums) within
1e-3 * max(1, ||ref||_inf).
"""

import math

import numpy as np
import pytest
import torch

import deepseek_sparse_attention_dsa_amd as dsa
from gpu_helpers import DEV, f64, i64, say
from oracle import dsa_oracle as O
from workloads import make_custom

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    dsa.load_library()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _indices(T, kw, T_kv, rng, dup=True, invalid=True, active=None):
    idx = np.full((T, kw), -1, dtype=np.int32)
    tl = np.zeros(T, dtype=np.int32)
    for t in range(T):
        if active is not None and not active[t]:
            continue
        n = min(kw, t + 1, T_kv)
        c = np.sort(rng.choice(min(t + 1, T_kv), n, replace=False))
        idx[t, :n] = c
        tl[t] = n
        if dup and n >= 3 and t % 5 == 1:
            idx[t, n - 1] = idx[t, 0]          # duplicated slot
        if invalid and n >= 4 and t % 7 == 3:
            idx[t, 1] = T_kv + 9               # out-of-range id: invalid slot
    return idx, tl


def _check(name, got, ref, rel_max=2e-2, rel_fro=1e-2):
    g = got.astype(np.float64)
    scale = max(np.abs(ref).max(), 1e-30)
    err = np.abs(g - ref).max() / scale
    fro = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)
    say(f"  {name}: max {err:.2e} fro {fro:.2e}")
    assert err <= rel_max, (name, err)
    assert fro <= rel_fro, (name, fro)


def _run(T, H, D, kw, seed, sink=True, stress=False, use_tl=True, active=None, rows=None):
    wl = make_custom([T], H=H, D_qk=D, D_v=512, H_idx=0, seed=seed, device=DEV, sink=sink,
                     stress=stress, topk=kw)
    rng = np.random.default_rng(seed)
    idx, tl = _indices(T, kw, T, rng, active=active)
    idx_t = torch.from_numpy(idx).to(DEV)
    tl_t = torch.from_numpy(tl).to(DEV) if use_tl else None
    out, lse, _ = dsa.dsa_sparse_attn_fwd(wl.q, wl.kv, idx_t, topk_length=tl_t, attn_sink=wl.sink,
                                          softmax_scale=wl.scale, return_max_logits=False)
    g = torch.Generator(device=DEV).manual_seed(seed + 1)
    dout = (torch.randn((T, H, 512), generator=g, device=DEV) / math.sqrt(512)).to(torch.bfloat16)
    dq, dkv, ds = dsa.dsa_sparse_attn_bwd(wl.q, wl.kv, idx_t, out, dout, lse, topk_length=tl_t,
                                          attn_sink=wl.sink, softmax_scale=wl.scale)
    torch.cuda.synchronize()
    sk = None if wl.sink is None else f64(wl.sink)
    tl_ref = tl if use_tl else None
    rq, rk, rs = O.sparse_attention_backward(f64(wl.q), f64(wl.kv), idx.astype(np.int64), tl_ref,
                                             sk, wl.scale, f64(dout), 512, rows=rows)
    sel = np.arange(T) if rows is None else np.asarray(rows)
    _check("dq", f64(dq)[sel], rq[sel])
    _check("dkv", f64(dkv), rk)
    ds_np = ds.cpu().numpy().astype(np.float64)
    if sk is None:
        assert np.all(ds_np == 0.0)
    else:
        err = np.abs(ds_np - rs).max()
        say(f"  d_sink: max abs {err:.2e} (ref max {np.abs(rs).max():.2e})")
        assert err <= 1e-3 * max(1.0, np.abs(rs).max())


def _kv_tiles(T_kv, kw):
    """The library's choice of dkv scheme for these sizes (KV tiles or one
    dkv row per slot)."""
    return dsa.dsa_sparse_attn_bwd_kv_tiles(T_kv, kw)


SMALL = [
    # KV tiles
    (64, 16, 576, 32, True, False, True),
    (150, 64, 576, 64, True, True, True),
    (97, 33, 512, 40, False, False, True),
    (128, 128, 576, 96, True, True, False),
    (70, 64, 512, 33, True, True, True),
    (60, 80, 576, 48, True, False, True),
    (45, 96, 512, 40, True, True, True),
    (300, 64, 576, 40, True, False, True),   # several parts and tiles, a ragged last tile
    # one dkv row per slot
    (300, 64, 576, 32, True, True, True),
    (200, 33, 512, 24, True, False, True),
    (400, 128, 576, 40, True, True, False),
    (270, 96, 512, 33, False, False, True),
    (300, 16, 576, 32, True, False, True),   # one 32-head block: 32-head parts
    (260, 24, 512, 24, False, True, True),
]


def test_small_cases_cover_both_dkv_schemes():
    kinds = {_kv_tiles(T, kw) for T, _, _, kw, *_ in SMALL}
    assert kinds == {True, False}


def test_small_per_slot_cases_cover_every_head_block_count():
    """The per-slot dkv path at 1, 2, 3 and 4 blocks of 32 heads (head parts
    of 32 or 64 heads, one to three of them), at both D_qk."""
    blocks = {(-(-H // 32), D) for T, H, D, kw, *_ in SMALL if not _kv_tiles(T, kw)}
    assert {b for b, _ in blocks} == {1, 2, 3, 4}
    assert {D for _, D in blocks} == {512, 576}


@pytest.mark.parametrize("T,H,D,kw,sink,stress,use_tl", SMALL)
def test_backward_small(T, H, D, kw, sink, stress, use_tl):
    say("attention backward", T, H, D, kw, sink, stress, use_tl,
        "kv tiles" if _kv_tiles(T, kw) else "per-slot rows")
    _run(T, H, D, kw, seed=T + H, sink=sink, stress=stress, use_tl=use_tl)


def test_backward_full_size_sampled_rows():
    """T = 4096, 64 heads, K = 2048 (the single_T4096 shapes, KV tiles): only
    sampled rows carry slots, so dkv is the sum of their contributions alone
    and the oracle covers every output. The rows sit on both sides of the
    64-row part and 128-row tile edges."""
    T = 4096
    rows = [0, 1, 63, 64, 127, 128, 1000, 2047, 2048, 2049, 3000, 3071, 3072, 4031, 4095]
    active = np.zeros(T, dtype=bool)
    active[rows] = True
    say("attention backward, full size, rows", rows)
    _run(T, 64, 576, 2048, seed=7, stress=True, active=active, rows=rows)


def test_backward_empty_rows_and_no_slots():
    say("attention backward, empty rows")
    T, H = 40, 16
    wl = make_custom([T], H=H, D_qk=576, D_v=512, H_idx=0, seed=3, device=DEV)
    idx = torch.full((T, 32), -1, dtype=torch.int32, device=DEV)
    out, lse, _ = dsa.dsa_sparse_attn_fwd(wl.q, wl.kv, idx, attn_sink=wl.sink,
                                          softmax_scale=wl.scale)
    dout = torch.ones((T, H, 512), dtype=torch.bfloat16, device=DEV)
    dq, dkv, ds = dsa.dsa_sparse_attn_bwd(wl.q, wl.kv, idx, out, dout, lse, attn_sink=wl.sink,
                                          softmax_scale=wl.scale)
    torch.cuda.synchronize()
    assert torch.all(dq == 0) and torch.all(dkv == 0) and torch.all(ds == 0)


def test_backward_kv_beyond_2gib():
    """A latent KV spanning more than 2^31 bytes: the gathers then take 64-bit
    addresses instead of 32-bit buffer offsets. Ids above 2^31 / row bytes are
    drawn on purpose. The oracle sees the gathered rows only (remapped to a
    compact KV); every KV row no slot selects must get a zero gradient."""
    D, H, T_q, kw = 576, 64, 24, 64
    T_kv = (1 << 31) // (2 * D) + 40000
    say("attention backward, KV beyond 2 GiB", T_kv)
    gen = torch.Generator(device=DEV).manual_seed(21)
    kv = (torch.randn((T_kv, D), generator=gen, device=DEV) / math.sqrt(D)).to(torch.bfloat16)
    q = (torch.randn((T_q, H, D), generator=gen, device=DEV) / math.sqrt(D)).to(torch.bfloat16)
    sink = torch.randn((H,), generator=gen, device=DEV)
    rng = np.random.default_rng(8)
    lo = (1 << 31) // (2 * D) - 2000
    idx = np.empty((T_q, kw), dtype=np.int64)
    for t in range(T_q):
        idx[t] = np.sort(np.concatenate([rng.choice(np.arange(lo, T_kv), kw // 2, replace=False),
                                         rng.choice(lo, kw // 2, replace=False)]))
    idx[3, 5] = -1
    scale = 1.0 / math.sqrt(D)
    idx_t = torch.from_numpy(idx.astype(np.int32)).to(DEV)
    out, lse, _ = dsa.dsa_sparse_attn_fwd(q, kv, idx_t, attn_sink=sink, softmax_scale=scale,
                                          return_max_logits=False)
    dout = (torch.randn((T_q, H, 512), generator=gen, device=DEV) / math.sqrt(512)).to(torch.bfloat16)
    dq, dkv, ds = dsa.dsa_sparse_attn_bwd(q, kv, idx_t, out, dout, lse, attn_sink=sink,
                                          softmax_scale=scale)
    torch.cuda.synchronize()
    uniq = np.unique(idx[idx >= 0])
    remap = np.full(idx.shape, -1, dtype=np.int64)
    remap[idx >= 0] = np.searchsorted(uniq, idx[idx >= 0])
    ut = torch.from_numpy(uniq).to(DEV)
    touched = torch.zeros(T_kv, dtype=torch.bool, device=DEV)
    touched[ut] = True
    assert not torch.any(dkv[~touched] != 0), "a KV row no slot selects got a gradient"
    kv_small = kv[ut].contiguous()
    dkv_small = dkv[ut].contiguous()
    del kv, dkv
    rq, rk, rs = O.sparse_attention_backward(f64(q), f64(kv_small), remap, None, f64(sink), scale,
                                             f64(dout), 512)
    _check("dq", f64(dq), rq)
    _check("dkv", f64(dkv_small), rk)
    err = np.abs(ds.cpu().numpy().astype(np.float64) - rs).max()
    assert err <= 1e-3 * max(1.0, np.abs(rs).max())


@pytest.mark.parametrize("kw", [256, 64])
def test_backward_reproducible_and_chunked(kw):
    """No atomics decide a sum of dkv: the per-slot rows are summed per KV
    row in ascending slot order (a stable radix sort of the slots), the KV
    tiles' partials in ascending part order with repeated ids merged in
    ascending slot order. So repeated calls give identical bits, also with a
    workspace holding stale data; a workspace that holds only a few rows at a
    time (several chunks) stays within the oracle's tolerance. k_width 256
    takes KV tiles, 64 the per-slot rows (T_kv = 600 needs two 8-bit sort
    passes); most KV rows are selected by hundreds of rows and every fifth
    row repeats a slot."""
    T, H, D = 600, 64, 576
    assert _kv_tiles(T, kw) == (kw == 256)
    wl = make_custom([T], H=H, D_qk=D, D_v=512, H_idx=0, seed=31, device=DEV, sink=True,
                     topk=kw)
    rng = np.random.default_rng(31)
    idx, tl = _indices(T, kw, T, rng)
    idx_t = torch.from_numpy(idx).to(DEV)
    tl_t = torch.from_numpy(tl).to(DEV)
    out, lse, _ = dsa.dsa_sparse_attn_fwd(wl.q, wl.kv, idx_t, topk_length=tl_t, attn_sink=wl.sink,
                                          softmax_scale=wl.scale, return_max_logits=False)
    g = torch.Generator(device=DEV).manual_seed(32)
    dout = (torch.randn((T, H, 512), generator=g, device=DEV) / math.sqrt(512)).to(torch.bfloat16)
    need = dsa.dsa_sparse_attn_bwd_workspace_bytes(T, H, T, D, kw)
    runs = []
    for fill in (0, 0xA5, 0x3C):
        ws = torch.full((need,), fill, dtype=torch.uint8, device=DEV)
        runs.append(dsa.dsa_sparse_attn_bwd(wl.q, wl.kv, idx_t, out, dout, lse, topk_length=tl_t,
                                            attn_sink=wl.sink, softmax_scale=wl.scale,
                                            workspace=ws))
        torch.cuda.synchronize()
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(a, b)
    say("  three calls: identical dq, dkv, d_sink")
    # a workspace for about 37 rows: many chunks
    full = dsa.dsa_sparse_attn_bwd_workspace_bytes(37, H, T, D, kw)
    ws = torch.full((full,), 0x5A, dtype=torch.uint8, device=DEV)
    dq, dkv, ds = dsa.dsa_sparse_attn_bwd(wl.q, wl.kv, idx_t, out, dout, lse, topk_length=tl_t,
                                          attn_sink=wl.sink, softmax_scale=wl.scale, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(dq, runs[0][0])
    rq, rk, rs = O.sparse_attention_backward(f64(wl.q), f64(wl.kv), idx.astype(np.int64), tl,
                                             f64(wl.sink), wl.scale, f64(dout), 512)
    _check("dq", f64(dq), rq)
    _check("dkv", f64(dkv), rk)
    _check("dkv (one chunk)", f64(runs[0][1]), rk)
    err = np.abs(ds.cpu().numpy().astype(np.float64) - rs).max()
    assert err <= 1e-3 * max(1.0, np.abs(rs).max())
