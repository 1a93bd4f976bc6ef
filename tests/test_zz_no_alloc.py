"""dsa_sparse_attn_bwd_noalloc (the backward on the library's own device
scratch, for callers that cannot allocate) against dsa_sparse_attn_bwd.

Both are called through the C ABI. Given a caller workspace of the scratch's
size, dsa_sparse_attn_bwd runs the same chunks of query rows, so the two must
agree bit for bit; the no-alloc results are also checked against the fp64
oracle (every row, since dkv sums over all of them). Two calls in a row, the second smaller and with other
head / dim / sink settings, so that the second runs on the first one's stale
scratch contents.
"""

import ctypes
import math

import numpy as np
import pytest
import torch

import deepseek_sparse_attention_dsa_amd as dsa
from gpu_helpers import DEV, f64, say
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


def _inputs(T, H, D, kw, seed, sink):
    wl = make_custom([T], H=H, D_qk=D, D_v=512, H_idx=0, seed=seed, device=DEV, sink=sink,
                     topk=kw)
    rng = np.random.default_rng(seed)
    idx = np.full((T, kw), -1, dtype=np.int32)
    tl = np.zeros(T, dtype=np.int32)
    for t in range(T):
        n = min(kw, t + 1)
        idx[t, :n] = np.sort(rng.choice(t + 1, n, replace=False))
        tl[t] = n
        if n >= 3 and t % 5 == 1:
            idx[t, n - 1] = idx[t, 0]          # duplicated slot
    idx_t = torch.from_numpy(idx).to(DEV)
    tl_t = torch.from_numpy(tl).to(DEV)
    out, lse, _ = dsa.dsa_sparse_attn_fwd(wl.q, wl.kv, idx_t, topk_length=tl_t, attn_sink=wl.sink,
                                          softmax_scale=wl.scale, return_max_logits=False)
    g = torch.Generator(device=DEV).manual_seed(seed + 1)
    dout = (torch.randn((T, H, 512), generator=g, device=DEV) / math.sqrt(512)).to(torch.bfloat16)
    return wl, idx, tl, idx_t, tl_t, out, lse, dout


def _call(lib, name, wl, idx_t, tl_t, out, lse, dout, workspace=None):
    T, H, D = wl.q.shape
    dq = torch.full_like(wl.q, float("nan"))
    dkv = torch.full((wl.kv.shape[0], D), float("nan"), dtype=torch.bfloat16, device=DEV)
    d_sink = torch.full((H,), float("nan"), dtype=torch.float32, device=DEV)
    p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    args = [p(wl.q), T, H, D, p(wl.kv), wl.kv.shape[0], wl.kv.stride(0), 512, p(idx_t),
            idx_t.stride(0), idx_t.shape[1], p(tl_t), p(wl.sink), ctypes.c_float(wl.scale),
            p(out), p(dout), p(lse), p(dq), p(dkv), p(d_sink)]
    if workspace is not None:
        args += [p(workspace), workspace.numel()]
    args.append(torch.cuda.current_stream().cuda_stream)
    rc = getattr(lib, name)(*args)
    assert rc == 0, (name, rc, lib.dsa_last_error().decode())
    return dq, dkv, d_sink


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _check_vs_oracle(wl, idx, tl, dout, dq, dkv, d_sink, rows):
    sk = None if wl.sink is None else f64(wl.sink)
    rq, rk, rs = O.sparse_attention_backward(f64(wl.q), f64(wl.kv), idx.astype(np.int64), tl, sk,
                                             wl.scale, f64(dout), 512, rows=rows)
    for name, got, ref in (("dq", f64(dq)[rows], rq[rows]), ("dkv", f64(dkv), rk)):
        scale = max(np.abs(ref).max(), 1e-30)
        err = np.abs(got - ref).max() / scale
        say(f"  {name} vs oracle: max {err:.2e}")
        assert err <= 2e-2, (name, err)


# first call: 1600 rows of up to 1024 slots at 32 heads, dkv by KV tiles, two
# chunks of query rows on the 256 MiB scratch (300 MB of buffers); second call:
# smaller, 16 heads, D_qk 512, no sink, dkv by per-slot rows
@pytest.mark.parametrize("calls", [[(1600, 32, 576, 1024, 41, True, True),
                                    (300, 16, 512, 32, 42, False, False)]])
def test_noalloc_matches_workspace_entry(calls):
    lib = dsa.load_library()
    ws = torch.empty(dsa.DSA_NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device=DEV)
    for (T, H, D, kw, seed, sink, tiles) in calls:
        assert dsa.dsa_sparse_attn_bwd_kv_tiles(T, kw) == tiles
        say("no-alloc backward", dict(T=T, H=H, D=D, kw=kw, sink=sink, kv_tiles=tiles))
        wl, idx, tl, idx_t, tl_t, out, lse, dout = _inputs(T, H, D, kw, seed, sink)
        a = _call(lib, "dsa_sparse_attn_bwd_noalloc", wl, idx_t, tl_t, out, lse, dout)
        b = _call(lib, "dsa_sparse_attn_bwd", wl, idx_t, tl_t, out, lse, dout, workspace=ws)
        torch.cuda.synchronize()
        for name, x, y in zip(("dq", "dkv", "d_sink"), a, b):
            assert torch.equal(_bits(x), _bits(y)), name
        # dkv sums over every row, so the oracle runs every row
        _check_vs_oracle(wl, idx, tl, dout, a[0], a[1], a[2], np.arange(T))
        if sink:
            assert torch.isfinite(a[2]).all()
        else:
            assert torch.all(a[2] == 0)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    lib = dsa.load_library()
    wl, idx, tl, idx_t, tl_t, out, lse, dout = _inputs(64, 16, 576, 64, 43, True)
    T, H, D = wl.q.shape
    p = lambda t: t.data_ptr()  # noqa: E731
    dq = torch.empty_like(wl.q)
    dkv = torch.empty((wl.kv.shape[0], D), dtype=torch.bfloat16, device=DEV)
    # a claimed key count whose fp32 dkv accumulator alone exceeds the scratch:
    # rejected on the host before anything is launched or read
    rc = lib.dsa_sparse_attn_bwd_noalloc(p(wl.q), T, H, D, p(wl.kv), 1 << 17, wl.kv.stride(0),
                                         512, p(idx_t), idx_t.stride(0), idx_t.shape[1], p(tl_t),
                                         None, ctypes.c_float(wl.scale), p(out), p(dout), p(lse),
                                         p(dq), p(dkv), None,
                                         torch.cuda.current_stream().cuda_stream)
    assert rc == dsa.DSA_ERR_VALUE
    assert "no-alloc scratch" in lib.dsa_last_error().decode()
