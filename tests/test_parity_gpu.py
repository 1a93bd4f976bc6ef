"""Parity of the HIP path (through the C ABI) against the CPU oracle.

Small shapes are compared element by element; the named workloads at full
size are compared on sampled rows (every row the oracle can afford) plus
whole-tensor properties. Top-K is bit-exact against the oracle run on the
GPU's own fp32 scores; indexer scores are within 1e-2 * ||row||_inf (and a
tighter 1e-4 internal gate); attention out within 1e-2 max-abs plus a per-row
2e-2 relative gate, lse within 1e-3.
"""

import math

import numpy as np
import pytest
import torch

import deepseek_sparse_attention_dsa_amd as dsa
from gpu_helpers import DEV, check_attention, check_indexer, f64, i64, say
from oracle import dsa_oracle as O
from workloads import make_config, make_custom

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    dsa.load_library()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _meta(wl):
    rs, sl = dsa.dsa_packed_metadata(wl.cu_seqlens, wl.T)
    return rs, sl


# ------------------------------------------------------------------ metadata

@pytest.mark.parametrize("doc_lens", [[256], [3, 4], [1, 0, 7, 0, 0, 300, 2], [4096] * 3])
def test_metadata(doc_lens):
    cu = np.concatenate([[0], np.cumsum(doc_lens)]).astype(np.int32)
    T = int(cu[-1])
    say("metadata", doc_lens)
    rs, sl = dsa.dsa_packed_metadata(torch.from_numpy(cu).to(DEV), T)
    st_ref, sl_ref = O.packed_metadata(cu, T)
    assert np.array_equal(i64(rs), st_ref) and np.array_equal(i64(sl), sl_ref)


# ------------------------------------------------------------------- indexer

@pytest.mark.parametrize("doc_lens,H,D,wdt", [
    ([256], 4, 64, torch.bfloat16),
    ([1, 70, 5, 130, 64], 64, 128, torch.bfloat16),
    ([200, 9], 3, 128, torch.float32),
    ([77, 300], 17, 64, torch.float32),
    ([513], 64, 128, torch.float32),
])
def test_indexer_small(doc_lens, H, D, wdt):
    say("indexer", doc_lens, H, D, wdt)
    wl = make_custom(doc_lens, H=1, D_qk=256, D_v=256, H_idx=H, D_idx=D, seed=11, device=DEV)
    if wdt == torch.float32:
        wl.w = wl.w.float()  # exact widening; the oracle reads the same values
    rs, sl = _meta(wl)
    sc = dsa.dsa_indexer_fwd(wl.q_idx, wl.k_idx, wl.w, rs, sl, width=max(doc_lens))
    torch.cuda.synchronize()
    err = check_indexer(sc, wl, np.arange(wl.T), i64(rs), i64(sl))
    say("  worst rel err", err)


@pytest.mark.parametrize("wdt", [torch.bfloat16, torch.float32])
def test_indexer_weights_at_any_offset(wdt):
    # W views at a storage offset that breaks the four-weight alignment take
    # the one-weight loads; the scores are the same bits as from aligned W
    say("indexer W offset", wdt)
    wl = make_custom([300, 190], H=1, D_qk=256, D_v=256, H_idx=64, D_idx=128, seed=13, device=DEV)
    w = wl.w.to(wdt)
    base = torch.empty(w.numel() + 1, dtype=wdt, device=DEV)
    base[1:].copy_(w.reshape(-1))
    w_off = base[1:].view(w.shape)
    assert w_off.data_ptr() % (4 * w_off.element_size()) != 0
    rs, sl = _meta(wl)
    a = dsa.dsa_indexer_fwd(wl.q_idx, wl.k_idx, w, rs, sl, width=300)
    b = dsa.dsa_indexer_fwd(wl.q_idx, wl.k_idx, w_off, rs, sl, width=300)
    torch.cuda.synchronize()
    sln = i64(sl)
    ga, gb = a.cpu().numpy(), b.cpu().numpy()
    for t in range(wl.T):
        assert np.array_equal(ga[t, :sln[t]].view(np.uint32), gb[t, :sln[t]].view(np.uint32)), t
    wl.w = w
    check_indexer(b, wl, np.arange(wl.T), i64(rs), sln)


def test_indexer_chunk_offsets_and_untouched_columns():
    say("indexer chunk offsets")
    wl = make_custom([150, 333], H=1, D_qk=256, D_v=256, H_idx=64, D_idx=128, seed=5, device=DEV)
    rs, sl = _meta(wl)
    ld = 400
    r0, n = 97, 190
    buf = torch.full((n, ld), float("nan"), device=DEV)
    dsa.dsa_indexer_fwd(wl.q_idx, wl.k_idx, wl.w, rs, sl, row_begin=r0, n_rows=n, scores=buf)
    torch.cuda.synchronize()
    rows = np.arange(r0, r0 + n)
    check_indexer(buf, wl, rows, i64(rs), i64(sl))
    g = buf.cpu().numpy()
    sln = i64(sl)[rows]
    for i in range(n):
        assert np.all(np.isfinite(g[i, :sln[i]]))
        assert np.all(np.isnan(g[i, sln[i]:])), "columns past seq_len must stay untouched"


# --------------------------------------------------------------------- top-K

def _topk_check(scores: torch.Tensor, seq_lens: torch.Tensor, k: int, row_starts=None,
                n_cols=None):
    """Bit-exact top-K on both output paths of dsa_topk.

    Without values the kernels stage the selected slots in LDS and write them
    with 16-byte stores (and rows of at most k columns take the 16-byte closed
    form): the path the pipeline uses. With values they write slot by slot.
    Both calls write into buffers pre-filled with a sentinel, so an unwritten
    slot shows up, and both are compared with the oracle on the same scores.
    """
    n_rows = scores.shape[0]
    sc = scores.detach().cpu().numpy()
    st = None if row_starts is None else i64(row_starts)
    ref_idx, ref_len = O.topk(sc.astype(np.float64), i64(seq_lens), k, row_starts=st,
                              n_cols=n_cols)
    res = {}
    for with_values in (False, True):
        idx = torch.full((n_rows, k), 0x7F7F7F7F, dtype=torch.int32, device=DEV)
        tl = torch.full((n_rows,), -7, dtype=torch.int32, device=DEV)
        _, _, vals = dsa.dsa_topk(scores, seq_lens, k, row_starts=row_starts, n_cols=n_cols,
                                  indices=idx, topk_length=tl, return_values=with_values)
        torch.cuda.synchronize()
        gi, gl = i64(idx), i64(tl)
        bad = np.nonzero(np.any(gi != ref_idx, axis=1))[0]
        assert len(bad) == 0, (with_values, bad[:5], gi[bad[:1]], ref_idx[bad[:1]])
        assert np.array_equal(gl, ref_len), with_values
        res[with_values] = (idx, tl)
        if not with_values:
            continue
        # values: the selected scores (-0.0 may come back as +0.0), -inf padding
        gv = vals.cpu().numpy().astype(np.float64)
        for r in range(n_rows):
            m = ref_len[r]
            loc = ref_idx[r, :m] - (0 if st is None else st[r])
            assert np.array_equal(gv[r, :m], sc[r, loc].astype(np.float64))
            assert np.all(gv[r, m:] == -np.inf)
    return res[False]


@pytest.mark.parametrize("n_cols", [100, 256, 1000, 4096, 5000, 16384, 20000, 40000, 65536])
@pytest.mark.parametrize("kind", ["gauss", "ties"])
def test_topk_synthetic(n_cols, kind):
    say("topk", n_cols, kind)
    g = torch.Generator().manual_seed(n_cols + (7 if kind == "ties" else 0))
    n_rows = 24 if n_cols > 16384 else 64
    x = torch.randn((n_rows, n_cols), generator=g)
    if kind == "ties":
        x = torch.round(x * 4) / 4          # heavy exact ties, incl. 0.0
        neg = torch.rand((n_rows, n_cols), generator=g) < 0.5
        x = torch.where((x == 0) & neg, torch.full_like(x, -0.0), x)
    ld = (n_cols + 3) // 4 * 4 + (4 if n_cols % 3 == 0 else 0)
    buf = torch.zeros((n_rows, ld))
    buf[:, :n_cols] = x
    for k in ([1, 7, 64, 2048] if n_cols >= 2048 else [1, 7, 64]):
        lens = torch.randint(0, n_cols + 1, (n_rows,), generator=g)
        lens[0] = n_cols
        lens[1] = min(k, n_cols)
        lens[2] = min(k + 1, n_cols)
        lens[3] = max(k - 1, 0)
        lens[4] = 0
        lens[5] = n_cols + 100          # clamped to n_cols
        starts = torch.randint(0, 1 << 20, (n_rows,), generator=g).to(torch.int32)
        _topk_check(buf.to(DEV), lens.to(torch.int32).to(DEV), k,
                    row_starts=starts.to(DEV) if k != 7 else None, n_cols=n_cols)


@pytest.mark.parametrize("n_cols", [200, 1000, 3000, 6000, 12000])
def test_topk_special_rows(n_cols):
    say("topk special rows", n_cols)
    k = 64
    rows = []
    rows.append(np.full(n_cols, 0.25))                       # all equal -> first K
    rows.append(np.arange(n_cols, dtype=np.float64))         # increasing -> last K
    rows.append(-np.arange(n_cols, dtype=np.float64))        # decreasing -> first K
    r = np.zeros(n_cols)
    r[::2] = -0.0
    rows.append(r)                                           # +-0 ties -> first K
    r = np.full(n_cols, -np.inf)
    r[100:110] = 1.0
    rows.append(r)                                           # -inf is a value
    r = np.random.default_rng(0).standard_normal(n_cols)
    r[r < 1.5] = 1.5                                         # huge tie at the boundary
    rows.append(r)
    r = np.random.default_rng(1).standard_normal(n_cols)
    r[[5, 17, n_cols - 1]] = np.inf                          # +inf scores
    rows.append(r)
    one_up = float(np.nextafter(np.float32(1.0), np.float32(2.0)))
    rows.append(np.where(np.arange(n_cols) % 3 == 0, one_up, 1.0))  # span of one ulp
    r = np.random.default_rng(2).standard_normal(n_cols)
    low = r < 2.5                                            # the boundary falls inside it
    r[low] = 1.0 + np.float32(2.0 ** -20) * np.cumsum(low)[low]     # dense distinct cluster
    rows.append(r)
    x = torch.tensor(np.stack(rows), dtype=torch.float32)
    lens = torch.full((len(rows),), n_cols, dtype=torch.int32)
    idx, _ = _topk_check(x.to(DEV), lens.to(DEV), k)
    gi = i64(idx)
    assert gi[0].tolist() == list(range(k))
    assert gi[1].tolist() == list(range(n_cols - k, n_cols))
    assert gi[2].tolist() == list(range(k))
    assert gi[3].tolist() == list(range(k))


@pytest.mark.parametrize("n_cols", [65536, 20000])
def test_topk_adversarial_sample_rows(n_cols):
    """Rows built against the kernel's sample of long rows (64 runs of 64
    columns, run q starting at (q * (n - 64) // 63) rounded down to a multiple
    of 4): the sampled lower bound then either admits fewer than K keys or
    more than the candidate list holds, and the radix passes that re-stream
    the row must take over. The oracle is independent of all this."""
    say("topk adversarial sample rows", n_cols)
    k = 2048
    starts = ((np.arange(64) * (n_cols - 64)) // 63) & ~3
    samp = np.unique((starts[:, None] + np.arange(64)[None, :]).ravel())
    rng = np.random.default_rng(n_cols)
    rows = []
    r = -1.0 - rng.random(n_cols)
    r[samp] = 1.0 + rng.random(len(samp))           # only the samples are large
    rows.append(r)
    r = 1.0 + rng.random(n_cols)
    r[samp] = -1.0 - rng.random(len(samp))          # the samples are the smallest
    rows.append(r)
    r = np.round(1.0 + rng.random(n_cols), 1)       # ... with heavy ties
    r[samp] = -1.0
    rows.append(r)
    r = rng.standard_normal(n_cols)                 # ordinary row (candidate path)
    rows.append(r)
    x = torch.tensor(np.stack(rows), dtype=torch.float32)
    lens = torch.full((len(rows),), n_cols, dtype=torch.int32)
    starts = torch.arange(len(rows), dtype=torch.int32) * 1000
    _topk_check(x.to(DEV), lens.to(DEV), k, row_starts=starts.to(DEV), n_cols=n_cols)


# ----------------------------------------------------------------- attention

def _attn_case(T_kv, T_q, H, Dqk, Dv, shared, kw, seed, tl_mode="none", sink=True,
               stress=False, dup=False):
    g = np.random.default_rng(seed)
    wl = make_custom([max(T_q, T_kv)], H=H, D_qk=Dqk, D_v=Dv, shared_kv=shared, H_idx=0,
                     sink=sink, seed=seed, device=DEV, stress=stress, topk=kw,
                     value_std=(1 / 16 if Dqk == 256 else None))
    q = wl.q[:T_q].contiguous()
    kv = wl.kv[:T_kv].contiguous()
    v = None if shared else wl.v[:T_kv].contiguous()
    idx = g.integers(0, T_kv, size=(T_q, kw)).astype(np.int32)
    if not dup:
        for t in range(T_q):
            idx[t] = g.permutation(T_kv)[:kw] if kw <= T_kv else idx[t]
    # sprinkle invalid slots: -1, negative and out-of-range ids
    m = g.random((T_q, kw))
    idx[m < 0.05] = -1
    idx[(m >= 0.05) & (m < 0.07)] = T_kv + 3
    idx[(m >= 0.07) & (m < 0.08)] = -5
    tl = None
    if tl_mode == "prefix":
        tl = g.integers(-3, kw + 5, size=T_q).astype(np.int32)
        tl[0] = 0
        tl[1] = kw
    return wl, q, kv, v, torch.from_numpy(idx).to(DEV), \
        (None if tl is None else torch.from_numpy(tl).to(DEV))


@pytest.mark.parametrize("Dqk,Dv,shared,H,kw,tl_mode,sink,stress", [
    (576, 512, True, 16, 64, "none", True, False),
    (576, 512, True, 64, 100, "prefix", True, False),
    (576, 512, True, 64, 37, "none", False, True),
    (576, 512, True, 128, 96, "prefix", True, True),
    (576, 512, True, 20, 33, "none", True, True),
    (576, 512, True, 1, 5, "none", True, False),
    (512, 512, True, 64, 70, "prefix", True, True),
    (256, 256, False, 12, 64, "none", False, False),
    (256, 256, False, 12, 129, "prefix", False, True),
    (256, 256, True, 24, 40, "none", True, True),
    (256, 256, False, 128, 32, "none", True, False),
])
def test_attention_small(Dqk, Dv, shared, H, kw, tl_mode, sink, stress):
    say("attention", Dqk, Dv, shared, H, kw, tl_mode, sink, stress)
    T_kv, T_q = 300, 41
    wl, q, kv, v, idx, tl = _attn_case(T_kv, T_q, H, Dqk, Dv, shared, kw, seed=H * 7 + kw,
                                       tl_mode=tl_mode, sink=sink, stress=stress,
                                       dup=(kw == 37))
    sk = wl.sink
    out, lse, mx = dsa.dsa_sparse_attn_fwd(q, kv, idx, topk_length=tl, attn_sink=sk,
                                           softmax_scale=wl.scale, v=v, d_v=Dv)
    torch.cuda.synchronize()
    e_out, e_rel = check_attention(out, lse, mx, q, kv, v, idx, tl, sk, wl.scale, Dv,
                                   np.arange(T_q))
    say("  max|dout|", e_out, "row rel", e_rel)


def test_attention_edge_rows():
    say("attention edge rows")
    H, Dqk, Dv, kw, T_kv = 64, 576, 512, 48, 80
    wl = make_custom([T_kv], H=H, D_qk=Dqk, D_v=Dv, H_idx=0, seed=3, device=DEV, stress=True)
    q = wl.q[:8].contiguous()
    kv = wl.kv
    idx = np.full((8, kw), -1, dtype=np.int32)
    idx[1, :3] = [5, 5, 5]                       # one key three times
    idx[2, :] = np.arange(kw)                    # all valid, compact
    idx[3, 10] = 7                               # a single valid slot deep in the row
    idx[4, :] = T_kv + np.arange(kw)             # all out of range -> empty
    idx[5, ::2] = np.arange(kw // 2)             # interleaved -1
    idx[6, :] = np.arange(kw)                    # topk_length clamps below
    idx[7, :] = np.arange(kw)                    # topk_length 0 -> empty
    tl = np.array([kw, kw, kw, kw, kw, kw, 5, 0], dtype=np.int32)
    idx_t = torch.from_numpy(idx).to(DEV)
    tl_t = torch.from_numpy(tl).to(DEV)
    for sink in (None, wl.sink):
        out, lse, mx = dsa.dsa_sparse_attn_fwd(q, kv, idx_t, topk_length=tl_t, attn_sink=sink,
                                               softmax_scale=wl.scale)
        torch.cuda.synchronize()
        check_attention(out, lse, mx, q, kv, None, idx_t, tl_t, sink, wl.scale, Dv,
                        np.arange(8))
        l = lse.cpu().numpy()
        assert np.all(np.isposinf(l[[0, 4, 7]]))
        assert np.all(out[[0, 4, 7]].float().cpu().numpy() == 0)
    # k_width = 0: every row is empty
    out, lse, mx = dsa.dsa_sparse_attn_fwd(q, kv, idx_t[:, :0].contiguous(), softmax_scale=0.1)
    torch.cuda.synchronize()
    assert torch.all(torch.isposinf(lse)) and torch.all(out == 0)
    assert torch.all(torch.isneginf(mx))


def test_attention_reference_paths():
    """First valid key late in the row, and logits far above the first tile's max."""
    say("attention reference paths")
    H, T_kv, kw = 64, 200, 160
    wl = make_custom([T_kv], H=H, D_qk=576, D_v=512, H_idx=0, seed=17, device=DEV)
    kv = wl.kv.clone()
    q = wl.q[:4].clone()
    # keys 100..199 get a large component along dim 0; q rows 2, 3 point at it
    kv[100:, 0] = 32.0
    q[2:, :, 0] = 64.0  # logit gap ~ 2048 * scale = 85 nats = 123 log2 units
    idx = np.full((4, kw), -1, dtype=np.int32)
    idx[0, 50] = 3                               # first valid key in the 2nd tile
    idx[0, 120:125] = [7, 8, 9, 10, 11]
    idx[1, 40:] = np.arange(kw - 40)             # leading invalid tile
    idx[2, :] = np.arange(kw)                    # keys 0..99 small, 100..159 huge
    idx[3, :100] = np.arange(100)                # huge key appears only in the last tile
    idx[3, 150] = 150
    idx_t = torch.from_numpy(idx).to(DEV)
    for sink in (None, wl.sink):
        out, lse, mx = dsa.dsa_sparse_attn_fwd(q, kv, idx_t, attn_sink=sink,
                                               softmax_scale=wl.scale)
        torch.cuda.synchronize()
        # V dim 0 is 32 for keys >= 100, so outputs reach ~32 where one bf16 ulp
        # is 0.25: the absolute bound scales with that, the per-row relative
        # gate stays at 2e-2.
        check_attention(out, lse, mx, q, kv, None, idx_t, None, sink, wl.scale, 512,
                        np.arange(4), atol_out=0.1)


@pytest.mark.parametrize("H,kw,tl_mode,sink,stress,dup", [
    (12, 512, "none", False, False, False),
    (16, 96, "prefix", True, True, False),
    (1, 33, "none", True, False, False),
    (5, 200, "prefix", False, True, False),
    (13, 47, "none", True, True, True),
    (16, 1, "none", False, False, False),
])
def test_gqa_one_wave_per_row(H, kw, tl_mode, sink, stress, dup):
    """The block-routed GQA form (D 256, separate V, at most 16 heads) runs on
    its own one-wave-per-row kernel: head counts 1..16, widths that are not
    multiples of the 32-slot tile, sinks, topk_length prefixes, duplicates."""
    say("gqa", H, kw, tl_mode, sink, stress, dup)
    T_kv, T_q = 700, 37
    wl, q, kv, v, idx, tl = _attn_case(T_kv, T_q, H, 256, 256, False, kw, seed=H * 11 + kw,
                                       tl_mode=tl_mode, sink=sink, stress=stress, dup=dup)
    out, lse, mx = dsa.dsa_sparse_attn_fwd(q, kv, idx, topk_length=tl, attn_sink=wl.sink,
                                           softmax_scale=wl.scale, v=v, d_v=256)
    torch.cuda.synchronize()
    check_attention(out, lse, mx, q, kv, v, idx, tl, wl.sink, wl.scale, 256, np.arange(T_q))


def test_gqa_edge_rows_and_reference_paths():
    """Empty rows (all ids invalid, topk_length 0, k_width 0), a single valid
    slot deep in the row, the first valid key in a later tile, and logits far
    above the first tile's max (the row runs again with its exact max)."""
    say("gqa edge rows")
    H, T_kv, kw = 12, 300, 160
    wl = make_custom([T_kv], H=H, D_qk=256, D_v=256, shared_kv=False, H_idx=0, seed=21,
                     device=DEV, value_std=1 / 16)
    k = wl.kv.clone()
    v = wl.v.clone()
    q = wl.q[:8].clone()
    k[100:, 0] = 32.0
    q[6:, :, 0] = 64.0  # scaled logits ~ 2048 / 16 = 128 above the others (> 2^64 in exp2)
    idx = np.full((8, kw), -1, dtype=np.int32)
    idx[1, 70] = 9                               # one valid slot in the third tile
    idx[2, :] = T_kv + np.arange(kw)             # every id out of range: empty
    idx[3, 40:] = np.arange(kw - 40)             # first valid key in the second tile
    idx[4, ::3] = np.arange(0, kw, 3)            # interleaved -1
    idx[5, :] = np.arange(kw)                    # topk_length 0: empty
    idx[6, :] = np.arange(kw)                    # keys 100.. huge from tile 4 on
    idx[7, :100] = np.arange(100)                # the huge key only in the last tile
    idx[7, 150] = 150
    tl = np.full(8, kw, dtype=np.int32)
    tl[5] = 0
    idx_t = torch.from_numpy(idx).to(DEV)
    tl_t = torch.from_numpy(tl).to(DEV)
    sink = torch.randn((H,), generator=torch.Generator(device=DEV).manual_seed(4), device=DEV)
    for sk in (None, sink):
        out, lse, mx = dsa.dsa_sparse_attn_fwd(q, k, idx_t, topk_length=tl_t, attn_sink=sk,
                                               softmax_scale=1 / 16, v=v, d_v=256)
        torch.cuda.synchronize()
        check_attention(out, lse, mx, q, k, v, idx_t, tl_t, sk, 1 / 16, 256, np.arange(8))
        l = lse.cpu().numpy()
        assert np.all(np.isposinf(l[[0, 2, 5]]))
        assert np.all(out[[0, 2, 5]].float().cpu().numpy() == 0)
    out, lse, mx = dsa.dsa_sparse_attn_fwd(q, k, idx_t[:, :0].contiguous(), softmax_scale=0.1,
                                           v=v, d_v=256)
    torch.cuda.synchronize()
    assert torch.all(torch.isposinf(lse)) and torch.all(out == 0)
    assert torch.all(torch.isneginf(mx))


def test_attention_dense_identity_on_gpu():
    """Top-K covering every causal key and no sink == dense causal attention."""
    say("attention dense identity")
    T, H = 96, 16
    wl = make_custom([T], H=H, D_qk=576, D_v=512, H_idx=0, sink=False, seed=9, device=DEV,
                     stress=True)
    idx = np.full((T, T), -1, dtype=np.int32)
    for t in range(T):
        idx[t, : t + 1] = np.arange(t + 1)
    out, lse, _ = dsa.dsa_sparse_attn_fwd(wl.q, wl.kv, torch.from_numpy(idx).to(DEV),
                                          softmax_scale=wl.scale)
    torch.cuda.synchronize()
    qf = wl.q.float().cpu().double().permute(1, 0, 2)
    kf = wl.kv.float().cpu().double()
    ref = torch.nn.functional.scaled_dot_product_attention(
        qf, kf.expand(H, T, 576), kf[:, :512].expand(H, T, 512), is_causal=True,
        scale=wl.scale).permute(1, 0, 2).numpy()
    got = out.float().cpu().double().numpy()
    assert np.abs(got - ref).max() <= 2e-2 * np.abs(ref).max()


@pytest.mark.parametrize("shared", [True, False])
def test_attention_kv_beyond_2gib(shared):
    """K (and V) spanning more than 2^31 bytes: the kernel then gathers through
    64-bit addresses instead of 32-bit buffer offsets. Ids above 2^31 / row
    bytes are drawn on purpose. The oracle sees only the gathered rows (the
    attention of a row depends on nothing else), remapped to a compact KV."""
    Dqk, Dv, H = (576, 512, 64) if shared else (256, 256, 12)
    T_kv = (1 << 31) // (2 * Dqk) + 40000
    say("attention KV beyond 2 GiB", shared, T_kv)
    gen = torch.Generator(device=DEV).manual_seed(11)
    kv = torch.randn((T_kv, Dqk), generator=gen, device=DEV, dtype=torch.float32)
    kv = (kv / math.sqrt(Dqk)).to(torch.bfloat16)
    v = None
    if not shared:
        v = (torch.randn((T_kv, Dv), generator=gen, device=DEV) / math.sqrt(Dv)).to(torch.bfloat16)
    T_q, kw = 24, 96
    q = (torch.randn((T_q, H, Dqk), generator=gen, device=DEV) / math.sqrt(Dqk)).to(torch.bfloat16)
    g = np.random.default_rng(5)
    lo = (1 << 31) // (2 * Dqk) - 2000
    idx = np.where(g.random((T_q, kw)) < 0.5, g.integers(lo, T_kv, size=(T_q, kw)),
                   g.integers(0, T_kv, size=(T_q, kw))).astype(np.int64)
    idx[g.random((T_q, kw)) < 0.05] = -1
    idx[0, :4] = [T_kv - 1, 0, T_kv - 1, -1]
    scale = 1.0 / math.sqrt(Dqk)
    sink = torch.randn((H,), generator=gen, device=DEV)
    out, lse, mx = dsa.dsa_sparse_attn_fwd(q, kv, torch.from_numpy(idx.astype(np.int32)).to(DEV),
                                           attn_sink=sink, softmax_scale=scale, v=v, d_v=Dv)
    torch.cuda.synchronize()
    uniq = np.unique(idx[idx >= 0])
    remap = np.full(idx.shape, -1, dtype=np.int32)
    remap[idx >= 0] = np.searchsorted(uniq, idx[idx >= 0])
    ut = torch.from_numpy(uniq).to(DEV)
    kv_small = kv[ut].contiguous()
    v_small = None if v is None else v[ut].contiguous()
    del kv, v
    check_attention(out, lse, mx, q, kv_small, v_small, torch.from_numpy(remap).to(DEV), None,
                    sink, scale, Dv, np.arange(T_q))


# ------------------------------------------------------- named workloads

def _assert_topk_is_oracle(idx, tl, scores, seq_lens, k, row_starts, n_cols=None):
    """The selection a pipeline used equals the oracle's on the same fp32 scores."""
    ref_idx, ref_len = O.topk(scores.detach().cpu().numpy().astype(np.float64), i64(seq_lens), k,
                              row_starts=i64(row_starts), n_cols=n_cols)
    gi = i64(idx)
    bad = np.nonzero(np.any(gi != ref_idx, axis=1))[0]
    assert len(bad) == 0, (bad[:5], gi[bad[:1]], ref_idx[bad[:1]])
    assert np.array_equal(i64(tl), ref_len)


def _pipeline(wl, max_seqlen=None, fused=None):
    idx, tl = dsa.indexer_topk(wl.q_idx, wl.k_idx, wl.w, wl.cu_seqlens, wl.topk,
                               max_seqlen=max_seqlen, fused=fused)[:2]
    out, lse, mx = dsa.dsa_sparse_attn_fwd(wl.q, wl.kv, idx, topk_length=tl, attn_sink=wl.sink,
                                           softmax_scale=wl.scale)
    return idx, tl, out, lse, mx


def test_config1_full():
    say("config 1 full")
    wl = make_config(1, device=DEV)
    rs, sl = _meta(wl)
    sc = dsa.dsa_indexer_fwd(wl.q_idx, wl.k_idx, wl.w, rs, sl, width=wl.T)
    idx, tl, vals = dsa.dsa_topk(sc, sl, wl.topk, row_starts=rs)
    out, lse, mx = dsa.dsa_sparse_attn_fwd(wl.q, wl.kv, idx, topk_length=tl, attn_sink=wl.sink,
                                           softmax_scale=wl.scale)
    torch.cuda.synchronize()
    check_indexer(sc, wl, np.arange(wl.T), i64(rs), i64(sl))
    _assert_topk_is_oracle(idx, tl, sc, sl, wl.topk, rs)  # the pipeline's own selection
    _topk_check(sc, sl, wl.topk, row_starts=rs)
    check_attention(out, lse, mx, wl.q, wl.kv, None, idx, tl, wl.sink, wl.scale, 512,
                    np.arange(wl.T))
    # end to end against the oracle's own scores: overlap ratio (reported)
    q = f64(wl.q_idx)
    ref_sc = O.indexer_scores(q, f64(wl.k_idx), f64(wl.w), i64(rs), i64(sl), np.arange(wl.T),
                              width=wl.T)
    ref_idx, _ = O.topk(ref_sc, i64(sl), wl.topk, row_starts=i64(rs))
    gi = i64(idx)
    inter = sum(len(set(gi[t][gi[t] >= 0]) & set(ref_idx[t][ref_idx[t] >= 0]))
                for t in range(wl.T))
    total = int((ref_idx >= 0).sum())
    say("  end-to-end top-K overlap", inter / total)
    assert inter / total > 0.99


@pytest.mark.parametrize("stress", [False, True])
def test_config2(stress):
    say("config 2", "stress" if stress else "")
    wl = make_config(2, device=DEV, stress=stress)
    rs, sl = _meta(wl)
    sc = dsa.dsa_indexer_fwd(wl.q_idx, wl.k_idx, wl.w, rs, sl, width=wl.T)
    idx, tl, _ = dsa.dsa_topk(sc, sl, wl.topk, row_starts=rs)
    out, lse, mx = dsa.dsa_sparse_attn_fwd(wl.q, wl.kv, idx, topk_length=tl, attn_sink=wl.sink,
                                           softmax_scale=wl.scale)
    torch.cuda.synchronize()
    _assert_topk_is_oracle(idx, tl, sc, sl, wl.topk, rs)  # the pipeline's own selection
    if not stress:
        check_indexer(sc, wl, np.arange(wl.T), i64(rs), i64(sl))
        _topk_check(sc, sl, wl.topk, row_starts=rs)
    rows = np.unique(np.concatenate([[0, 1, 2047, 2048, 2049, 4095],
                                     np.random.default_rng(2).integers(0, wl.T, 18)]))
    check_attention(out, lse, mx, wl.q, wl.kv, None, idx, tl, wl.sink, wl.scale, 512, rows)
    # rows t < 2048 keep every causal key, -1 after
    gi = i64(idx)
    for t in (0, 5, 2047):
        assert gi[t, : t + 1].tolist() == list(range(t + 1))
        assert np.all(gi[t, t + 1:] == -1)


def test_config3_sampled():
    say("config 3")
    wl = make_config(3, device=DEV)
    mx_len = max(wl.doc_lens)
    idx, tl, out, lse, mx = _pipeline(wl, max_seqlen=mx_len)
    torch.cuda.synchronize()
    rs, sl = _meta(wl)
    cu = np.cumsum([0] + wl.doc_lens)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([cu[:-1], cu[1:] - 1, cu[:-1] + 2048, cu[:-1] + 2047,
                                     rng.integers(0, wl.T, 24)]))
    rows = rows[rows < wl.T]
    # indexer + top-K on the sampled rows (scores recomputed row by row)
    for r in rows:
        sc = dsa.dsa_indexer_fwd(wl.q_idx, wl.k_idx, wl.w, rs, sl, row_begin=int(r), n_rows=1,
                                 width=mx_len)
        torch.cuda.synchronize()
        check_indexer(sc, wl, [r], i64(rs), i64(sl))
        ref_idx, ref_len = O.topk(sc.cpu().numpy().astype(np.float64), i64(sl)[[r]], wl.topk,
                                  row_starts=i64(rs)[[r]], n_cols=mx_len)
        assert np.array_equal(i64(idx)[r], ref_idx[0]) and i64(tl)[r] == ref_len[0]
    check_attention(out, lse, mx, wl.q, wl.kv, None, idx, tl, wl.sink, wl.scale, 512,
                    rows[:: max(1, len(rows) // 16)])
    # stress variant of the attention (same indexer inputs, so the same selection)
    del out, lse, mx
    wls = make_config(3, device=DEV, stress=True)
    out, lse, mx = dsa.dsa_sparse_attn_fwd(wls.q, wls.kv, idx, topk_length=tl, attn_sink=wls.sink,
                                           softmax_scale=wls.scale)
    torch.cuda.synchronize()
    check_attention(out, lse, mx, wls.q, wls.kv, None, idx, tl, wls.sink, wls.scale, 512,
                    rows[:: max(1, len(rows) // 16)])


def _c4_rows(T, chunk_rows, K):
    """Sampled rows of the T=65536 workload: the first and last rows of every
    score chunk, both sides of the top-K regimes (closed form up to K columns,
    rows held on chip up to 8192 columns, streamed rows beyond), and seeded
    random rows; 64 in all."""
    edges = []
    for c0 in range(0, T, chunk_rows):
        edges += [c0, c0 + 1, c0 + chunk_rows - 1]
    regimes = [K - 2, K - 1, K, K + 1, 4095, 4096, 8191, 8192, 8193, 16385, 32768, T - 2, T - 1]
    base = np.unique(np.array([r for r in edges + regimes if 0 <= r < T]))
    rng = np.random.default_rng(4)
    extra = rng.choice(np.setdiff1d(np.arange(T), base), 64 - len(base), replace=False)
    return np.sort(np.concatenate([base, extra]))


@pytest.mark.parametrize("fused", [False, True], ids=["score_chunks", "candidates"])
def test_config4_sampled(fused):
    """Both indexer + top-K paths at T = 65536: score chunks + dsa_topk, and
    the combined path's candidate buffer."""
    say("config 4", "candidates" if fused else "score chunks")
    wl = make_config(4, device=DEV)
    idx, tl, out, lse, mx = _pipeline(wl, fused=fused)
    torch.cuda.synchronize()
    rs, sl = _meta(wl)
    rows = _c4_rows(wl.T, dsa.chunk_rows(wl.T, wl.T), wl.topk)
    assert len(rows) == 64
    gi_all, gl_all = i64(idx), i64(tl)
    for r in rows:
        sc = dsa.dsa_indexer_fwd(wl.q_idx, wl.k_idx, wl.w, rs, sl, row_begin=int(r), n_rows=1,
                                 width=wl.T)
        torch.cuda.synchronize()
        check_indexer(sc, wl, [r], i64(rs), i64(sl))
        ref_idx, ref_len = O.topk(sc.cpu().numpy().astype(np.float64), i64(sl)[[r]], wl.topk,
                                  row_starts=i64(rs)[[r]], n_cols=wl.T)
        assert np.array_equal(gi_all[r], ref_idx[0]) and gl_all[r] == ref_len[0], int(r)
    check_attention(out, lse, mx, wl.q, wl.kv, None, idx, tl, wl.sink, wl.scale, 512, rows)
    # whole-tensor properties at full size
    gi = idx.cpu().numpy()
    tln = tl.cpu().numpy()
    t = np.arange(wl.T)
    assert np.array_equal(tln, np.minimum(t + 1, wl.topk))
    valid = gi >= 0
    assert np.array_equal(valid.sum(1), tln)
    assert np.all(np.where(valid, gi <= t[:, None], True))
    assert np.all(np.diff(np.where(valid, gi, np.iinfo(np.int32).max), axis=1)[:, :] >= 0)
    assert torch.isfinite(lse).all() and torch.isfinite(out.float()).all()
    if fused:
        return
    # stress variant of the attention (same indexer inputs, so the same selection;
    # queries scaled to logits of std ~4, sinks near the LSE)
    del out, lse, mx
    wls = make_config(4, device=DEV, stress=True)
    del wl
    out, lse, mx = dsa.dsa_sparse_attn_fwd(wls.q, wls.kv, idx, topk_length=tl, attn_sink=wls.sink,
                                           softmax_scale=wls.scale)
    torch.cuda.synchronize()
    check_attention(out, lse, mx, wls.q, wls.kv, None, idx, tl, wls.sink, wls.scale, 512,
                    rows[::2])


def test_config5_sampled():
    say("config 5")
    wl = make_config(5, device=DEV)
    out, lse, mx = dsa.dsa_sparse_attn_fwd(wl.q, wl.kv, wl.routes, attn_sink=None,
                                           softmax_scale=wl.scale, v=wl.v)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 3, 4, 8191, 8192, 8195, 32767],
                                     np.random.default_rng(5).integers(0, wl.T, 40)]))
    check_attention(out, lse, mx, wl.q, wl.kv, wl.v, wl.routes, None, None, wl.scale, 256, rows)
    wls = make_config(5, device=DEV, stress=True)
    out, lse, mx = dsa.dsa_sparse_attn_fwd(wls.q, wls.kv, wls.routes, softmax_scale=wls.scale,
                                           v=wls.v)
    torch.cuda.synchronize()
    check_attention(out, lse, mx, wls.q, wls.kv, wls.v, wls.routes, None, None, wls.scale, 256,
                    rows)


# -------------------------------------------------------------- determinism

def test_bitwise_determinism():
    say("determinism")
    wl = make_config(2, device=DEV)
    a = _pipeline(wl)
    b = _pipeline(wl)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y)
