"""C ABI checks that need no GPU: exports, version, host-side validation.

Argument validation runs before any HIP call, so bad calls return their status
without a device. Every call here passes fake (never dereferenced) pointers, so
all of them run in a child process with every GPU hidden: even a missing check
can then only reach the device lookup and report DSA_ERR_RUNTIME.
"""

import json
import os
import re
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

import deepseek_sparse_attention_dsa_amd as dsa  # noqa: E402

OK, ETYPE, EVALUE, ERUNTIME = 0, 1, 2, 3
FAKE = 1 << 20      # 16-byte aligned
FAKE2 = 3 << 20     # a second, distinct fake buffer

TOPK_BASE = dict(scores=FAKE, ld=4096, n_rows=8, n_cols=4096, seq_lens=FAKE, row_starts=None,
                 k=64, indices=FAKE, ld_idx=64, tl=None, vals=None, stream=None)
IDX_BASE = dict(q=FAKE, k=FAKE, w=FAKE, wd=0, rs=FAKE, sl=FAKE, T=256, Tkv=256, H=4, D=64, rb=0,
                nr=256, scores=FAKE, ld=256, stream=None)
ATTN_BASE = dict(q=FAKE, Tq=16, H=16, Dqk=576, k=FAKE, Tkv=16, ldk=576, v=None, ldv=0, Dv=512,
                 idx=FAKE, ldi=64, kw=64, tl=None, sink=None, scale=0.04, out=FAKE, lse=FAKE,
                 mx=None, stream=None)
META_BASE = dict(cu=FAKE, n_seq=1, T=4, rs=FAKE, sl=FAKE, stream=None)
F8_BASE = dict(q=FAKE, qs=FAKE2, k=FAKE, ks=FAKE2, sc=1, w=FAKE, wd=0, rs=FAKE, sl=FAKE, T=256,
               Tkv=256, H=64, D=128, rb=0, nr=256, scores=FAKE, ld=256, stream=None)
FUSED_BASE = dict(q=FAKE, qs=None, k=FAKE, ks=None, prec=0, w=FAKE, wd=0, rs=FAKE, sl=FAKE,
                  T=256, Tkv=256, H=64, D=128, rb=0, nr=256, nc=4096, kk=2048, idx=FAKE, ldi=2048,
                  tl=None, lg=None, so=None, lse=None, cb=None, cbn=0, stream=None)
# floats of the candidate buffer for 256 rows of 4097 columns: 4-word header,
# counts and queue (256 words each), 256 rescue rows of 4100 floats, and 256
# lists of 8192 (key, column) pairs
CAND_4097 = 4 + 256 + 256 + 256 * 4100 + 256 * 8192 * 2
BWD_BASE = dict(q=FAKE, Tq=16, H=16, Dqk=576, kv=FAKE, Tkv=16, ldkv=576, Dv=512, idx=FAKE, ldi=64,
                kw=64, tl=None, sink=None, scale=0.04, out=FAKE, dout=FAKE, lse=FAKE, dq=FAKE,
                dkv=FAKE, ds=None, ws=FAKE2, wsb=1 << 24, stream=None)
NOALLOC_BASE = {k: v for k, v in BWD_BASE.items() if k not in ("ws", "wsb")}
RMETA_BASE = dict(cq=FAKE, ck=FAKE2, off=None, n_seq=2, T=4, ratio=4, rs=FAKE, sl=FAKE,
                  stream=None)

ORDER = {
    "topk": ["scores", "ld", "n_rows", "n_cols", "seq_lens", "row_starts", "k", "indices",
             "ld_idx", "tl", "vals", "stream"],
    "idx": ["q", "k", "w", "wd", "rs", "sl", "T", "Tkv", "H", "D", "rb", "nr", "scores", "ld",
            "stream"],
    "attn": ["q", "Tq", "H", "Dqk", "k", "Tkv", "ldk", "v", "ldv", "Dv", "idx", "ldi", "kw", "tl",
             "sink", "scale", "out", "lse", "mx", "stream"],
    "meta": ["cu", "n_seq", "T", "rs", "sl", "stream"],
    "rmeta": ["cq", "ck", "off", "n_seq", "T", "ratio", "rs", "sl", "stream"],
    "f8": ["q", "qs", "k", "ks", "sc", "w", "wd", "rs", "sl", "T", "Tkv", "H", "D", "rb", "nr",
           "scores", "ld", "stream"],
    "fused": ["q", "qs", "k", "ks", "prec", "w", "wd", "rs", "sl", "T", "Tkv", "H", "D", "rb", "nr",
              "nc", "kk", "idx", "ldi", "tl", "lg", "so", "lse", "cb", "cbn", "stream"],
    "bwd": ["q", "Tq", "H", "Dqk", "kv", "Tkv", "ldkv", "Dv", "idx", "ldi", "kw", "tl", "sink",
            "scale", "out", "dout", "lse", "dq", "dkv", "ds", "ws", "wsb", "stream"],
    "noalloc": ["q", "Tq", "H", "Dqk", "kv", "Tkv", "ldkv", "Dv", "idx", "ldi", "kw", "tl",
                "sink", "scale", "out", "dout", "lse", "dq", "dkv", "ds", "stream"],
}
BASE = {"topk": TOPK_BASE, "idx": IDX_BASE, "attn": ATTN_BASE, "meta": META_BASE,
        "rmeta": RMETA_BASE, "f8": F8_BASE, "fused": FUSED_BASE, "bwd": BWD_BASE,
        "noalloc": NOALLOC_BASE}
FN = {"topk": "dsa_topk", "idx": "dsa_indexer_fwd", "attn": "dsa_sparse_attn_fwd",
      "meta": "dsa_packed_metadata", "rmeta": "dsa_ratio_causal_metadata",
      "f8": "dsa_indexer_fwd_fp8", "fused": "dsa_indexer_topk_fused", "bwd": "dsa_sparse_attn_bwd",
      "noalloc": "dsa_sparse_attn_bwd_noalloc"}

CASES = [
    # top-K
    ("topk", dict(k=0), EVALUE), ("topk", dict(k=2049), EVALUE), ("topk", dict(n_cols=0), EVALUE),
    ("topk", dict(n_cols=65537, ld=65540), EVALUE), ("topk", dict(ld=4095), EVALUE),
    ("topk", dict(ld=4094, n_cols=4094), EVALUE), ("topk", dict(ld_idx=63), EVALUE),
    ("topk", dict(n_rows=-1), EVALUE), ("topk", dict(scores=None), EVALUE),
    ("topk", dict(seq_lens=None), EVALUE), ("topk", dict(indices=None), EVALUE),
    ("topk", dict(scores=FAKE + 4), EVALUE),
    ("topk", dict(n_rows=0, scores=None, seq_lens=None, indices=None), OK),
    ("topk", dict(), ERUNTIME),
    # indexer
    ("idx", dict(wd=5), ETYPE), ("idx", dict(H=0), EVALUE), ("idx", dict(H=65), EVALUE),
    ("idx", dict(D=96), EVALUE), ("idx", dict(rb=200, nr=100), EVALUE),
    ("idx", dict(ld=254), EVALUE), ("idx", dict(q=None), EVALUE), ("idx", dict(k=FAKE + 2), EVALUE),
    ("idx", dict(scores=FAKE + 8), EVALUE), ("idx", dict(wd=1, w=FAKE + 2), EVALUE),
    ("idx", dict(T=-1), EVALUE), ("idx", dict(nr=0, q=None, k=None, w=None), OK),
    ("idx", dict(Tkv=-1), EVALUE), ("idx", dict(Tkv=2 ** 31), EVALUE),
    ("idx", dict(Tkv=0, q=None, k=None, w=None), OK), ("idx", dict(Tkv=64), ERUNTIME),
    ("idx", dict(), ERUNTIME), ("idx", dict(wd=1, D=128, H=64), ERUNTIME),
    # attention
    ("attn", dict(H=0), EVALUE), ("attn", dict(H=129), EVALUE),
    ("attn", dict(Dqk=128, Dv=128, ldk=128), EVALUE), ("attn", dict(Dqk=576, Dv=576), EVALUE),
    ("attn", dict(v=FAKE2, ldv=512), EVALUE),
    ("attn", dict(Dqk=512, Dv=512, ldk=512, v=FAKE2, ldv=512), EVALUE),
    ("attn", dict(ldk=570), EVALUE), ("attn", dict(ldk=580), EVALUE),
    ("attn", dict(scale=0.0), EVALUE), ("attn", dict(scale=-1.0), EVALUE),
    ("attn", dict(scale="nan"), EVALUE), ("attn", dict(scale="inf"), EVALUE),
    ("attn", dict(kw=65), EVALUE), ("attn", dict(kw=-1), EVALUE), ("attn", dict(q=None), EVALUE),
    ("attn", dict(out=None), EVALUE), ("attn", dict(lse=None), EVALUE),
    ("attn", dict(idx=None), EVALUE), ("attn", dict(q=FAKE + 2), EVALUE),
    ("attn", dict(out=FAKE + 8), EVALUE),
    ("attn", dict(Dqk=256, Dv=256, ldk=256, v=FAKE2, ldv=250), EVALUE),
    ("attn", dict(Dqk=256, Dv=256, ldk=256, v=FAKE2 + 2, ldv=256), EVALUE),
    ("attn", dict(Tq=0, q=None, out=None, lse=None, idx=None), OK),
    ("attn", dict(), ERUNTIME), ("attn", dict(Dqk=256, Dv=256, ldk=256, v=FAKE2, ldv=256), ERUNTIME),
    ("attn", dict(kw=0), ERUNTIME), ("attn", dict(kw=0, idx=None), ERUNTIME),
    # metadata
    ("meta", dict(n_seq=0), EVALUE), ("meta", dict(T=-1), EVALUE), ("meta", dict(cu=None), EVALUE),
    ("meta", dict(T=0, cu=None, rs=None, sl=None), OK), ("meta", dict(), ERUNTIME),
    # ratio-causal metadata
    ("rmeta", dict(n_seq=0), EVALUE), ("rmeta", dict(T=-1), EVALUE),
    ("rmeta", dict(ratio=0), EVALUE), ("rmeta", dict(ratio=-4), EVALUE),
    ("rmeta", dict(cq=None), EVALUE), ("rmeta", dict(ck=None), EVALUE),
    ("rmeta", dict(sl=None), EVALUE),
    ("rmeta", dict(T=0, cq=None, ck=None, rs=None, sl=None), OK),
    ("rmeta", dict(), ERUNTIME), ("rmeta", dict(off=FAKE2, ratio=1), ERUNTIME),
    # FP8 indexer
    ("f8", dict(wd=3), ETYPE), ("f8", dict(sc=2), EVALUE), ("f8", dict(sc=-1), EVALUE),
    ("f8", dict(D=64), EVALUE), ("f8", dict(H=0), EVALUE), ("f8", dict(H=65), EVALUE),
    ("f8", dict(qs=None), EVALUE), ("f8", dict(ks=None), EVALUE), ("f8", dict(k=FAKE + 8), EVALUE),
    ("f8", dict(ks=FAKE2 + 2), EVALUE), ("f8", dict(sc=0, qs=FAKE2 + 2), EVALUE),
    ("f8", dict(sc=1, qs=FAKE2 + 1), ERUNTIME), ("f8", dict(ld=250), EVALUE),
    ("f8", dict(rb=100, nr=200), EVALUE), ("f8", dict(Tkv=-1), EVALUE),
    ("f8", dict(nr=0, q=None, k=None), OK), ("f8", dict(Tkv=0, q=None), OK),
    ("f8", dict(), ERUNTIME), ("f8", dict(sc=0, wd=1), ERUNTIME),
    # combined indexer + top-K
    ("fused", dict(wd=2), ETYPE), ("fused", dict(prec=3), EVALUE), ("fused", dict(nc=0), EVALUE),
    ("fused", dict(nc=65537), EVALUE), ("fused", dict(kk=0), EVALUE), ("fused", dict(kk=2049), EVALUE),
    # rows longer than the on-chip path: a candidate buffer of the queried size
    ("fused", dict(nc=4097), EVALUE), ("fused", dict(nc=4097, cb=FAKE2, cbn=CAND_4097 - 1), EVALUE),
    ("fused", dict(nc=4097, cb=FAKE2 + 4, cbn=CAND_4097), EVALUE),
    ("fused", dict(nc=4097, cb=FAKE2, cbn=CAND_4097, prec=1, qs=FAKE2, ks=FAKE2), ERUNTIME),
    ("fused", dict(nc=4097, cb=FAKE2, cbn=CAND_4097, prec=2, qs=FAKE2, ks=FAKE2), ERUNTIME),
    ("fused", dict(nc=4097, cb=FAKE2, cbn=CAND_4097 - 1, prec=2, qs=FAKE2, ks=FAKE2), EVALUE),
    ("fused", dict(nc=4097, cb=FAKE2, cbn=CAND_4097), ERUNTIME),
    ("fused", dict(nc=65536, nr=0, cb=None), OK),
    ("fused", dict(ldi=2047), EVALUE), ("fused", dict(D=96), EVALUE),
    ("fused", dict(prec=1, D=64), EVALUE), ("fused", dict(prec=1), EVALUE),
    ("fused", dict(prec=2, qs=FAKE2, ks=FAKE2 + 1), EVALUE), ("fused", dict(idx=None), EVALUE),
    ("fused", dict(H=65), EVALUE), ("fused", dict(rb=1), EVALUE), ("fused", dict(q=FAKE + 4), EVALUE),
    ("fused", dict(nr=0, q=None, idx=None), OK), ("fused", dict(), ERUNTIME),
    ("fused", dict(prec=2, qs=FAKE2 + 1, ks=FAKE2), ERUNTIME),
    ("fused", dict(Tkv=0, D=64, kk=1, ldi=1), ERUNTIME),
    # attention backward
    ("bwd", dict(H=0), EVALUE), ("bwd", dict(H=129), EVALUE), ("bwd", dict(Dv=256), EVALUE),
    ("bwd", dict(Dqk=256), EVALUE), ("bwd", dict(ldkv=570), EVALUE), ("bwd", dict(kw=65), EVALUE),
    ("bwd", dict(scale=0.0), EVALUE), ("bwd", dict(scale="nan"), EVALUE),
    ("bwd", dict(dout=None), EVALUE), ("bwd", dict(lse=None), EVALUE), ("bwd", dict(dkv=None), EVALUE),
    ("bwd", dict(ws=None), EVALUE), ("bwd", dict(wsb=1024), EVALUE), ("bwd", dict(ws=FAKE2 + 16), EVALUE),
    ("bwd", dict(out=FAKE + 8), EVALUE), ("bwd", dict(idx=None), EVALUE),
    ("bwd", dict(), ERUNTIME), ("bwd", dict(Dqk=512, ldkv=512, sink=FAKE, ds=FAKE), ERUNTIME),
    # attention backward on the no-alloc scratch: the same checks, plus sizes
    # whose fixed buffers and one query row exceed the scratch
    ("noalloc", dict(H=0), EVALUE), ("noalloc", dict(Dv=256), EVALUE),
    ("noalloc", dict(scale=0.0), EVALUE), ("noalloc", dict(dout=None), EVALUE),
    ("noalloc", dict(out=FAKE + 8), EVALUE),
    ("noalloc", dict(Tkv=1 << 17), EVALUE),     # fp32 dkv accumulator alone: 302 MB
    ("noalloc", dict(Tq=1 << 20, H=128), EVALUE),  # [T_q, H] statistics: 1 GiB
    ("noalloc", dict(), ERUNTIME), ("noalloc", dict(Tkv=1 << 16), ERUNTIME),
]

_CHILD = r"""
import json, math, sys
sys.path.insert(0, {root!r})
import deepseek_sparse_attention_dsa_amd as dsa
lib = dsa.load_library()
calls = json.loads(sys.stdin.read())
res = []
for fn, args in calls:
    args = [float(a) if isinstance(a, str) else a for a in args]
    rc = getattr(lib, fn)(*args)
    res.append([rc, lib.dsa_last_error().decode()])
print(json.dumps(res))
"""


def _hidden_env():
    return dict(os.environ, HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="",
                CUDA_VISIBLE_DEVICES="")


@pytest.fixture(scope="module")
def results():
    calls = []
    for kind, kw, _ in CASES:
        a = dict(BASE[kind])
        a.update(kw)
        calls.append([FN[kind], [a[n] for n in ORDER[kind]]])
    r = subprocess.run([sys.executable, "-c", _CHILD.format(root=ROOT)], input=json.dumps(calls),
                       capture_output=True, text=True, env=_hidden_env(), timeout=300)
    assert r.returncode == 0, r.stderr
    return json.loads(r.stdout.strip().splitlines()[-1])


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|const char\*)\s+(dsa_\w+)\s*\(", text,
                                 flags=re.M)))


def test_header_declares_the_path():
    names = _declared_functions()
    for fn in ["dsa_packed_metadata", "dsa_ratio_causal_metadata", "dsa_indexer_fwd",
               "dsa_indexer_fwd_fp8", "dsa_indexer_topk_fused", "dsa_topk", "dsa_sparse_attn_fwd",
               "dsa_sparse_attn_bwd", "dsa_sparse_attn_bwd_workspace_bytes",
               "dsa_sparse_attn_bwd_kv_tiles", "dsa_topk_workspace_bytes",
               "dsa_indexer_topk_cand_buffer_size", "dsa_last_error", "dsa_abi_version"]:
        assert fn in names


def test_library_exports_every_declared_symbol():
    lib = dsa.load_library()
    for fn in _declared_functions():
        assert hasattr(lib, fn), fn
    out = subprocess.run(["nm", "-D", "--defined-only", dsa.library_path()], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\bT\s+(dsa_\w+)", out))
    assert set(_declared_functions()) <= exported


def test_abi_version():
    text = open(HEADER).read()
    v = int(re.search(r"#define DSA_ABI_VERSION (\d+)", text).group(1))
    assert dsa.load_library().dsa_abi_version() == v


@pytest.mark.parametrize("case", range(len(CASES)),
                         ids=[f"{c[0]}-{'-'.join(f'{k}={v}' for k, v in c[1].items()) or 'valid'}"
                              for c in CASES])
def test_validation_status(results, case):
    kind, kw, code = CASES[case]
    rc, msg = results[case]
    assert rc == code, (kind, kw, rc, msg)
    if code != OK:
        assert msg.startswith(FN[kind]), msg


def test_python_binding_type_and_shape_errors():
    import torch
    # dtype and device checks happen in the binding, before the library
    with pytest.raises(TypeError):
        dsa.dsa_topk(torch.zeros(2, 4, dtype=torch.float64), torch.zeros(2, dtype=torch.int32), 1)
    with pytest.raises(TypeError):
        dsa.dsa_sparse_attn_fwd(torch.zeros(1, 1, 576), torch.zeros(1, 576),
                                torch.zeros(1, 1, dtype=torch.int32))
    with pytest.raises(ValueError):  # host tensors are rejected
        dsa.dsa_sparse_attn_fwd(torch.zeros(1, 1, 576, dtype=torch.bfloat16),
                                torch.zeros(1, 576, dtype=torch.bfloat16),
                                torch.zeros(1, 1, dtype=torch.int32))
    with pytest.raises(TypeError):
        dsa.dsa_indexer_fwd(torch.zeros(4, 2, 64, dtype=torch.bfloat16),
                            torch.zeros(4, 64, dtype=torch.bfloat16),
                            torch.zeros(4, 2, dtype=torch.float16),
                            torch.zeros(4, dtype=torch.int32), torch.zeros(4, dtype=torch.int32))


def test_backward_workspace_size_rule():
    lib = dsa.load_library()
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    # Per-slot dkv (fewer than one key in eight selected: 8 * 64 < 1024):
    # statistics, dkv accumulator, per-KV-row counts and offsets and the radix
    # sort's 256 digit totals, then P, dS, the per-slot dkv rows, the slot
    # list and the sort's two key / value buffers of every row, and the sort's
    # 256 digit counts per 4096 slots, when they fit in 4 GiB
    n = lib.dsa_sparse_attn_bwd_workspace_bytes(256, 16, 1024, 576, 64)
    fixed = 2 * up(256 * 16 * 4) + up(1024 * 576 * 4) + up(1024 * 4) + up(1025 * 4) + up(1024)
    rows = (2 * up(256 * 64 * 32 * 2) + up(256 * 64 * 576 * 2) + 5 * up(256 * 64 * 4)
            + up(4 * 1024))
    assert n == fixed + rows
    # KV-tile dkv (8 * 64 >= 256): P and dS, the int16 slot map of every row
    # over the KV rows rounded up to 128, an fp32 partial per part of 64 rows
    # and its tile flags, the repeated-id queue and its count
    n = lib.dsa_sparse_attn_bwd_workspace_bytes(256, 16, 256, 576, 64)
    fixed = 2 * up(256 * 16 * 4) + up(256 * 576 * 4) + up(256 * 4) + up(257 * 4) + up(1024)
    rows = (2 * up(256 * 64 * 32 * 2) + up(256 * 256 * 2) + up(4 * 256 * 576 * 4)
            + up(4 * 2 * 4) + up(4) + up(256 * 4))
    assert n == fixed + rows
    # the rule's edges: 8 * k_width >= T_kv, at most 32768 KV rows and 8192 slots
    def layout(tq, tkv, kw, d=512, h=16):
        fx = 2 * up(tq * h * 4) + up(tkv * d * 4) + up(tkv * 4) + up((tkv + 1) * 4) + up(1024)
        kwp, hp, ld = (kw + 31) // 32 * 32, (h + 31) // 32 * 32, (tkv + 127) // 128 * 128
        npart = (tq + 63) // 64
        tile = (2 * up(tq * kwp * hp * 2) + up(tq * ld * 2) + up(npart * ld * d * 4)
                + up(npart * (ld // 128) * 4) + up(4) + up(tq * 4))
        slot = (2 * up(tq * kwp * hp * 2) + up(tq * kwp * d * 2) + 5 * up(tq * kwp * 4)
                + up((tq * kwp + 4095) // 4096 * 1024))
        return fx + tile, fx + slot
    for tq, tkv, kw, want_tiles in [(8, 800, 100, True), (8, 801, 100, False),
                                    (8, 32768, 4096, True), (8, 32769, 8192, False),
                                    (8, 4096, 8192, True), (8, 4096, 8193, False)]:
        tile, slot = layout(tq, tkv, kw)
        got = lib.dsa_sparse_attn_bwd_workspace_bytes(tq, 16, tkv, 512, kw)
        assert got == (tile if want_tiles else slot), (tq, tkv, kw)
        assert lib.dsa_sparse_attn_bwd_kv_tiles(tkv, kw) == int(want_tiles)
        assert dsa.dsa_sparse_attn_bwd_kv_tiles(tkv, kw) is want_tiles
    assert lib.dsa_sparse_attn_bwd_kv_tiles(0, 8) == 0
    assert lib.dsa_sparse_attn_bwd_kv_tiles(8, 0) == 0
    assert lib.dsa_sparse_attn_bwd_kv_tiles(-1, 8) == -1
    assert lib.dsa_sparse_attn_bwd_kv_tiles(8, -1) == -1
    assert lib.dsa_sparse_attn_bwd_workspace_bytes(10, 0, 10, 576, 8) == -1
    assert lib.dsa_sparse_attn_bwd_workspace_bytes(10, 8, 10, 256, 8) == -1


def test_cand_buffer_size_query():
    # no buffer for rows the on-chip path takes; the layout's size otherwise;
    # -1 exactly for the sizes the combined call rejects
    lib = dsa.load_library()
    assert lib.dsa_indexer_topk_cand_buffer_size(65536, 4096, 2048) == 0
    assert lib.dsa_indexer_topk_cand_buffer_size(0, 65536, 2048) == 0
    assert lib.dsa_indexer_topk_cand_buffer_size(256, 4097, 2048) == CAND_4097
    assert dsa.dsa_indexer_topk_cand_buffer_size(256, 4097, 1) == CAND_4097
    n = dsa.dsa_indexer_topk_cand_buffer_size(65536, 65536, 2048)
    assert n == 4 + 2 * 65536 + 256 * 65536 + 65536 * 8192 * 2
    for args in [(-1, 8192, 64), (8, 0, 64), (8, 65537, 64), (8, 8192, 0), (8, 8192, 2049),
                 (2 ** 31, 8192, 64)]:
        assert lib.dsa_indexer_topk_cand_buffer_size(*args) == -1, args
        with pytest.raises(ValueError):
            dsa.dsa_indexer_topk_cand_buffer_size(*args)


def test_topk_workspace_query():
    # dsa_topk needs no workspace for any size it accepts, and the query
    # rejects exactly the sizes dsa_topk rejects
    lib = dsa.load_library()
    assert lib.dsa_topk_workspace_bytes(65536, 65536, 2048) == 0
    assert lib.dsa_topk_workspace_bytes(0, 1, 1) == 0
    assert dsa.dsa_topk_workspace_bytes(8192, 4096, 64) == 0
    for args in [(-1, 4096, 64), (8, 0, 64), (8, 65537, 64), (8, 4096, 0), (8, 4096, 2049),
                 (2 ** 31, 4096, 64)]:
        assert lib.dsa_topk_workspace_bytes(*args) == -1, args
    with pytest.raises(ValueError):
        dsa.dsa_topk_workspace_bytes(8, 4096, 4096)


PEAKS_HEADER = os.path.join(ROOT, "include", "dsa_peaks.h")
PEAKS_LIB = os.path.join(ROOT, "deepseek_sparse_attention_dsa_amd", "libdsa_peaks.so")


def _peaks_lib():
    import ctypes
    lib = ctypes.CDLL(PEAKS_LIB)
    lib.dsa_peak_mfma_flop.restype = ctypes.c_double
    lib.dsa_peak_mfma_flop.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32]
    lib.dsa_peak_mfma.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                  ctypes.c_void_p]
    lib.dsa_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                  ctypes.c_int32, ctypes.c_void_p]
    lib.dsa_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_void_p, ctypes.c_void_p]
    return lib


def test_peaks_library_exports_and_work_counts():
    """The measurement probes: every declared symbol exported, the FLOP each
    MFMA form performs, and invalid arguments rejected before any launch."""
    text = re.sub(r"/\*.*?\*/", "", open(PEAKS_HEADER).read(), flags=re.S)
    names = set(re.findall(r"^\s*(?:int|double)\s+(dsa_\w+)\s*\(", text, flags=re.M))
    assert {"dsa_peak_mfma", "dsa_peak_mfma_flop", "dsa_peak_copy", "dsa_peak_read",
            "dsa_peak_threads_per_block"} <= names
    out = subprocess.run(["nm", "-D", "--defined-only", PEAKS_LIB], capture_output=True,
                         text=True).stdout
    assert names <= set(re.findall(r"\bT\s+(dsa_\w+)", out))
    lib = _peaks_lib()
    assert lib.dsa_peak_threads_per_block() == 256
    # 4 chains x iters MFMAs per wave, 4 waves per workgroup
    assert lib.dsa_peak_mfma_flop(0, 10, 3) == 2 * 32 * 32 * 16 * 4 * 10 * 4 * 3
    assert lib.dsa_peak_mfma_flop(1, 10, 3) == 2 * 32 * 32 * 64 * 4 * 10 * 4 * 3
    assert lib.dsa_peak_mfma_flop(2, 1, 1) == 2 * 32 * 32 * 64 * 4 * 4
    for bad in [(3, 10, 3), (0, 0, 3), (0, 10, 0)]:
        assert lib.dsa_peak_mfma_flop(*bad) == -1.0
    assert lib.dsa_peak_mfma(0, 0, 4, FAKE, None) == 1
    assert lib.dsa_peak_mfma(0, 10, 0, FAKE, None) == 1
    assert lib.dsa_peak_mfma(0, 10, 4, None, None) == 1
    assert lib.dsa_peak_mfma(0, 10, 4, FAKE + 4, None) == 1
    assert lib.dsa_peak_mfma(7, 10, 4, FAKE, None) == 1
    assert lib.dsa_peak_copy(FAKE, FAKE2, 100, 4, None) == 1
    assert lib.dsa_peak_copy(FAKE, FAKE2, 0, 4, None) == 1
    assert lib.dsa_peak_copy(FAKE + 8, FAKE2, 4096, 4, None) == 1
    assert lib.dsa_peak_copy(None, FAKE2, 4096, 4, None) == 1
    assert lib.dsa_peak_read(FAKE, 4096, 0, FAKE2, None) == 1
    assert lib.dsa_peak_read(FAKE, 4096, 4, None, None) == 1


def test_batched_gqa_validation():
    """sparse_gqa_attention rejects bad types, shapes, head layouts and scales
    before touching a device (CPU tensors: shape checks come first)."""
    bf = torch.bfloat16
    q = torch.zeros((2, 8, 24, 256), dtype=bf)
    k = torch.zeros((2, 8, 2, 256), dtype=bf)
    ids = torch.zeros((2, 8, 4), dtype=torch.int32)
    with pytest.raises(TypeError):
        dsa.sparse_gqa_attention(q.float(), k, k, ids)
    with pytest.raises(TypeError):
        dsa.sparse_gqa_attention(q, k, k, ids.float())
    with pytest.raises(ValueError):  # 24 query heads over 5 KV heads
        dsa.sparse_gqa_attention(q, torch.zeros((2, 8, 5, 256), dtype=bf),
                                 torch.zeros((2, 8, 5, 256), dtype=bf), ids)
    with pytest.raises(ValueError):  # 24 query heads over one KV head: a group of 24
        dsa.sparse_gqa_attention(q, k[:, :, :1], k[:, :, :1], ids)
    with pytest.raises(ValueError):  # head dim 128
        dsa.sparse_gqa_attention(q[..., :128], k[..., :128], k[..., :128], ids)
    with pytest.raises(ValueError):  # value shape
        dsa.sparse_gqa_attention(q, k, k[:, :7], ids)
    with pytest.raises(ValueError):  # ids not [B, S, W]
        dsa.sparse_gqa_attention(q, k, k, ids[:, :7])
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(ValueError):
            dsa.sparse_gqa_attention(q, k, k, ids, softmax_scale=bad)
