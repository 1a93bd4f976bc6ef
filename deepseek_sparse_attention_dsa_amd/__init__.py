"""MI355X (gfx950) DeepSeek Sparse Attention forward path.

Python binding of libdsa.so. The functions carry the C ABI's names and only
marshal arguments: they check torch dtypes, devices and shapes, allocate
outputs the caller did not pass (torch is used for device memory and streams),
and enqueue the HIP kernels on the current torch stream. Every step of the
path runs in the library's kernels; there is no fallback.

Status codes map to the exception classes of the NeMo cudnn_dsa API pages:
DSA_ERR_TYPE -> TypeError, DSA_ERR_VALUE -> ValueError,
DSA_ERR_RUNTIME -> RuntimeError.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = [
    "DSA_BF16", "DSA_F32", "DSA_MAX_TOPK", "DSA_TOPK_MAX_COLS", "DSA_MAX_HEADS",
    "load_library", "library_path", "dsa_abi_version", "dsa_last_error",
    "dsa_packed_metadata", "dsa_ratio_causal_metadata", "dsa_indexer_fwd",
    "dsa_indexer_fwd_fp8", "DSA_FP8_PER_TOKEN", "DSA_MXFP8", "dsa_topk",
    "dsa_topk_workspace_bytes",
    "dsa_indexer_topk_fused", "dsa_indexer_topk_cand_buffer_size", "DSA_FUSED_MAX_COLS",
    "dsa_sparse_attn_fwd", "dsa_sparse_attn_bwd", "dsa_sparse_attn_bwd_workspace_bytes",
    "dsa_sparse_attn_bwd_kv_tiles", "indexer_topk", "chunk_rows", "sparse_gqa_attention",
]

DSA_OK, DSA_ERR_TYPE, DSA_ERR_VALUE, DSA_ERR_RUNTIME = 0, 1, 2, 3
DSA_BF16, DSA_F32 = 0, 1
DSA_FP8_PER_TOKEN, DSA_MXFP8 = 0, 1
DSA_MAX_TOPK = 2048
DSA_TOPK_MAX_COLS = 65536
DSA_MAX_HEADS = 128
DSA_FUSED_MAX_COLS = 4096
DSA_INDEXER_BF16, DSA_INDEXER_FP8, DSA_INDEXER_MXFP8 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F32 = ctypes.c_float

_SIGNATURES = {
    "dsa_last_error": ([], ctypes.c_char_p),
    "dsa_abi_version": ([], ctypes.c_int),
    "dsa_packed_metadata": ([_P, _I32, _I64, _P, _P, _P], ctypes.c_int),
    "dsa_ratio_causal_metadata": ([_P, _P, _P, _I32, _I64, _I32, _P, _P, _P], ctypes.c_int),
    "dsa_indexer_fwd": ([_P, _P, _P, _I32, _P, _P, _I64, _I64, _I32, _I32, _I64, _I64, _P, _I64,
                         _P], ctypes.c_int),
    "dsa_indexer_fwd_fp8": ([_P, _P, _P, _P, _I32, _P, _I32, _P, _P, _I64, _I64, _I32, _I32,
                             _I64, _I64, _P, _I64, _P], ctypes.c_int),
    "dsa_indexer_topk_fused": ([_P, _P, _P, _P, _I32, _P, _I32, _P, _P, _I64, _I64, _I32, _I32,
                                _I64, _I64, _I64, _I32, _P, _I64, _P, _P, _P, _P, _P, _I64,
                                _P], ctypes.c_int),
    "dsa_indexer_topk_cand_buffer_size": ([_I64, _I64, _I32], ctypes.c_int64),
    "dsa_topk": ([_P, _I64, _I64, _I64, _P, _P, _I32, _P, _I64, _P, _P, _P], ctypes.c_int),
    "dsa_topk_workspace_bytes": ([_I64, _I64, _I32], ctypes.c_int64),
    "dsa_sparse_attn_bwd_workspace_bytes": ([_I64, _I32, _I64, _I32, _I32], ctypes.c_int64),
    "dsa_sparse_attn_bwd_kv_tiles": ([_I64, _I32], ctypes.c_int),
    "dsa_sparse_attn_bwd": ([_P, _I64, _I32, _I32, _P, _I64, _I64, _I32, _P, _I64, _I32, _P, _P,
                             _F32, _P, _P, _P, _P, _P, _P, _P, _I64, _P], ctypes.c_int),
    "dsa_sparse_attn_fwd": ([_P, _I64, _I32, _I32, _P, _I64, _I64, _P, _I64, _I32, _P, _I64,
                             _I32, _P, _P, _F32, _P, _P, _P, _P], ctypes.c_int),
    "dsa_sparse_attn_bwd_noalloc": ([_P, _I64, _I32, _I32, _P, _I64, _I64, _I32, _P, _I64, _I32,
                                     _P, _P, _F32, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
}
DSA_NOALLOC_SCRATCH_BYTES = 256 * 1024 * 1024


def library_path() -> str:
    return os.environ.get("DSA_LIBRARY", os.path.join(_HERE, "libdsa.so"))


def load_library(path: Optional[str] = None):
    """Load libdsa.so (built in-tree by build.py). Raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or library_path()
    if not os.path.exists(p):
        raise RuntimeError(
            f"libdsa.so not found at {p}; build it with "
            "`python -m deepseek_sparse_attention_dsa_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (args, res) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def dsa_abi_version() -> int:
    return load_library().dsa_abi_version()


def dsa_last_error() -> str:
    return load_library().dsa_last_error().decode()


def _check(rc: int):
    if rc == DSA_OK:
        return
    msg = dsa_last_error()
    if rc == DSA_ERR_TYPE:
        raise TypeError(msg)
    if rc == DSA_ERR_VALUE:
        raise ValueError(msg)
    raise RuntimeError(msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _need(t, name, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t if t.is_contiguous() else t.contiguous()


def _out(t, name, dtype, device):
    """Validate a caller-provided output buffer (never copied)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.stride(-1) != 1:
        raise ValueError(f"{name} must have a unit innermost stride")
    return t


def dsa_packed_metadata(cu_seqlens: torch.Tensor, T: int, row_starts=None, seq_lens=None,
                        stream=None):
    """Per-token document start and causal length of packed THD sequences."""
    cu = _need(cu_seqlens, "cu_seqlens", torch.int32)
    dev = cu.device
    row_starts = (torch.empty(T, dtype=torch.int32, device=dev) if row_starts is None
                  else _out(row_starts, "row_starts", torch.int32, dev))
    seq_lens = (torch.empty(T, dtype=torch.int32, device=dev) if seq_lens is None
                else _out(seq_lens, "seq_lens", torch.int32, dev))
    if row_starts.numel() < T or seq_lens.numel() < T:
        raise ValueError("row_starts and seq_lens need T entries")
    lib = load_library()
    _check(lib.dsa_packed_metadata(_ptr(cu), cu.numel() - 1, T, _ptr(row_starts), _ptr(seq_lens),
                                   _stream(stream)))
    return row_starts, seq_lens


def dsa_ratio_causal_metadata(cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, T_q: int,
                              ratio: int = 1, q_causal_offsets: Optional[torch.Tensor] = None,
                              row_starts=None, seq_lens=None, stream=None):
    """Per-query key-segment start and visible key count of the ratio-causal mask."""
    cu_q = _need(cu_seqlens_q, "cu_seqlens_q", torch.int32)
    dev = cu_q.device
    cu_k = _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, dev)
    n_seq = cu_q.numel() - 1
    if cu_k.numel() != n_seq + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k need the same number of segments")
    if q_causal_offsets is not None:
        q_causal_offsets = _need(q_causal_offsets, "q_causal_offsets", torch.int32, dev)
        if q_causal_offsets.numel() != n_seq:
            raise ValueError("q_causal_offsets needs one entry per segment")
    row_starts = (torch.empty(T_q, dtype=torch.int32, device=dev) if row_starts is None
                  else _out(row_starts, "row_starts", torch.int32, dev))
    seq_lens = (torch.empty(T_q, dtype=torch.int32, device=dev) if seq_lens is None
                else _out(seq_lens, "seq_lens", torch.int32, dev))
    if row_starts.numel() < T_q or seq_lens.numel() < T_q:
        raise ValueError("row_starts and seq_lens need T_q entries")
    lib = load_library()
    _check(lib.dsa_ratio_causal_metadata(_ptr(cu_q), _ptr(cu_k), _ptr(q_causal_offsets), n_seq,
                                         T_q, int(ratio), _ptr(row_starts), _ptr(seq_lens),
                                         _stream(stream)))
    return row_starts, seq_lens


def dsa_indexer_fwd(q_idx: torch.Tensor, k_idx: torch.Tensor, w: torch.Tensor,
                    row_starts: torch.Tensor, seq_lens: torch.Tensor, row_begin: int = 0,
                    n_rows: Optional[int] = None, scores: Optional[torch.Tensor] = None,
                    width: Optional[int] = None, stream=None) -> torch.Tensor:
    """Indexer scores [n_rows, ld] fp32 for rows [row_begin, row_begin + n_rows).

    `width` (>= the longest causal length of the rows) sizes a new score
    buffer; its row stride is rounded up to a multiple of 4. k_idx [T_kv, D]
    may have another row count than q_idx (compressed keys).
    """
    if not isinstance(w, torch.Tensor) or w.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"w must be a bfloat16 or float32 tensor (got {getattr(w, 'dtype', w)})")
    q_idx = _need(q_idx, "q_idx", torch.bfloat16)
    dev = q_idx.device
    k_idx = _need(k_idx, "k_idx", torch.bfloat16, dev)
    w = _need(w, "w", w.dtype, dev)
    row_starts = _need(row_starts, "row_starts", torch.int32, dev)
    seq_lens = _need(seq_lens, "seq_lens", torch.int32, dev)
    if q_idx.dim() != 3 or k_idx.dim() != 2 or w.dim() != 2:
        raise ValueError("expected q_idx [T,H,D], k_idx [T_kv,D], w [T,H]")
    T, H, D = q_idx.shape
    T_kv = k_idx.shape[0]
    if k_idx.shape[1] != D or w.shape != (T, H):
        raise ValueError(f"shape mismatch: q_idx {tuple(q_idx.shape)}, k_idx "
                         f"{tuple(k_idx.shape)}, w {tuple(w.shape)}")
    if n_rows is None:
        n_rows = T - row_begin
    if scores is None:
        if width is None:
            width = T_kv
        ld = max(4, (int(width) + 3) // 4 * 4)
        scores = torch.empty((n_rows, ld), dtype=torch.float32, device=dev)
    else:
        scores = _out(scores, "scores", torch.float32, dev)
        if scores.dim() != 2 or scores.shape[0] < n_rows:
            raise ValueError("scores must be 2-D with at least n_rows rows")
    lib = load_library()
    _check(lib.dsa_indexer_fwd(_ptr(q_idx), _ptr(k_idx), _ptr(w),
                               DSA_BF16 if w.dtype == torch.bfloat16 else DSA_F32,
                               _ptr(row_starts), _ptr(seq_lens), T, T_kv, H, D, row_begin, n_rows,
                               _ptr(scores), scores.stride(0), _stream(stream)))
    return scores


def _fp8_bytes(t, name, dev):
    if not isinstance(t, torch.Tensor) or t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError(f"{name} must be a uint8 or float8_e4m3fn tensor")
    return _need(t.view(torch.uint8), name, torch.uint8, dev)


def dsa_indexer_fwd_fp8(q8: torch.Tensor, q_scale: torch.Tensor, k8: torch.Tensor,
                        k_scale: torch.Tensor, w: torch.Tensor, row_starts: torch.Tensor,
                        seq_lens: torch.Tensor, scaling: int = DSA_MXFP8, row_begin: int = 0,
                        n_rows: Optional[int] = None, scores: Optional[torch.Tensor] = None,
                        width: Optional[int] = None, stream=None) -> torch.Tensor:
    """Indexer scores from FP8 E4M3 q8 [T,H,128] / k8 [T_kv,128].

    scaling DSA_FP8_PER_TOKEN: q_scale fp32 [T,H], k_scale fp32 [T_kv]
    descales; DSA_MXFP8: q_scale uint8 E8M0 [T,H,4], k_scale uint8 [T_kv,4].
    Other arguments as dsa_indexer_fwd.
    """
    if not isinstance(w, torch.Tensor) or w.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"w must be a bfloat16 or float32 tensor (got {getattr(w, 'dtype', w)})")
    if scaling not in (DSA_FP8_PER_TOKEN, DSA_MXFP8):
        raise ValueError(f"unknown scaling {scaling}")
    dev = q8.device
    q8 = _fp8_bytes(q8, "q8", dev)
    k8 = _fp8_bytes(k8, "k8", dev)
    sdt = torch.float32 if scaling == DSA_FP8_PER_TOKEN else torch.uint8
    if isinstance(q_scale, torch.Tensor) and q_scale.dtype == torch.float8_e8m0fnu:
        q_scale = q_scale.view(torch.uint8)
    if isinstance(k_scale, torch.Tensor) and k_scale.dtype == torch.float8_e8m0fnu:
        k_scale = k_scale.view(torch.uint8)
    q_scale = _need(q_scale, "q_scale", sdt, dev)
    k_scale = _need(k_scale, "k_scale", sdt, dev)
    w = _need(w, "w", w.dtype, dev)
    row_starts = _need(row_starts, "row_starts", torch.int32, dev)
    seq_lens = _need(seq_lens, "seq_lens", torch.int32, dev)
    if q8.dim() != 3 or k8.dim() != 2 or w.dim() != 2:
        raise ValueError("expected q8 [T,H,D], k8 [T_kv,D], w [T,H]")
    T, H, D = q8.shape
    T_kv = k8.shape[0]
    nb = D // 32
    qs_shape = (T, H) if scaling == DSA_FP8_PER_TOKEN else (T, H, nb)
    ks_shape = (T_kv,) if scaling == DSA_FP8_PER_TOKEN else (T_kv, nb)
    if (k8.shape[1] != D or w.shape != (T, H) or tuple(q_scale.shape) != qs_shape
            or tuple(k_scale.shape) != ks_shape):
        raise ValueError(f"shape mismatch: q8 {tuple(q8.shape)}, k8 {tuple(k8.shape)}, w "
                         f"{tuple(w.shape)}, q_scale {tuple(q_scale.shape)}, k_scale "
                         f"{tuple(k_scale.shape)}")
    if n_rows is None:
        n_rows = T - row_begin
    if scores is None:
        width = T_kv if width is None else width
        ld = max(4, (int(width) + 3) // 4 * 4)
        scores = torch.empty((n_rows, ld), dtype=torch.float32, device=dev)
    else:
        scores = _out(scores, "scores", torch.float32, dev)
        if scores.dim() != 2 or scores.shape[0] < n_rows:
            raise ValueError("scores must be 2-D with at least n_rows rows")
    lib = load_library()
    _check(lib.dsa_indexer_fwd_fp8(_ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), int(scaling),
                                   _ptr(w), DSA_BF16 if w.dtype == torch.bfloat16 else DSA_F32,
                                   _ptr(row_starts), _ptr(seq_lens), T, T_kv, H, D, row_begin,
                                   n_rows, _ptr(scores), scores.stride(0), _stream(stream)))
    return scores


def dsa_topk(scores: torch.Tensor, seq_lens: torch.Tensor, k: int,
             row_starts: Optional[torch.Tensor] = None, n_cols: Optional[int] = None,
             indices: Optional[torch.Tensor] = None, topk_length: Optional[torch.Tensor] = None,
             return_values: bool = False, stream=None):
    """Top-k per row -> (indices int32 [n_rows, k], topk_length int32 [n_rows], values|None)."""
    if not isinstance(scores, torch.Tensor) or scores.dtype != torch.float32:
        raise TypeError("scores must be a float32 tensor")
    if scores.dim() != 2 or scores.stride(1) != 1:
        raise ValueError("scores must be 2-D with unit column stride")
    dev = scores.device
    n_rows = scores.shape[0]
    n_cols = scores.shape[1] if n_cols is None else int(n_cols)
    seq_lens = _need(seq_lens, "seq_lens", torch.int32, dev)
    if seq_lens.numel() != n_rows:
        raise ValueError("seq_lens must have one entry per score row")
    if row_starts is not None:
        row_starts = _need(row_starts, "row_starts", torch.int32, dev)
        if row_starts.numel() != n_rows:
            raise ValueError("row_starts must have one entry per score row")
    indices = (torch.empty((n_rows, k), dtype=torch.int32, device=dev) if indices is None
               else _out(indices, "indices", torch.int32, dev))
    topk_length = (torch.empty((n_rows,), dtype=torch.int32, device=dev) if topk_length is None
                   else _out(topk_length, "topk_length", torch.int32, dev))
    values = torch.empty((n_rows, indices.stride(0)), dtype=torch.float32,
                         device=dev)[:, :k] if return_values else None
    lib = load_library()
    _check(lib.dsa_topk(_ptr(scores), scores.stride(0), n_rows, n_cols, _ptr(seq_lens),
                        _ptr(row_starts), k, _ptr(indices), indices.stride(0), _ptr(topk_length),
                        _ptr(values), _stream(stream)))
    return indices, topk_length, values


def dsa_topk_workspace_bytes(n_rows: int, n_cols: int, k: int) -> int:
    """Device workspace dsa_topk needs (0: it keeps each row on chip)."""
    n = int(load_library().dsa_topk_workspace_bytes(n_rows, n_cols, k))
    if n < 0:
        raise ValueError("sizes out of contract for dsa_topk")
    return n


def dsa_sparse_attn_fwd(q: torch.Tensor, kv: torch.Tensor, indices: torch.Tensor,
                        topk_length: Optional[torch.Tensor] = None,
                        attn_sink: Optional[torch.Tensor] = None,
                        softmax_scale: Optional[float] = None, v: Optional[torch.Tensor] = None,
                        d_v: Optional[int] = None, out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None,
                        max_logits: Optional[torch.Tensor] = None,
                        return_max_logits: bool = True, stream=None):
    """Sparse attention forward -> (out bf16 [T_q,H,D_v], lse fp32 [T_q,H], max_logits|None).

    kv: [T_kv, D_qk] (or [T_kv, 1, D_qk]) key rows; V = kv[:, :d_v] unless a
    separate v [T_kv, D_v] is given. d_v defaults to 512 for D_qk = 576 and to
    D_qk otherwise. softmax_scale defaults to 1/sqrt(D_qk).
    """
    q = _need(q, "q", torch.bfloat16)
    dev = q.device
    if kv.dim() == 3 and kv.shape[1] == 1:
        kv = kv[:, 0, :]
    kv = _need(kv, "kv", torch.bfloat16, dev)
    if v is not None:
        if v.dim() == 3 and v.shape[1] == 1:
            v = v[:, 0, :]
        v = _need(v, "v", torch.bfloat16, dev)
    if indices.dim() == 3 and indices.shape[1] == 1:
        indices = indices[:, 0, :]
    indices = _need(indices, "indices", torch.int32, dev)
    if topk_length is not None:
        topk_length = _need(topk_length, "topk_length", torch.int32, dev)
    if attn_sink is not None:
        attn_sink = _need(attn_sink, "attn_sink", torch.float32, dev)
    if q.dim() != 3 or kv.dim() != 2 or indices.dim() != 2:
        raise ValueError("expected q [T_q,H,D_qk], kv [T_kv,D_qk], indices [T_q,K]")
    T_q, H, D_qk = q.shape
    if kv.shape[1] != D_qk or indices.shape[0] != T_q:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, kv {tuple(kv.shape)}, "
                         f"indices {tuple(indices.shape)}")
    if v is not None:
        d_v = v.shape[1]
        if v.shape[0] != kv.shape[0]:
            raise ValueError("v and kv must have the same number of rows")
    elif d_v is None:
        d_v = 512 if D_qk == 576 else D_qk
    if attn_sink is not None and attn_sink.numel() != H:
        raise ValueError("attn_sink must have one entry per head")
    if topk_length is not None and topk_length.numel() != T_q:
        raise ValueError("topk_length must have one entry per query row")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D_qk)
    out = (torch.empty((T_q, H, d_v), dtype=torch.bfloat16, device=dev) if out is None
           else _out(out, "out", torch.bfloat16, dev))
    if not out.is_contiguous() or out.shape != (T_q, H, d_v):
        raise ValueError("out must be a contiguous [T_q, H, D_v] tensor")
    lse = (torch.empty((T_q, H), dtype=torch.float32, device=dev) if lse is None
           else _out(lse, "lse", torch.float32, dev))
    if max_logits is None and return_max_logits:
        max_logits = torch.empty((T_q, H), dtype=torch.float32, device=dev)
    elif max_logits is not None:
        max_logits = _out(max_logits, "max_logits", torch.float32, dev)
    for name, t in (("lse", lse), ("max_logits", max_logits)):
        if t is not None and (not t.is_contiguous() or t.shape != (T_q, H)):
            raise ValueError(f"{name} must be a contiguous [T_q, H] tensor")
    lib = load_library()
    _check(lib.dsa_sparse_attn_fwd(
        _ptr(q), T_q, H, D_qk, _ptr(kv), kv.shape[0], kv.stride(0), _ptr(v),
        0 if v is None else v.stride(0), d_v, _ptr(indices), indices.stride(0), indices.shape[1],
        _ptr(topk_length), _ptr(attn_sink), float(softmax_scale), _ptr(out), _ptr(lse),
        _ptr(max_logits), _stream(stream)))
    return out, lse, max_logits


def dsa_indexer_topk_fused(q_idx: torch.Tensor, k_idx: torch.Tensor, w: torch.Tensor,
                           row_starts: torch.Tensor, seq_lens: torch.Tensor, k: int, n_cols: int,
                           q_scale: Optional[torch.Tensor] = None,
                           k_scale: Optional[torch.Tensor] = None,
                           fp8_scaling: Optional[int] = None, row_begin: int = 0,
                           n_rows: Optional[int] = None, indices: Optional[torch.Tensor] = None,
                           topk_length: Optional[torch.Tensor] = None, return_logits: bool = False,
                           return_softmax: bool = False, return_lse: bool = False,
                           cand_buffer: Optional[torch.Tensor] = None, stream=None):
    """Indexer scores + top-k without dense scores.

    Returns (indices int32 [n_rows, k], topk_length int32 [n_rows], logits |
    None, softmax | None, lse | None). bf16 q_idx / k_idx, or FP8 ones with
    q_scale, k_scale and fp8_scaling as dsa_indexer_fwd_fp8 takes them. Rows
    longer than DSA_FUSED_MAX_COLS go through the candidate path and need
    cand_buffer, a
    float32 device tensor of dsa_indexer_topk_cand_buffer_size(n_rows,
    n_cols, k) elements (allocated when None).
    """
    if not isinstance(w, torch.Tensor) or w.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"w must be a bfloat16 or float32 tensor (got {getattr(w, 'dtype', w)})")
    dev = q_idx.device
    fp8 = isinstance(q_idx, torch.Tensor) and q_idx.dtype in (torch.uint8, torch.float8_e4m3fn)
    if fp8:
        if fp8_scaling not in (DSA_FP8_PER_TOKEN, DSA_MXFP8):
            raise ValueError("FP8 inputs need fp8_scaling DSA_FP8_PER_TOKEN or DSA_MXFP8")
        precision = DSA_INDEXER_FP8 if fp8_scaling == DSA_FP8_PER_TOKEN else DSA_INDEXER_MXFP8
        q_idx = _fp8_bytes(q_idx, "q_idx", dev)
        k_idx = _fp8_bytes(k_idx, "k_idx", dev)
        sdt = torch.float32 if fp8_scaling == DSA_FP8_PER_TOKEN else torch.uint8
        q_scale = _need(q_scale.view(torch.uint8) if q_scale is not None and
                        q_scale.dtype == torch.float8_e8m0fnu else q_scale, "q_scale", sdt, dev)
        k_scale = _need(k_scale.view(torch.uint8) if k_scale is not None and
                        k_scale.dtype == torch.float8_e8m0fnu else k_scale, "k_scale", sdt, dev)
    else:
        precision = DSA_INDEXER_BF16
        q_idx = _need(q_idx, "q_idx", torch.bfloat16)
        k_idx = _need(k_idx, "k_idx", torch.bfloat16, dev)
    w = _need(w, "w", w.dtype, dev)
    row_starts = _need(row_starts, "row_starts", torch.int32, dev)
    seq_lens = _need(seq_lens, "seq_lens", torch.int32, dev)
    if q_idx.dim() != 3 or k_idx.dim() != 2 or w.dim() != 2:
        raise ValueError("expected q_idx [T,H,D], k_idx [T_kv,D], w [T,H]")
    T, H, D = q_idx.shape
    T_kv = k_idx.shape[0]
    if k_idx.shape[1] != D or w.shape != (T, H):
        raise ValueError(f"shape mismatch: q_idx {tuple(q_idx.shape)}, k_idx "
                         f"{tuple(k_idx.shape)}, w {tuple(w.shape)}")
    if fp8:
        nb = D // 32
        qs_shape = (T, H) if fp8_scaling == DSA_FP8_PER_TOKEN else (T, H, nb)
        ks_shape = (T_kv,) if fp8_scaling == DSA_FP8_PER_TOKEN else (T_kv, nb)
        if tuple(q_scale.shape) != qs_shape or tuple(k_scale.shape) != ks_shape:
            raise ValueError("scale shapes do not match q_idx / k_idx")
    if n_rows is None:
        n_rows = T - row_begin
    indices = (torch.empty((n_rows, k), dtype=torch.int32, device=dev) if indices is None
               else _out(indices, "indices", torch.int32, dev))
    topk_length = (torch.empty((n_rows,), dtype=torch.int32, device=dev) if topk_length is None
                   else _out(topk_length, "topk_length", torch.int32, dev))
    ld = indices.stride(0)
    logits = (torch.empty((n_rows, ld), dtype=torch.float32, device=dev)[:, :k]
              if return_logits else None)
    softmax = (torch.empty((n_rows, ld), dtype=torch.float32, device=dev)[:, :k]
               if return_softmax else None)
    lse = torch.empty((n_rows,), dtype=torch.float32, device=dev) if return_lse else None
    need = dsa_indexer_topk_cand_buffer_size(n_rows, int(n_cols), int(k))
    if need > 0 and cand_buffer is None:
        cand_buffer = torch.empty((need,), dtype=torch.float32, device=dev)
    elif cand_buffer is not None:
        cand_buffer = _out(cand_buffer, "cand_buffer", torch.float32, dev)
    lib = load_library()
    _check(lib.dsa_indexer_topk_fused(
        _ptr(q_idx), _ptr(q_scale) if fp8 else None, _ptr(k_idx), _ptr(k_scale) if fp8 else None,
        precision, _ptr(w), DSA_BF16 if w.dtype == torch.bfloat16 else DSA_F32, _ptr(row_starts),
        _ptr(seq_lens), T, T_kv, H, D, row_begin, n_rows, int(n_cols), int(k), _ptr(indices), ld,
        _ptr(topk_length), _ptr(logits), _ptr(softmax), _ptr(lse), _ptr(cand_buffer),
        0 if cand_buffer is None else cand_buffer.numel(), _stream(stream)))
    return indices, topk_length, logits, softmax, lse


def dsa_indexer_topk_cand_buffer_size(n_rows: int, n_cols: int, k: int) -> int:
    """Floats of the candidate buffer dsa_indexer_topk_fused needs (0: none)."""
    n = int(load_library().dsa_indexer_topk_cand_buffer_size(n_rows, n_cols, k))
    if n < 0:
        raise ValueError("sizes out of contract for dsa_indexer_topk_fused")
    return n


def dsa_sparse_attn_bwd_workspace_bytes(T_q: int, H: int, T_kv: int, D_qk: int,
                                        k_width: int) -> int:
    n = int(load_library().dsa_sparse_attn_bwd_workspace_bytes(T_q, H, T_kv, D_qk, k_width))
    if n < 0:
        raise ValueError("sizes out of contract for dsa_sparse_attn_bwd")
    return n


def dsa_sparse_attn_bwd_kv_tiles(T_kv: int, k_width: int) -> bool:
    """Whether dsa_sparse_attn_bwd computes dkv by KV tiles (dense selections)
    rather than by per-slot rows, for these sizes."""
    r = int(load_library().dsa_sparse_attn_bwd_kv_tiles(T_kv, k_width))
    if r < 0:
        raise ValueError("T_kv and k_width must be >= 0")
    return r == 1


def dsa_sparse_attn_bwd(q: torch.Tensor, kv: torch.Tensor, indices: torch.Tensor,
                        out: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor,
                        topk_length: Optional[torch.Tensor] = None,
                        attn_sink: Optional[torch.Tensor] = None,
                        softmax_scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
                        dq: Optional[torch.Tensor] = None, dkv: Optional[torch.Tensor] = None,
                        d_sink: Optional[torch.Tensor] = None, stream=None):
    """Sparse attention backward for shared latent KV -> (dq, dkv, d_sink).

    q [T_q,H,D_qk], kv [T_kv,D_qk] (V = kv[:, :512]), indices [T_q, k], out
    and dout [T_q,H,512] bf16, lse [T_q,H] fp32 (the forward's). workspace:
    a uint8 device tensor (allocated when None).
    """
    q = _need(q, "q", torch.bfloat16)
    dev = q.device
    kv = _need(kv, "kv", torch.bfloat16, dev)
    if kv.dim() == 3 and kv.shape[1] == 1:
        kv = kv[:, 0]
    out = _need(out, "out", torch.bfloat16, dev)
    dout = _need(dout, "dout", torch.bfloat16, dev)
    lse = _need(lse, "lse", torch.float32, dev)
    if indices.dtype != torch.int32:
        raise TypeError("indices must be int32")
    if indices.dim() != 2 or indices.stride(1) != 1:
        raise ValueError("indices must be 2-D with unit column stride")
    T_q, H, D = q.shape
    T_kv = kv.shape[0]
    if kv.shape[1] < D or out.shape != (T_q, H, 512) or dout.shape != (T_q, H, 512) or \
            lse.shape != (T_q, H) or indices.shape[0] != T_q:
        raise ValueError("shape mismatch among q, kv, indices, out, dout, lse")
    if topk_length is not None:
        topk_length = _need(topk_length, "topk_length", torch.int32, dev)
    if attn_sink is not None:
        attn_sink = _need(attn_sink, "attn_sink", torch.float32, dev)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    k_width = indices.shape[1]
    need = dsa_sparse_attn_bwd_workspace_bytes(T_q, H, T_kv, D, k_width)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    else:
        workspace = _out(workspace, "workspace", torch.uint8, dev)
    dq = torch.empty_like(q) if dq is None else _out(dq, "dq", torch.bfloat16, dev)
    dkv = (torch.empty((T_kv, D), dtype=torch.bfloat16, device=dev) if dkv is None
           else _out(dkv, "dkv", torch.bfloat16, dev))
    d_sink = (torch.empty((H,), dtype=torch.float32, device=dev) if d_sink is None
              else _out(d_sink, "d_sink", torch.float32, dev))
    lib = load_library()
    _check(lib.dsa_sparse_attn_bwd(_ptr(q), T_q, H, D, _ptr(kv), T_kv, kv.stride(0), 512,
                                   _ptr(indices), indices.stride(0), k_width, _ptr(topk_length),
                                   _ptr(attn_sink), float(scale), _ptr(out), _ptr(dout), _ptr(lse),
                                   _ptr(dq), _ptr(dkv), _ptr(d_sink), _ptr(workspace),
                                   workspace.numel(), _stream(stream)))
    return dq, dkv, d_sink


# Score-buffer cap per chunk of rows (2 GiB, the cap the NeMo cudnn_dsa page
# applies to its score / top-K scratch).
SCORE_CHUNK_BYTES = 2 * 1024 * 1024 * 1024


def chunk_rows(T: int, width: int, cap_bytes: int = SCORE_CHUNK_BYTES) -> int:
    """Rows per score chunk so that [rows, width] fp32 stays under the cap."""
    ld = max(4, (int(width) + 3) // 4 * 4)
    return max(1, min(T, cap_bytes // (4 * ld)))


def sparse_gqa_attention(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                         selected_token_ids: torch.Tensor,
                         softmax_scale: Optional[float] = None) -> torch.Tensor:
    """Block-routed sparse GQA over batched tensors -> out bf16 [B, S, H_q, 256].

    The layout of NeMo-QSA `cudnn_sparse_gqa_attention`: query [B, S, H_q,
    256], key / value [B, S, H_kv, 256] (bf16), selected_token_ids [B, S, W]
    int32 / int64 ids into the same batch row's sequence (ids outside [0, S)
    are padding), one route set per token shared by the KV heads. Each KV
    head and its H_q / H_kv query heads form an independent head group, run
    as its own dsa_sparse_attn_fwd call per batch row (the pages' (24, 2)
    case is two (12, 1) groups); strided inputs are copied to contiguous
    per-group buffers first; everything runs on the current stream.
    softmax_scale defaults to 1/sqrt(256). Raises
    TypeError for non-bf16 tensors or non-integer ids, ValueError for shapes,
    head counts (H_q a multiple of H_kv, at most 16 query heads per group)
    or the scale.
    """
    for name, t in (("query", query), ("key", key), ("value", value)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be a bfloat16 tensor")
    if not isinstance(selected_token_ids, torch.Tensor) or selected_token_ids.dtype not in (
            torch.int32, torch.int64):
        raise TypeError("selected_token_ids must be an int32 or int64 tensor")
    if query.dim() != 4 or key.dim() != 4 or query.shape[3] != 256:
        raise ValueError("expected query [B, S, H_q, 256] and key / value [B, S, H_kv, 256]")
    B, S, H_q, D = query.shape
    H_kv = key.shape[2]
    if tuple(key.shape) != (B, S, H_kv, D) or tuple(value.shape) != tuple(key.shape):
        raise ValueError(f"shape mismatch: query {tuple(query.shape)}, key {tuple(key.shape)}, "
                         f"value {tuple(value.shape)}")
    if H_kv < 1 or H_q % H_kv != 0 or H_q // H_kv > 16:
        raise ValueError(f"unsupported heads ({H_q}, {H_kv}): H_q must be a multiple of H_kv "
                         "with at most 16 query heads per KV head")
    if (selected_token_ids.dim() != 3 or tuple(selected_token_ids.shape[:2]) != (B, S)
            or selected_token_ids.shape[2] < 1):
        raise ValueError("selected_token_ids must be [B, S, W] with W >= 1")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if not (math.isfinite(softmax_scale) and softmax_scale > 0):
        raise ValueError("softmax_scale must be finite and positive")
    dev = query.device
    for name, t in (("key", key), ("value", value), ("selected_token_ids", selected_token_ids)):
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
    ids = selected_token_ids
    if ids.dtype == torch.int64:  # narrowing must not turn an invalid id into a valid one
        ids = torch.where((ids < 0) | (ids >= S), torch.full_like(ids, -1), ids)
    ids = ids.to(torch.int32)
    G = H_q // H_kv
    out = torch.empty((B, S, H_q, D), dtype=torch.bfloat16, device=dev)
    for b in range(B):
        idx = ids[b].contiguous()
        for g in range(H_kv):
            o, _, _ = dsa_sparse_attn_fwd(
                query[b, :, G * g:G * (g + 1), :].contiguous(), key[b, :, g, :].contiguous(),
                idx, softmax_scale=softmax_scale, v=value[b, :, g, :].contiguous(), d_v=D,
                return_max_logits=False)
            out[b, :, G * g:G * (g + 1), :] = o
    return out


def indexer_topk(q_idx: torch.Tensor, k_idx: torch.Tensor, w: torch.Tensor,
                 cu_seqlens: torch.Tensor, k: int, max_seqlen: Optional[int] = None,
                 rows_per_chunk: Optional[int] = None, cu_seqlens_k: Optional[torch.Tensor] = None,
                 ratio: int = 1, q_causal_offsets: Optional[torch.Tensor] = None,
                 q_scale: Optional[torch.Tensor] = None, k_scale: Optional[torch.Tensor] = None,
                 fp8_scaling: Optional[int] = None, fused: Optional[bool] = None,
                 return_softmax: bool = False, stream=None):
    """Metadata + indexer scores + top-K over all rows, in score chunks.

    Returns (indices int32 [T, k] global ascending with -1 suffix,
    topk_length int32 [T]). With only cu_seqlens the mask is the causal mask
    of packed documents and max_seqlen (the longest document, default T)
    sizes each chunk's score buffer. Passing cu_seqlens_k, a ratio other than
    1 or q_causal_offsets selects the ratio-causal mask (cu_seqlens then
    locates the query segments, cu_seqlens_k the key segments, default
    cu_seqlens); max_seqlen is then the longest key segment (default T_kv).
    FP8 inputs (q_idx / k_idx as uint8 or float8_e4m3fn) take q_scale,
    k_scale and fp8_scaling as dsa_indexer_fwd_fp8 does.
    fused=True (or return_softmax=True) replaces the score chunks by one
    dsa_indexer_topk_fused call (no score buffer: rows of at most
    DSA_FUSED_MAX_COLS columns stay on chip, longer rows go through a
    candidate buffer); only that path gives return_softmax, which returns
    (indices, topk_length, logits, softmax, lse). fused=None takes the
    candidate buffer for rows longer than DSA_FUSED_MAX_COLS (the faster path
    there on MI355X) and score chunks otherwise.
    """
    fp8 = q_idx.dtype in (torch.uint8, torch.float8_e4m3fn)
    if fp8 and (q_scale is None or k_scale is None or fp8_scaling is None):
        raise ValueError("FP8 indexer inputs need q_scale, k_scale and fp8_scaling")
    T = q_idx.shape[0]
    T_kv = k_idx.shape[0]
    dev = q_idx.device
    ratio_causal = cu_seqlens_k is not None or int(ratio) != 1 or q_causal_offsets is not None
    if ratio_causal:
        width = T_kv if max_seqlen is None else int(max_seqlen)
        row_starts, seq_lens = dsa_ratio_causal_metadata(
            cu_seqlens, cu_seqlens if cu_seqlens_k is None else cu_seqlens_k, T, ratio,
            q_causal_offsets, stream=stream)
    else:
        width = T if max_seqlen is None else int(max_seqlen)
        row_starts, seq_lens = dsa_packed_metadata(cu_seqlens, T, stream=stream)
    if fused is None:
        fused = return_softmax or width > DSA_FUSED_MAX_COLS
    if return_softmax and not fused:
        raise ValueError("return_softmax needs the fused path")
    if fused:
        res = dsa_indexer_topk_fused(q_idx, k_idx, w, row_starts, seq_lens, k, max(width, 1),
                                     q_scale=q_scale, k_scale=k_scale, fp8_scaling=fp8_scaling,
                                     return_logits=return_softmax, return_softmax=return_softmax,
                                     return_lse=return_softmax, stream=stream)
        return res if return_softmax else res[:2]
    rows = chunk_rows(T, width) if rows_per_chunk is None else int(rows_per_chunk)
    indices = torch.empty((T, k), dtype=torch.int32, device=dev)
    topk_length = torch.empty((T,), dtype=torch.int32, device=dev)
    ld = max(4, (width + 3) // 4 * 4)
    scores = torch.empty((min(rows, T), ld), dtype=torch.float32, device=dev)
    for r0 in range(0, T, rows):
        n = min(rows, T - r0)
        if fp8:
            dsa_indexer_fwd_fp8(q_idx, q_scale, k_idx, k_scale, w, row_starts, seq_lens,
                                scaling=fp8_scaling, row_begin=r0, n_rows=n, scores=scores,
                                stream=stream)
        else:
            dsa_indexer_fwd(q_idx, k_idx, w, row_starts, seq_lens, row_begin=r0, n_rows=n,
                            scores=scores, stream=stream)
        # plain causal rows never see more than r0 + n keys
        n_cols = width if ratio_causal else min(width, r0 + n)
        dsa_topk(scores[:n], seq_lens[r0:r0 + n], k, row_starts=row_starts[r0:r0 + n],
                 n_cols=n_cols, indices=indices[r0:r0 + n],
                 topk_length=topk_length[r0:r0 + n],
                 stream=stream)
    return indices, topk_length

