"""split_kv_merge_amd -- attention forward with a per-row log2 LSE, split-KV decode
partials and their stable merge, as hand-written HIP kernels for MI355X (gfx950).

This module is a thin ctypes binding over ``libskv.so`` (C ABI in include/skv.h):
it checks tensor metadata, allocates outputs with torch (device memory and the
current stream are the only things torch provides) and passes raw pointers.
Every step of the computation runs in the library's kernels.  There is no CPU
fallback: if the library is missing, every call raises.

Functions (same names as the C entry points without the ``skv_`` prefix):
    attn_fwd, attn_fwd_varlen, attn_splitkv_partial, attn_splitkv_decode,
    attn_splitkv_decode_noalloc, splitkv_decode_noalloc_max_bytes, merge_state,
    workspace_bytes, splitkv_workspace_bytes, pick_num_splits, lse_varlen_to_dense,
    sage_quant, sage_fwd, sage_workspace_bytes
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["attn_fwd", "attn_fwd_varlen", "attn_splitkv_partial", "attn_splitkv_decode",
           "attn_splitkv_decode_noalloc", "splitkv_decode_noalloc_max_bytes",
           "merge_state", "workspace_bytes", "splitkv_workspace_bytes", "pick_num_splits",
           "lse_varlen_to_dense", "sage_quant", "sage_fwd", "sage_workspace_bytes", "SkvError",
           "lib_path"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libskv.so")

SKV_BF16, SKV_FP16, SKV_FP32 = 0, 1, 2
SKV_HND, SKV_NHD = 0, 1
_STATUS = {0: "SKV_OK", 1: "SKV_EINVAL", 2: "SKV_EUNSUPPORTED", 3: "SKV_ELAUNCH"}

_lib = None


class SkvError(RuntimeError):
    """A non-OK status from libskv; ``.status`` holds the code."""

    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


def lib_path() -> str:
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m split_kv_merge_amd.build` "
                           "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, SZ, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_int64
    I64P = ctypes.POINTER(ctypes.c_int64)
    lib.skv_attn_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, I, P, SZ, P]
    lib.skv_attn_fwd.restype = I
    lib.skv_attn_fwd_varlen.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, I, P, SZ, P]
    lib.skv_attn_fwd_varlen.restype = I
    lib.skv_attn_splitkv_partial.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, P, P]
    lib.skv_attn_splitkv_partial.restype = I
    lib.skv_attn_splitkv_decode.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, P, P, SZ, P]
    lib.skv_attn_splitkv_decode.restype = I
    lib.skv_attn_splitkv_decode_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, P, P]
    lib.skv_attn_splitkv_decode_noalloc.restype = I
    lib.skv_splitkv_decode_noalloc_max_bytes.argtypes = []
    lib.skv_splitkv_decode_noalloc_max_bytes.restype = SZ
    lib.skv_splitkv_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.skv_splitkv_workspace_bytes.restype = SZ
    lib.skv_merge_state.argtypes = [I, I, I, I, I, P, I, I64, I64P, P, I64, I64P, P, I, I64P, P, I64P, P]
    lib.skv_merge_state.restype = I
    lib.skv_workspace_bytes.argtypes = [I, I, I, I]
    lib.skv_workspace_bytes.restype = SZ
    lib.skv_pick_num_splits.argtypes = [I, I, I, I, I]
    lib.skv_pick_num_splits.restype = I
    lib.skv_sage_quant.argtypes = [P, P, I, I, I, I, I, I, I, I, I, P, P, P, P, P, P]
    lib.skv_sage_quant.restype = I
    lib.skv_sage_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, I, P, SZ, P]
    lib.skv_sage_fwd.restype = I
    lib.skv_sage_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I]
    lib.skv_sage_workspace_bytes.restype = SZ
    lib.skv_status_str.argtypes = [I]
    lib.skv_status_str.restype = ctypes.c_char_p
    lib.skv_last_error.argtypes = []
    lib.skv_last_error.restype = ctypes.c_char_p
    _check_single_hip_runtime()
    _lib = lib
    return lib


def _check_single_hip_runtime():
    """torch ships its own libamdhip64; libskv must bind to that same runtime, or
    torch's streams and allocations would be foreign to the library's launches."""
    try:
        maps = open("/proc/self/maps").read()
    except OSError:
        return
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    if len(libs) > 1:
        raise RuntimeError(f"two HIP runtimes are mapped ({sorted(libs)}); import torch before "
                           "loading libskv")


def _check(status: int):
    if status != 0:
        raise SkvError(status, _lib.skv_last_error().decode() or _lib.skv_status_str(status).decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SKV_BF16
    if t.dtype == torch.float16:
        return SKV_FP16
    if t.dtype == torch.float32:
        return SKV_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need_cuda_contig(name, t):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_kv_len(kv_len, B):
    """kv_len: None, or an int32 GPU tensor of B filled lengths (read on the device)."""
    if kv_len is None:
        return
    _need_cuda_contig("kv_len", kv_len)
    if kv_len.dtype != torch.int32 or tuple(kv_len.shape) != (B,):
        raise ValueError(f"kv_len must be an int32 tensor of shape ({B},)")


def workspace_bytes(b_or_nseq: int, hkv: int, d: int, smooth_k: bool) -> int:
    return int(_load().skv_workspace_bytes(b_or_nseq, hkv, d, int(bool(smooth_k))))


def pick_num_splits(B: int, Hkv: int, rows_per_kv_head: int, Lkv: int, D: int) -> int:
    return int(_load().skv_pick_num_splits(B, Hkv, rows_per_kv_head, Lkv, D))


def _dims(q, k, layout):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be 4-D")
    if layout == "HND":
        B, Hq, Sq, D = q.shape
        Bk, Hkv, Sk, Dk = k.shape
    elif layout == "NHD":
        B, Sq, Hq, D = q.shape
        Bk, Sk, Hkv, Dk = k.shape
    else:
        raise ValueError(f"layout must be 'HND' or 'NHD', got {layout!r}")
    if Bk != B or Dk != D:
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} disagree on batch or head dim")
    return B, Hq, Hkv, Sq, Sk, D


def attn_fwd(q, k, v, scale=None, layout="HND", causal=False, smooth_k=False, return_lse=False,
             out=None, lse=None):
    """Attention forward on GPU tensors in HND [B,H,S,D] or NHD [B,S,H,D] layout.

    Returns ``out`` (q's shape and dtype), or ``(out, lse)`` with lse float32
    [B, Hq, Sq] in log2 units when ``return_lse``.  ``scale`` defaults to D**-0.5.
    ``smooth_k`` subtracts mean(k) from the keys inside the kernel and adds the
    matching term back into the LSE, which therefore does not change.
    """
    lib = _load()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need_cuda_contig(n, t)
    if v.shape != k.shape or v.dtype != k.dtype or q.dtype != k.dtype:
        raise ValueError("k and v must match in shape, and q, k, v in dtype")
    B, Hq, Hkv, Sq, Sk, D = _dims(q, k, layout)
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty_like(q)
    _need_cuda_contig("out", out)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must have q's shape and dtype")
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need_cuda_contig("lse", lse)
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Sq):
            raise ValueError(f"lse must be float32 {(B, Hq, Sq)}")
    ws_n = workspace_bytes(B, Hkv, D, smooth_k)
    ws = torch.empty(max(ws_n // 4, 1), dtype=torch.float32, device=q.device) if ws_n else None
    _check(lib.skv_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Sq, Sk, D,
                            _dt(q), SKV_HND if layout == "HND" else SKV_NHD, float(scale),
                            int(bool(causal)), int(bool(smooth_k)), _ptr(ws), ws_n,
                            _stream(q.device)))
    return (out, lse) if (return_lse or lse is not None) else out


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, scale=None, causal=False,
                    smooth_k=False, return_lse=False, out=None, lse=None):
    """Packed varlen attention: q [total_q,Hq,D], k/v [total_k,Hkv,D], cu_seqlens int32
    GPU tensors [nseq+1].  Returns ``out`` or ``(out, lse)`` with lse float32
    [Hq, total_q] (2-D, log2)."""
    lib = _load()
    for n, t in (("q", q), ("k", k), ("v", v), ("cu_seqlens_q", cu_seqlens_q),
                 ("cu_seqlens_k", cu_seqlens_k)):
        _need_cuda_contig(n, t)
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
        raise ValueError("q must be [total_q,Hq,D] and k, v [total_k,Hkv,D]")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both have nseq + 1 entries")
    total_q, Hq, D = q.shape
    total_k, Hkv, Dk = k.shape
    if Dk != D or q.dtype != k.dtype or v.dtype != k.dtype:
        raise ValueError("q, k, v must agree on head dim and dtype")
    nseq = cu_seqlens_q.numel() - 1
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty_like(q)
    _need_cuda_contig("out", out)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must have q's shape and dtype")
    if return_lse and lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need_cuda_contig("lse", lse)
        if lse.dtype != torch.float32 or tuple(lse.shape) != (Hq, total_q):
            raise ValueError(f"lse must be float32 {(Hq, total_q)}")
    ws_n = workspace_bytes(nseq, Hkv, D, smooth_k)
    ws = torch.empty(max(ws_n // 4, 1), dtype=torch.float32, device=q.device) if ws_n else None
    _check(lib.skv_attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                   _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), nseq, total_q, total_k,
                                   int(max_seqlen_q), Hq, Hkv, D, _dt(q), float(scale),
                                   int(bool(causal)), int(bool(smooth_k)), _ptr(ws), ws_n,
                                   _stream(q.device)))
    return (out, lse) if (return_lse or lse is not None) else out


def attn_splitkv_partial(q, k, v, num_splits=None, scale=None, layout="HND", out_part=None,
                         lse_part=None, kv_len=None):
    """Split-KV decode partials: returns (out_part float32 [S, *q.shape],
    lse_part float32 [S, B, Hq, Lq]) for S = num_splits chunks of the keys
    (default: pick_num_splits).  ``kv_len`` (int32 GPU tensor [B], optional): the
    filled KV length per batch element; only those keys are read, split evenly
    over the chunks."""
    lib = _load()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need_cuda_contig(n, t)
    if v.shape != k.shape or q.dtype != k.dtype or v.dtype != k.dtype:
        raise ValueError("k and v must match in shape, and q, k, v in dtype")
    B, Hq, Hkv, Lq, Lkv, D = _dims(q, k, layout)
    if Hkv <= 0 or Hq % Hkv:
        raise ValueError(f"Hq ({Hq}) must be a multiple of Hkv ({Hkv})")
    _check_kv_len(kv_len, B)
    if num_splits is None:
        num_splits = pick_num_splits(B, Hkv, (Hq // Hkv) * Lq, Lkv, D)
    if scale is None:
        scale = D ** -0.5
    S = int(num_splits)
    if out_part is None:
        out_part = torch.empty((S,) + tuple(q.shape), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((S, B, Hq, Lq), dtype=torch.float32, device=q.device)
    _need_cuda_contig("out_part", out_part)
    _need_cuda_contig("lse_part", lse_part)
    if out_part.dtype != torch.float32 or tuple(out_part.shape) != (S,) + tuple(q.shape):
        raise ValueError("out_part must be float32 [num_splits, *q.shape]")
    if lse_part.dtype != torch.float32 or tuple(lse_part.shape) != (S, B, Hq, Lq):
        raise ValueError("lse_part must be float32 [num_splits, B, Hq, Lq]")
    _check(lib.skv_attn_splitkv_partial(_ptr(q), _ptr(k), _ptr(v), _ptr(out_part), _ptr(lse_part),
                                        B, Hq, Hkv, Lq, Lkv, D, _dt(q),
                                        SKV_HND if layout == "HND" else SKV_NHD, float(scale), S,
                                        _ptr(kv_len), _stream(q.device)))
    return out_part, lse_part


def splitkv_workspace_bytes(B: int, Hq: int, Lq: int, D: int, num_splits: int, Hkv: int) -> int:
    return int(_load().skv_splitkv_workspace_bytes(B, Hq, Lq, D, num_splits, Hkv))


def attn_splitkv_decode(q, k, v, num_splits=None, scale=None, layout="HND", out=None, lse=None,
                        workspace=None, return_lse=True, kv_len=None):
    """Split-KV decode in one launch (partials + stable merge): returns (out, lse) with
    out in q's shape and dtype and lse float32 [B, Hq, Lq] (log2).

    ``workspace`` (uint8 GPU tensor of splitkv_workspace_bytes(...) bytes) must be
    zero-filled before its first use; the call leaves it zero-filled again, so it can
    be reused by later calls and graph replays.  A fresh zeroed one is made if None.
    ``kv_len``: as in attn_splitkv_partial.
    """
    lib = _load()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need_cuda_contig(n, t)
    if v.shape != k.shape or q.dtype != k.dtype or v.dtype != k.dtype:
        raise ValueError("k and v must match in shape, and q, k, v in dtype")
    B, Hq, Hkv, Lq, Lkv, D = _dims(q, k, layout)
    if Hkv <= 0 or Hq % Hkv:
        raise ValueError(f"Hq ({Hq}) must be a multiple of Hkv ({Hkv})")
    _check_kv_len(kv_len, B)
    if num_splits is None:
        num_splits = pick_num_splits(B, Hkv, (Hq // Hkv) * Lq, Lkv, D)
    if scale is None:
        scale = D ** -0.5
    S = int(num_splits)
    if out is None:
        out = torch.empty_like(q)
    _need_cuda_contig("out", out)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must have q's shape and dtype")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need_cuda_contig("lse", lse)
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Lq):
            raise ValueError(f"lse must be float32 {(B, Hq, Lq)}")
    need = splitkv_workspace_bytes(B, Hq, Lq, D, S, Hkv)
    if workspace is None:
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=q.device)
    _need_cuda_contig("workspace", workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.skv_attn_splitkv_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv,
                                       Lq, Lkv, D, _dt(q), SKV_HND if layout == "HND" else SKV_NHD,
                                       float(scale), S, _ptr(kv_len), _ptr(workspace), ws_bytes,
                                       _stream(q.device)))
    return (out, lse) if lse is not None else out


def splitkv_decode_noalloc_max_bytes() -> int:
    return int(_load().skv_splitkv_decode_noalloc_max_bytes())


def attn_splitkv_decode_noalloc(q, k, v, out, lse=None, num_splits=None, scale=None,
                                layout="HND", kv_len=None):
    """The single-launch decode of ``attn_splitkv_decode`` with its partial states in
    the library's fixed device scratch instead of a workspace: the call allocates
    nothing, so ``out`` (q's shape and dtype) must be given, and ``lse`` (float32
    [B, Hq, Lq]) too if wanted.  Calls that may overlap on one GPU share that scratch
    and must not run at the same time.  Returns (out, lse), or out when lse is None."""
    lib = _load()
    for n, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _need_cuda_contig(n, t)
    if v.shape != k.shape or q.dtype != k.dtype or v.dtype != k.dtype:
        raise ValueError("k and v must match in shape, and q, k, v in dtype")
    B, Hq, Hkv, Lq, Lkv, D = _dims(q, k, layout)
    if Hkv <= 0 or Hq % Hkv:
        raise ValueError(f"Hq ({Hq}) must be a multiple of Hkv ({Hkv})")
    _check_kv_len(kv_len, B)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must have q's shape and dtype")
    if lse is not None:
        _need_cuda_contig("lse", lse)
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Lq):
            raise ValueError(f"lse must be float32 {(B, Hq, Lq)}")
    if num_splits is None:
        num_splits = pick_num_splits(B, Hkv, (Hq // Hkv) * Lq, Lkv, D)
    if scale is None:
        scale = D ** -0.5
    _check(lib.skv_attn_splitkv_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B,
                                               Hq, Hkv, Lq, Lkv, D, _dt(q),
                                               SKV_HND if layout == "HND" else SKV_NHD,
                                               float(scale), int(num_splits), _ptr(kv_len),
                                               _stream(q.device)))
    return (out, lse) if lse is not None else out


def _rows3(t: torch.Tensor, lead: int, tail: int):
    """Sizes and element strides of the row dims of t (skipping `lead` leading and
    `tail` trailing dims), left-padded to exactly three."""
    dims = list(t.shape[lead:t.dim() - tail])
    strides = list(t.stride()[lead:t.dim() - tail])
    if len(dims) > 3:
        raise ValueError("at most three row dimensions are supported")
    while len(dims) < 3:
        dims.insert(0, 1)
        strides.insert(0, 0)
    return dims, strides


def merge_state(o_parts, lse_parts, out_dtype=None, out=None, lse=None, return_lse=True):
    """Stable merge of partial states: o_parts [S, *rows, D] (float32, bf16 or fp16;
    any strides with D contiguous), lse_parts float32 [S, *rows] (1 to 3 row dims).
    Returns (out [*rows, D] in ``out_dtype`` (default: o_parts' dtype), lse float32
    [*rows]); or just out when ``return_lse`` is False and no ``lse`` is given."""
    lib = _load()
    if not (o_parts.is_cuda and lse_parts.is_cuda):
        raise ValueError("o_parts and lse_parts must be GPU tensors")
    if o_parts.stride(-1) != 1:
        raise ValueError("o_parts must be contiguous along D")
    if lse_parts.dtype != torch.float32:
        raise TypeError("lse_parts must be float32")
    if tuple(lse_parts.shape) != tuple(o_parts.shape[:-1]):
        raise ValueError(f"lse_parts {tuple(lse_parts.shape)} must be o_parts {tuple(o_parts.shape)} "
                         "without its last axis")
    S, D = o_parts.shape[0], o_parts.shape[-1]
    rows_shape = tuple(o_parts.shape[1:-1])
    if out is None:
        out = torch.empty(rows_shape + (D,), dtype=out_dtype or o_parts.dtype, device=o_parts.device)
    if out.stride(-1) != 1 or tuple(out.shape) != rows_shape + (D,):
        raise ValueError("out must be [*rows, D] and contiguous along D")
    if lse is None and return_lse:
        lse = torch.empty(rows_shape, dtype=torch.float32, device=o_parts.device)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != rows_shape):
        raise ValueError(f"lse must be float32 {rows_shape}")
    (R0, R1, R2), po = _rows3(o_parts, 1, 1)
    _, pl = _rows3(lse_parts, 1, 0)
    _, oo = _rows3(out, 0, 1)
    arr = ctypes.c_int64 * 3
    lo = arr(*(_rows3(lse, 0, 0)[1])) if lse is not None else None
    _check(lib.skv_merge_state(S, R0, R1, R2, D, _ptr(o_parts), _dt(o_parts), o_parts.stride(0),
                               arr(*po), _ptr(lse_parts), lse_parts.stride(0), arr(*pl), _ptr(out),
                               _dt(out), arr(*oo), _ptr(lse), lo, _stream(o_parts.device)))
    return (out, lse) if lse is not None else out


def lse_varlen_to_dense(lse: torch.Tensor, B: int, S: int, cu_seqlens=None) -> torch.Tensor:
    """View a varlen LSE [H, B*S] of B sequences of S tokens each as the dense [B, H, S]
    layout (SGLang PR #33840 review thread: reshape to (H, B, S), swap the first two
    axes).  The shape is checked first.  The LSE alone cannot show where one sequence
    ends, so only with ``cu_seqlens`` (the int32 [B + 1] boundaries the varlen call
    used; a GPU tensor is copied to the host, which synchronises) are sequences of
    unequal length detected and rejected; without it the caller vouches that every
    sequence has S tokens."""
    if lse.dim() != 2 or lse.shape[1] != B * S:
        raise ValueError(f"expected a varlen LSE [H, {B}*{S}], got {tuple(lse.shape)}")
    if cu_seqlens is not None:
        cu = [int(x) for x in torch.as_tensor(cu_seqlens).cpu().tolist()]
        if cu != [b * S for b in range(B + 1)]:
            raise ValueError(f"cu_seqlens {cu} does not describe {B} sequences of {S} tokens")
    return lse.reshape(lse.shape[0], B, S).transpose(0, 1)


# ------------------------------------------------------------- INT8 QK^T path

def sage_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, dtype, smooth_k=True) -> int:
    dt = dtype if isinstance(dtype, int) else _dt(torch.empty(0, dtype=dtype))
    return int(_load().skv_sage_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, dt, int(bool(smooth_k))))


def sage_quant(q, k, layout="HND", smooth_k=True):
    """Per-block INT8 quantisation of q and of k - mean(k) (skv_sage_quant).

    Returns dict(q_codes int8 [B,Hq,Sq,D], q_scale float32 [B,Hq,ceil(Sq/32)],
    k_codes int8 [B,Hkv,Sk,D], k_scale float32 [B,Hkv,ceil(Sk/32)], kbar float32
    [B,Hkv,D] or None); codes are in HND order whatever the input layout.
    """
    lib = _load()
    for n, t in (("q", q), ("k", k)):
        _need_cuda_contig(n, t)
    if q.dtype != k.dtype:
        raise ValueError("q and k must have the same dtype")
    B, Hq, Hkv, Sq, Sk, D = _dims(q, k, layout)
    dev = q.device
    qc = torch.empty((B, Hq, Sq, D), dtype=torch.int8, device=dev)
    qs = torch.empty((B, Hq, (Sq + 31) // 32), dtype=torch.float32, device=dev)
    kc = torch.empty((B, Hkv, Sk, D), dtype=torch.int8, device=dev)
    ks = torch.empty((B, Hkv, (Sk + 31) // 32), dtype=torch.float32, device=dev)
    kb = torch.empty((B, Hkv, D), dtype=torch.float32, device=dev) if smooth_k else None
    _check(lib.skv_sage_quant(_ptr(q), _ptr(k), B, Hq, Hkv, Sq, Sk, D, _dt(q),
                              SKV_HND if layout == "HND" else SKV_NHD, int(bool(smooth_k)),
                              _ptr(qc), _ptr(qs), _ptr(kc), _ptr(ks), _ptr(kb), _stream(dev)))
    return dict(q_codes=qc, q_scale=qs, k_codes=kc, k_scale=ks, kbar=kb)


def sage_fwd(q, k, v, scale=None, layout="HND", causal=False, smooth_k=True, return_lse=False,
             out=None, lse=None, workspace=None):
    """Attention with INT8 QK^T and half-precision P.V (skv_sage_fwd).

    Arguments and results as ``attn_fwd``; smoothing is on by default.  The LSE
    (float32 [B, Hq, Sq], log2) refers to the unsmoothed logits.  ``workspace``: a
    uint8 GPU tensor of at least ``sage_workspace_bytes(...)`` bytes, or None to
    allocate one.
    """
    lib = _load()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need_cuda_contig(n, t)
    if v.shape != k.shape or v.dtype != k.dtype or q.dtype != k.dtype:
        raise ValueError("k and v must match in shape, and q, k, v in dtype")
    B, Hq, Hkv, Sq, Sk, D = _dims(q, k, layout)
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty_like(q)
    _need_cuda_contig("out", out)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must have q's shape and dtype")
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need_cuda_contig("lse", lse)
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Sq):
            raise ValueError(f"lse must be float32 {(B, Hq, Sq)}")
    dt = _dt(q)
    ws_n = int(lib.skv_sage_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, dt, int(bool(smooth_k))))
    if workspace is None:
        workspace = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=q.device)
    _need_cuda_contig("workspace", workspace)
    if workspace.numel() * workspace.element_size() < ws_n:
        raise ValueError(f"workspace must hold {ws_n} bytes")
    _check(lib.skv_sage_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Sq, Sk,
                            D, dt, SKV_HND if layout == "HND" else SKV_NHD, float(scale),
                            int(bool(causal)), int(bool(smooth_k)), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(q.device)))
    return (out, lse) if (return_lse or lse is not None) else out
