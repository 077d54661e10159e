"""fp64 CPU oracle for attention with a per-row log2 LSE, split-KV partials and merge.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with the
HIP library and imports nothing from it.

The arithmetic lives in ``oracle.c`` (plain loops in double precision, OpenMP over
rows); this module only marshals numpy arrays through ctypes.  Inputs are the raw
16-bit patterns (``numpy.uint16``) of bf16 / fp16 tensors, decoded inside the C
code, so the oracle consumes exactly the values handed to the GPU.

Which page passage each routine follows is stated next to the C function.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

BF16, FP16 = 0, 1
HND, NHD = 0, 1

_lib = None


def build() -> str:
    """Compile liboracle.so with gcc (plain -O2, no fast-math: inf/NaN must survive)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-o", LIB_PATH + ".tmp", SRC_PATH, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    D = ctypes.c_double
    I64 = ctypes.c_int64
    lib.oracle_decode.argtypes = [P, I64, I, P]
    lib.oracle_decode.restype = None
    lib.oracle_kmean.argtypes = [P, I, I, I, I, I, I, P]
    lib.oracle_kmean.restype = None
    lib.oracle_attn.argtypes = [P, P, P, I, I, I, I, I, I, I, I, D, I, I, P, P]
    lib.oracle_attn.restype = I
    lib.oracle_attn_rows.argtypes = [P, P, P, I, I, I, I, I, I, I, I, D, I, P, I64, P, P]
    lib.oracle_attn_rows.restype = I
    lib.oracle_attn_varlen.argtypes = [P, P, P, I, P, P, I, I, I, I, D, I, P, P]
    lib.oracle_attn_varlen.restype = I
    lib.oracle_splitkv_partials.argtypes = [P, P, P, I, I, I, I, I, I, I, I, D, I, P, P]
    lib.oracle_splitkv_partials.restype = I
    lib.oracle_merge.argtypes = [I, I64, I, P, P, P, P]
    lib.oracle_merge.restype = None
    lib.oracle_sage_kbar.argtypes = [P, I, I, I, I, I, I, P]
    lib.oracle_sage_kbar.restype = None
    lib.oracle_sage_quant.argtypes = [P, I, I, I, I, I, I, P, P, P]
    lib.oracle_sage_quant.restype = I
    lib.oracle_sage_attn.argtypes = [P, P, P, I, I, I, I, I, I, I, I, D, I, I, P, I64, P, P]
    lib.oracle_sage_attn.restype = I
    _lib = lib
    return lib


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected raw 16-bit patterns (uint16), got {a.dtype}")
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dt(dtype) -> int:
    if dtype in (BF16, "bf16", "bfloat16"):
        return BF16
    if dtype in (FP16, "fp16", "float16"):
        return FP16
    raise ValueError(f"unknown dtype {dtype!r}")


def _lay(layout) -> int:
    if layout in (HND, "HND"):
        return HND
    if layout in (NHD, "NHD"):
        return NHD
    raise ValueError(f"unknown layout {layout!r}")


def _dims(q, k, layout):
    """(B, Hq, Hkv, Sq, Sk, D) from 4-D HND [B,H,S,D] or NHD [B,S,H,D] arrays."""
    if q.ndim != 4 or k.ndim != 4:
        raise ValueError("q and k must be 4-D")
    if _lay(layout) == HND:
        B, Hq, Sq, D = q.shape
        _, Hkv, Sk, _ = k.shape
    else:
        B, Sq, Hq, D = q.shape
        _, Sk, Hkv, _ = k.shape
    return B, Hq, Hkv, Sq, Sk, D


def decode(bits, dtype) -> np.ndarray:
    """Decode raw bf16/fp16 patterns to float64 with the oracle's own decoder."""
    a = _u16(bits)
    out = np.empty(a.shape, np.float64)
    _load().oracle_decode(_ptr(a), a.size, _dt(dtype), _ptr(out))
    return out


def kmean(k, dtype, layout="HND") -> np.ndarray:
    """mean over keys of k per (batch, kv head), float64 [B, Hkv, D]."""
    k = _u16(k)
    if _lay(layout) == HND:
        B, Hkv, Sk, D = k.shape
    else:
        B, Sk, Hkv, D = k.shape
    out = np.empty((B, Hkv, D), np.float64)
    _load().oracle_kmean(_ptr(k), _dt(dtype), _lay(layout), B, Hkv, Sk, D, _ptr(out))
    return out


def attn(q, k, v, dtype, layout="HND", scale=None, causal=False, smoothed=False):
    """Dense attention: (out float64 in q's layout, lse float64 [B, Hq, Sq] in log2).

    ``scale`` defaults to D**-0.5 rounded to float32, the value the GPU receives.
    ``smoothed=True`` returns the LSE of the smoothed logits (k - mean(k)) with no
    add-back; it exists only for the add-back identity check.
    """
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, Hq, Hkv, Sq, Sk, D = _dims(q, k, layout)
    if v.shape != k.shape:
        raise ValueError("v must have k's shape")
    if scale is None:
        scale = float(np.float32(D ** -0.5))
    out = np.empty(q.shape, np.float64)
    lse = np.empty((B, Hq, Sq), np.float64)
    rc = _load().oracle_attn(_ptr(q), _ptr(k), _ptr(v), _dt(dtype), _lay(layout), B, Hq, Hkv,
                             Sq, Sk, D, float(scale), int(bool(causal)), int(bool(smoothed)),
                             _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_attn rejected its arguments")
    return out, lse


def attn_rows(q, k, v, dtype, rows, layout="HND", scale=None, causal=False):
    """Attention for selected rows only; rows is an int array of (b, h, i) triples.

    Returns (out float64 [n, D], lse float64 [n]).
    """
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, Hq, Hkv, Sq, Sk, D = _dims(q, k, layout)
    rows = np.ascontiguousarray(np.asarray(rows, np.int64).reshape(-1, 3))
    n = rows.shape[0]
    if scale is None:
        scale = float(np.float32(D ** -0.5))
    out = np.empty((n, D), np.float64)
    lse = np.empty((n,), np.float64)
    rc = _load().oracle_attn_rows(_ptr(q), _ptr(k), _ptr(v), _dt(dtype), _lay(layout), B, Hq,
                                  Hkv, Sq, Sk, D, float(scale), int(bool(causal)), _ptr(rows),
                                  n, _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_attn_rows rejected its arguments")
    return out, lse


def attn_varlen(q, k, v, dtype, cu_seqlens_q, cu_seqlens_k, scale=None, causal=False):
    """Packed varlen attention: q [total_q,Hq,D], k/v [total_k,Hkv,D].

    Returns (out float64 [total_q, Hq, D], lse float64 [Hq, total_q] in log2).
    """
    q, k, v = _u16(q), _u16(k), _u16(v)
    cu_q = np.ascontiguousarray(np.asarray(cu_seqlens_q, np.int32))
    cu_k = np.ascontiguousarray(np.asarray(cu_seqlens_k, np.int32))
    total_q, Hq, D = q.shape
    _, Hkv, _ = k.shape
    nseq = cu_q.size - 1
    if cu_k.size != nseq + 1 or cu_q[-1] != total_q or cu_k[-1] != k.shape[0]:
        raise ValueError("cu_seqlens do not match the packed tensors")
    if scale is None:
        scale = float(np.float32(D ** -0.5))
    out = np.empty(q.shape, np.float64)
    lse = np.empty((Hq, total_q), np.float64)
    rc = _load().oracle_attn_varlen(_ptr(q), _ptr(k), _ptr(v), _dt(dtype), _ptr(cu_q),
                                    _ptr(cu_k), nseq, Hq, Hkv, D, float(scale),
                                    int(bool(causal)), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_attn_varlen rejected its arguments")
    return out, lse


def splitkv_partials(q, k, v, dtype, num_splits, layout="HND", scale=None):
    """Per-chunk partial states: (o float64 [S,B,Hq,Lq,D], lse float64 [S,B,Hq,Lq])."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, Hq, Hkv, Lq, Lkv, D = _dims(q, k, layout)
    if scale is None:
        scale = float(np.float32(D ** -0.5))
    S = int(num_splits)
    o = np.empty((S, B, Hq, Lq, D), np.float64)
    lse = np.empty((S, B, Hq, Lq), np.float64)
    rc = _load().oracle_splitkv_partials(_ptr(q), _ptr(k), _ptr(v), _dt(dtype), _lay(layout),
                                         B, Hq, Hkv, Lq, Lkv, D, float(scale), S, _ptr(o),
                                         _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_splitkv_partials rejected its arguments")
    return o, lse


def merge(o_parts, lse_parts):
    """Stable LSE-weighted merge of S partial states.

    o_parts [S, ..., D] and lse_parts [S, ...] (float64); returns (out [..., D], lse [...]).
    """
    o = np.ascontiguousarray(np.asarray(o_parts, np.float64))
    l = np.ascontiguousarray(np.asarray(lse_parts, np.float64))
    S = o.shape[0]
    D = o.shape[-1]
    if l.shape != o.shape[:-1]:
        raise ValueError("lse_parts must be o_parts without its last axis")
    R = int(np.prod(l.shape[1:], dtype=np.int64))
    out = np.empty(o.shape[1:], np.float64)
    lse = np.empty(l.shape[1:], np.float64)
    _load().oracle_merge(S, R, D, _ptr(o), _ptr(l), _ptr(out), _ptr(lse))
    return out, lse


# ----------------------------------------------------- INT8 QK^T (Sage-v1 reading)

SAGE_BLOCK = 32  # rows (query rows or keys) per quantisation block


def sage_kbar(k, dtype, layout="HND") -> np.ndarray:
    """mean(k) over keys per (batch, kv head), exact then rounded to float32 [B, Hkv, D]."""
    k = _u16(k)
    if _lay(layout) == HND:
        B, Hkv, Sk, D = k.shape
    else:
        B, Sk, Hkv, D = k.shape
    out = np.empty((B, Hkv, D), np.float32)
    _load().oracle_sage_kbar(_ptr(k), _dt(dtype), _lay(layout), B, Hkv, Sk, D, _ptr(out))
    return out


def sage_quant_tensor(x, dtype, layout="HND", center=None):
    """Per-block INT8 codes of x (minus center [B,H,D] float32 if given).

    Returns (codes int8 [B,H,S,D] in HND order, scales float32 [B,H,ceil(S/32)]).
    """
    x = _u16(x)
    if x.ndim != 4:
        raise ValueError("x must be 4-D")
    if _lay(layout) == HND:
        B, H, S, D = x.shape
    else:
        B, S, H, D = x.shape
    nb = (S + SAGE_BLOCK - 1) // SAGE_BLOCK
    codes = np.empty((B, H, S, D), np.int8)
    scales = np.empty((B, H, nb), np.float32)
    c = None
    if center is not None:
        c = np.ascontiguousarray(np.asarray(center, np.float32))
        if c.shape != (B, H, D):
            raise ValueError("center must be [B, H, D]")
    rc = _load().oracle_sage_quant(_ptr(x), _dt(dtype), _lay(layout), B, H, S, D,
                                   _ptr(c) if c is not None else None, _ptr(codes),
                                   _ptr(scales))
    if rc != 0:
        raise ValueError("oracle_sage_quant rejected its arguments")
    return codes, scales


def sage_quant(q, k, dtype, layout="HND", smooth_k=True):
    """The quantisation step of the INT8 path.

    Returns dict(q_codes, q_scale, k_codes, k_scale, kbar) with kbar float32
    [B, Hkv, D] (zeros without smoothing); codes are HND-ordered int8.
    """
    q, k = _u16(q), _u16(k)
    B, Hq, Hkv, Sq, Sk, D = _dims(q, k, layout)
    kbar = sage_kbar(k, dtype, layout) if smooth_k else np.zeros((B, Hkv, D), np.float32)
    qc, qs = sage_quant_tensor(q, dtype, layout)
    kc, ks = sage_quant_tensor(k, dtype, layout, kbar if smooth_k else None)
    return dict(q_codes=qc, q_scale=qs, k_codes=kc, k_scale=ks, kbar=kbar)


def sage_attn(q, k, v, dtype, layout="HND", scale=None, causal=False, smooth_k=True, rows=None):
    """INT8-QK^T attention: (out float64, lse float64 in log2 with the add-back).

    rows=None: out in q's layout and lse [B, Hq, Sq]; else rows is an int array of
    (b, h, i) triples and out is [n, D], lse [n].
    """
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, Hq, Hkv, Sq, Sk, D = _dims(q, k, layout)
    if v.shape != k.shape:
        raise ValueError("v must have k's shape")
    if scale is None:
        scale = float(np.float32(D ** -0.5))
    if rows is None:
        r, n = None, 0
        out = np.empty(q.shape, np.float64)
        lse = np.empty((B, Hq, Sq), np.float64)
    else:
        r = np.ascontiguousarray(np.asarray(rows, np.int64).reshape(-1, 3))
        n = r.shape[0]
        out = np.empty((n, D), np.float64)
        lse = np.empty((n,), np.float64)
    rc = _load().oracle_sage_attn(_ptr(q), _ptr(k), _ptr(v), _dt(dtype), _lay(layout), B, Hq,
                                  Hkv, Sq, Sk, D, float(scale), int(bool(causal)),
                                  int(bool(smooth_k)), _ptr(r) if r is not None else None, n,
                                  _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_sage_attn rejected its arguments")
    return out, lse
