"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random tensors and lays them out; it holds none of the
attention arithmetic.  Both the HIP path and the fp64 oracle consume the tensors
it returns (the oracle through their raw 16-bit patterns, see ``bits``).

Recipe, shared by every generator: a ``torch.Generator("cpu")`` seeded with the
given seed; fp32 draws first, scaled or offset in fp32, then rounded to the
16-bit dtype (round-to-nearest-even), which is how the ARK return_lse bug report
(auto-round #2556, Reproduction Steps) builds its rows of distinct magnitude.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw 16-bit patterns of a bf16/fp16 CPU tensor as a contiguous numpy uint16 array."""
    if t.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"expected a 16-bit float tensor, got {t.dtype}")
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def default_scale(D: int) -> float:
    """D**-0.5 rounded to float32: the value that crosses the C ABI."""
    return float(np.float32(D ** -0.5))


def _to(x: torch.Tensor, dtype) -> torch.Tensor:
    return x.to(DTYPES[dtype] if isinstance(dtype, str) else dtype)


def hnd_to_nhd(t: torch.Tensor) -> torch.Tensor:
    """[B,H,S,D] -> contiguous [B,S,H,D]."""
    return t.transpose(1, 2).contiguous()


@dataclass
class Attn:
    """One dense attention problem (HND or NHD, contiguous CPU tensors)."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    layout: str
    scale: float
    causal: bool = False
    meta: dict = field(default_factory=dict)

    @property
    def dims(self):
        """(B, Hq, Hkv, Sq, Sk, D)."""
        if self.layout == "HND":
            B, Hq, Sq, D = self.q.shape
            Hkv, Sk = self.k.shape[1], self.k.shape[2]
        else:
            B, Sq, Hq, D = self.q.shape
            Sk, Hkv = self.k.shape[1], self.k.shape[2]
        return B, Hq, Hkv, Sq, Sk, D


def attn_problem(B, Hq, Hkv, Sq, Sk, D, dtype="bf16", layout="HND", seed=0,
                 q_mag=(0.25, 4.0), k_offset=0.0, q_mul=1.0, causal=False) -> Attn:
    """Generic problem: q/k/v ~ N(0,1); each q row times a magnitude ~ U(q_mag) (one
    scalar per (b, h, row)), times q_mul; k + k_offset; all in fp32 before one rounding."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, Sq, D, generator=g)
    if q_mag is not None:
        lo, hi = q_mag
        q = q * (lo + (hi - lo) * torch.rand(B, Hq, Sq, 1, generator=g))
    q = _to(q * q_mul, dtype)
    k = _to(torch.randn(B, Hkv, Sk, D, generator=g) + k_offset, dtype)
    v = _to(torch.randn(B, Hkv, Sk, D, generator=g), dtype)
    if layout == "NHD":
        q, k, v = hnd_to_nhd(q), hnd_to_nhd(k), hnd_to_nhd(v)
    return Attn(q, k, v, layout, default_scale(D), causal,
                dict(seed=seed, q_mag=q_mag, k_offset=k_offset, q_mul=q_mul))


# ------------------------------------------------------------------ config 1

def tiny_lse(seed=0, dtype="bf16"):
    """Config 1, the shape of the ARK return_lse report (auto-round #2556, Reproduction
    Steps): batch 1, 4 heads, 64 queries, 1000 keys, head dim 128, HND, scale D**-0.5.

    Draws q, k, v ~ N(0,1) (in that order, each rounded once) and derives three inputs
    from them: ``q_graded``, whose query row i carries the magnitude 0.25 + 3.75 i / 63
    (evenly spaced from 0.25 to 4), so every row has its own LSE; ``q_grouped``, where
    each group of 16 consecutive rows repeats the group's first graded row, the control
    in which a 16-row-block LSE bug is invisible; and ``k_shifted`` = k + 0.5, a common
    key offset that smoothing must absorb.
    """
    n_q, n_k, d = 64, 1000, 128
    gen = torch.Generator().manual_seed(seed)
    q, k, v = (_to(torch.randn(1, 4, n, d, generator=gen), dtype) for n in (n_q, n_k, n_k))
    magnitude = torch.linspace(0.25, 4.0, n_q)
    graded = _to(q.float() * magnitude[:, None], dtype)
    group_lead = (torch.arange(n_q) // 16) * 16
    grouped = graded.index_select(2, group_lead)
    shifted = _to(k.float() + 0.5, dtype)
    return dict(q=q, k=k, v=v, q_graded=graded, q_grouped=grouped, k_shifted=shifted,
                scale=default_scale(d), B=1, H=4, Sq=n_q, Sk=n_k, D=d, seed=seed)


# ------------------------------------------------------------------ config 2

def decode_gqa(Lkv, seed=None, B=8, Hq=32, Hkv=8, Lq=1, D=128, dtype="bf16"):
    """Split-KV decode with GQA: q [B,Hq,Lq,D] ~ N(0,1) times U(0.25,4) per row;
    K, V [B,Hkv,Lkv,D] ~ N(0,1), HND.  K and V are drawn one batch element at a
    time (k[b] then v[b]) to bound host memory.  Default seeds 21/22/23 for
    Lkv 4096/8192/32768."""
    if seed is None:
        seed = {4096: 21, 8192: 22, 32768: 23}.get(Lkv, 20)
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, Lq, D, generator=g)
    q = _to(q * (0.25 + 3.75 * torch.rand(B, Hq, Lq, 1, generator=g)), dtype)
    k = torch.empty(B, Hkv, Lkv, D, dtype=DTYPES[dtype])
    v = torch.empty_like(k)
    for b in range(B):
        k[b] = _to(torch.randn(Hkv, Lkv, D, generator=g), dtype)
        v[b] = _to(torch.randn(Hkv, Lkv, D, generator=g), dtype)
    return Attn(q, k, v, "HND", default_scale(D), False, dict(seed=seed, Lkv=Lkv))


# ------------------------------------------------------------------ config 3

def wide_decode(Lkv, sign=+1, seed=None, B=4, Hq=16, Hkv=4, Lq=4, D=256, dtype="bf16"):
    """Wide heads and a large score range: q = 8 * N(0,1) [B,Hq,Lq,D];
    K = N(0,1) + 2*sign; V ~ N(0,1); HND, non-causal."""
    if seed is None:
        seed = {(16384, 1): 31, (16384, -1): 32, (32768, 1): 33, (32768, -1): 34}.get(
            (Lkv, sign), 30)
    g = torch.Generator().manual_seed(seed)
    q = _to(8.0 * torch.randn(B, Hq, Lq, D, generator=g), dtype)
    k = torch.empty(B, Hkv, Lkv, D, dtype=DTYPES[dtype])
    v = torch.empty_like(k)
    for b in range(B):
        k[b] = _to(torch.randn(Hkv, Lkv, D, generator=g) + 2.0 * sign, dtype)
        v[b] = _to(torch.randn(Hkv, Lkv, D, generator=g), dtype)
    return Attn(q, k, v, "HND", default_scale(D), False, dict(seed=seed, Lkv=Lkv, sign=sign))


def extreme_logits(sign=+1, Lkv=4096, B=1, Hq=16, Hkv=4, Lq=1, D=256, seed=35, dtype="bf16"):
    """Overflow (sign=+1) / underflow (sign=-1) fixture: q = 4*sign everywhere,
    K = N(0,1) + 2, so every logit is about sign * 128 nats: outside the fp32 exp
    range at any fixed offset."""
    g = torch.Generator().manual_seed(seed)
    q = _to(torch.full((B, Hq, Lq, D), 4.0 * sign), dtype)
    k = _to(torch.randn(B, Hkv, Lkv, D, generator=g) + 2.0, dtype)
    v = _to(torch.randn(B, Hkv, Lkv, D, generator=g), dtype)
    return Attn(q, k, v, "HND", default_scale(D), False, dict(seed=seed, sign=sign))


# ------------------------------------------------------------------ config 4

@dataclass
class Varlen:
    q: torch.Tensor          # [total_q, Hq, D]
    k: torch.Tensor          # [total_k, Hkv, D]
    v: torch.Tensor
    cu_seqlens_q: torch.Tensor   # int32 [nseq+1]
    cu_seqlens_k: torch.Tensor
    lengths: list
    scale: float
    causal: bool
    meta: dict = field(default_factory=dict)


def varlen_prefill(seed=4, nseq=16, lo=128, hi=4096, Hq=32, Hkv=8, D=128, dtype="bf16",
                   causal=True, lengths=None):
    """Packed prefill: nseq lengths ~ U[lo, hi] (integers, inclusive), q [T,Hq,D]
    ~ N(0,1) times U(0.25,4) per (token, head), K/V [T,Hkv,D] ~ N(0,1), NHD packed,
    cu_seqlens int32.  Query and key lengths are equal per sequence."""
    g = torch.Generator().manual_seed(seed)
    if lengths is None:
        lengths = torch.randint(lo, hi + 1, (nseq,), generator=g).tolist()
    T = int(sum(lengths))
    q = torch.randn(T, Hq, D, generator=g)
    q = _to(q * (0.25 + 3.75 * torch.rand(T, Hq, 1, generator=g)), dtype)
    k = _to(torch.randn(T, Hkv, D, generator=g), dtype)
    v = _to(torch.randn(T, Hkv, D, generator=g), dtype)
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return Varlen(q, k, v, cu, cu.clone(), list(lengths), default_scale(D), causal,
                  dict(seed=seed, T=T))


# ------------------------------------------------------------------ config 5

def ring_chunks(seed=5, B=1, H=16, S=8192, D=64, n_chunks=4, dtype="fp16"):
    """Ring-attention-style chunked prefill: q, k, v [B,H,S,D] ~ N(0,1); K chunk c
    (keys [c*S/n, (c+1)*S/n)) gets its own scalar offset ~ U(-1,1) added in fp32
    before rounding.  The chunks come back as separate contiguous tensors, the way
    a ring hop delivers them; k/v also hold the full (concatenated) tensors."""
    g = torch.Generator().manual_seed(seed)
    q = _to(torch.randn(B, H, S, D, generator=g), dtype)
    offs = (2.0 * torch.rand(n_chunks, generator=g) - 1.0).tolist()
    kf = torch.randn(B, H, S, D, generator=g)
    v = _to(torch.randn(B, H, S, D, generator=g), dtype)
    n = S // n_chunks
    for c in range(n_chunks):
        kf[:, :, c * n:(c + 1) * n] += offs[c]
    k = _to(kf, dtype)
    k_chunks = [k[:, :, c * n:(c + 1) * n].contiguous() for c in range(n_chunks)]
    v_chunks = [v[:, :, c * n:(c + 1) * n].contiguous() for c in range(n_chunks)]
    return dict(q=q, k=k, v=v, k_chunks=k_chunks, v_chunks=v_chunks, offsets=offs,
                scale=default_scale(D), seed=seed)


def prefill_flops(lengths, Hq, D, causal=True):
    """Algorithmic flops of attention: 4*D per attended (query, key) pair (QK^T and
    PV, a multiply-add each); with causal masking only the lower triangle counts."""
    pairs = sum((L * (L + 1)) // 2 if causal else L * L for L in lengths)
    return 4 * Hq * D * pairs
