"""Randomised shapes: every entry point against the oracle on shapes drawn from a
fixed seed.

The fixed-case tests pin chosen shapes (tile multiples, ragged tails, empty inputs);
this sweep draws 64 more per entry point (32 for the varlen and INT8 calls) -- batch, head counts and grouping, query
and key lengths from 1 to a few tiles past the tile size, head dimension, dtype,
layout, causal masking, smoothing, key offsets, split counts, filled KV lengths --
from numpy's default generator with seed 2026, so a shape class the chosen cases
missed still meets the parity bar.  Sizes stay small enough for the fp64 oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.tolerance import assert_lse_close, assert_out_close

pytestmark = pytest.mark.gpu

DEV = "cuda"
N_CASES = 64


@pytest.fixture(scope="module")
def skv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import split_kv_merge_amd as m
    m._load()
    return m


def _heads(g):
    hkv = int(g.choice([1, 2, 4, 8]))
    return hkv * int(g.choice([1, 2, 4, 8])), hkv


def _fwd_cases():
    g = np.random.default_rng(2026)
    out = []
    for i in range(N_CASES):
        hq, hkv = _heads(g)
        out.append(dict(B=int(g.integers(1, 4)), Hq=hq, Hkv=hkv, Sq=int(g.integers(1, 700)),
                        Sk=int(g.integers(1, 900)), D=int(g.choice([64, 128, 256])),
                        dtype=str(g.choice(["bf16", "fp16"])), layout=str(g.choice(["HND", "NHD"])),
                        causal=bool(g.integers(0, 2)), smooth=bool(g.integers(0, 2)),
                        k_offset=float(g.uniform(-3, 3)), seed=3000 + i))
    return out


@pytest.mark.parametrize("c", _fwd_cases(), ids=lambda c: f"s{c['seed']}")
def test_attn_fwd_random(skv, c):
    p = wl.attn_problem(c["B"], c["Hq"], c["Hkv"], c["Sq"], c["Sk"], c["D"], dtype=c["dtype"],
                        layout=c["layout"], seed=c["seed"], k_offset=c["k_offset"])
    ro, rl = oracle.attn(wl.bits(p.q), wl.bits(p.k), wl.bits(p.v), c["dtype"], c["layout"],
                         p.scale, c["causal"])
    out, lse = skv.attn_fwd(p.q.to(DEV), p.k.to(DEV), p.v.to(DEV), scale=p.scale,
                            layout=c["layout"], causal=c["causal"], smooth_k=c["smooth"],
                            return_lse=True)
    torch.cuda.synchronize()
    assert_lse_close(lse.cpu(), rl)
    assert_out_close(out.cpu(), ro)


def _varlen_cases():
    g = np.random.default_rng(2027)
    out = []
    for i in range(N_CASES // 2):
        hq, hkv = _heads(g)
        n = int(g.integers(1, 6))
        lq = [int(x) for x in g.integers(0, 600, size=n)]
        same = bool(g.integers(0, 2))
        lk = lq if same else [int(x) for x in g.integers(0, 700, size=n)]
        out.append(dict(Hq=hq, Hkv=hkv, lq=lq, lk=lk, D=int(g.choice([64, 128, 256])),
                        dtype=str(g.choice(["bf16", "fp16"])), causal=bool(g.integers(0, 2)),
                        smooth=bool(g.integers(0, 2)), seed=3100 + i))
    return out


@pytest.mark.parametrize("c", _varlen_cases(), ids=lambda c: f"s{c['seed']}")
def test_attn_fwd_varlen_random(skv, c):
    """Packed sequences of independent query and key lengths (zero-length ones too)."""
    gen = torch.Generator().manual_seed(c["seed"])
    T, Tk, D = sum(c["lq"]), sum(c["lk"]), c["D"]
    to = (lambda x: x.to(torch.bfloat16)) if c["dtype"] == "bf16" else (lambda x: x.to(torch.float16))
    q = to(torch.randn(max(T, 1), c["Hq"], D, generator=gen))[:T]
    k = to(torch.randn(max(Tk, 1), c["Hkv"], D, generator=gen) + 0.5)[:Tk]
    v = to(torch.randn(max(Tk, 1), c["Hkv"], D, generator=gen))[:Tk]
    cq = np.concatenate([[0], np.cumsum(c["lq"])]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(c["lk"])]).astype(np.int32)
    scale = wl.default_scale(D)
    if T == 0:
        pytest.skip("no query token drawn")
    ro, rl = oracle.attn_varlen(wl.bits(q), wl.bits(k.contiguous()), wl.bits(v.contiguous()),
                                c["dtype"], cq, ck, scale=scale, causal=c["causal"])
    out, lse = skv.attn_fwd_varlen(q.contiguous().to(DEV), k.contiguous().to(DEV),
                                   v.contiguous().to(DEV), torch.from_numpy(cq).to(DEV),
                                   torch.from_numpy(ck).to(DEV), max(c["lq"]), scale=scale,
                                   causal=c["causal"], smooth_k=c["smooth"], return_lse=True)
    torch.cuda.synchronize()
    assert_lse_close(lse.cpu(), rl)
    assert_out_close(out.cpu(), ro)


def _decode_cases():
    g = np.random.default_rng(2028)
    out = []
    for i in range(N_CASES):
        hkv = int(g.choice([1, 2, 4, 8]))
        grp = int(g.choice([1, 2, 4, 8, 16]))
        lq = int(g.integers(1, 16 // grp + 1))
        out.append(dict(B=int(g.integers(1, 5)), Hq=hkv * grp, Hkv=hkv, Lq=lq,
                        Lkv=int(g.integers(0, 5000)), D=int(g.choice([64, 128, 256])),
                        dtype=str(g.choice(["bf16", "fp16"])), layout=str(g.choice(["HND", "NHD"])),
                        S=int(g.choice([0, 1, 3, 8, 17, 64])), kv_len=bool(g.integers(0, 2)),
                        seed=3200 + i))
    return out


@pytest.mark.parametrize("c", _decode_cases(), ids=lambda c: f"s{c['seed']}")
def test_decode_random(skv, c):
    """The single-launch decode and the two-kernel form (partials, then merge_state)
    with a random split count (0: the heuristic's) and, half the time, random filled
    lengths per batch element."""
    B, Hq, Hkv, Lq, Lkv, D = c["B"], c["Hq"], c["Hkv"], c["Lq"], c["Lkv"], c["D"]
    p = wl.attn_problem(B, Hq, Hkv, Lq, Lkv, D, dtype=c["dtype"], layout=c["layout"],
                        seed=c["seed"])
    g = np.random.default_rng(c["seed"])
    lens = g.integers(0, Lkv + 1, size=B).astype(np.int32) if c["kv_len"] else None
    S = c["S"] or skv.pick_num_splits(B, Hkv, (Hq // Hkv) * Lq, Lkv, D)
    # oracle: dense attention over each element's filled keys
    outs, lses = [], []
    for b in range(B):
        L = Lkv if lens is None else int(lens[b])
        sl = (slice(b, b + 1), slice(None), slice(0, L)) if c["layout"] == "HND" else \
             (slice(b, b + 1), slice(0, L))
        o, l = oracle.attn(wl.bits(p.q[b:b + 1]), wl.bits(p.k[sl].contiguous()),
                           wl.bits(p.v[sl].contiguous()), c["dtype"], c["layout"], p.scale)
        outs.append(o)
        lses.append(l)
    ro, rl = np.concatenate(outs), np.concatenate(lses)
    q, k, v = p.q.to(DEV), p.k.to(DEV), p.v.to(DEV)
    kvl = None if lens is None else torch.from_numpy(lens).to(DEV)
    out, lse = skv.attn_splitkv_decode(q, k, v, num_splits=min(S, 256), scale=p.scale,
                                       layout=c["layout"], kv_len=kvl)
    op, lp = skv.attn_splitkv_partial(q, k, v, num_splits=S, scale=p.scale, layout=c["layout"],
                                      kv_len=kvl)
    if c["layout"] == "HND":
        out2, lse2 = skv.merge_state(op, lp, out_dtype=q.dtype)
    else:   # partial outputs in q's [B, Lq, Hq] row order, partial LSEs [B, Hq, Lq]
        out2, lse2 = skv.merge_state(op, lp.transpose(2, 3), out_dtype=q.dtype)
        lse2 = lse2.transpose(1, 2)
    torch.cuda.synchronize()
    for o, l in ((out, lse), (out2, lse2)):
        assert_lse_close(l.cpu(), rl)
        assert_out_close(o.cpu(), ro)


def _sage_cases():
    g = np.random.default_rng(2029)
    out = []
    for i in range(N_CASES // 2):
        hq, hkv = _heads(g)
        out.append(dict(B=int(g.integers(1, 3)), Hq=hq, Hkv=hkv, Sq=int(g.integers(1, 600)),
                        Sk=int(g.integers(0, 800)), D=int(g.choice([64, 128])),
                        dtype=str(g.choice(["bf16", "fp16"])), layout=str(g.choice(["HND", "NHD"])),
                        causal=bool(g.integers(0, 2)), smooth=bool(g.integers(0, 2)),
                        k_offset=float(g.uniform(-3, 3)), seed=3300 + i))
    return out


@pytest.mark.parametrize("c", _sage_cases(), ids=lambda c: f"s{c['seed']}")
def test_sage_fwd_random(skv, c):
    p = wl.attn_problem(c["B"], c["Hq"], c["Hkv"], c["Sq"], c["Sk"], c["D"], dtype=c["dtype"],
                        layout=c["layout"], seed=c["seed"], k_offset=c["k_offset"])
    ro, rl = oracle.sage_attn(wl.bits(p.q), wl.bits(p.k), wl.bits(p.v), c["dtype"], c["layout"],
                              scale=p.scale, causal=c["causal"], smooth_k=c["smooth"])
    out, lse = skv.sage_fwd(p.q.to(DEV), p.k.to(DEV), p.v.to(DEV), scale=p.scale,
                            layout=c["layout"], causal=c["causal"], smooth_k=c["smooth"],
                            return_lse=True)
    torch.cuda.synchronize()
    assert_lse_close(lse.cpu(), rl)
    assert_out_close(out.cpu(), ro)
