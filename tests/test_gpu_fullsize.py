"""GPU parity at the measured sizes, in the launch configuration bench.py times.

Decode problems have 256 query rows: the oracle computes every one (about a second
each), and every row is compared.  The prefill problems are too large for the oracle
whole, so they compare a seeded sample of query rows (always including the first and
last row of every batch element or sequence) with the oracle's per-row attention.
Every row of the output is also checked for what holds at any size: it is finite
(each row here sees at least one key), and for decode it lies inside the per-column
range of V over the keys its head reads (a softmax average of V's rows cannot leave
that range).
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


@pytest.fixture(scope="module")
def skv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import split_kv_merge_amd as m
    m._load()
    return m


def _sample_rows(B, H, L, n, seed):
    """n seeded (b, h, i) triples plus the first and last row of every b."""
    g = np.random.default_rng(seed)
    rows = [(b, h, i) for b in range(B) for (h, i) in ((0, 0), (H - 1, L - 1))]
    rows += [(int(g.integers(B)), int(g.integers(H)), int(g.integers(L))) for _ in range(n)]
    return np.array(sorted(set(rows)), np.int64)


_PROBLEMS = {}


def _decode_problem(kind, *key):
    """Generated once per module: (problem, oracle out, oracle lse) of a full-size decode
    problem; the oracle runs over every query row (256 rows per problem)."""
    if (kind,) + key not in _PROBLEMS:
        p = wl.decode_gqa(*key) if kind == "gqa" else wl.wide_decode(*key)
        ro, rl = oracle.attn(wl.bits(p.q), wl.bits(p.k), wl.bits(p.v), "bf16", scale=p.scale)
        _PROBLEMS.clear()            # keep one problem's tensors alive at a time
        _PROBLEMS[(kind,) + key] = (p, ro, rl)
    return _PROBLEMS[(kind,) + key]


def _check_decode_rows(p, out, lse, ro, rl):
    """Every row against the oracle, plus the range property: a softmax average of V's
    rows stays inside the per-column range of V over the keys its head reads."""
    B, Hq, Hkv, Lq, Lkv, D = p.dims
    G = Hq // Hkv
    v = p.v.to(DEV)
    vmin = v.float().amin(dim=2).repeat_interleave(G, dim=1)[:, :, None, :]
    vmax = v.float().amax(dim=2).repeat_interleave(G, dim=1)[:, :, None, :]
    torch.cuda.synchronize()
    o = out.float()
    assert torch.isfinite(lse).all() and torch.isfinite(o).all()
    slack = 1e-2 + 1e-2 * torch.maximum(vmin.abs(), vmax.abs())
    assert ((o >= vmin - slack) & (o <= vmax + slack)).all()
    assert_lse_close(lse.cpu(), rl)
    assert_out_close(o.cpu(), ro)


def _single_launch(skv, p, S):
    B, Hq, Hkv, Lq, Lkv, D = p.dims
    q, k, v = p.q.to(DEV), p.k.to(DEV), p.v.to(DEV)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, Lq), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.zeros(skv.splitkv_workspace_bytes(B, Hq, Lq, D, S, Hkv), dtype=torch.uint8,
                     device=DEV)
    skv.attn_splitkv_decode(q, k, v, num_splits=S, scale=p.scale, out=out, lse=lse, workspace=ws)
    return out, lse


@pytest.mark.parametrize("S", [0, 8, 16, 32])
@pytest.mark.parametrize("Lkv", [4096, 8192, 32768])
def test_decode_gqa_full_size(skv, Lkv, S):
    """B8 Hq32 Hkv8 Lq1 D128 bf16 decode, all 256 rows against the oracle.

    S = 0: the split count pick_num_splits chooses, in one launch (partials + in-kernel
    merge), as bench.py times it.  S = 8, 16, 32: config 2 as written, the keys split
    into S chunks: every chunk's partial (out, LSE) against the oracle's partial of that
    chunk, their merge_state against the oracle's unsplit run, and the single-launch
    decode at the same S against it too."""
    p, ro, rl = _decode_problem("gqa", Lkv)
    B, Hq, Hkv, Lq, Lkv, D = p.dims
    if S == 0:
        out, lse = _single_launch(skv, p, skv.pick_num_splits(B, Hkv, (Hq // Hkv) * Lq, Lkv, D))
        _check_decode_rows(p, out, lse, ro, rl)
        return
    q, k, v = p.q.to(DEV), p.k.to(DEV), p.v.to(DEV)
    op = torch.full((S,) + tuple(q.shape), float("nan"), dtype=torch.float32, device=DEV)
    lp = torch.full((S, B, Hq, Lq), float("nan"), dtype=torch.float32, device=DEV)
    skv.attn_splitkv_partial(q, k, v, num_splits=S, scale=p.scale, out_part=op, lse_part=lp)
    mo = torch.full_like(q, float("nan"))
    ml = torch.full((B, Hq, Lq), float("nan"), dtype=torch.float32, device=DEV)
    skv.merge_state(op, lp, out=mo, lse=ml)
    torch.cuda.synchronize()
    po, pl = oracle.splitkv_partials(wl.bits(p.q), wl.bits(p.k), wl.bits(p.v), "bf16", S,
                                     scale=p.scale)
    assert_lse_close(lp.cpu(), pl, "partial lse")
    assert_out_close(op.cpu(), po, "partial out")
    _check_decode_rows(p, mo, ml, ro, rl)
    out, lse = _single_launch(skv, p, S)
    _check_decode_rows(p, out, lse, ro, rl)


@pytest.mark.parametrize("Lkv,sign", [(16384, 1), (16384, -1), (32768, 1), (32768, -1)])
def test_wide_decode_full_size(skv, Lkv, sign):
    """B4 Hq16 Hkv4 Lq4 D256 decode, q = 8 N(0,1), K offset by +-2 (score range of
    hundreds of nats), the split count bench.py uses: all 256 rows."""
    p, ro, rl = _decode_problem("wide", Lkv, sign)
    B, Hq, Hkv, Lq, Lkv, D = p.dims
    S = skv.pick_num_splits(B, Hkv, (Hq // Hkv) * Lq, Lkv, D)
    out, lse = _single_launch(skv, p, S)
    _check_decode_rows(p, out, lse, ro, rl)


@pytest.mark.parametrize("G", [8, 16])
def test_many_row_decode_full_size(skv, G):
    """B8 Hkv8 Lkv8192 D128 decode with G query heads per kv head at Lq = 4 (32 and 64
    rows per kv head), the problems of bench.py's many-row lines, at the split count it
    uses: 160 sampled rows (plus the first and last of every batch element) against the
    oracle, every row against the range property."""
    p = wl.decode_gqa(8192, seed=40 + G, Hq=8 * G, Lq=4)
    B, Hq, Hkv, Lq, Lkv, D = p.dims
    S = skv.pick_num_splits(B, Hkv, G * Lq, Lkv, D)
    out, lse = _single_launch(skv, p, S)
    v = p.v.to(DEV)
    vmin = v.float().amin(dim=2).repeat_interleave(G, dim=1)[:, :, None, :]
    vmax = v.float().amax(dim=2).repeat_interleave(G, dim=1)[:, :, None, :]
    torch.cuda.synchronize()
    o = out.float()
    assert torch.isfinite(lse).all() and torch.isfinite(o).all()
    slack = 1e-2 + 1e-2 * torch.maximum(vmin.abs(), vmax.abs())
    assert ((o >= vmin - slack) & (o <= vmax + slack)).all()
    rows = _sample_rows(B, Hq, Lq, 160, seed=60 + G)
    ro, rl = oracle.attn_rows(wl.bits(p.q), wl.bits(p.k), wl.bits(p.v), "bf16", rows,
                              scale=p.scale)
    o_c, l_c = o.cpu().numpy(), lse.cpu().numpy()
    assert_lse_close(np.array([l_c[b, h, i] for b, h, i in rows]), rl, "lse")
    assert_out_close(np.stack([o_c[b, h, i] for b, h, i in rows]), ro, "out")


def test_varlen_causal_full_size(skv):
    """16 packed sequences, lengths U[128, 4096], Hq32 Hkv8 D128 bf16, causal."""
    vl = wl.varlen_prefill(seed=4)
    q, k, v = vl.q.to(DEV), vl.k.to(DEV), vl.v.to(DEV)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((q.shape[1], q.shape[0]), float("nan"), dtype=torch.float32, device=DEV)
    skv.attn_fwd_varlen(q, k, v, vl.cu_seqlens_q.to(DEV), vl.cu_seqlens_k.to(DEV),
                        max(vl.lengths), scale=vl.scale, causal=True, out=out, lse=lse)
    torch.cuda.synchronize()
    o_c, l_c = out.float().cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(o_c).all() and np.isfinite(l_c).all()
    cu = vl.cu_seqlens_q.tolist()
    Hq = q.shape[1]
    for s in range(len(vl.lengths)):
        a, e = cu[s], cu[s + 1]
        L = e - a
        # one sequence = a B=1 NHD problem; rows (0, h, i) in that sequence
        rows = _sample_rows(1, Hq, L, 6, seed=100 + s)
        qs, ks, vs = (wl.bits(t[a:e])[None] for t in (vl.q, vl.k, vl.v))
        ro, rl = oracle.attn_rows(qs, ks, vs, "bf16", rows, layout="NHD", scale=vl.scale,
                                  causal=True)
        got_o = np.stack([o_c[a + i, h] for _, h, i in rows])
        got_l = np.array([l_c[h, a + i] for _, h, i in rows])
        assert_lse_close(got_l, rl, f"seq {s} lse")
        assert_out_close(got_o, ro, f"seq {s} out")


def _ring_outputs(skv, rc):
    q = rc["q"].to(DEV)
    H, S = q.shape[1], q.shape[2]
    n = len(rc["k_chunks"])
    po = torch.empty((n,) + tuple(q.shape), dtype=q.dtype, device=DEV)
    pl = torch.empty((n, 1, H, S), dtype=torch.float32, device=DEV)
    for c in range(n):
        skv.attn_fwd(q, rc["k_chunks"][c].to(DEV), rc["v_chunks"][c].to(DEV), scale=rc["scale"],
                     smooth_k=True, out=po[c], lse=pl[c])
    mo = torch.full_like(q, float("nan"))
    ml = torch.full((1, H, S), float("nan"), dtype=torch.float32, device=DEV)
    skv.merge_state(po, pl, out=mo, lse=ml)
    fo = torch.full_like(q, float("nan"))
    fl = torch.full((1, H, S), float("nan"), dtype=torch.float32, device=DEV)
    skv.attn_fwd(q, rc["k"].to(DEV), rc["v"].to(DEV), scale=rc["scale"], out=fo, lse=fl)
    torch.cuda.synchronize()
    return (mo.float().cpu().numpy(), ml.cpu().numpy()), (fo.float().cpu().numpy(),
                                                           fl.cpu().numpy())


def test_ring_chunks_full_size(skv):
    """B1 H16 S8192 D64 fp16: four K/V chunks, each with its own K offset, run with
    smoothing and merged, and the unchunked run, both against the oracle."""
    rc = wl.ring_chunks(seed=5)
    (mo, ml), (fo, fl) = _ring_outputs(skv, rc)
    H, S = rc["q"].shape[1], rc["q"].shape[2]
    rows = _sample_rows(1, H, S, 40, seed=55)
    ro, rl = oracle.attn_rows(wl.bits(rc["q"]), wl.bits(rc["k"]), wl.bits(rc["v"]), "fp16", rows,
                              scale=rc["scale"])
    for name, o, l in (("merged", mo, ml), ("full", fo, fl)):
        assert np.isfinite(o).all() and np.isfinite(l).all(), name
        assert_lse_close(np.array([l[b, h, i] for b, h, i in rows]), rl, f"{name} lse")
        assert_out_close(np.stack([o[b, h, i] for b, h, i in rows]), ro, f"{name} out")


@pytest.mark.parametrize("Sq,causal", [(8192, False), (8192, True), (1024, True)])
def test_dense_d128_full_size(skv, Sq, causal):
    """B1 Hq32 Hkv8 D128 bf16 against 8192 keys: the dense prefill bench problem
    (Sq 8192, non-causal), the same causal, and a causal chunk of 1024 new rows after
    7168 cached keys (row i sees keys up to i + 7168).  Sampled rows against the oracle,
    including the rows on both sides of 256-row tile and 32-row wave-block boundaries,
    and every output finite."""
    p = wl.attn_problem(1, 32, 8, Sq, 8192, 128, seed=7 + (Sq != 8192))
    q, k, v = p.q.to(DEV), p.k.to(DEV), p.v.to(DEV)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((1, 32, Sq), float("nan"), dtype=torch.float32, device=DEV)
    skv.attn_fwd(q, k, v, scale=p.scale, causal=causal, out=out, lse=lse)
    torch.cuda.synchronize()
    o_c, l_c = out.float().cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(o_c).all() and np.isfinite(l_c).all()
    rows = set(map(tuple, _sample_rows(1, 32, Sq, 32, seed=70 + causal + Sq).tolist()))
    rows |= {(0, h, i % Sq) for h, i in ((3, 4095), (3, 4096), (17, 4127), (17, 4128),
                                          (31, 255), (31, 256), (8, 1), (8, 8190))}
    rows = np.array(sorted(rows), np.int64)
    ro, rl = oracle.attn_rows(wl.bits(p.q), wl.bits(p.k), wl.bits(p.v), "bf16", rows,
                              scale=p.scale, causal=causal)
    assert_lse_close(np.array([l_c[b, h, i] for b, h, i in rows]), rl, "lse")
    assert_out_close(np.stack([o_c[b, h, i] for b, h, i in rows]), ro, "out")
