"""GPU parity of the INT8 QK^T path (skv_sage_quant, skv_sage_fwd) with the oracle.

The quantisation decides integers from float32 arithmetic that both sides do in
the same precision (exact mean(k) rounded once, float32 k - mean, correctly
rounded divisions, one float32 product, round half to even), so codes, scales
and mean(k) must agree bit for bit.  The attention output and LSE are compared
with the oracle's INT8 path (same codes, fp64 afterwards) at the parity bar
(out 1e-2 + 1e-2 |ref|, LSE 1e-2 log2 units): the kernel's own rounding (fp32
softmax, P and V in fp16) stays far inside it.
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


QUANT_CASES = [
    # B, Hq, Hkv, Sq, Sk, D, dtype, layout, smooth, k_offset
    (1, 4, 4, 64, 1000, 128, "bf16", "HND", True, 0.5),
    (2, 8, 2, 70, 333, 64, "fp16", "NHD", True, -1.0),
    (1, 2, 1, 1, 1, 128, "bf16", "HND", False, 0.0),
    (2, 4, 4, 257, 129, 64, "bf16", "NHD", False, 2.0),
    (1, 16, 4, 512, 4096, 128, "fp16", "HND", True, 3.0),
]


@pytest.mark.parametrize("case", QUANT_CASES)
def test_quant_is_bit_exact(skv, case):
    B, Hq, Hkv, Sq, Sk, D, dtype, layout, smooth, off = case
    p = wl.attn_problem(B, Hq, Hkv, Sq, Sk, D, dtype=dtype, layout=layout, seed=Sq + Sk,
                        k_offset=off)
    ref = oracle.sage_quant(wl.bits(p.q), wl.bits(p.k), dtype, layout, smooth_k=smooth)
    got = skv.sage_quant(p.q.to(DEV), p.k.to(DEV), layout=layout, smooth_k=smooth)
    torch.cuda.synchronize()
    for name in ("q_codes", "q_scale", "k_codes", "k_scale"):
        g = got[name].cpu().numpy()
        assert g.shape == ref[name].shape, name
        bad = int((g != ref[name]).sum())
        assert bad == 0, f"{name}: {bad} of {g.size} differ"
    if smooth:
        assert np.array_equal(got["kbar"].cpu().numpy(), ref["kbar"])


FWD_CASES = [
    # B, Hq, Hkv, Sq, Sk, D, dtype, layout, causal, smooth, k_offset
    (1, 4, 4, 64, 1000, 128, "bf16", "HND", False, True, 0.5),
    (1, 4, 4, 64, 1000, 128, "bf16", "HND", False, False, 0.5),
    (2, 8, 2, 300, 700, 128, "bf16", "NHD", True, True, 1.0),
    (2, 8, 4, 513, 513, 64, "fp16", "HND", True, True, -2.0),
    (1, 6, 2, 257, 1200, 64, "bf16", "NHD", False, False, 0.0),
    (3, 4, 1, 100, 77, 128, "fp16", "HND", False, True, 0.3),
    (1, 4, 2, 700, 300, 128, "bf16", "HND", True, True, 0.0),   # Sq > Sk: empty rows
    (1, 2, 2, 1, 1, 64, "fp16", "NHD", False, True, 0.0),
    (1, 2, 1, 33, 1, 128, "bf16", "HND", True, False, 0.0),
]


def _run(skv, p, causal, smooth):
    q, k, v = p.q.to(DEV), p.k.to(DEV), p.v.to(DEV)
    out = torch.full_like(q, float("nan"))
    B, Hq, Hkv, Sq, Sk, D = p.dims
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=DEV)
    ws_n = skv.sage_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, q.dtype, smooth)
    ws = torch.full((max(ws_n, 1),), 0xFF, dtype=torch.uint8, device=DEV)   # NaN-ish garbage
    skv.sage_fwd(q, k, v, scale=p.scale, layout=p.layout, causal=causal, smooth_k=smooth,
                 out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("case", FWD_CASES)
def test_sage_fwd_matches_oracle(skv, case):
    B, Hq, Hkv, Sq, Sk, D, dtype, layout, causal, smooth, off = case
    p = wl.attn_problem(B, Hq, Hkv, Sq, Sk, D, dtype=dtype, layout=layout, seed=3 * Sq + Sk,
                        k_offset=off)
    ro, rl = oracle.sage_attn(wl.bits(p.q), wl.bits(p.k), wl.bits(p.v), dtype, layout,
                              scale=p.scale, causal=causal, smooth_k=smooth)
    o, l = _run(skv, p, causal, smooth)
    assert_lse_close(l, rl)
    assert_out_close(o, ro)


def test_empty_keys_give_zero_rows(skv):
    p = wl.attn_problem(1, 4, 2, 40, 0, 128, seed=1)
    o, l = _run(skv, p, False, True)
    assert np.isneginf(l).all() and not o.any()


def test_zero_blocks(skv):
    """An all-zero query block and an all-zero key block have delta = 0."""
    p = wl.attn_problem(1, 2, 1, 70, 100, 64, seed=2, dtype="fp16")
    p.q[:, :, 32:64] = 0
    p.k[:, :, 64:96] = 0
    for smooth in (False, True):
        ro, rl = oracle.sage_attn(wl.bits(p.q), wl.bits(p.k), wl.bits(p.v), "fp16", "HND",
                                  scale=p.scale, smooth_k=smooth)
        o, l = _run(skv, p, False, smooth)
        assert_lse_close(l, rl)
        assert_out_close(o, ro)


def test_pages_workload_against_exact_attention(skv):
    """B1 H4 Sq64 Sk1000 D128 bf16, rows of distinct magnitude, K and K + 0.5, smooth_k
    on and off: every row gets its own LSE (no 16-row sharing), and the INT8 LSE is
    within the INT8 error the ARK report prints for this workload (0.051 at most)
    of the exact LSE of the unsmoothed logits."""
    d = wl.tiny_lse(seed=0)
    for qn in ("q_graded", "q_grouped"):
        for kn in ("k", "k_shifted"):
            for smooth in (True, False):
                p = wl.Attn(d[qn], d[kn], d["v"], "HND", d["scale"])
                o, l = _run(skv, p, False, smooth)
                _, exact = oracle.attn(wl.bits(d[qn]), wl.bits(d[kn]), wl.bits(d["v"]), "bf16",
                                       scale=d["scale"])
                err = np.abs(l - exact).max()
                lim = 0.051 if qn == "q_grouped" else 0.15
                assert err <= lim, (qn, kn, smooth, err)
                if qn == "q_graded":
                    assert len(np.unique(l[0, 0])) == l.shape[2]


def test_ring_chunk_shape_full_size(skv):
    """B1 H16 D64 fp16 at the ring-hop shape: Sq 8192 queries against one 2048-key
    chunk with its own offset, smoothing on; sampled rows against the oracle."""
    rc = wl.ring_chunks(seed=5)
    q, k, v = rc["q"], rc["k_chunks"][1], rc["v_chunks"][1]
    p = wl.Attn(q, k, v, "HND", rc["scale"])
    o, l = _run(skv, p, False, True)
    assert np.isfinite(o).all() and np.isfinite(l).all()
    g = np.random.default_rng(8)
    rows = sorted({(0, int(g.integers(16)), int(g.integers(8192))) for _ in range(40)}
                  | {(0, 0, 0), (0, 15, 8191)})
    rows = np.array(rows, np.int64)
    ro, rl = oracle.sage_attn(wl.bits(q), wl.bits(k), wl.bits(v), "fp16", scale=rc["scale"],
                              smooth_k=True, rows=rows)
    assert_lse_close(np.array([l[b, h, i] for b, h, i in rows]), rl)
    assert_out_close(np.stack([o[b, h, i] for b, h, i in rows]), ro)


def test_sage_fwd_graph_replays(skv):
    """One captured INT8 forward (mean(k), quantisation and attention; no memset in
    the graph), replayed while q and k change on the device between replays: each
    replay matches the oracle on the inputs of that moment."""
    B, Hq, Hkv, Sq, Sk, D = 1, 8, 2, 300, 500, 128
    q = torch.empty((B, Hq, Sq, D), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((B, Hkv, Sk, D), dtype=torch.bfloat16, device=DEV)
    v = torch.empty_like(k)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=DEV)
    ws = torch.empty(skv.sage_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, q.dtype, True),
                     dtype=torch.uint8, device=DEV)
    scale = wl.default_scale(D)
    fn = lambda: skv.sage_fwd(q, k, v, scale=scale, causal=True, smooth_k=True, out=out, lse=lse,
                              workspace=ws)
    p0 = wl.attn_problem(B, Hq, Hkv, Sq, Sk, D, seed=40, k_offset=1.0)
    q.copy_(p0.q), k.copy_(p0.k), v.copy_(p0.v)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        fn()
    torch.cuda.current_stream().wait_stream(st)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for seed, off in ((41, 0.0), (42, -2.0), (43, 3.0)):
        p = wl.attn_problem(B, Hq, Hkv, Sq, Sk, D, seed=seed, k_offset=off)
        q.copy_(p.q), k.copy_(p.k), v.copy_(p.v)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ro, rl = oracle.sage_attn(wl.bits(p.q), wl.bits(p.k), wl.bits(p.v), "bf16", scale=scale,
                                  causal=True, smooth_k=True)
        assert_lse_close(lse.cpu().numpy(), rl, f"lse, replay with seed {seed}")
        assert_out_close(out.float().cpu().numpy(), ro, f"out, replay with seed {seed}")


def test_dense_d128_bench_shape_full_size(skv):
    """B1 Hq32 Hkv8 S8192 D128 bf16, non-causal, smoothing on, K offset by +1 (the dense
    problem bench.py times, with an offset so smoothing matters): sampled rows against
    the oracle's INT8 path; every row finite."""
    p = wl.attn_problem(1, 32, 8, 8192, 8192, 128, seed=7, k_offset=1.0)
    o, l = _run(skv, p, False, True)
    assert np.isfinite(o).all() and np.isfinite(l).all()
    g = np.random.default_rng(9)
    rows = sorted({(0, int(g.integers(32)), int(g.integers(8192))) for _ in range(32)}
                  | {(0, 0, 0), (0, 31, 8191)})
    rows = np.array(rows, np.int64)
    ro, rl = oracle.sage_attn(wl.bits(p.q), wl.bits(p.k), wl.bits(p.v), "bf16", scale=p.scale,
                              smooth_k=True, rows=rows)
    assert_lse_close(np.array([l[b, h, i] for b, h, i in rows]), rl)
    assert_out_close(np.stack([o[b, h, i] for b, h, i in rows]), ro)
