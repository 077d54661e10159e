"""Fresh-seed sweep: five more seeds per workload shape, for correctness only.

The fixed-seed tests pin particular inputs; this sweep draws new ones from the same
recipes (seeds 1000..1004) at sizes the oracle finishes quickly but that still span
several tiles and a ragged tail, and compares every output element and LSE with the
oracle at the parity bar.
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
SEEDS = [1000, 1001, 1002, 1003, 1004]


@pytest.fixture(scope="module")
def skv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import split_kv_merge_amd as m
    m._load()
    return m


@pytest.mark.parametrize("seed", SEEDS)
def test_tiny_lse_shape(skv, seed):
    """B1 H4 Sq64 Sk1000 D128 bf16, rows of distinct magnitude, K + 0.5, smooth_k on
    and off, HND and NHD."""
    d = wl.tiny_lse(seed=seed)
    for qn, kn, smooth, layout in (("q_graded", "k", False, "HND"), ("q_graded", "k_shifted", True, "HND"),
                                   ("q_grouped", "k_shifted", True, "NHD")):
        q, k, v = d[qn], d[kn], d["v"]
        if layout == "NHD":
            q, k, v = wl.hnd_to_nhd(q), wl.hnd_to_nhd(k), wl.hnd_to_nhd(v)
        ro, rl = oracle.attn(wl.bits(q), wl.bits(k), wl.bits(v), "bf16", layout, scale=d["scale"])
        out, lse = skv.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=d["scale"], layout=layout,
                                smooth_k=smooth, return_lse=True)
        torch.cuda.synchronize()
        assert_lse_close(lse.cpu(), rl, f"{qn}/{kn}/{layout} lse")
        assert_out_close(out.cpu(), ro, f"{qn}/{kn}/{layout} out")


@pytest.mark.parametrize("seed", SEEDS)
def test_decode_gqa_shape(skv, seed):
    """B2 Hq32 Hkv8 Lq1 D128 bf16 decode over 3000 keys, the split count the heuristic
    picks, one launch."""
    p = wl.attn_problem(2, 32, 8, 1, 3000, 128, seed=seed)
    ro, rl = oracle.attn(wl.bits(p.q), wl.bits(p.k), wl.bits(p.v), "bf16", scale=p.scale)
    out, lse = skv.attn_splitkv_decode(p.q.to(DEV), p.k.to(DEV), p.v.to(DEV), scale=p.scale)
    torch.cuda.synchronize()
    assert_lse_close(lse.cpu(), rl)
    assert_out_close(out.cpu(), ro)


@pytest.mark.parametrize("seed", SEEDS)
def test_wide_decode_shape(skv, seed):
    """B1 Hq16 Hkv4 Lq4 D256 bf16, q = 8 N(0,1), K offset +-2 (sign alternating with the
    seed), 5000 keys in 16 chunks, partials then merge_state."""
    sign = 1 if seed % 2 else -1
    p = wl.wide_decode(5000, sign, seed=seed, B=1)
    ro, rl = oracle.attn(wl.bits(p.q), wl.bits(p.k), wl.bits(p.v), "bf16", scale=p.scale)
    op, lp = skv.attn_splitkv_partial(p.q.to(DEV), p.k.to(DEV), p.v.to(DEV), num_splits=16,
                                      scale=p.scale)
    out, lse = skv.merge_state(op, lp, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_lse_close(lse.cpu(), rl)
    assert_out_close(out.cpu(), ro)


@pytest.mark.parametrize("seed", SEEDS)
def test_varlen_causal_shape(skv, seed):
    """5 packed sequences, lengths U[40, 700], Hq16 Hkv4 D128 bf16, causal, 2-D LSE."""
    vl = wl.varlen_prefill(seed=seed, nseq=5, lo=40, hi=700, Hq=16, Hkv=4)
    ro, rl = oracle.attn_varlen(wl.bits(vl.q), wl.bits(vl.k), wl.bits(vl.v), "bf16",
                                vl.cu_seqlens_q.numpy(), vl.cu_seqlens_k.numpy(), scale=vl.scale,
                                causal=True)
    out, lse = skv.attn_fwd_varlen(vl.q.to(DEV), vl.k.to(DEV), vl.v.to(DEV),
                                   vl.cu_seqlens_q.to(DEV), vl.cu_seqlens_k.to(DEV),
                                   max(vl.lengths), scale=vl.scale, causal=True, return_lse=True)
    torch.cuda.synchronize()
    assert_lse_close(lse.cpu(), rl)
    assert_out_close(out.cpu(), ro)


@pytest.mark.parametrize("seed", SEEDS)
def test_ring_chunks_shape(skv, seed):
    """B1 H4 S1024 D64 fp16: four K/V chunks with their own offsets, each run with
    smoothing, merged; equals the oracle on the whole sequence."""
    rc = wl.ring_chunks(seed=seed, B=1, H=4, S=1024, D=64, n_chunks=4)
    q = rc["q"].to(DEV)
    parts = [skv.attn_fwd(q, kc.to(DEV), vc.to(DEV), scale=rc["scale"], smooth_k=True,
                          return_lse=True) for kc, vc in zip(rc["k_chunks"], rc["v_chunks"])]
    out, lse = skv.merge_state(torch.stack([o for o, _ in parts]),
                               torch.stack([l for _, l in parts]))
    ro, rl = oracle.attn(wl.bits(rc["q"]), wl.bits(rc["k"]), wl.bits(rc["v"]), "fp16",
                         scale=rc["scale"])
    torch.cuda.synchronize()
    assert_lse_close(lse.cpu(), rl)
    assert_out_close(out.cpu(), ro)


@pytest.mark.parametrize("seed", SEEDS)
def test_int8_path_shape(skv, seed):
    """INT8 QK^T with smoothing: B2 Hq8 Hkv2 Sq300 Sk700 D128 bf16 causal, K offset 1,
    against the oracle's INT8 path."""
    p = wl.attn_problem(2, 8, 2, 300, 700, 128, seed=seed, k_offset=1.0)
    ro, rl = oracle.sage_attn(wl.bits(p.q), wl.bits(p.k), wl.bits(p.v), "bf16", scale=p.scale,
                              causal=True, smooth_k=True)
    out, lse = skv.sage_fwd(p.q.to(DEV), p.k.to(DEV), p.v.to(DEV), scale=p.scale, causal=True,
                            smooth_k=True, return_lse=True)
    torch.cuda.synchronize()
    assert_lse_close(lse.cpu(), rl)
    assert_out_close(out.cpu(), ro)
    assert np.isfinite(out.float().cpu().numpy()).all()
