"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every comparison uses the bar in tests/tolerance.py.  Output buffers are filled
with NaN before each call so that a row the kernels fail to write shows up.
"""
from __future__ import annotations

import math

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


def _gpu(t):
    return t.to(DEV)


def _poison(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


def _oracle_attn(p: wl.Attn, dtype, causal=None):
    return oracle.attn(wl.bits(p.q), wl.bits(p.k), wl.bits(p.v), dtype, p.layout, p.scale,
                       p.causal if causal is None else causal)


def _run_attn(skv, p: wl.Attn, smooth_k=False):
    q, k, v = _gpu(p.q), _gpu(p.k), _gpu(p.v)
    B, Hq, Hkv, Sq, Sk, D = p.dims
    out = _poison(q.shape, q.dtype)
    lse = _poison((B, Hq, Sq), torch.float32)
    skv.attn_fwd(q, k, v, scale=p.scale, layout=p.layout, causal=p.causal, smooth_k=smooth_k,
                 out=out, lse=lse)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


# ----------------------------------------------------------------- config 1

@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("layout", ["HND", "NHD"])
@pytest.mark.parametrize("regime", ["rows", "blocks", "blocks_koff"])
@pytest.mark.parametrize("smooth_k", [False, True])
def test_tiny_lse_per_row(skv, dtype, layout, regime, smooth_k):
    """B1 H4 Sq64 Sk1000 D128: each q row scaled by linspace(0.25, 4), the 16-equal-row
    control, and K + 0.5; one LSE per row against the oracle, smoothing on and off."""
    d = wl.tiny_lse(seed=0, dtype=dtype)
    q = d["q_graded"] if regime == "rows" else d["q_grouped"]
    k = d["k_shifted"] if regime == "blocks_koff" else d["k"]
    v = d["v"]
    if layout == "NHD":
        q, k, v = (wl.hnd_to_nhd(t) for t in (q, k, v))
    p = wl.Attn(q, k, v, layout, d["scale"])
    ro, rl = _oracle_attn(p, dtype)
    out, lse = _run_attn(skv, p, smooth_k=smooth_k)
    assert_lse_close(lse, rl)
    assert_out_close(out, ro)


# ------------------------------------------------------------ dense sweeps

DENSE_CASES = [
    # B, Hq, Hkv, Sq, Sk, D, causal
    (2, 8, 2, 200, 333, 128, False),
    (2, 8, 2, 200, 333, 128, True),
    (1, 4, 4, 257, 257, 64, True),
    (1, 4, 1, 130, 70, 256, False),
    (1, 2, 2, 64, 190, 256, True),
    (3, 6, 3, 1, 500, 128, False),
    (1, 4, 2, 300, 100, 64, True),    # Sq > Sk: early rows see no key (bottom-right)
    (1, 4, 2, 777, 900, 128, True),   # four 256-row tiles, ragged last one
    (2, 2, 1, 600, 513, 64, False),
    (1, 2, 2, 530, 530, 256, True),   # five 128-row tiles at D = 256
]


@pytest.mark.parametrize("case", DENSE_CASES)
@pytest.mark.parametrize("dtype,layout", [("bf16", "HND"), ("fp16", "NHD")])
def test_dense_parity(skv, case, dtype, layout):
    B, Hq, Hkv, Sq, Sk, D, causal = case
    p = wl.attn_problem(B, Hq, Hkv, Sq, Sk, D, dtype=dtype, layout=layout, seed=101, causal=causal)
    ro, rl = _oracle_attn(p, dtype)
    out, lse = _run_attn(skv, p)
    assert_lse_close(lse, rl)
    assert_out_close(out, ro)


def test_empty_key_set_gives_zero_and_neg_inf(skv):
    p = wl.attn_problem(1, 2, 1, 5, 0, 128, seed=3)
    out, lse = _run_attn(skv, p)
    assert (out == 0).all() and torch.isneginf(lse).all()


def test_zero_query_gives_log2_sk(skv):
    p = wl.attn_problem(1, 2, 2, 70, 1000, 128, seed=5)
    p.q.zero_()
    out, lse = _run_attn(skv, p)
    assert np.abs(lse.numpy() - math.log2(1000)).max() < 1e-3


def test_deterministic(skv):
    p = wl.attn_problem(2, 8, 2, 200, 333, 128, seed=9, causal=True)
    a = _run_attn(skv, p)
    b = _run_attn(skv, p)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])


# ------------------------------------------------------------------ varlen

@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("smooth_k", [False, True])
def test_varlen_parity(skv, causal, smooth_k):
    vl = wl.varlen_prefill(seed=41, Hq=8, Hkv=2, D=128, causal=causal,
                           lengths=[1, 127, 128, 129, 300, 5, 64, 513])
    ro, rl = oracle.attn_varlen(wl.bits(vl.q), wl.bits(vl.k), wl.bits(vl.v), "bf16",
                                vl.cu_seqlens_q, vl.cu_seqlens_k, vl.scale, causal)
    q, k, v = _gpu(vl.q), _gpu(vl.k), _gpu(vl.v)
    out = _poison(q.shape, q.dtype)
    lse = _poison((q.shape[1], q.shape[0]), torch.float32)
    skv.attn_fwd_varlen(q, k, v, _gpu(vl.cu_seqlens_q), _gpu(vl.cu_seqlens_k),
                        max(vl.lengths), scale=vl.scale, causal=causal, smooth_k=smooth_k,
                        out=out, lse=lse)
    torch.cuda.synchronize()
    assert_lse_close(lse.cpu(), rl)
    assert_out_close(out.cpu(), ro)


@pytest.mark.parametrize("D,dtype,Hq,Hkv", [(64, "fp16", 8, 2), (256, "bf16", 4, 1)])
@pytest.mark.parametrize("causal", [True, False])
def test_varlen_parity_other_heads(skv, D, dtype, Hq, Hkv, causal):
    """Varlen at D = 64 (128-key tiles) and D = 256 (the 4-wave kernel), with smoothing
    and GQA; lengths straddle the 128/256-row and 32/128-key tile edges."""
    vl = wl.varlen_prefill(seed=43 + D, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, causal=causal,
                           lengths=[3, 129, 255, 256, 257, 130, 1, 400])
    ro, rl = oracle.attn_varlen(wl.bits(vl.q), wl.bits(vl.k), wl.bits(vl.v), dtype,
                                vl.cu_seqlens_q, vl.cu_seqlens_k, vl.scale, causal)
    q, k, v = _gpu(vl.q), _gpu(vl.k), _gpu(vl.v)
    out = _poison(q.shape, q.dtype)
    lse = _poison((q.shape[1], q.shape[0]), torch.float32)
    skv.attn_fwd_varlen(q, k, v, _gpu(vl.cu_seqlens_q), _gpu(vl.cu_seqlens_k),
                        max(vl.lengths), scale=vl.scale, causal=causal, smooth_k=True,
                        out=out, lse=lse)
    torch.cuda.synchronize()
    assert_lse_close(lse.cpu(), rl)
    assert_out_close(out.cpu(), ro)


# ------------------------------------------------------ split-KV + merge

SPLIT_CASES = [
    # B, Hq, Hkv, Lq, Lkv, D, S
    (2, 32, 8, 1, 1000, 128, 8),
    (2, 32, 8, 1, 1000, 128, 32),
    (1, 16, 4, 4, 777, 256, 16),
    (1, 8, 8, 1, 100, 128, 32),       # trailing chunks hold no key
    (2, 8, 2, 2, 1, 64, 4),           # one key: three empty chunks
    (1, 16, 1, 1, 4096, 128, 1),      # 16 rows per kv head, one chunk
    (1, 4, 2, 1, 0, 128, 3),          # no key at all
    (2, 64, 8, 4, 1500, 128, 8),      # G = 8, Lq = 4: 32 rows per kv head
    (1, 64, 4, 4, 999, 128, 5),       # G = 16, Lq = 4: 64 rows per kv head
    (2, 32, 2, 3, 700, 64, 16),       # 48 rows per kv head at D = 64
    (1, 16, 2, 3, 2049, 64, 3),       # 24 rows per kv head, ragged key tail
]


@pytest.mark.parametrize("case", SPLIT_CASES)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_splitkv_partials_and_merge(skv, case, dtype):
    B, Hq, Hkv, Lq, Lkv, D, S = case
    p = wl.attn_problem(B, Hq, Hkv, Lq, Lkv, D, dtype=dtype, seed=202)
    ro_p, rl_p = oracle.splitkv_partials(wl.bits(p.q), wl.bits(p.k), wl.bits(p.v), dtype, S,
                                         scale=p.scale)
    ro, rl = _oracle_attn(p, dtype)
    q, k, v = _gpu(p.q), _gpu(p.k), _gpu(p.v)
    op = _poison((S, B, Hq, Lq, D), torch.float32)
    lp = _poison((S, B, Hq, Lq), torch.float32)
    skv.attn_splitkv_partial(q, k, v, num_splits=S, scale=p.scale, out_part=op, lse_part=lp)
    out = _poison(q.shape, q.dtype)
    lse = _poison((B, Hq, Lq), torch.float32)
    skv.merge_state(op, lp, out=out, lse=lse)
    torch.cuda.synchronize()
    assert_lse_close(lp.cpu(), rl_p, "partial lse")
    assert_out_close(op.cpu(), ro_p, "partial out")
    assert_lse_close(lse.cpu(), rl)
    assert_out_close(out.cpu(), ro)


@pytest.mark.parametrize("sign", [+1, -1])
def test_extreme_logits_stay_finite(skv, sign):
    """Logits near +-128 nats: outside the fp32 exp range at any fixed offset."""
    p = wl.extreme_logits(sign=sign, Lkv=4096, B=1, Hq=16, Hkv=4, Lq=1, D=256)
    ro, rl = _oracle_attn(p, "bf16")
    q, k, v = _gpu(p.q), _gpu(p.k), _gpu(p.v)
    op, lp = skv.attn_splitkv_partial(q, k, v, num_splits=16, scale=p.scale)
    out, lse = skv.merge_state(op, lp, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    assert_lse_close(lse.cpu(), rl)
    assert_out_close(out.cpu(), ro)


def test_merge_fp16_parts_ring_style(skv):
    """Four chunk runs with smoothing (each chunk has its own mean(k)) merged equal
    the unsmoothed full run -- the ring-attention use of the LSE."""
    d = wl.ring_chunks(seed=5, B=1, H=4, S=512, D=64, n_chunks=4)
    q = _gpu(d["q"])
    parts_o = torch.empty((4,) + tuple(q.shape), dtype=q.dtype, device=DEV)
    parts_l = torch.empty((4, 1, 4, 512), dtype=torch.float32, device=DEV)
    for c in range(4):
        skv.attn_fwd(q, _gpu(d["k_chunks"][c]), _gpu(d["v_chunks"][c]), scale=d["scale"],
                     smooth_k=True, out=parts_o[c], lse=parts_l[c])
    out, lse = skv.merge_state(parts_o, parts_l)
    torch.cuda.synchronize()
    p = wl.Attn(d["q"], d["k"], d["v"], "HND", d["scale"])
    ro, rl = _oracle_attn(p, "fp16")
    assert_lse_close(lse.cpu(), rl)
    assert_out_close(out.cpu(), ro)


# ------------------------------------------------------ merge_state alone

@pytest.mark.parametrize("S", [1, 2, 3, 7, 16, 33, 64, 100])
@pytest.mark.parametrize("D,pdt", [(64, torch.float16), (128, torch.float32), (256, torch.float32),
                                   (128, torch.bfloat16)])
def test_merge_state_random_parts(skv, S, D, pdt):
    """Random partial states, including parts with lse = -inf and a row whose parts
    are all -inf, against the oracle's merge of the same (rounded) values."""
    g = torch.Generator().manual_seed(S * 1000 + D)
    R = (3, 5, 7)
    o = torch.randn((S,) + R + (D,), generator=g).to(pdt)
    lse = (torch.rand((S,) + R, generator=g) * 80 - 40).float()
    lse[torch.rand((S,) + R, generator=g) < 0.2] = float("-inf")
    lse[:, 1, 2, 3] = float("-inf")
    ro, rl = oracle.merge(o.double().numpy(), lse.double().numpy())
    out, ml = skv.merge_state(o.to(DEV), lse.to(DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_lse_close(ml.cpu(), rl)
    assert_out_close(out.cpu(), ro)
    assert (out[1, 2, 3] == 0).all() and torch.isneginf(ml[1, 2, 3])


def test_merge_state_strided_nhd_output(skv):
    """Parts in HND row order merged straight into an NHD output (strides only)."""
    S, B, H, L, D = 5, 2, 4, 9, 128
    g = torch.Generator().manual_seed(7)
    o = torch.randn(S, B, H, L, D, generator=g)
    lse = torch.randn(S, B, H, L, generator=g) * 10
    ro, rl = oracle.merge(o.double().numpy(), lse.double().numpy())
    out_nhd = _poison((B, L, H, D), torch.bfloat16)
    lse_out = _poison((B, H, L), torch.float32)
    skv.merge_state(o.to(DEV), lse.to(DEV), out=out_nhd.transpose(1, 2), lse=lse_out)
    torch.cuda.synchronize()
    assert_out_close(out_nhd.transpose(1, 2).cpu(), ro)
    assert_lse_close(lse_out.cpu(), rl)


# ------------------------------------------------ single-launch decode

@pytest.mark.parametrize("case", SPLIT_CASES)
@pytest.mark.parametrize("layout", ["HND", "NHD"])
def test_splitkv_decode_single_launch(skv, case, layout):
    """Partials + in-kernel merge by the last work group; three calls share one
    workspace (the arrival counters must come back to zero each time)."""
    B, Hq, Hkv, Lq, Lkv, D, S = case
    p = wl.attn_problem(B, Hq, Hkv, Lq, Lkv, D, seed=303, layout=layout)
    ro, rl = _oracle_attn(p, "bf16")
    q, k, v = _gpu(p.q), _gpu(p.k), _gpu(p.v)
    ws = torch.zeros(skv.splitkv_workspace_bytes(B, Hq, Lq, D, S, Hkv), dtype=torch.uint8,
                     device=DEV)
    for _ in range(3):
        out = _poison(q.shape, q.dtype)
        lse = _poison((B, Hq, Lq), torch.float32)
        skv.attn_splitkv_decode(q, k, v, num_splits=S, scale=p.scale, layout=layout, out=out,
                                lse=lse, workspace=ws)
        torch.cuda.synchronize()
        assert_lse_close(lse.cpu(), rl)
        assert_out_close(out.cpu(), ro)
    # the counters (the block at the start of the workspace) are back at zero
    assert (ws[:65536 * 4] == 0).all()


def test_splitkv_decode_graph_replays(skv):
    """Captured once, replayed with different inputs copied in between: every replay
    matches the oracle (the workspace stays reusable across replays)."""
    B, Hq, Hkv, Lq, Lkv, D, S = 2, 32, 8, 1, 3000, 128, 8
    probs = [wl.attn_problem(B, Hq, Hkv, Lq, Lkv, D, seed=400 + i) for i in range(3)]
    q = _gpu(probs[0].q); k = _gpu(probs[0].k); v = _gpu(probs[0].v)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=DEV)
    ws = torch.zeros(skv.splitkv_workspace_bytes(B, Hq, Lq, D, S, Hkv), dtype=torch.uint8,
                     device=DEV)
    fn = lambda: skv.attn_splitkv_decode(q, k, v, num_splits=S, scale=probs[0].scale, out=out,
                                         lse=lse, workspace=ws)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        fn()
    torch.cuda.current_stream().wait_stream(st)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for p in probs + probs[:1]:
        q.copy_(p.q); k.copy_(p.k); v.copy_(p.v)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ro, rl = _oracle_attn(p, "bf16")
        assert_lse_close(lse.cpu(), rl)
        assert_out_close(out.cpu(), ro)
