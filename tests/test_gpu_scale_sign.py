"""GPU parity for logit scales of either sign and for scale 0.

The kernels take the running max over raw dot products; for a negative scale they
negate q (exactly) and use |scale|, and in masked tiles a masked logit contributes
p = 0 also when the logit scale is 0 (scale 0, or an all-zero INT8 K block).  Each
case is compared with the fp64 oracle, whose logits are scale * q . k for any scale:
causal masks and ragged key tails put masked logits into the masked-tile path.
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


CASES = [
    # B, Hq, Hkv, Sq, Sk, D, causal, dtype, layout
    (1, 4, 2, 300, 300, 128, True, "bf16", "HND"),
    (2, 4, 4, 130, 200, 64, True, "fp16", "NHD"),    # bottom-right causal, ragged tiles
    (1, 2, 1, 70, 333, 256, False, "bf16", "HND"),   # ragged key tail only
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("scale", [-0.09, 0.0])
@pytest.mark.parametrize("smooth_k", [False, True])
def test_attn_fwd_any_scale(skv, case, scale, smooth_k):
    B, Hq, Hkv, Sq, Sk, D, causal, dtype, layout = case
    p = wl.attn_problem(B, Hq, Hkv, Sq, Sk, D, dtype=dtype, layout=layout, seed=211,
                        causal=causal, k_offset=0.5)
    ro, rl = oracle.attn(wl.bits(p.q), wl.bits(p.k), wl.bits(p.v), dtype, layout, scale, causal)
    q, k, v = p.q.to(DEV), p.k.to(DEV), p.v.to(DEV)
    out, lse = skv.attn_fwd(q, k, v, scale=scale, layout=layout, causal=causal,
                            smooth_k=smooth_k, return_lse=True)
    torch.cuda.synchronize()
    assert_lse_close(lse.cpu(), rl)
    assert_out_close(out.cpu(), ro)


def test_scale_zero_is_uniform_over_visible_keys(skv):
    """scale 0: every visible logit is 0, so LSE = log2(number of visible keys) and
    out is the mean of the visible V rows (row i of a causal square problem sees i + 1
    keys)."""
    p = wl.attn_problem(1, 2, 2, 200, 200, 64, seed=212, causal=True)
    q, k, v = p.q.to(DEV), p.k.to(DEV), p.v.to(DEV)
    out, lse = skv.attn_fwd(q, k, v, scale=0.0, causal=True, return_lse=True)
    torch.cuda.synchronize()
    want = np.log2(np.arange(1, 201, dtype=np.float64))
    assert np.abs(lse.cpu().numpy()[0] - want[None, :]).max() < 1e-3


def test_varlen_negative_scale(skv):
    vl = wl.varlen_prefill(seed=213, nseq=3, lengths=[100, 257, 1], Hq=4, Hkv=2, D=128)
    ro, rl = oracle.attn_varlen(wl.bits(vl.q), wl.bits(vl.k), wl.bits(vl.v), "bf16",
                                vl.cu_seqlens_q.numpy(), vl.cu_seqlens_k.numpy(), scale=-0.1,
                                causal=True)
    out, lse = skv.attn_fwd_varlen(vl.q.to(DEV), vl.k.to(DEV), vl.v.to(DEV),
                                   vl.cu_seqlens_q.to(DEV), vl.cu_seqlens_k.to(DEV), 257,
                                   scale=-0.1, causal=True, return_lse=True)
    torch.cuda.synchronize()
    assert_lse_close(lse.cpu(), rl)
    assert_out_close(out.cpu(), ro)


@pytest.mark.parametrize("scale", [-0.11, 0.0])
@pytest.mark.parametrize("causal", [False, True])
def test_sage_fwd_any_scale(skv, scale, causal):
    p = wl.attn_problem(1, 4, 2, 150, 150, 64, dtype="fp16", seed=214, k_offset=1.0)
    ro, rl = oracle.sage_attn(wl.bits(p.q), wl.bits(p.k), wl.bits(p.v), "fp16", scale=scale,
                              causal=causal, smooth_k=True)
    out, lse = skv.sage_fwd(p.q.to(DEV), p.k.to(DEV), p.v.to(DEV), scale=scale, causal=causal,
                            smooth_k=True, return_lse=True)
    torch.cuda.synchronize()
    assert_lse_close(lse.cpu(), rl)
    assert_out_close(out.cpu(), ro)


def test_sage_fwd_all_zero_key_blocks_in_masked_tiles(skv):
    """Identical keys: with smoothing every key block of k - mean(k) is zero (its scale
    0), so every logit is 0; causal masking and a ragged tail must still give the
    uniform average over the visible keys, not NaN."""
    B, H, S, D = 1, 2, 173, 128
    g = torch.Generator().manual_seed(215)
    q = torch.randn(B, H, S, D, generator=g).to(torch.bfloat16)
    k = (torch.randn(1, 1, 1, D, generator=g) * 2).expand(B, H, S, D).contiguous().to(torch.bfloat16)
    v = torch.randn(B, H, S, D, generator=g).to(torch.bfloat16)
    ro, rl = oracle.sage_attn(wl.bits(q), wl.bits(k), wl.bits(v), "bf16", scale=0.125,
                              causal=True, smooth_k=True)
    out, lse = skv.sage_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=0.125, causal=True,
                            smooth_k=True, return_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    assert_lse_close(lse.cpu(), rl)
    assert_out_close(out.cpu(), ro)


DECODE_CASES = [
    # B, Hq, Hkv, Lq, Lkv, D, S: 4, 32 and 64 query rows per kv head, and 24 at D = 64
    (2, 8, 2, 1, 777, 128, 3),
    (1, 32, 4, 4, 777, 128, 3),
    (1, 64, 4, 4, 650, 128, 2),
    (1, 16, 2, 3, 901, 64, 4),
]


@pytest.mark.parametrize("case", DECODE_CASES)
@pytest.mark.parametrize("scale", [-0.09, 0.0])
def test_splitkv_decode_any_scale(skv, case, scale):
    """Split partials + merge and the single-launch decode with a negative or zero logit
    scale, ragged key tails included, against the oracle."""
    B, Hq, Hkv, Lq, Lkv, D, S = case
    p = wl.attn_problem(B, Hq, Hkv, Lq, Lkv, D, seed=321)
    ro, rl = oracle.attn(wl.bits(p.q), wl.bits(p.k), wl.bits(p.v), "bf16", scale=scale)
    q, k, v = p.q.to(DEV), p.k.to(DEV), p.v.to(DEV)
    op = torch.full((S,) + tuple(q.shape), float("nan"), dtype=torch.float32, device=DEV)
    lp = torch.full((S, B, Hq, Lq), float("nan"), dtype=torch.float32, device=DEV)
    skv.attn_splitkv_partial(q, k, v, num_splits=S, scale=scale, out_part=op, lse_part=lp)
    mo = torch.full_like(q, float("nan"))
    ml = torch.full((B, Hq, Lq), float("nan"), dtype=torch.float32, device=DEV)
    skv.merge_state(op, lp, out=mo, lse=ml)
    ws = torch.zeros(skv.splitkv_workspace_bytes(B, Hq, Lq, D, S, Hkv), dtype=torch.uint8,
                     device=DEV)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, Lq), float("nan"), dtype=torch.float32, device=DEV)
    skv.attn_splitkv_decode(q, k, v, num_splits=S, scale=scale, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    for name, o, l in (("partials + merge", mo, ml), ("single launch", out, lse)):
        assert_lse_close(l.cpu(), rl, f"{name} lse")
        assert_out_close(o.float().cpu(), ro, f"{name} out")
