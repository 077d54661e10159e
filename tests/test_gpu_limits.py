"""Size limits.

The single-launch decode at its documented limit, 65536 (batch, kv head) units (the
size of the workspace's fixed ticket block): every unit's last work group must merge
its own rows, and every ticket must be back at zero after the call, so that the next
call (here: the same one again) starts clean; one unit more is refused.  And tensors
past 2^31 elements, where every offset into K and V must be 64-bit.
"""
from __future__ import annotations

import pytest
import torch

import oracle
import workloads as wl
from tests.tolerance import assert_lse_close, assert_out_close

pytestmark = pytest.mark.gpu

DEV = "cuda"
MAX_UNITS = 65536


@pytest.fixture(scope="module")
def skv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import split_kv_merge_amd as m
    m._load()
    return m


def test_decode_at_the_unit_limit(skv):
    B, Hq, Hkv, Lq, Lkv, D, S = MAX_UNITS // 8, 8, 8, 1, 40, 64, 3
    p = wl.attn_problem(B, Hq, Hkv, Lq, Lkv, D, seed=640)
    ro, rl = oracle.attn(wl.bits(p.q), wl.bits(p.k), wl.bits(p.v), "bf16", "HND", p.scale)
    q, k, v = p.q.to(DEV), p.k.to(DEV), p.v.to(DEV)
    ws = torch.zeros(skv.splitkv_workspace_bytes(B, Hq, Lq, D, S, Hkv), dtype=torch.uint8,
                     device=DEV)
    for _ in range(2):
        out = torch.full_like(q, float("nan"))
        lse = torch.full((B, Hq, Lq), float("nan"), dtype=torch.float32, device=DEV)
        skv.attn_splitkv_decode(q, k, v, num_splits=S, scale=p.scale, out=out, lse=lse,
                                workspace=ws)
        torch.cuda.synchronize()
        assert_lse_close(lse.cpu(), rl)
        assert_out_close(out.cpu(), ro)
        assert (ws[:MAX_UNITS * 4] == 0).all()


def test_decode_one_unit_past_the_limit_is_refused(skv):
    B, Hq, Hkv = MAX_UNITS // 8 + 1, 8, 8
    q = torch.zeros(B, Hq, 1, 64, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(B, Hkv, 16, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(skv.SkvError) as e:
        skv.attn_splitkv_decode(q, k, k, num_splits=2)
    assert e.value.status == 2


def test_decode_past_2_31_elements(skv):
    """K and V of 2.15e9 elements each (B16 Hkv8 Lkv131200 D128 bf16, 4.3 GB apiece),
    so the last batch element's keys lie past element 2^31: the offsets must be 64-bit.
    The inputs are drawn on the device with a seeded generator; the first and the last
    batch element are checked against the oracle, the rest for finite output."""
    B, Hq, Hkv, Lq, Lkv, D = 16, 32, 8, 1, 131200, 128
    assert B * Hkv * Lkv * D > 2 ** 31
    gen = torch.Generator(device=DEV).manual_seed(650)
    q = torch.randn(B, Hq, Lq, D, generator=gen, device=DEV).to(torch.bfloat16)
    k = torch.randn(B, Hkv, Lkv, D, generator=gen, device=DEV, dtype=torch.bfloat16)
    v = torch.randn(B, Hkv, Lkv, D, generator=gen, device=DEV, dtype=torch.bfloat16)
    scale = wl.default_scale(D)
    S = skv.pick_num_splits(B, Hkv, (Hq // Hkv) * Lq, Lkv, D)
    out, lse = skv.attn_splitkv_decode(q, k, v, num_splits=S, scale=scale)
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all() and torch.isfinite(out.float()).all()
    for b in (0, B - 1):
        qb, kb, vb = q[b:b + 1].cpu(), k[b:b + 1].cpu(), v[b:b + 1].cpu()
        ro, rl = oracle.attn(wl.bits(qb), wl.bits(kb), wl.bits(vb), "bf16", "HND", scale)
        assert_lse_close(lse[b:b + 1].cpu(), rl)
        assert_out_close(out[b:b + 1].cpu(), ro)
    del k, v
    torch.cuda.empty_cache()


def test_prefill_past_2_31_elements(skv):
    """The attention forward with K and V of 2.15e9 elements each (B2 Hkv8 Sk1050000
    D128 bf16): the second batch element's keys lie past element 2^31.  Sampled rows of
    that element are checked against the oracle, every output for finiteness."""
    B, Hq, Hkv, Sq, Sk, D = 2, 32, 8, 256, 1050000, 128
    assert B * Hkv * Sk * D > 2 ** 31
    gen = torch.Generator(device=DEV).manual_seed(660)
    q = torch.randn(B, Hq, Sq, D, generator=gen, device=DEV).to(torch.bfloat16)
    k = torch.randn(B, Hkv, Sk, D, generator=gen, device=DEV, dtype=torch.bfloat16)
    v = torch.randn(B, Hkv, Sk, D, generator=gen, device=DEV, dtype=torch.bfloat16)
    scale = wl.default_scale(D)
    out, lse = skv.attn_fwd(q, k, v, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all() and torch.isfinite(out.float()).all()
    b = B - 1
    qb, kb, vb = q[b:b + 1].cpu(), k[b:b + 1].cpu(), v[b:b + 1].cpu()
    rows = [(0, h, i) for h in (0, 13, Hq - 1) for i in (0, 131, Sq - 1)]
    ro, rl = oracle.attn_rows(wl.bits(qb), wl.bits(kb), wl.bits(vb), "bf16", rows, scale=scale)
    got_o = torch.stack([out[b, h, i] for _, h, i in rows]).cpu()
    got_l = torch.stack([lse[b, h, i] for _, h, i in rows]).cpu()
    assert_lse_close(got_l, rl)
    assert_out_close(got_o, ro)
    del k, v
    torch.cuda.empty_cache()
