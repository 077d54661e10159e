"""The single-launch decode at its documented limit: 65536 (batch, kv head) units,
the size of the workspace's fixed ticket block.  Every unit's last work group must
merge its own rows, and every ticket must be back at zero after the call, so that
the next call (here: the same one again) starts clean."""
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
