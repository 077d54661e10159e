"""GPU checks of skv_attn_splitkv_decode_noalloc, the single-launch decode whose
partial states live in the library's fixed device scratch instead of a workspace.

Its results are compared with skv_attn_splitkv_decode (the workspace form, the same
kernels: bit for bit) and with the fp64 oracle (the parity bar), on consecutive calls
of different sizes that share the scratch, and on replays of a captured graph."""
from __future__ import annotations

import pytest
import torch

import oracle
import workloads as wl
from tolerance import assert_lse_close, assert_out_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def skv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import split_kv_merge_amd as m
    m._load()
    return m


def _problem(B, Hq, Hkv, Lq, Lkv, D, seed):
    p = wl.attn_problem(B, Hq, Hkv, Lq, Lkv, D, seed=seed)
    return p, p.q.cuda(), p.k.cuda(), p.v.cuda()


def _check(skv, p, q, k, v, S):
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    skv.attn_splitkv_decode_noalloc(q, k, v, out, lse, num_splits=S, scale=p.scale)
    ref_out, ref_lse = skv.attn_splitkv_decode(q, k, v, num_splits=S, scale=p.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), "no-allocation decode differs from the workspace form"
    assert torch.equal(lse, ref_lse)
    ro, rl = oracle.attn(wl.bits(p.q), wl.bits(p.k), wl.bits(p.v), "bf16", scale=p.scale)
    assert_out_close(out, ro)
    assert_lse_close(lse, rl)


def test_noalloc_decode_consecutive_calls_shrinking(skv):
    """A full-size config-2 decode, then a smaller one on the same scratch, then the
    first again: each equals the workspace form and the oracle."""
    big = _problem(8, 32, 8, 1, 4096, 128, seed=61)
    small = _problem(2, 16, 4, 2, 700, 128, seed=62)
    _check(skv, *big, S=16)
    _check(skv, *small, S=5)
    _check(skv, *big, S=32)


def test_noalloc_decode_wide_heads_and_kv_len(skv):
    """D = 256 with 16 rows per kv head, then a kv_len-bounded call."""
    p, q, k, v = _problem(2, 16, 4, 4, 3000, 256, seed=63)
    _check(skv, p, q, k, v, S=7)
    p2, q2, k2, v2 = _problem(3, 8, 2, 1, 2048, 128, seed=64)
    kvl = torch.tensor([2048, 17, 0], dtype=torch.int32, device="cuda")
    out = torch.empty_like(q2)
    lse = torch.empty(q2.shape[:3], dtype=torch.float32, device="cuda")
    skv.attn_splitkv_decode_noalloc(q2, k2, v2, out, lse, num_splits=8, scale=p2.scale,
                                    kv_len=kvl)
    ref_out, ref_lse = skv.attn_splitkv_decode(q2, k2, v2, num_splits=8, scale=p2.scale,
                                               kv_len=kvl)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)


def test_noalloc_decode_graph_replays(skv):
    """Captured once, replayed with eager work and synchronisations in between: every
    replay equals the eager workspace form."""
    p, q, k, v = _problem(4, 32, 8, 1, 2500, 128, seed=65)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    ref_out, ref_lse = skv.attn_splitkv_decode(q, k, v, num_splits=12, scale=p.scale)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        skv.attn_splitkv_decode_noalloc(q, k, v, out, lse, num_splits=12, scale=p.scale)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        skv.attn_splitkv_decode_noalloc(q, k, v, out, lse, num_splits=12, scale=p.scale)
    torch.cuda.synchronize()
    for r in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        # eager work between replays, on the same scratch with another shape
        small = _problem(1, 8, 2, 1, 300, 128, seed=66 + r)
        _check(skv, *small, S=3)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {r}"
        assert torch.equal(lse, ref_lse), f"replay {r}"


def test_noalloc_decode_rejects_oversized(skv):
    """A problem whose partial states exceed the scratch is refused before launch."""
    q = torch.empty((64, 64, 1, 256), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((64, 8, 128, 256), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(skv.SkvError) as e:
        skv.attn_splitkv_decode_noalloc(q, k, k, out, num_splits=64)
    assert e.value.status == 2
