"""Calls on separate streams and shared workspaces.

A call only enqueues on the stream it is given, so independent calls on two
streams may run at the same time on the device.  Each single-launch decode keeps
its arrival tickets in its own workspace, and each smoothed forward its mean(k) in
its own: concurrent calls must not see each other's state.  A decode workspace is
sized for the largest problem it serves and returns its tickets to zero after every
call, so one workspace can serve problems of different shapes in turn.  Every
result is compared with the oracle at the parity bar.
"""
from __future__ import annotations

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


def _oracle(p, dtype="bf16", causal=False):
    return oracle.attn(wl.bits(p.q), wl.bits(p.k), wl.bits(p.v), dtype, p.layout, p.scale, causal)


def test_decodes_on_two_streams(skv):
    """Two single-launch decodes of different shapes, each with its own workspace,
    enqueued on two streams without waiting in between, three times over."""
    probs = [wl.attn_problem(4, 32, 8, 1, 3000, 128, seed=501),
             wl.attn_problem(2, 16, 4, 4, 5000, 128, seed=502)]
    refs = [_oracle(p) for p in probs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    gpu, ws = [], []
    for p in probs:
        B, Hq, Hkv, Lq, Lkv, D = p.dims
        S = skv.pick_num_splits(B, Hkv, (Hq // Hkv) * Lq, Lkv, D)
        gpu.append((p.q.to(DEV), p.k.to(DEV), p.v.to(DEV), S))
        ws.append(torch.zeros(skv.splitkv_workspace_bytes(B, Hq, Lq, D, S, Hkv),
                              dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    for _ in range(3):
        outs = []
        for (q, k, v, S), w, st, p in zip(gpu, ws, streams, probs):
            with torch.cuda.stream(st):
                out = torch.full_like(q, float("nan"))
                lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
                skv.attn_splitkv_decode(q, k, v, num_splits=S, scale=p.scale, out=out, lse=lse,
                                        workspace=w)
                outs.append((out, lse))
        torch.cuda.synchronize()
        for (out, lse), (ro, rl) in zip(outs, refs):
            assert_lse_close(lse.cpu(), rl)
            assert_out_close(out.cpu(), ro)


def test_smoothed_forwards_on_two_streams(skv):
    """Two smoothed forwards whose keys have different offsets (so their mean(k)
    differ) on two streams at once."""
    probs = [wl.attn_problem(1, 8, 2, 700, 900, 128, seed=511, k_offset=2.0),
             wl.attn_problem(2, 4, 4, 300, 1300, 64, dtype="fp16", seed=512, k_offset=-3.0)]
    dts = ["bf16", "fp16"]
    refs = [_oracle(p, dt, causal=True) for p, dt in zip(probs, dts)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    gpu = [(p.q.to(DEV), p.k.to(DEV), p.v.to(DEV)) for p in probs]
    torch.cuda.synchronize()
    outs = []
    for (q, k, v), st, p in zip(gpu, streams, probs):
        with torch.cuda.stream(st):
            outs.append(skv.attn_fwd(q, k, v, scale=p.scale, causal=True, smooth_k=True,
                                     return_lse=True))
    torch.cuda.synchronize()
    for (out, lse), (ro, rl) in zip(outs, refs):
        assert_lse_close(lse.cpu(), rl)
        assert_out_close(out.cpu(), ro)


def test_one_decode_workspace_for_several_shapes(skv):
    """One zero-filled workspace, sized for the largest of three decode problems,
    serves all three in turn and twice over; its tickets are zero after each call."""
    shapes = [(8, 32, 8, 1, 2000, 128), (1, 16, 1, 16 // 16, 4096, 128), (2, 8, 2, 3, 777, 64)]
    probs = [wl.attn_problem(*sh, seed=520 + i) for i, sh in enumerate(shapes)]
    refs = [_oracle(p) for p in probs]
    plans = []
    for p in probs:
        B, Hq, Hkv, Lq, Lkv, D = p.dims
        S = skv.pick_num_splits(B, Hkv, (Hq // Hkv) * Lq, Lkv, D)
        plans.append((S, skv.splitkv_workspace_bytes(B, Hq, Lq, D, S, Hkv)))
    ws = torch.zeros(max(n for _, n in plans), dtype=torch.uint8, device=DEV)
    gpu = [(p.q.to(DEV), p.k.to(DEV), p.v.to(DEV)) for p in probs]
    for _ in range(2):
        for (q, k, v), (S, n), p, (ro, rl) in zip(gpu, plans, probs, refs):
            out, lse = skv.attn_splitkv_decode(q, k, v, num_splits=S, scale=p.scale, workspace=ws)
            torch.cuda.synchronize()
            assert_lse_close(lse.cpu(), rl)
            assert_out_close(out.cpu(), ro)
