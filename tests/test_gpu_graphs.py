"""HIP-graph replay of the prefill, varlen and merge calls.

Every call only enqueues on its stream and reads lengths on the device, so a captured
graph must follow new inputs, and new device-side sequence boundaries, from replay to
replay.  Each test captures once, then replays several times with fresh inputs written
into the captured tensors between replays (with eager work and synchronisations in
between), and checks every replay against the fp64 oracle at the parity bar.  The
decode and INT8 graphs are covered in test_gpu_parity.py, test_gpu_kvlen.py and
test_gpu_sage.py.
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


def _capture(fn):
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        fn()                                   # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def test_smoothed_causal_fwd_graph_replays(skv):
    """mean(k) and the attention kernel in one graph; k's offset changes per replay,
    so a stale mean would shift the LSE."""
    probs = [wl.attn_problem(1, 8, 2, 300, 420, 128, seed=610 + i, k_offset=off)
             for i, off in enumerate((2.0, -1.5, 0.0))]
    p0 = probs[0]
    q, k, v = p0.q.to(DEV), p0.k.to(DEV), p0.v.to(DEV)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    g = _capture(lambda: skv.attn_fwd(q, k, v, scale=p0.scale, causal=True, smooth_k=True,
                                      out=out, lse=lse))
    for p in probs + probs[:1]:
        q.copy_(p.q); k.copy_(p.k); v.copy_(p.v)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ro, rl = oracle.attn(wl.bits(p.q), wl.bits(p.k), wl.bits(p.v), "bf16", "HND", p.scale, True)
        assert_lse_close(lse.cpu(), rl)
        assert_out_close(out.cpu(), ro)


def test_varlen_graph_follows_device_seqlens(skv):
    """Three sequences packed in 900 tokens; the boundaries in cu_seqlens (on the
    device) and the data change between replays, within the captured max_seqlen."""
    Hq, Hkv, D, T, maxL = 8, 2, 128, 900, 500
    splits = [[300, 300, 300], [100, 500, 300], [450, 50, 400], [500, 400, 0]]
    gen = torch.Generator().manual_seed(620)
    datas = [tuple(torch.randn(T, h, D, generator=gen).to(torch.bfloat16) for h in (Hq, Hkv, Hkv))
             for _ in splits]
    q = torch.empty(T, Hq, D, dtype=torch.bfloat16, device=DEV)
    k = torch.empty(T, Hkv, D, dtype=torch.bfloat16, device=DEV)
    v = torch.empty_like(k)
    cu = torch.zeros(len(splits[0]) + 1, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty(Hq, T, dtype=torch.float32, device=DEV)
    scale = wl.default_scale(D)

    def load(i):
        qq, kk, vv = datas[i]
        q.copy_(qq); k.copy_(kk); v.copy_(vv)
        cu.copy_(torch.from_numpy(np.concatenate([[0], np.cumsum(splits[i])]).astype(np.int32)))

    load(0)
    g = _capture(lambda: skv.attn_fwd_varlen(q, k, v, cu, cu, maxL, scale=scale, causal=True,
                                             out=out, lse=lse))
    for i in (1, 2, 3, 0):
        load(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        cuh = np.concatenate([[0], np.cumsum(splits[i])]).astype(np.int32)
        qq, kk, vv = datas[i]
        ro, rl = oracle.attn_varlen(wl.bits(qq), wl.bits(kk), wl.bits(vv), "bf16", cuh, cuh,
                                    scale=scale, causal=True)
        assert_lse_close(lse.cpu(), rl)
        assert_out_close(out.cpu(), ro)


def test_merge_state_graph_replays(skv):
    """Four fp32 partial states of 3 x 16 x 50 rows (some parts -inf, one row -inf in
    every part) merged in a graph; the parts change between replays."""
    S, B, H, R, D = 4, 3, 16, 50, 128
    gen = torch.Generator().manual_seed(630)
    sets = []
    for _ in range(3):
        o = torch.randn(S, B, H, R, D, generator=gen)
        l = torch.randn(S, B, H, R, generator=gen) * 20
        l[1, 0, :, :7] = -float("inf")
        l[:, 2, 3, 11] = -float("inf")
        sets.append((o, l))
    o_dev = torch.empty(S, B, H, R, D, dtype=torch.float32, device=DEV)
    l_dev = torch.empty(S, B, H, R, dtype=torch.float32, device=DEV)
    out = torch.empty(B, H, R, D, dtype=torch.float32, device=DEV)
    lse = torch.empty(B, H, R, dtype=torch.float32, device=DEV)
    o_dev.copy_(sets[0][0]); l_dev.copy_(sets[0][1])
    g = _capture(lambda: skv.merge_state(o_dev, l_dev, out=out, lse=lse))
    for o, l in sets[1:] + sets[:1]:
        o_dev.copy_(o); l_dev.copy_(l)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ro, rl = oracle.merge(o.numpy().astype(np.float64), l.numpy().astype(np.float64))
        assert_lse_close(lse.cpu(), rl)
        assert_out_close(out.cpu(), ro)
        assert torch.isneginf(lse[2, 3, 11]).item() and (out[2, 3, 11] == 0).all().item()
