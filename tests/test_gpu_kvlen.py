"""GPU parity of the kv_len-bounded split-KV decode (a partly filled KV cache).

Protocol of the ExecuTorch PR #22133 review ("Prevent Voxtral NaNs in CUDA split-K
attention", reviewer item 3): every key and value past a batch element's filled
length is NaN, every partial slot is pre-filled with NaN, and L_kv is swept from 1
to 40000.  The expected result is the oracle on the filled keys only: the merged
output and LSE of dense attention over keys [0, kv_len[b]), and each chunk's partial
state over the same even split of that length.
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


def _problem(B, Hq, Hkv, Lq, Lkv, D, seed, dtype="bf16"):
    """A seeded problem plus per-batch filled lengths (0 and Lkv included when B >= 2);
    positions past the filled length are NaN in K and V."""
    p = wl.attn_problem(B, Hq, Hkv, Lq, Lkv, D, dtype=dtype, seed=seed)
    g = np.random.default_rng(seed)
    lens = g.integers(0, Lkv + 1, size=B)
    if B >= 2:
        lens[0], lens[-1] = Lkv, 0
    if B >= 3:
        lens[1] = min(Lkv, 1)
    k, v = p.k.clone(), p.v.clone()
    for b in range(B):
        k[b, :, lens[b]:] = float("nan")
        v[b, :, lens[b]:] = float("nan")
    return p, k, v, lens.astype(np.int32)


def _oracle_per_batch(p, lens, dtype, S=None):
    """Dense attention (and, with S, the chunk partials) over each element's filled keys."""
    outs, lses, pos, pls = [], [], [], []
    for b, L in enumerate(lens):
        q = wl.bits(p.q[b:b + 1])
        k = wl.bits(p.k[b:b + 1, :, :L].contiguous())
        v = wl.bits(p.v[b:b + 1, :, :L].contiguous())
        o, l = oracle.attn(q, k, v, dtype, scale=p.scale)
        outs.append(o)
        lses.append(l)
        if S is not None:
            po, pl = oracle.splitkv_partials(q, k, v, dtype, S, scale=p.scale)
            pos.append(po)
            pls.append(pl)
    ro, rl = np.concatenate(outs), np.concatenate(lses)
    if S is None:
        return ro, rl
    return ro, rl, np.concatenate(pos, axis=1), np.concatenate(pls, axis=1)


SWEEP = [
    # B, Hq, Hkv, Lq, Lkv, D, S
    (3, 8, 2, 2, 1, 128, 4),
    (3, 8, 2, 1, 2, 128, 8),
    (4, 8, 2, 2, 33, 128, 4),
    (3, 16, 4, 1, 257, 64, 8),
    (2, 8, 2, 4, 1000, 256, 16),
    (3, 32, 8, 1, 4097, 128, 4),
    (2, 8, 1, 2, 12345, 128, 32),
    (2, 8, 2, 1, 40000, 128, 8),
    (2, 32, 1, 2, 3001, 128, 24),     # 64 rows per kv head
    (3, 16, 1, 2, 777, 64, 8),        # 32 rows per kv head (one 32-row block), lengths 777, 1, 0
    (2, 24, 1, 1, 100, 128, 16),      # 24 rows, 7-key chunks and empty ones
]


@pytest.mark.parametrize("case", SWEEP)
def test_kv_len_partials_and_merge_nan_poisoned(skv, case):
    B, Hq, Hkv, Lq, Lkv, D, S = case
    p, k_nan, v_nan, lens = _problem(B, Hq, Hkv, Lq, Lkv, D, seed=500 + Lkv)
    ro, rl, ro_p, rl_p = _oracle_per_batch(p, lens, "bf16", S)
    q, k, v = p.q.to(DEV), k_nan.to(DEV), v_nan.to(DEV)
    kv_len = torch.from_numpy(lens).to(DEV)
    op = torch.full((S, B, Hq, Lq, D), float("nan"), dtype=torch.float32, device=DEV)
    lp = torch.full((S, B, Hq, Lq), float("nan"), dtype=torch.float32, device=DEV)
    skv.attn_splitkv_partial(q, k, v, num_splits=S, scale=p.scale, out_part=op, lse_part=lp,
                             kv_len=kv_len)
    out, lse = skv.merge_state(op, lp, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_lse_close(lp.cpu(), rl_p, "partial lse")
    assert_out_close(op.cpu(), ro_p, "partial out")
    assert_lse_close(lse.cpu(), rl)
    assert_out_close(out.cpu(), ro)


@pytest.mark.parametrize("case", SWEEP)
def test_kv_len_single_launch_decode_nan_poisoned(skv, case):
    B, Hq, Hkv, Lq, Lkv, D, S = case
    p, k_nan, v_nan, lens = _problem(B, Hq, Hkv, Lq, Lkv, D, seed=600 + Lkv)
    ro, rl = _oracle_per_batch(p, lens, "bf16")
    q, k, v = p.q.to(DEV), k_nan.to(DEV), v_nan.to(DEV)
    kv_len = torch.from_numpy(lens).to(DEV)
    ws = torch.zeros(skv.splitkv_workspace_bytes(B, Hq, Lq, D, S, Hkv), dtype=torch.uint8,
                     device=DEV)
    # poison the partial-state part of the workspace (the counter block at its start
    # must stay zero): all-ones bytes are NaN in float32 and in both 16-bit types
    ws[65536 * 4:].fill_(0xFF)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, Lq), float("nan"), dtype=torch.float32, device=DEV)
    skv.attn_splitkv_decode(q, k, v, num_splits=S, scale=p.scale, out=out, lse=lse,
                            workspace=ws, kv_len=kv_len)
    torch.cuda.synchronize()
    assert_lse_close(lse.cpu(), rl)
    assert_out_close(out.cpu(), ro)


def test_kv_len_out_of_range_is_clamped(skv):
    """Lengths below 0 read as 0 (out 0, LSE -inf); above Lkv as Lkv."""
    B, Hq, Hkv, Lq, Lkv, D, S = 2, 8, 2, 1, 300, 128, 4
    p = wl.attn_problem(B, Hq, Hkv, Lq, Lkv, D, seed=77)
    ro, rl = _oracle_per_batch(p, np.array([0, Lkv]), "bf16")
    out, lse = skv.attn_splitkv_decode(p.q.to(DEV), p.k.to(DEV), p.v.to(DEV), num_splits=S,
                                       scale=p.scale,
                                       kv_len=torch.tensor([-5, 10 ** 6], dtype=torch.int32,
                                                           device=DEV))
    torch.cuda.synchronize()
    assert_lse_close(lse.cpu(), rl)
    assert_out_close(out.cpu(), ro)


def test_kv_len_graph_replays_follow_the_length(skv):
    """One captured decode, replayed while kv_len grows on the device between
    replays: each replay matches the oracle at its own lengths (graph-safe)."""
    B, Hq, Hkv, Lq, Lkv, D, S = 2, 32, 8, 1, 2048, 128, 4
    p = wl.attn_problem(B, Hq, Hkv, Lq, Lkv, D, seed=88)
    q, k, v = p.q.to(DEV), p.k.to(DEV), p.v.to(DEV)
    kv_len = torch.zeros(B, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=DEV)
    ws = torch.zeros(skv.splitkv_workspace_bytes(B, Hq, Lq, D, S, Hkv), dtype=torch.uint8,
                     device=DEV)
    fn = lambda: skv.attn_splitkv_decode(q, k, v, num_splits=S, scale=p.scale, out=out, lse=lse,
                                         workspace=ws, kv_len=kv_len)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        fn()
    torch.cuda.current_stream().wait_stream(st)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for lens in ([1, 7], [100, 64], [1000, 2048], [2048, 5]):
        kv_len.copy_(torch.tensor(lens, dtype=torch.int32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ro, rl = _oracle_per_batch(p, np.array(lens), "bf16")
        assert_lse_close(lse.cpu(), rl, f"lse at {lens}")
        assert_out_close(out.cpu(), ro, f"out at {lens}")
