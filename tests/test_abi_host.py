"""CPU checks of the C ABI: the library loads, exports every declared entry point,
and rejects malformed arguments before touching the GPU."""
from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch  # noqa: F401  (the HIP runtime torch ships must be the one libskv binds to)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "skv.h")
LIB = os.path.join(ROOT, "split_kv_merge_amd", "libskv.so")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(skv_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libskv.so is not built (run __graft_entry__.build())")
    import split_kv_merge_amd as skv
    return skv._load()


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("skv_attn_fwd", "skv_attn_fwd_varlen", "skv_attn_splitkv_partial", "skv_merge_state"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), f"{name} declared in skv.h but not exported"


def test_single_hip_runtime_mapped(lib):
    maps = open("/proc/self/maps").read()
    libs = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
    assert len(libs) <= 1, libs


def test_status_strings(lib):
    assert lib.skv_status_str(0) == b"ok"
    assert lib.skv_status_str(1) == b"invalid argument"
    assert lib.skv_status_str(2) == b"unsupported configuration"


def test_workspace_and_split_heuristic(lib):
    # mean(k) [B, Hkv, D] float32, then fp64 sums of min(32, ceil(512 / (B*Hkv))) splits
    assert lib.skv_workspace_bytes(2, 8, 128, 1) == 2 * 8 * 128 * 4 + 2 * 8 * 32 * 128 * 8
    assert lib.skv_workspace_bytes(16, 8, 64, 1) == 16 * 8 * 64 * 4 + 16 * 8 * 4 * 64 * 8
    assert lib.skv_workspace_bytes(64, 8, 128, 1) == 64 * 8 * 128 * 4      # one split
    assert lib.skv_workspace_bytes(2, 8, 128, 0) == 0
    for B, Hkv, Lkv in [(8, 8, 4096), (8, 8, 32768), (4, 4, 16384), (1, 1, 10), (1, 2, 0)]:
        s = lib.skv_pick_num_splits(B, Hkv, 4, Lkv, 128)
        assert 1 <= s <= max(1, Lkv // 128)


# A fake but 256-byte aligned device-looking address: validation must reject the
# call before any launch, so nothing ever dereferences it.
FAKE = ctypes.c_void_p(0x10000)


def _fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, B=1, Hq=4, Hkv=2, Sq=8, Sk=8, D=128,
             dtype=0, layout=0, scale=0.1, causal=0, smooth_k=0, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.skv_attn_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                            a["Sq"], a["Sk"], a["D"], a["dtype"], a["layout"], a["scale"],
                            a["causal"], a["smooth_k"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1),
    (dict(Hq=6, Hkv=4), 1),           # not a multiple
    (dict(Hkv=0), 1),
    (dict(B=-1), 1),
    (dict(Sq=-3), 1),
    (dict(D=96), 2),                  # well-formed, not built
    (dict(D=0), 1),
    (dict(dtype=2), 2),               # fp32 attention not built
    (dict(dtype=7), 1),
    (dict(layout=5), 1),
    (dict(scale=float("nan")), 1),
    (dict(scale=float("inf")), 1),
    (dict(q=ctypes.c_void_p(0x10008)), 1),   # misaligned
    (dict(smooth_k=1), 1),            # no workspace
    (dict(smooth_k=1, ws=FAKE, ws_bytes=16), 1),  # too small
])
def test_attn_fwd_rejects(lib, kw, status):
    assert _fwd(lib, **kw) == status
    assert lib.skv_last_error() != b""


def test_grid_limit_rejected_before_any_launch(lib):
    """Too many row tiles is refused before anything is launched, also with smoothing,
    whose mean-k kernel would otherwise run first and write the workspace."""
    ws = dict(smooth_k=1, ws=FAKE, ws_bytes=1 << 20)
    assert _fwd(lib, Sq=65536 * 256, **ws) == 2
    assert b"row tiles" in lib.skv_last_error()


def test_zero_sized_calls_succeed_without_launching(lib):
    assert _fwd(lib, B=0) == 0
    assert _fwd(lib, Sq=0) == 0


def test_varlen_rejects(lib):
    P = FAKE

    def call(**kw):
        a = dict(nseq=2, total_q=10, total_k=10, maxq=8, Hq=4, Hkv=2, D=128, dtype=0, cu=P)
        a.update(kw)
        return lib.skv_attn_fwd_varlen(P, P, P, P, None, a["cu"], a["cu"], a["nseq"], a["total_q"],
                                       a["total_k"], a["maxq"], a["Hq"], a["Hkv"], a["D"], a["dtype"],
                                       0.1, 1, 0, None, 0, None)
    assert call(cu=None) == 1
    assert call(maxq=11) == 1
    assert call(nseq=-1) == 1
    assert call(Hq=5) == 1
    assert call(D=48) == 2
    assert call(nseq=0) == 0


def test_splitkv_rejects(lib):
    P = FAKE

    def call(**kw):
        a = dict(B=1, Hq=32, Hkv=8, Lq=1, Lkv=64, D=128, S=4, kv_len=None)
        a.update(kw)
        return lib.skv_attn_splitkv_partial(P, P, P, P, P, a["B"], a["Hq"], a["Hkv"], a["Lq"],
                                            a["Lkv"], a["D"], 0, 0, 0.1, a["S"], a["kv_len"],
                                            None)
    assert call(S=0) == 1
    assert call(Lq=0) == 1
    assert call(Lkv=-1) == 1
    assert call(Hq=30) == 1
    assert call(Lq=17) == 2          # (32/8)*17 = 68 rows per kv head > 64
    assert call(Lq=5, D=256) == 2    # 20 rows > 16 at D = 256
    assert call(D=80) == 2
    assert call(kv_len=ctypes.c_void_p(0x10002)) == 1   # kv_len misaligned
    assert call(B=0) == 0


def test_merge_rejects(lib):
    P = FAKE
    arr = ctypes.c_int64 * 3
    good = arr(0, 128, 128)

    def call(**kw):
        a = dict(S=4, R=(1, 2, 3), D=128, pdt=2, odt=0, pstride=128 * 6, ps=good, ls=arr(0, 1, 1),
                 os_=good)
        a.update(kw)
        return lib.skv_merge_state(a["S"], *a["R"], a["D"], P, a["pdt"], a["pstride"], a["ps"], P,
                                   6, a["ls"], P, a["odt"], a["os_"], None, None, None)
    assert call(S=0) == 1
    assert call(R=(1, -2, 3)) == 1
    assert call(D=100) == 2
    assert call(pdt=9) == 1
    assert call(pstride=3) == 1       # not a multiple of 16 bytes
    assert call(ps=None) == 1
    assert call(R=(0, 2, 3)) == 0     # no rows: nothing to do


def test_python_binding_fails_loudly_without_gpu_tensors():
    import split_kv_merge_amd as skv
    q = torch.zeros(1, 2, 4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        skv.attn_fwd(q, q, q)


def test_lse_varlen_to_dense_checks_shape():
    import split_kv_merge_amd as skv
    lse = torch.arange(2 * 6, dtype=torch.float32).reshape(2, 6)   # H=2, B=3, S=2
    dense = skv.lse_varlen_to_dense(lse, 3, 2)
    assert dense.shape == (3, 2, 2)
    assert dense[1, 0, 1] == lse[0, 3]
    with pytest.raises(ValueError):
        skv.lse_varlen_to_dense(lse, 4, 2)
    # with the boundaries, equal lengths pass and unequal ones (same total) are refused
    cu_eq = torch.tensor([0, 2, 4, 6], dtype=torch.int32)
    assert torch.equal(skv.lse_varlen_to_dense(lse, 3, 2, cu_seqlens=cu_eq), dense)
    with pytest.raises(ValueError):
        skv.lse_varlen_to_dense(lse, 3, 2, cu_seqlens=torch.tensor([0, 1, 4, 6], dtype=torch.int32))


def test_splitkv_decode_rejects(lib):
    P = FAKE
    ws = ctypes.c_void_p(0x20000)   # 256-byte aligned

    def call(**kw):
        a = dict(B=2, Hq=32, Hkv=8, Lq=1, Lkv=4096, D=128, S=8, ws=ws, wsb=1 << 30, out=P,
                 kv_len=None)
        a.update(kw)
        return lib.skv_attn_splitkv_decode(P, P, P, a["out"], None, a["B"], a["Hq"], a["Hkv"],
                                           a["Lq"], a["Lkv"], a["D"], 0, 0, 0.1, a["S"],
                                           a["kv_len"], a["ws"], a["wsb"], None)
    assert call(S=257) == 2          # at most 256 splits in the single-launch form
    assert call(kv_len=ctypes.c_void_p(0x10001)) == 1   # kv_len misaligned
    assert call(ws=None) == 1
    assert call(ws=ctypes.c_void_p(0x20010)) == 1     # not 256-byte aligned
    assert call(wsb=16) == 1
    assert call(out=None) == 1
    assert call(B=0) == 0
    assert call(B=8193, Hkv=8, Hq=8, ws=None, wsb=0) == 2   # B*Hkv over 65536 counters
    need = lib.skv_splitkv_workspace_bytes(2, 32, 1, 128, 8, 8)
    rows = 8 * 2 * 32
    # the fixed counter block (65536 int32), 16-bit chunk outputs, float32 chunk LSEs
    assert need == 65536 * 4 + ((rows * 128 * 2 + 255) // 256 + (rows * 4 + 255) // 256) * 256


def test_splitkv_decode_noalloc_rejects_before_touching_the_device(lib):
    """The no-allocation decode validates like the workspace form and refuses a
    problem whose partial states do not fit its fixed scratch, all before any device
    call (so these run without a GPU)."""
    P = FAKE
    cap = lib.skv_splitkv_decode_noalloc_max_bytes()
    assert cap == 16 << 20

    def call(**kw):
        a = dict(B=8, Hq=32, Hkv=8, Lq=1, Lkv=4096, D=128, S=8, out=P, kv_len=None)
        a.update(kw)
        return lib.skv_attn_splitkv_decode_noalloc(P, P, P, a["out"], None, a["B"], a["Hq"],
                                                   a["Hkv"], a["Lq"], a["Lkv"], a["D"], 0, 0, 0.1,
                                                   a["S"], a["kv_len"], None)
    assert call(S=257) == 2
    assert call(out=None) == 1
    assert call(Hq=30) == 1
    assert call(B=0) == 0
    # a decode of 8 x 32 rows at D = 128 fits with up to 128 splits ...
    assert lib.skv_splitkv_workspace_bytes(8, 32, 1, 128, 128, 8) <= cap
    # ... a problem whose partial states exceed the scratch is refused with a message
    big = dict(B=64, Hq=64, Hkv=8, Lq=1, D=256, S=64)
    assert lib.skv_splitkv_workspace_bytes(64, 64, 1, 256, 64, 8) > cap
    assert call(**big) == 2
    assert b"scratch" in lib.skv_last_error()


def _sage_fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, B=1, Hq=4, Hkv=2, Sq=64, Sk=64, D=128,
             dtype=0, layout=0, scale=0.1, causal=0, smooth=1, ws=ctypes.c_void_p(0x20000),
             wsb=1 << 30)
    a.update(kw)
    return lib.skv_sage_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                            a["Sq"], a["Sk"], a["D"], a["dtype"], a["layout"], a["scale"],
                            a["causal"], a["smooth"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=256), 2),                 # the INT8 path is built for D 64 and 128
    (dict(D=96), 2),
    (dict(dtype=2), 2),
    (dict(Hq=5), 1),
    (dict(q=None), 1),
    (dict(out=None), 1),
    (dict(ws=None), 1),
    (dict(ws=ctypes.c_void_p(0x20010)), 1),   # not 256-byte aligned
    (dict(wsb=16), 1),
    (dict(scale=float("nan")), 1),
    (dict(layout=3), 1),
    (dict(Sq=65536 * 256), 2),        # more row tiles than the grid allows
])
def test_sage_fwd_rejects(lib, kw, status):
    assert _sage_fwd(lib, **kw) == status
    assert lib.skv_last_error() != b""


def test_sage_zero_sized_and_workspace(lib):
    assert _sage_fwd(lib, B=0) == 0
    assert _sage_fwd(lib, Sq=0) == 0
    # sections, each padded to 256 bytes: mean(k) fp32 [B,Hkv,D]; its fp64 split sums
    # (32 splits for 2 kv heads); q codes int8; q scales fp32 [B,Hq,Sq/32]; add-back fp32
    # [B,Hq,Sq]; k codes int8; k scales fp32; V in fp16 (bf16 input)
    r = lambda x: (x + 255) // 256 * 256
    B, Hq, Hkv, Sq, Sk, D = 1, 4, 2, 64, 64, 128
    want = (r(B * Hkv * D * 4) + r(B * Hkv * 32 * D * 8) + r(B * Hq * Sq * D) + r(B * Hq * 2 * 4)
            + r(B * Hq * Sq * 4) + r(B * Hkv * Sk * D) + r(B * Hkv * 2 * 4) + r(B * Hkv * Sk * D * 2))
    assert lib.skv_sage_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, 0, 1) == want
    # fp16 input: no V copy; no smoothing: no mean(k) and no add-back
    assert lib.skv_sage_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, 1, 0) == (
        r(B * Hq * Sq * D) + r(B * Hq * 2 * 4) + r(B * Hkv * Sk * D) + r(B * Hkv * 2 * 4))


def test_sage_quant_rejects(lib):
    P = FAKE

    def call(**kw):
        a = dict(q=P, k=P, B=1, Hq=4, Hkv=2, Sq=64, Sk=64, D=128, smooth=1, qc=P, qs=P, kc=P,
                 ks=P, kb=P)
        a.update(kw)
        return lib.skv_sage_quant(a["q"], a["k"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"],
                                  a["D"], 0, 0, a["smooth"], a["qc"], a["qs"], a["kc"], a["ks"],
                                  a["kb"], None)
    assert call(kb=None) == 1         # smoothing needs the mean(k) output
    assert call(qc=None) == 1
    assert call(qc=ctypes.c_void_p(0x10008)) == 1   # codes need 16-byte alignment
    assert call(D=256) == 2
    assert call(Hkv=3) == 1
    assert call(B=0) == 0


def _header_prototypes():
    """name -> parameter count of every skv_* prototype in include/skv.h."""
    import re
    text = open(os.path.join(ROOT, "include", "skv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    out = {}
    for m in re.finditer(r"\b(skv_\w+)\s*\(([^;{]*?)\)\s*;", text):
        params = " ".join(m.group(2).split())
        out[m.group(1)] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_argtypes_match_the_header(lib):
    """The ctypes binding declares, for every entry point, as many arguments as the
    C prototype has: a drift would shift arguments into the wrong slots silently."""
    import split_kv_merge_amd as skv
    protos = _header_prototypes()
    assert set(protos) == set(_declared())
    for name, n in protos.items():
        fn = getattr(skv._lib, name)
        assert fn.argtypes is not None, f"{name}: no argtypes in the binding"
        assert len(fn.argtypes) == n, f"{name}: binding {len(fn.argtypes)} args, header {n}"
