"""Benchmark of the split-KV decode step and the prefill forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--reps R]

Headline workload: split-KV decode with GQA, B=8, Hq=32, Hkv=8, Lq=1, D=128, bf16,
HND, with Lkv = 4096, 8192 and 32768.  One step runs the decode (split-KV partials
+ merge) of all three problems back to back, each with the split count
skv_pick_num_splits chooses; the 32768 problem (1.07 GB of K/V) evicts the
256 MB Infinity Cache, so every problem of the next step reads cold HBM.  The
step is captured once into a HIP graph and replayed; K replays are timed with
torch.cuda.synchronize() on both sides.

`value` = algorithmic bytes of a step (K + V + Q read, out + LSE written) / step
time, in GB/s.  The decode runs as skv_attn_splitkv_decode: one launch computes
the per-chunk partial states and the last work group of each (batch, kv head)
merges them.  `roofline` covers that kernel: its algorithmic bytes per launch over
its average launch duration, timed with HIP events on the launch stream in a
separate pass in which the launches are queued behind a spin kernel (so host
overhead does not open gaps); per problem it reports the mean (`us`, the figure the
roofline uses) and the 10th / 50th / 90th percentiles over the repetitions, and
`step_us` gives the same spread for the captured step.  The two-kernel form
(partials, then merge_state) is timed as well and reported per problem.
`cpu_baseline` times the fp64 oracle (oracle/, C + OpenMP) on a bounded sample of
the same workload.  `secondary` reports the other shapes of the same path
(the decode on a partly filled KV cache bounded by a device kv_len, wide-head
decode, varlen causal prefill, ring-style chunked prefill, a dense D128 prefill,
the tiny LSE case) in us, GB/s or TFLOP/s and as a fraction of the roofline, plus
the INT8 QK^T path (skv_sage_fwd, smoothing on) on the ring and dense problems, its
fraction taken against the combined int8 + fp16 MFMA peak.  Secondary figures are
the median (`us`) of 50 graph replays, each timed with its own HIP events, with
p10 / p90 and the mean beside it; the prefill lines rotate four input copies between
replays, so that no replay finds its inputs in the Infinity Cache.  `practical_ceilings` are the micro-benchmarks of
microbench/ceilings.hip run in the same process (HBM read stream with plain and with
nontemporal loads, bf16 MFMA, ...); every decode and prefill figure is also given
as a fraction of them (`frac_practical`, `frac_mfma_practical`, and for prefill
`frac_gemm_practical`: the rate over a bf16 8192^3 vendor-library GEMM's on the same GPU).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 / fp16 MFMA, TFLOP/s
INT8_PEAK_TOPS = 5033.2        # MI355X dense int8 MFMA, TOP/s
# INT8 QK^T + fp16 P.V: per (query, key) pair 2D int8 ops and 2D fp16 flops, so at both
# peaks the 4D "attention flops" of a pair take 2D/INT8 + 2D/FP16 seconds
INT8_FP16_PEAK_TFLOPS = 4.0 / (2.0 / INT8_PEAK_TOPS + 2.0 / MFMA_PEAK_TFLOPS)
METRIC = "split-KV decode µs & HBM GB/s (%peak); prefill TFLOP/s (%MFMA peak)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--reps", type=int, default=50,
                    help="graph replays per secondary figure (default 50; fewer for profiled runs)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# Phase markers for kernel traces: before each measured phase a float64 fill kernel
# (bench.py launches no other float64 kernel) marks where the phase's launches begin
# in a rocprofv3 kernel trace, and PHASES lists the phases in order, each with the
# labels of its launchers: the k-th library launch of a phase belongs to launcher
# k mod len(labels) (launchers there are single kernels, issued round-robin).  The
# JSON line carries PHASES, so a trace of this run splits into one row per workload.
PHASES = []
_MARK = []


def phase(name, labels=None):
    if not _MARK:
        _MARK.append(torch.empty(16, dtype=torch.float64, device="cuda"))
    _MARK[0].fill_(float(len(PHASES)))
    PHASES.append(dict(name=name, labels=list(labels or [name])))


# ------------------------------------------------------------------ helpers

class Decode:
    """One decode problem on the GPU with preallocated partial and output buffers."""

    def __init__(self, skv, prob, num_splits=None):
        self.skv = skv
        self.host = prob
        self.q, self.k, self.v = prob.q.cuda(), prob.k.cuda(), prob.v.cuda()
        self.scale = prob.scale
        B, Hq, Hkv, Lq, Lkv, D = prob.dims
        self.dims = (B, Hq, Hkv, Lq, Lkv, D)
        self.S = num_splits or skv.pick_num_splits(B, Hkv, (Hq // Hkv) * Lq, Lkv, D)
        self.op = torch.empty((self.S, B, Hq, Lq, D), dtype=torch.float32, device="cuda")
        self.lp = torch.empty((self.S, B, Hq, Lq), dtype=torch.float32, device="cuda")
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device="cuda")
        self.ws = torch.zeros(skv.splitkv_workspace_bytes(B, Hq, Lq, D, self.S, Hkv),
                              dtype=torch.uint8, device="cuda")

    def partial(self):
        self.skv.attn_splitkv_partial(self.q, self.k, self.v, num_splits=self.S, scale=self.scale,
                                      out_part=self.op, lse_part=self.lp)

    def merge(self):
        self.skv.merge_state(self.op, self.lp, out=self.out, lse=self.lse)

    def two_kernel(self):
        self.partial()
        self.merge()

    def step(self):
        """Single-launch decode: partials + in-kernel merge."""
        self.skv.attn_splitkv_decode(self.q, self.k, self.v, num_splits=self.S, scale=self.scale,
                                     out=self.out, lse=self.lse, workspace=self.ws)

    def kv_bytes(self):
        B, Hq, Hkv, Lq, Lkv, D = self.dims
        return 2 * B * Hkv * Lkv * D * 2

    def partial_bytes(self):
        """Algorithmic bytes of the partial pass alone: K + V + Q."""
        B, Hq, Hkv, Lq, Lkv, D = self.dims
        return self.kv_bytes() + B * Hq * Lq * D * 2

    def step_bytes(self):
        """Algorithmic bytes of the decode: K + V + Q read, out (16-bit) + LSE written."""
        B, Hq, Hkv, Lq, Lkv, D = self.dims
        return self.partial_bytes() + B * Hq * Lq * D * 2 + B * Hq * Lq * 4


def _ws_dims(d, S):
    B, Hq, Hkv, Lq, Lkv, D = d.dims
    return B, Hq, Lq, D, S, Hkv


def capture(fn):
    """Capture fn() (library calls only, all buffers preallocated) into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _pct(xs, q):
    """q-th percentile (0..100) of a list, linear interpolation."""
    ys = sorted(xs)
    if not ys:
        return float("nan")
    pos = (len(ys) - 1) * q / 100.0
    lo = int(pos)
    hi = min(lo + 1, len(ys) - 1)
    return ys[lo] + (ys[hi] - ys[lo]) * (pos - lo)


def stats(xs):
    """Mean, median and the 10th / 90th percentiles of per-replay times (us)."""
    return dict(mean=sum(xs) / len(xs), p10=_pct(xs, 10), p50=_pct(xs, 50), p90=_pct(xs, 90))


def time_graph(g, reps, warm=3):
    """Per-replay GPU times (us) of a captured graph, or of a list of graphs replayed in
    rotation (replay i runs g[i % len(g)]): HIP events around each of `reps` replays,
    all queued behind a spin kernel that outlasts the host's enqueue time, so host
    overhead opens no gaps.  Returns stats(): mean, p10, p50, p90."""
    gs = list(g) if isinstance(g, (list, tuple)) else [g]
    for i in range(max(warm, len(gs))):
        gs[i % len(gs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    gs[0].replay()                  # host enqueue cost of one replay
    host_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    torch.cuda._sleep(int(_spin_cycles_per_ms() * (3.0 * (host_ms + 0.05) * reps + 5.0)))
    for i, (a, b) in enumerate(evs):
        a.record()
        gs[i % len(gs)].replay()
        b.record()
    torch.cuda.synchronize()
    return stats([a.elapsed_time(b) * 1e3 for a, b in evs])


# Prefill lines replay NCOPY input copies in rotation, so that consecutive replays do not
# find their inputs in the 256 MB Infinity Cache (NCOPY copies of each problem's inputs
# exceed twice its size).
NCOPY = 4


def copies(*ts):
    """NCOPY copies of each tensor: the tensor itself, then clones."""
    return [[t] + [t.clone() for _ in range(NCOPY - 1)] for t in ts]


def _spin_cycles_per_ms():
    """Calibrate torch.cuda._sleep (a spin kernel counting device clock cycles)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    torch.cuda._sleep(1_000_000)
    e1.record()
    torch.cuda.synchronize()
    return 1_000_000 / max(e0.elapsed_time(e1), 1e-3)


def kernel_durations(launchers, reps, per_rep=False):
    """Per-launch GPU durations (us) of each callable, timed with HIP events on the
    current (launch) stream.  The launches are queued behind a spin kernel that
    outlasts the host's enqueue time, so host overhead cannot open idle gaps inside
    a measured interval.  Returns the mean per callable, or with per_rep the list of
    every repetition's duration per callable."""
    n = len(launchers)
    t0 = time.perf_counter()
    for fn in launchers:            # one unmeasured pass: host enqueue cost
        fn()
    torch.cuda.synchronize()
    host_ms = (time.perf_counter() - t0) * 1e3
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n)] for _ in range(reps)]
    cyc = _spin_cycles_per_ms()
    torch.cuda.synchronize()
    torch.cuda._sleep(int(cyc * (3.0 * host_ms * reps + 5.0)))
    for r in range(reps):
        for i, fn in enumerate(launchers):
            a, b = evs[r][i]
            a.record()
            fn()
            b.record()
    torch.cuda.synchronize()
    durs = [[evs[r][i][0].elapsed_time(evs[r][i][1]) * 1e3 for r in range(reps)]
            for i in range(n)]
    if per_rep:
        return durs
    return [sum(d) / reps for d in durs]


# ------------------------------------------------------------- workloads

def headline(skv, args):
    import workloads as wl
    lkvs = (4096, 8192, 32768)
    dec = []
    for L in lkvs:
        log(f"generating decode_gqa Lkv={L}")
        dec.append(Decode(skv, wl.decode_gqa(L)))

    def step():
        for d in dec:
            d.step()

    phase("decode_gqa step (graph)", [f"decode_gqa Lkv{L}" for L in lkvs])
    g = capture(step)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    step_bytes = sum(d.step_bytes() for d in dec)
    value = step_bytes / (ms * 1e-3) / 1e9

    # dominant kernel: the single-launch decode kernel (all of the step's work);
    # durations per launch from HIP events.  The two-kernel form (partials, then
    # merge_state) is timed too, for comparison.
    reps = max(5, args.steps)
    phase("decode_gqa single launch", [f"decode_gqa Lkv{L} S{d.S}" for L, d in zip(lkvs, dec)])
    fused = [stats(x) for x in kernel_durations([d.step for d in dec], reps, per_rep=True)]
    fused_us = [st["mean"] for st in fused]
    phase("decode_gqa step (graph, events)", [f"decode_gqa Lkv{L}" for L in lkvs])
    step_st = time_graph(g, reps)
    launchers = []
    for d in dec:
        launchers += [d.partial, d.merge]
    phase("decode_gqa two-kernel", [f"decode_gqa Lkv{L} {w}" for L in lkvs
                                      for w in ("partial", "merge")])
    durs = kernel_durations(launchers, reps)
    part_us = [durs[2 * i] for i in range(len(dec))]
    merge_us = [durs[2 * i + 1] for i in range(len(dec))]
    avg_us = sum(fused_us) / len(fused_us)
    avg_bytes = sum(d.step_bytes() for d in dec) / len(dec)
    achieved = avg_bytes / (avg_us * 1e-6) / 1e9

    # the single-launch decode at the chunk counts of config 2 (8 to 32) and at 4, the
    # three problems interleaved as in the step (cold HBM); same buffers, own workspaces
    sweep_S = (4, 8, 16, 32)
    sweep = {}
    for S in sweep_S:
        wss = [torch.zeros(d.skv.splitkv_workspace_bytes(*_ws_dims(d, S)), dtype=torch.uint8,
                           device="cuda") for d in dec]
        fns = [(lambda d=d, w=w, S=S: d.skv.attn_splitkv_decode(
            d.q, d.k, d.v, num_splits=S, scale=d.scale, out=d.out, lse=d.lse, workspace=w))
            for d, w in zip(dec, wss)]
        phase(f"decode_gqa single launch num_splits={S}",
              [f"decode_gqa Lkv{L} S{S}" for L in lkvs])
        sweep[S] = [stats(x) for x in kernel_durations(fns, reps, per_rep=True)]
        del wss

    # per problem, from the same event passes (problems run in step order: cold HBM)
    per = {}
    for i, (L, d) in enumerate(zip(lkvs, dec)):
        us = fused_us[i]
        gbs = d.step_bytes() / (us * 1e-6) / 1e9
        by_s = {}
        for S in sweep_S:
            u = sweep[S][i]["mean"]
            by_s[str(S)] = dict(us=round(u, 2), frac=round(d.step_bytes() / (u * 1e-6) / 1e9 /
                                                        HBM_PEAK_GBS, 4),
                                p50_us=round(sweep[S][i]["p50"], 2))
        per[str(L)] = dict(num_splits=d.S, us=round(us, 2), gbs=round(gbs, 1),
                           frac=round(gbs / HBM_PEAK_GBS, 4),
                           p10_us=round(fused[i]["p10"], 2), p50_us=round(fused[i]["p50"], 2),
                           p90_us=round(fused[i]["p90"], 2),
                           two_kernel_us=round(part_us[i] + merge_us[i], 2),
                           partial_us=round(part_us[i], 2), merge_us=round(merge_us[i], 2),
                           single_launch_by_num_splits=by_s)
    return dec, dict(ms=ms, value=value, step_bytes=step_bytes, achieved=achieved,
                     avg_us=avg_us, avg_bytes=avg_bytes, per=per, step_st=step_st)


def parity_sample(dec):
    """A few rows of the measured decode problems against the oracle (sanity only)."""
    import numpy as np

    import oracle
    import workloads as wl
    errs = []
    d = dec[0]
    prob_q, prob_k, prob_v = d.host.q, d.host.k, d.host.v
    B, Hq, Hkv, Lq, Lkv, D = d.dims
    rows = np.array([[0, 0, 0], [B - 1, Hq - 1, Lq - 1], [B // 2, Hq // 3, 0]])
    ro, rl = oracle.attn_rows(wl.bits(prob_q), wl.bits(prob_k), wl.bits(prob_v), "bf16", rows,
                              scale=d.scale)
    out, lse = d.out.float().cpu().numpy(), d.lse.cpu().numpy()
    for n, (b, h, i) in enumerate(rows):
        errs.append(max(abs(float(lse[b, h, i]) - rl[n]),
                        float(np.abs(out[b, h, i] - ro[n]).max())))
    return max(errs)


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), else what platform reports."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


# The oracle's config-1 attention (B1 H4 Sq64 Sk1000 D128: the graded-row query, fp64),
# timed in a child process started with OMP_NUM_THREADS=1 so that it runs on one core.
_C1_SINGLE_CORE = r"""
import json, sys, time
sys.path.insert(0, sys.argv[1])
import oracle, workloads as wl
d = wl.tiny_lse()
args = (wl.bits(d["q_graded"]), wl.bits(d["k"]), wl.bits(d["v"]), "bf16")
oracle.attn(*args, scale=d["scale"])
ts = []
for _ in range(5):
    t = time.perf_counter()
    oracle.attn(*args, scale=d["scale"])
    ts.append(time.perf_counter() - t)
print(json.dumps(sorted(ts)[2]))
"""


def c1_single_core_ms():
    """Milliseconds per call of the oracle's config-1 attention on one core (median of 5
    calls), or None when the child process fails."""
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1")
    try:
        r = subprocess.run([sys.executable, "-c", _C1_SINGLE_CORE, ROOT], env=env,
                           capture_output=True, text=True, timeout=300)
        return round(float(r.stdout.strip().splitlines()[-1]) * 1e3, 2)
    except (subprocess.SubprocessError, ValueError, IndexError):
        return None


def cpu_baseline(dec, args):
    """The oracle's decode step (fp64 per-chunk partials + merge, same split counts) on
    the same three problems, repeated until at least 10 s of host time has passed; with
    the host's CPU model, OMP_NUM_THREADS as set, and the config-1 oracle on one core."""
    import oracle
    import workloads as wl
    cores = len(os.sched_getaffinity(0))
    threads = min(int(os.environ.get("OMP_NUM_THREADS", cores)), cores)
    inputs = [(wl.bits(d.host.q), wl.bits(d.host.k), wl.bits(d.host.v), d) for d in dec]
    reps, t0 = 0, time.perf_counter()
    while True:
        for qb, kb, vb, d in inputs:
            o, l = oracle.splitkv_partials(qb, kb, vb, "bf16", d.S, scale=d.scale)
            oracle.merge(o, l)
        reps += 1
        sec = time.perf_counter() - t0
        if sec >= 10.0 or sec * (reps + 1) / reps > 30.0:
            break
    step_bytes = sum(d.step_bytes() for d in dec)
    return dict(value=round(step_bytes * reps / sec / 1e9, 4), unit="GB/s", cores=threads,
                kind="oracle",
                sample=f"the whole decode step (Lkv 4096, 8192, 32768; B=8 Hq=32 Hkv=8 D=128), "
                       f"fp64 partials + merge, {reps} repetition(s) in {sec:.1f} s",
                cpu=cpu_model(), cpus_available=cores,
                omp_num_threads=os.environ.get("OMP_NUM_THREADS"),
                c1_single_core_ms=c1_single_core_ms(),
                c1_single_core="the oracle's config-1 attention (B1 H4 Sq64 Sk1000 D128, fp64, "
                               "graded-row query) on one core (OMP_NUM_THREADS=1), median of "
                               "5 calls")


def secondary(skv, args, dec):
    import workloads as wl
    res = {}
    reps = max(3, args.reps)

    def pct(st):
        """Median (`us`) and spread of per-replay times, rounded."""
        return dict(us=round(st["p50"], 2), p10_us=round(st["p10"], 2), p90_us=round(st["p90"], 2),
                    mean_us=round(st["mean"], 2))

    # partly filled KV cache: the Lkv-32768 decode_gqa problem with every kv_len = 4096
    # (lengths on the device, split count chosen for the capacity, as a captured
    # serving loop would keep it); only the filled keys are read
    d32 = dec[-1]
    B, Hq, Hkv, Lq, Lkv, D = d32.dims
    filled = 4096
    kvl = torch.full((B,), filled, dtype=torch.int32, device="cuda")

    def partly_filled():
        skv.attn_splitkv_decode(d32.q, d32.k, d32.v, num_splits=d32.S, scale=d32.scale,
                                out=d32.out, lse=d32.lse, workspace=d32.ws, kv_len=kvl)
    # each timed launch follows a full decode of the 1.07 GB Lkv-32768 problem, which
    # evicts the 256 MB Infinity Cache: the filled keys are read cold
    phase("decode_gqa kv_len", ["capacity32768 kv_len4096", "evicting Lkv32768 decode"])
    st = stats(kernel_durations([partly_filled, d32.step], reps, per_rep=True)[0])
    us = st["p50"]
    fb = 2 * B * Hkv * filled * D * 2 + 2 * B * Hq * Lq * D * 2 + B * Hq * Lq * 4
    res["decode_gqa_capacity32768_kvlen4096"] = dict(
        **pct(st), gbs=round(fb / (us * 1e-6) / 1e9, 1), frac_hbm=round(fb / (us * 1e-6) / 1e9 /
                                                                       HBM_PEAK_GBS, 4),
        num_splits=d32.S, filled_bytes=fb, cache="cold (each launch follows a 1.07 GB decode)")

    # small-query GQA decode with more query rows per kv head (G x Lq = 32 and 64):
    # B8 Hkv8 D128 bf16 Lkv 8192, G = 8 and 16 with Lq = 4; the two problems alternate
    # (268 MB of K/V each), so each reads what the other evicted
    many = []
    for G in (8, 16):
        log(f"generating decode G={G} Lq=4")
        many.append((G, Decode(skv, wl.decode_gqa(8192, seed=40 + G, Hq=8 * G, Lq=4))))
    phase("decode many rows", [f"G{G} Lq4 rows{4 * G}" for G, _ in many])
    durs = kernel_durations([d.step for _, d in many], reps, per_rep=True)
    for i, (G, d) in enumerate(many):
        st = stats(durs[i])
        us = st["p50"]
        gbs = d.step_bytes() / (us * 1e-6) / 1e9
        res[f"decode_gqa_G{G}_Lq4_rows{4 * G}_B8_Hkv8_Lkv8192_D128"] = dict(
            **pct(st), gbs=round(gbs, 1), frac_hbm=round(gbs / HBM_PEAK_GBS, 4), num_splits=d.S)
    del many, durs
    torch.cuda.empty_cache()

    # wide-head decode: B4 Hq16 Hkv4 Lq4 D256, K offset +2; the two problems
    # alternate, so each reads what the other evicted
    wides = []
    for L in (16384, 32768):
        log(f"generating wide_decode Lkv={L}")
        wides.append((L, Decode(skv, wl.wide_decode(L, +1))))
    launchers = [d.step for _, d in wides]
    phase("decode wide D256", [f"wide Lkv{L}" for L, _ in wides])
    durs = kernel_durations(launchers, reps, per_rep=True)
    for i, (L, d) in enumerate(wides):
        st = stats(durs[i])
        us = st["p50"]
        gbs = d.step_bytes() / (us * 1e-6) / 1e9
        res[f"decode_wide_D256_Lq4_Lkv{L}"] = dict(
            **pct(st), gbs=round(gbs, 1), frac_hbm=round(gbs / HBM_PEAK_GBS, 4), num_splits=d.S)
    del wides, launchers
    torch.cuda.empty_cache()

    # varlen causal prefill: 16 sequences, lengths U[128, 4096], Hq32 Hkv8 D128 bf16
    log("generating varlen_prefill")
    vl = wl.varlen_prefill(seed=4)
    qs, ks, vs = copies(vl.q.cuda(), vl.k.cuda(), vl.v.cuda())
    cq, ck = vl.cu_seqlens_q.cuda(), vl.cu_seqlens_k.cuda()
    out = torch.empty_like(qs[0])
    lse = torch.empty((qs[0].shape[1], qs[0].shape[0]), dtype=torch.float32, device="cuda")
    mx = max(vl.lengths)

    def varlen(i):
        return lambda: skv.attn_fwd_varlen(qs[i], ks[i], vs[i], cq, ck, mx, scale=vl.scale,
                                           causal=True, out=out, lse=lse)
    phase("prefill varlen causal")
    st = time_graph([capture(varlen(i)) for i in range(NCOPY)], reps)
    us = st["p50"]
    fl = wl.prefill_flops(vl.lengths, 32, 128, causal=True)
    tf = fl / (us * 1e-6) / 1e12
    res["prefill_varlen_causal_16seq_Hq32_Hkv8_D128"] = dict(
        **pct(st), tflops=round(tf, 1), frac_mfma=round(tf / MFMA_PEAK_TFLOPS, 4),
        total_tokens=vl.meta["T"], flop=fl)
    del qs, ks, vs, out, lse
    torch.cuda.empty_cache()

    # ring-style chunked prefill: B1 H16 S8192 D64 fp16, 4 KV chunks with smoothing + merge
    log("generating ring_chunks")
    rc = wl.ring_chunks(seed=5)
    qs, kfs, vfs = copies(rc["q"].cuda(), rc["k"].cuda(), rc["v"].cuda())
    kcs = list(zip(*copies(*[t.cuda() for t in rc["k_chunks"]])))   # kcs[i][c]
    vcs = list(zip(*copies(*[t.cuda() for t in rc["v_chunks"]])))
    q = qs[0]
    po = torch.empty((4,) + tuple(q.shape), dtype=q.dtype, device="cuda")
    pl = torch.empty((4, 1, 16, 8192), dtype=torch.float32, device="cuda")
    mo = torch.empty_like(q)
    ml = torch.empty((1, 16, 8192), dtype=torch.float32, device="cuda")
    fo = torch.empty_like(q)
    fl_ = torch.empty((1, 16, 8192), dtype=torch.float32, device="cuda")

    def ring(i):
        def f():
            for c in range(4):
                skv.attn_fwd(qs[i], kcs[i][c], vcs[i][c], scale=rc["scale"], smooth_k=True,
                             out=po[c], lse=pl[c])
            skv.merge_state(po, pl, out=mo, lse=ml)
        return f

    def full(i):
        return lambda: skv.attn_fwd(qs[i], kfs[i], vfs[i], scale=rc["scale"], out=fo, lse=fl_)
    fl = 4 * 16 * 8192 * 8192 * 64
    for name, fn in (("prefill_ring_4chunks_smooth_merge_H16_S8192_D64_fp16", ring),
                     ("prefill_full_H16_S8192_D64_fp16", full)):
        phase(name)
        st = time_graph([capture(fn(i)) for i in range(NCOPY)], reps)
        us = st["p50"]
        tf = fl / (us * 1e-6) / 1e12
        res[name] = dict(**pct(st), tflops=round(tf, 1), frac_mfma=round(tf / MFMA_PEAK_TFLOPS, 4),
                         flop=fl)
    # INT8 QK^T with smoothing (fp16 P.V) on the same ring problem: per chunk + merge,
    # and unsplit.  Each call quantises its own q and chunk (mean(k), codes, scales),
    # all inside the timed region.
    wsr = torch.empty(skv.sage_workspace_bytes(1, 16, 16, 8192, 2048, 64, q.dtype, True),
                      dtype=torch.uint8, device="cuda")
    wsf = torch.empty(skv.sage_workspace_bytes(1, 16, 16, 8192, 8192, 64, q.dtype, True),
                      dtype=torch.uint8, device="cuda")

    def ring_int8(i):
        def f():
            for c in range(4):
                skv.sage_fwd(qs[i], kcs[i][c], vcs[i][c], scale=rc["scale"], smooth_k=True,
                             out=po[c], lse=pl[c], workspace=wsr)
            skv.merge_state(po, pl, out=mo, lse=ml)
        return f

    def full_int8(i):
        return lambda: skv.sage_fwd(qs[i], kfs[i], vfs[i], scale=rc["scale"], smooth_k=True,
                                    out=fo, lse=fl_, workspace=wsf)
    for name, fn in (("prefill_int8qk_ring_4chunks_smooth_merge_H16_S8192_D64_fp16", ring_int8),
                     ("prefill_int8qk_full_smooth_H16_S8192_D64_fp16", full_int8)):
        phase(name)
        st = time_graph([capture(fn(i)) for i in range(NCOPY)], reps)
        us = st["p50"]
        tf = fl / (us * 1e-6) / 1e12
        res[name] = dict(**pct(st), tflops=round(tf, 1),
                         frac_mfma_int8_fp16=round(tf / INT8_FP16_PEAK_TFLOPS, 4), flop=fl)
    del q, qs, kcs, vcs, kfs, vfs, po, pl, mo, ml, fo, fl_, wsr, wsf
    torch.cuda.empty_cache()

    # dense non-causal D128 bf16 (the varlen problem's heads at one 8192-token
    # sequence): 16-bit path and INT8 QK^T path with smoothing
    log("generating dense D128 problem")
    p = wl.attn_problem(1, 32, 8, 8192, 8192, 128, seed=7)
    qs, ks, vs = copies(p.q.cuda(), p.k.cuda(), p.v.cuda())
    out = torch.empty_like(qs[0])
    lse = torch.empty((1, 32, 8192), dtype=torch.float32, device="cuda")
    wsd = torch.empty(skv.sage_workspace_bytes(1, 32, 8, 8192, 8192, 128, qs[0].dtype, True),
                      dtype=torch.uint8, device="cuda")

    def dense16(i):
        return lambda: skv.attn_fwd(qs[i], ks[i], vs[i], scale=p.scale, out=out, lse=lse)

    def dense8(i):
        return lambda: skv.sage_fwd(qs[i], ks[i], vs[i], scale=p.scale, smooth_k=True, out=out,
                                    lse=lse, workspace=wsd)
    fl = 4 * 32 * 8192 * 8192 * 128
    phase("prefill_dense_H32_Hkv8_S8192_D128_bf16")
    st = time_graph([capture(dense16(i)) for i in range(NCOPY)], reps)
    us = st["p50"]
    tf = fl / (us * 1e-6) / 1e12
    res["prefill_dense_H32_Hkv8_S8192_D128_bf16"] = dict(
        **pct(st), tflops=round(tf, 1), frac_mfma=round(tf / MFMA_PEAK_TFLOPS, 4), flop=fl)
    phase("prefill_int8qk_dense_smooth_H32_Hkv8_S8192_D128_bf16")
    st = time_graph([capture(dense8(i)) for i in range(NCOPY)], reps)
    us = st["p50"]
    tf = fl / (us * 1e-6) / 1e12
    res["prefill_int8qk_dense_smooth_H32_Hkv8_S8192_D128_bf16"] = dict(
        **pct(st), tflops=round(tf, 1),
        frac_mfma_int8_fp16=round(tf / INT8_FP16_PEAK_TFLOPS, 4), flop=fl)
    del qs, ks, vs, out, lse, wsd
    torch.cuda.empty_cache()

    # tiny LSE case: B1 H4 Sq64 Sk1000 D128 bf16 (launch-bound)
    d = wl.tiny_lse()
    tq, tk, tv = d["q_graded"].cuda(), d["k"].cuda(), d["v"].cuda()
    to = torch.empty_like(tq)
    tl = torch.empty((1, 4, 64), dtype=torch.float32, device="cuda")

    def tiny():
        skv.attn_fwd(tq, tk, tv, scale=d["scale"], out=to, lse=tl)
    phase("tiny_lse_B1_H4_Sq64_Sk1000_D128")
    res["tiny_lse_B1_H4_Sq64_Sk1000_D128"] = pct(time_graph(capture(tiny), reps))
    return res


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "decode_gqa_splitkv_decode_hbm_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "split_kv_merge_amd", "csrc", f)
                  for f in ("splitkv.hip", "splitkv_tail.h", "device.h", "launch.h")]


def kernel_source_sha():
    """SHA-256 of the decode kernel's sources with comments and whitespace removed:
    splitkv.hip, splitkv_tail.h, device.h and, of launch.h, only the decode's argument block
    (struct SplitArgs), so that the counter record goes stale when the decode's code
    changes, not its comments or other kernels' declarations."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        text = open(f, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        if f.endswith("launch.h"):
            m = re.search(r"struct SplitArgs\s*\{.*?\};", text, flags=re.S)
            text = m.group(0) if m else text
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter record, or
    None when the record is missing or the kernel source changed since it was taken."""
    try:
        rec = json.load(open(TRAFFIC_RECORD))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def practical_ceilings():
    """The practical ceilings of microbench/ceilings.hip, measured in this run (HBM read
    stream with plain and with nontemporal loads, bf16 MFMA, LDS, exp/FMA rates alone and
    interleaved), or None when that library is not built."""
    if not os.path.exists(os.path.join(ROOT, "microbench", "libceilings.so")):
        return None
    sys.path.insert(0, os.path.join(ROOT, "microbench"))
    import ceilings
    return {k: round(v, 3) if abs(v) < 10 else round(v, 1) for k, v in ceilings.measure().items()}


def copy_probe():
    """A plain device copy of known size (256 MiB read + 256 MiB written), for
    scaling the FETCH_SIZE / WRITE_SIZE counters of a profiled run."""
    a = torch.empty(64 * 1024 * 1024, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import split_kv_merge_amd as skv
    skv._load()
    torch.cuda.init()
    dec, h = headline(skv, args)
    err = parity_sample(dec)
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(dec, args)
    sec = {} if args.no_secondary else secondary(skv, args, dec)
    copy_probe()
    ceil = None if args.no_secondary else practical_ceilings()
    if ceil:
        # the same figures against the practical ceilings measured above
        hbm = ceil["hbm_read_stream_nontemporal_GBs"]
        mfma = ceil["mfma_bf16_32x32x16_tflops"]
        gemm = ceil.get("gemm_bf16_8192_tflops")
        for v in h["per"].values():
            v["frac_practical"] = round(v["gbs"] / hbm, 4)
        for v in sec.values():
            if "gbs" in v:
                v["frac_practical"] = round(v["gbs"] / hbm, 4)
            if "frac_mfma" in v:
                v["frac_mfma_practical"] = round(v["tflops"] / mfma, 4)
                if gemm:
                    v["frac_gemm_practical"] = round(v["tflops"] / gemm, 4)
    line = {
        "metric": METRIC,
        "value": round(h["value"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "decode_gqa: split-KV decode (partials + stable merge, one launch), "
                        "B=8 Hq=32 Hkv=8 Lq=1 D=128 bf16 HND, Lkv 4096 + 8192 + 32768 per step",
            "global_batch": 8,
            "seq_len": [4096, 8192, 32768],
            "parallelism": "single GPU",
            "num_splits": {k: v["num_splits"] for k, v in h["per"].items()},
            "step_bytes": h["step_bytes"],
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(h["achieved"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(h["achieved"] / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "kernel": "splitkv_kernel<bf16, 128, single-launch> (skv_attn_splitkv_decode)",
            "avg_launch_us": round(h["avg_us"], 2),
            "algorithmic_bytes_per_launch": int(h["avg_bytes"]),
            "practical_peak": ceil["hbm_read_stream_nontemporal_GBs"] if ceil else None,
            "frac_practical": (round(h["achieved"] / ceil["hbm_read_stream_nontemporal_GBs"], 4)
                               if ceil else None),
        },
        "step_us": {k: round(v, 2) for k, v in h["step_st"].items()},
        "cpu_baseline": cpu,
        "per_problem": h["per"],
        "parity_sample_max_err": round(err, 5),
        "secondary": sec,
        "practical_ceilings": ceil,
        "trace_phases": PHASES,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
