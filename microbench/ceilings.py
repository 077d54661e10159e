"""Run the micro-benchmarks of ceilings.hip and print one line per ceiling.

    python microbench/ceilings.py        (needs microbench/libceilings.so, built by
                                          __graft_entry__.build())
Rates per compute unit assume the 2.4 GHz peak clock.
"""
import ctypes
import os
import sys

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libceilings.so")


def build():
    import subprocess
    subprocess.run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-shared", "-fPIC",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-o", LIB, os.path.join(HERE, "ceilings.hip")], check=True,
                   capture_output=True)
    return LIB


def measure():
    lib = ctypes.CDLL(LIB)
    lib.run.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                        ctypes.c_int, ctypes.c_void_p]
    out = torch.zeros(1 << 20, dtype=torch.int32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def t(which, grid, iters, p=None, n=0, reps=5):
        for _ in range(2):
            assert lib.run(which, p, n, ctypes.c_void_p(out.data_ptr()), grid, iters, st) == 0
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            lib.run(which, p, n, ctypes.c_void_p(out.data_ptr()), grid, iters, st)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    CU, CLK = 256, 2.4e9
    res = {}
    g, it = CU * 4, 2000
    sec = t(0, g, it)
    res["lds_read_b128_B_per_clk_per_cu"] = g * 256 * 16 * 16 * it / sec / CU / CLK
    sec = t(1, g, it)
    res["lds_read_tr16_b64_B_per_clk_per_cu"] = g * 256 * 8 * 16 * it / sec / CU / CLK
    g2 = CU * 2
    sec = t(2, g2, 2000)
    res["mfma_bf16_32x32x16_tflops"] = g2 * 4 * 4 * 32768 * 2000 / sec / 1e12
    g2 = CU * 4
    sec = t(3, g2, 2000)
    res["exp_f32_lanes_per_clk_per_cu"] = g2 * 256 * 8 * 2000 / sec / CU / CLK
    sec = t(4, g2, 2000)
    res["fma_f32_lanes_per_clk_per_cu"] = g2 * 256 * 8 * 2000 / sec / CU / CLK
    # Two waves per SIMD (the prefill kernels' occupancy): exponentials alone, then with
    # one and three independent FMAs each.  A time ratio near 1 + (FMA time / exp time)
    # means one shared pipe; near max(1, FMA time / exp time), separate pipes.
    g3 = CU * 2
    t_exp = t(7, g3, 4000)
    t_fma = t(4, g3, 4000)
    res["exp_only_f32_lanes_per_clk_per_cu"] = g3 * 256 * 8 * 4000 / t_exp / CU / CLK
    res["fma_over_exp_time_2waves"] = t_fma / t_exp
    res["exp_plus_fma_over_exp_time_2waves"] = t(8, g3, 4000) / t_exp
    res["exp_plus_3fma_over_exp_time_2waves"] = t(9, g3, 4000) / t_exp
    # The same MFMA stream for about a quarter of a second per launch, when the chip's power
    # management has settled: the rate and the shader clock it holds (s_memtime ticks
    # per s_memrealtime tick at 100 MHz, from work group 0)
    g4, it4 = CU * 2, 2_000_000
    sec = t(10, g4, it4, reps=2)
    clk = out[:6].cpu().view(torch.int64)
    res["mfma_bf16_32x32x16_sustained_tflops"] = g4 * 4 * 4 * 32768 * it4 / sec / 1e12
    res["mfma_sustained_shader_clock_ghz"] = float(clk[0]) / float(clk[1]) * 0.1
    buf = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    for which, key in ((5, "hbm_read_stream_GBs"), (6, "hbm_read_stream_nontemporal_GBs")):
        best = 0.0
        for grid in (512, 1024, 2048, 4096, 8192):   # each divides the element count
            sec = t(which, grid, 0, ctypes.c_void_p(buf.data_ptr()), buf.numel() // 16)
            best = max(best, buf.numel() / sec / 1e9)
        res[key] = best
    del buf
    # A vendor-library GEMM (torch.matmul, hipBLASLt on ROCm), bf16 8192^3: what a kernel
    # that streams its MFMA operands through memory and LDS reaches on this machine, as
    # opposed to the register-only MFMA loop above.
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        a @ b
    e1.record()
    torch.cuda.synchronize()
    res["gemm_bf16_8192_tflops"] = 2 * 8192 ** 3 / (e0.elapsed_time(e1) / 20 * 1e-3) / 1e12
    return res


if __name__ == "__main__":
    if not os.path.exists(LIB):
        sys.exit("microbench/libceilings.so is not built")
    for k, v in measure().items():
        print(f"{k}: {v:.3g}", flush=True)
