// ceilings.hip -- micro-benchmarks for the practical ceilings the attention kernels
// are measured against on MI355X (gfx950): LDS read bandwidth (16-byte reads and
// the 64-bit transpose read), bf16 MFMA throughput, v_exp_f32 and v_fma_f32 issue
// rates, alone and interleaved (whether exponentials and FMAs share one pipe), the MFMA
// rate and shader clock sustained over a long run, and an HBM read stream (plain and nontemporal loads).  Measurement infrastructure only; nothing
// in the attention library uses it.
#include <hip/hip_runtime.h>
#include <stdint.h>
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// LDS read bandwidth: each lane reads 16 B at a conflict-free address, ITER times.
__global__ __launch_bounds__(256) void lds_b128(uint32_t* out, int iters) {
  __shared__ u32x4 buf[4096];  // 64 KB
  int t = threadIdx.x;
  for (int i = t; i < 4096; i += 256) buf[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  u32x4 acc = {0, 0, 0, 0};
  int base = (threadIdx.x >> 6) * 1024 + (threadIdx.x & 63);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      u32x4 v = buf[(base + u * 64 + it) & 4095];
      acc ^= v;
    }
  }
  if (acc.x == 0x12345678) out[blockIdx.x] = acc.y;
}
__global__ __launch_bounds__(256) void lds_tr(uint32_t* out, int iters) {
  __shared__ short buf[32768];  // 64 KB
  int t = threadIdx.x;
  for (int i = t; i < 32768; i += 256) buf[i] = (short)i;
  __syncthreads();
  u32x2 acc = {0, 0};
  int lane = t & 63;
  int base = (t >> 6) * 8192 + lane * 4;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(buf + ((base + u * 256 + it * 4) & 32767)));
      acc ^= __builtin_bit_cast(u32x2, r);
    }
  }
  if (acc.x == 0x12345678) out[blockIdx.x] = acc.y;
}
// MFMA throughput: 4 independent accumulators
__global__ __launch_bounds__(256) void mfma_bf16(float* out, int iters) {
  bf16x8 a, b;
  for (int j = 0; j < 8; ++j) { a[j] = (__bf16)(threadIdx.x * 0.001f + j); b[j] = (__bf16)(j * 0.5f); }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  f32x16 s = c0 + c1 + c2 + c3;
  float r = 0; for (int j = 0; j < 16; ++j) r += s[j];
  if (r == 1234.5f) out[blockIdx.x] = r;
}
// The same MFMA stream, long enough (tens to hundreds of ms) for the chip's power
// management to settle, with the shader clock it ran at: work group 0's first lane
// records s_memtime (shader clock) and s_memrealtime (100 MHz) at its start and end.
__global__ __launch_bounds__(256) void mfma_bf16_clocked(unsigned long long* out, int iters) {
  unsigned long long t0 = 0, r0 = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  bf16x8 a, b;
  for (int j = 0; j < 8; ++j) { a[j] = (__bf16)(threadIdx.x * 0.001f + j); b[j] = (__bf16)(j * 0.5f); }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  f32x16 s = c0 + c1 + c2 + c3;
  float r = 0; for (int j = 0; j < 16; ++j) r += s[j];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    out[0] = t1 - t0;
    out[1] = r1 - r0;
    out[2] = r == 1234.5f ? 1ull : 0ull;   // keeps the accumulators live
  }
}
// exp2 throughput
__global__ __launch_bounds__(256) void exp_f32(float* out, int iters) {
  float x0 = threadIdx.x * 1e-3f, x1 = x0 + 0.1f, x2 = x0 + 0.2f, x3 = x0 + 0.3f, x4 = x0+0.4f, x5=x0+0.5f, x6=x0+0.6f, x7=x0+0.7f;
  for (int it = 0; it < iters; ++it) {
    x0 = __builtin_amdgcn_exp2f(x0) * -0.5f; x1 = __builtin_amdgcn_exp2f(x1) * -0.5f;
    x2 = __builtin_amdgcn_exp2f(x2) * -0.5f; x3 = __builtin_amdgcn_exp2f(x3) * -0.5f;
    x4 = __builtin_amdgcn_exp2f(x4) * -0.5f; x5 = __builtin_amdgcn_exp2f(x5) * -0.5f;
    x6 = __builtin_amdgcn_exp2f(x6) * -0.5f; x7 = __builtin_amdgcn_exp2f(x7) * -0.5f;
  }
  float r = x0 + x1 + x2 + x3 + x4 + x5 + x6 + x7;
  if (r == 1234.5f) out[blockIdx.x] = r;
}
// fma throughput
__global__ __launch_bounds__(256) void fma_f32(float* out, int iters) {
  float x0 = threadIdx.x * 1e-3f, x1 = x0 + 0.1f, x2 = x0 + 0.2f, x3 = x0 + 0.3f, x4 = x0+0.4f, x5=x0+0.5f, x6=x0+0.6f, x7=x0+0.7f;
  for (int it = 0; it < iters; ++it) {
    x0 = fmaf(x0, 0.999f, 0.001f); x1 = fmaf(x1, 0.999f, 0.001f); x2 = fmaf(x2, 0.999f, 0.001f); x3 = fmaf(x3, 0.999f, 0.001f);
    x4 = fmaf(x4, 0.999f, 0.001f); x5 = fmaf(x5, 0.999f, 0.001f); x6 = fmaf(x6, 0.999f, 0.001f); x7 = fmaf(x7, 0.999f, 0.001f);
  }
  float r = x0 + x1 + x2 + x3 + x4 + x5 + x6 + x7;
  if (r == 1234.5f) out[blockIdx.x] = r;
}
// v_exp_f32 alone (the -|x| folds into the source modifiers: one instruction per
// element), then with one and with three independent FMAs per exponential.
__global__ __launch_bounds__(256) void exp_only(float* out, int iters) {
  float x0 = threadIdx.x * 1e-3f, x1 = x0 + 0.1f, x2 = x0 + 0.2f, x3 = x0 + 0.3f, x4 = x0+0.4f, x5=x0+0.5f, x6=x0+0.6f, x7=x0+0.7f;
  for (int it = 0; it < iters; ++it) {
    x0 = __builtin_amdgcn_exp2f(-__builtin_fabsf(x0)); x1 = __builtin_amdgcn_exp2f(-__builtin_fabsf(x1));
    x2 = __builtin_amdgcn_exp2f(-__builtin_fabsf(x2)); x3 = __builtin_amdgcn_exp2f(-__builtin_fabsf(x3));
    x4 = __builtin_amdgcn_exp2f(-__builtin_fabsf(x4)); x5 = __builtin_amdgcn_exp2f(-__builtin_fabsf(x5));
    x6 = __builtin_amdgcn_exp2f(-__builtin_fabsf(x6)); x7 = __builtin_amdgcn_exp2f(-__builtin_fabsf(x7));
  }
  float r = x0 + x1 + x2 + x3 + x4 + x5 + x6 + x7;
  if (r == 1234.5f) out[blockIdx.x] = r;
}
template <int NF>
__global__ __launch_bounds__(256) void exp_fma(float* out, int iters) {
  float x[8], y[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) { x[j] = threadIdx.x * 1e-3f + 0.1f * j; y[j] = x[j] + 1.f; }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[j] = __builtin_amdgcn_exp2f(-__builtin_fabsf(x[j]));
#pragma unroll
      for (int f = 0; f < NF; ++f) y[j] = fmaf(y[j], 0.999f - 0.001f * f, 0.001f);
    }
  }
  float r = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) r += x[j] + y[j];
  if (r == 1234.5f) out[blockIdx.x] = r;
}
// HBM read stream: each work group streams its own contiguous range with eight
// 16-byte loads in flight per thread, as plain loads or with the nontemporal hint.
template <bool NT>
__global__ __launch_bounds__(256) void hbm_read(const u32x4* in, int64_t n, uint32_t* out) {
  u32x4 acc = {0,0,0,0};
  const int64_t C = n / gridDim.x;
  const u32x4* p = in + (int64_t)blockIdx.x * C;
  int64_t i = threadIdx.x;
  for (; i + 7 * 256 < C; i += 8 * 256) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = NT ? __builtin_nontemporal_load(p + i + u * 256) : p[i + u * 256];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  for (; i < C; i += 256) acc ^= p[i];
  if (acc.x == 0x12345678) out[blockIdx.x] = acc.y;
}
extern "C" int run(int which, void* p, int64_t n, void* out, int grid, int iters, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  switch (which) {
    case 0: hipLaunchKernelGGL(lds_b128, dim3(grid), dim3(256), 0, s, (uint32_t*)out, iters); break;
    case 1: hipLaunchKernelGGL(lds_tr, dim3(grid), dim3(256), 0, s, (uint32_t*)out, iters); break;
    case 2: hipLaunchKernelGGL(mfma_bf16, dim3(grid), dim3(256), 0, s, (float*)out, iters); break;
    case 3: hipLaunchKernelGGL(exp_f32, dim3(grid), dim3(256), 0, s, (float*)out, iters); break;
    case 4: hipLaunchKernelGGL(fma_f32, dim3(grid), dim3(256), 0, s, (float*)out, iters); break;
    case 5: hipLaunchKernelGGL(hbm_read<false>, dim3(grid), dim3(256), 0, s, (const u32x4*)p, n, (uint32_t*)out); break;
    case 6: hipLaunchKernelGGL(hbm_read<true>, dim3(grid), dim3(256), 0, s, (const u32x4*)p, n, (uint32_t*)out); break;
    case 7: hipLaunchKernelGGL(exp_only, dim3(grid), dim3(256), 0, s, (float*)out, iters); break;
    case 8: hipLaunchKernelGGL(exp_fma<1>, dim3(grid), dim3(256), 0, s, (float*)out, iters); break;
    case 9: hipLaunchKernelGGL(exp_fma<3>, dim3(grid), dim3(256), 0, s, (float*)out, iters); break;
    case 10: hipLaunchKernelGGL(mfma_bf16_clocked, dim3(grid), dim3(256), 0, s, (unsigned long long*)out, iters); break;
  }
  return (int)hipGetLastError();
}
