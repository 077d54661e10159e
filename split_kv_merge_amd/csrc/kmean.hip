// kmean.hip -- mean of k over the keys of one call, per (batch | sequence, kv head).
//
// The smoothing of auto-round #2556 "ARK return_lse gives the same LSE for every
// 16 query rows" (Problem Description, second issue; Reproduction Steps part 3)
// subtracts mean(k), taken along the key axis, from every key; the attention
// kernel turns that into a per-row logit bias and adds it back into the LSE.
// One work group streams the keys of one (batch, kv head) with 16-byte loads,
// accumulates in fp32 and reduces through LDS.
#include "device.h"
#include "launch.h"

namespace skv {

namespace {

template <typename T, int D, bool VARLEN>
__global__ __launch_bounds__(256) void kmean_kernel(KmeanArgs a) {
    using E = Elem<T>;
    constexpr int CPR = D / 8;      // threads per key row
    constexpr int RPP = 256 / CPR;  // key rows per pass
    __shared__ float red[RPP * D];

    const int tid = threadIdx.x, g = blockIdx.x, b = blockIdx.y;
    int Lk;
    int64_t off;
    if (VARLEN) {
        const int k0 = a.cu_k[b];
        Lk = a.cu_k[b + 1] - k0;
        off = (int64_t)k0 * a.kv_row;
    } else {
        Lk = a.Sk;
        off = (int64_t)b * a.kv_batch;
    }
    const uint16_t* kp = (const uint16_t*)a.k + off + (int64_t)g * a.kv_head + (tid % CPR) * 8;

    // Eight rows in flight per thread: the loop is latency-bound otherwise.
    constexpr int U = 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int j = tid / CPR;
    for (; j + (U - 1) * RPP < Lk; j += U * RPP) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = load16(kp + (int64_t)(j + u * RPP) * a.kv_row);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                acc[2 * w] += E::to_float((uint16_t)(v[u][w] & 0xffff));
                acc[2 * w + 1] += E::to_float((uint16_t)(v[u][w] >> 16));
            }
    }
    for (; j < Lk; j += RPP) {
        const u32x4 v = load16(kp + (int64_t)j * a.kv_row);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            acc[2 * w] += E::to_float((uint16_t)(v[w] & 0xffff));
            acc[2 * w + 1] += E::to_float((uint16_t)(v[w] >> 16));
        }
    }
#pragma unroll
    for (int w = 0; w < 8; ++w) red[(tid / CPR) * D + (tid % CPR) * 8 + w] = acc[w];
    __syncthreads();
    if (tid < D) {
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < RPP; ++r) sum += red[r * D + tid];
        a.kbar[((int64_t)b * a.Hkv + g) * D + tid] = Lk > 0 ? sum / (float)Lk : 0.f;
    }
}

template <typename T, int D>
hipError_t launch_kmean_t(const KmeanArgs& a, bool varlen, dim3 grid, hipStream_t st) {
    if (varlen)
        hipLaunchKernelGGL((kmean_kernel<T, D, true>), grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((kmean_kernel<T, D, false>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_kmean_d(const KmeanArgs& a, int D, bool varlen, dim3 grid, hipStream_t st) {
    switch (D) {
        case 64: return launch_kmean_t<T, 64>(a, varlen, grid, st);
        case 128: return launch_kmean_t<T, 128>(a, varlen, grid, st);
        case 256: return launch_kmean_t<T, 256>(a, varlen, grid, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_kmean(const KmeanArgs& a, int dtype, int D, bool varlen, int grid_b,
                        hipStream_t stream) {
    const dim3 grid((unsigned)a.Hkv, (unsigned)grid_b);
    if (dtype == 0) return launch_kmean_d<__bf16>(a, D, varlen, grid, stream);
    return launch_kmean_d<_Float16>(a, D, varlen, grid, stream);
}

}  // namespace skv
