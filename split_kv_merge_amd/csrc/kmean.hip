// kmean.hip -- mean of k over the keys of one call, per (batch | sequence, kv head).
//
// The smoothing of auto-round #2556 "ARK return_lse gives the same LSE for every
// 16 query rows" (Problem Description, second issue; Reproduction Steps part 3)
// subtracts mean(k), taken along the key axis, from every key; the attention
// kernel turns that into a per-row logit bias and adds it back into the LSE.
// One work group streams the keys of one (batch, kv head) with 16-byte loads,
// accumulates in fp64 and reduces through LDS: the sum of 16-bit inputs is then
// exact whatever the order (their significant bits span far less than 53 bits
// for any realistic key range), so mean(k) is the exact mean rounded once to
// float32 -- the value the INT8 path's codes are defined on.
#include "device.h"
#include "launch.h"

namespace skv {

namespace {

// Grid (kv head, batch | sequence, split): split s sums keys [s*C, min((s+1)*C, Lk))
// with C = ceil(Lk / nsplit), so even one (batch, kv head) spreads over many
// compute units.  With one split the mean is written directly; otherwise each
// split writes its fp64 column sums and kmean_finish_kernel adds them in order.
template <typename T, int D, bool VARLEN>
__global__ __launch_bounds__(256) void kmean_kernel(KmeanArgs a) {
    using E = Elem<T>;
    constexpr int CPR = D / 8;      // threads per key row
    constexpr int RPP = 256 / CPR;  // key rows per pass
    __shared__ double red[RPP * D];

    const int tid = threadIdx.x, g = blockIdx.x, b = blockIdx.y, sp = blockIdx.z;
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
    const int64_t C = ((int64_t)Lk + a.nsplit - 1) / a.nsplit;
    const int j0 = (int)min((int64_t)sp * C, (int64_t)Lk);
    const int j1 = (int)min((int64_t)j0 + C, (int64_t)Lk);
    const uint16_t* kp = (const uint16_t*)a.k + off + (int64_t)g * a.kv_head + (tid % CPR) * 8;

    // Sixteen rows in flight per thread (64 KB per work group): with one work group
    // per (batch, kv head) the loop is latency-bound otherwise.
    constexpr int U = 16;
    double acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    int j = j0 + tid / CPR;
    for (; j + (U - 1) * RPP < j1; j += U * RPP) {
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
    for (; j < j1; j += RPP) {
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
        double sum = 0.0;
#pragma unroll
        for (int r = 0; r < RPP; ++r) sum += red[r * D + tid];
        const int64_t bg = (int64_t)b * a.Hkv + g;
        if (a.nsplit == 1)
            a.kbar[bg * D + tid] = Lk > 0 ? (float)(sum / (double)Lk) : 0.f;
        else
            a.partial[(bg * a.nsplit + sp) * D + tid] = sum;
    }
}

// mean = (sum of the split sums, in split order) / Lk, rounded once to float32.
template <int D, bool VARLEN>
__global__ __launch_bounds__(D) void kmean_finish_kernel(KmeanArgs a) {
    const int g = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    const int Lk = VARLEN ? a.cu_k[b + 1] - a.cu_k[b] : a.Sk;
    const int64_t bg = (int64_t)b * a.Hkv + g;
    // all loads first (independent), then the sum in split order
    double part[kMaxKmeanSplits];
#pragma unroll
    for (int sp = 0; sp < kMaxKmeanSplits; ++sp)
        part[sp] = sp < a.nsplit ? a.partial[(bg * a.nsplit + sp) * D + d] : 0.0;
    double sum = 0.0;
#pragma unroll
    for (int sp = 0; sp < kMaxKmeanSplits; ++sp) sum += part[sp];
    a.kbar[bg * D + d] = Lk > 0 ? (float)(sum / (double)Lk) : 0.f;
}

template <typename T, int D>
hipError_t launch_kmean_t(const KmeanArgs& a, bool varlen, dim3 grid, hipStream_t st) {
    if (varlen)
        hipLaunchKernelGGL((kmean_kernel<T, D, true>), grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((kmean_kernel<T, D, false>), grid, dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    const dim3 g2(grid.x, grid.y);
    if (varlen)
        hipLaunchKernelGGL((kmean_finish_kernel<D, true>), g2, dim3(D), 0, st, a);
    else
        hipLaunchKernelGGL((kmean_finish_kernel<D, false>), g2, dim3(D), 0, st, a);
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

// One work group per (batch, kv head) while its keys fit in 512 KB (a split costs a
// second launch, ~4 us); beyond that about two work groups per compute unit over
// the whole launch, each with at least 128 keys, at most kMaxKmeanSplits per
// (batch, kv head).
int kmean_splits(int64_t units, int64_t keys_per_unit, int D) {
    if (units <= 0) return 1;
    if (keys_per_unit * D * 2 <= (int64_t)512 * 1024) return 1;
    int64_t s = (512 + units - 1) / units;
    const int64_t by_len = keys_per_unit / 128 + (keys_per_unit % 128 != 0);
    if (s > by_len) s = by_len;
    if (s > kMaxKmeanSplits) s = kMaxKmeanSplits;
    return s < 1 ? 1 : (int)s;
}

hipError_t launch_kmean(const KmeanArgs& a, int dtype, int D, bool varlen, int grid_b,
                        hipStream_t stream) {
    const dim3 grid((unsigned)a.Hkv, (unsigned)grid_b, (unsigned)a.nsplit);
    if (dtype == 0) return launch_kmean_d<__bf16>(a, D, varlen, grid, stream);
    return launch_kmean_d<_Float16>(a, D, varlen, grid, stream);
}

}  // namespace skv
