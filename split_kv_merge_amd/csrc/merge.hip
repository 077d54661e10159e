// merge.hip -- stable merge of partial attention states (o_s, lse_s).
//
// Per row: M = max_s lse_s, w_s = 2^(lse_s - M), out = sum_s w_s o_s / sum_s w_s,
// lse = M + log2 sum_s w_s; a part with lse_s = -inf weighs 0 and an all -inf
// row yields (0, -inf).  This is the global-max rescale of ExecuTorch PR #22133
// "Prevent Voxtral NaNs in CUDA split-K attention" (Copilot overview), laid out
// as that PR's reviewer asked for (item 2): the max is a separate, parallel pass
// and the weighted sum is spread over the head dimension, so no exponential sits
// on a loop-carried chain.
//
// Layout: a row is handled by D/VEC lanes, each owning VEC contiguous elements
// (one 16-byte load per part); a wave covers 64/(D/VEC) rows and a work group 4
// waves.  The max pass strides the parts over the row's lanes and reduces with
// xor shuffles inside the row's lane group; every lane then walks all parts,
// reading each lse_s as a broadcast and accumulating w_s * o_s for its slice.
#include "device.h"
#include "launch.h"

namespace skv {

namespace {

template <typename TP> struct PartLoad;
template <> struct PartLoad<float> {
    static constexpr int VEC = 4;
    static __device__ __forceinline__ void load(const void* p, float* x) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(p);
        x[0] = v[0]; x[1] = v[1]; x[2] = v[2]; x[3] = v[3];
    }
};
template <> struct PartLoad<__bf16> {
    static constexpr int VEC = 8;
    static __device__ __forceinline__ void load(const void* p, float* x) {
        const u32x4 v = load16(p);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = Elem<__bf16>::to_float((uint16_t)(v[j] & 0xffff));
            x[2 * j + 1] = Elem<__bf16>::to_float((uint16_t)(v[j] >> 16));
        }
    }
};
template <> struct PartLoad<_Float16> {
    static constexpr int VEC = 8;
    static __device__ __forceinline__ void load(const void* p, float* x) {
        const u32x4 v = load16(p);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = Elem<_Float16>::to_float((uint16_t)(v[j] & 0xffff));
            x[2 * j + 1] = Elem<_Float16>::to_float((uint16_t)(v[j] >> 16));
        }
    }
};

template <typename TO, int VEC> struct OutStore;
template <int VEC> struct OutStore<float, VEC> {
    static __device__ __forceinline__ void store(void* p, const float* x) {
#pragma unroll
        for (int j = 0; j < VEC; j += 4)
            *reinterpret_cast<f32x4*>((float*)p + j) = f32x4{x[j], x[j + 1], x[j + 2], x[j + 3]};
    }
};
template <typename TO, int VEC> struct OutStore {
    static __device__ __forceinline__ void store(void* p, const float* x) {
        if constexpr (VEC == 8) {
            u32x4 w;
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = Elem<TO>::pack2(x[2 * j], x[2 * j + 1]);
            store16(p, w);
        } else {
            u32x2 w;
#pragma unroll
            for (int j = 0; j < 2; ++j) w[j] = Elem<TO>::pack2(x[2 * j], x[2 * j + 1]);
            *reinterpret_cast<u32x2*>(p) = w;
        }
    }
};

template <typename TP, typename TO, int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
    constexpr int VEC = PartLoad<TP>::VEC;
    constexpr int LPR = D / VEC;   // lanes per row
    constexpr int RPW = 64 / LPR;  // rows per wave
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % LPR;
    const int64_t row = ((int64_t)blockIdx.x * 4 + wave) * RPW + lane / LPR;
    if (row >= a.rows) return;  // whole lane groups leave together

    const int64_t r2 = row % a.R2, r1 = (row / a.R2) % a.R1, r0 = row / ((int64_t)a.R1 * a.R2);
    const float* lp = a.parts_lse + r0 * a.pl_s0 + r1 * a.pl_s1 + r2 * a.pl_s2;
    const TP* op = (const TP*)a.parts_out + r0 * a.po_s0 + r1 * a.po_s1 + r2 * a.po_s2 + sub * VEC;

    // pass 1: global max of the partial LSEs
    float M = -INFINITY;
    for (int s = sub; s < a.num_parts; s += LPR) M = fmaxf(M, lp[(int64_t)s * a.pl_part]);
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) M = fmaxf(M, xor_shfl(M, off));
    const float Mu = M == -INFINITY ? 0.f : M;

    // pass 2: weights and the weighted sum of this lane's slice
    float acc[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) acc[j] = 0.f;
    float W = 0.f;
    int s = 0;
    for (; s + 2 <= a.num_parts; s += 2) {
        const float w0 = fast_exp2(lp[(int64_t)s * a.pl_part] - Mu);
        const float w1 = fast_exp2(lp[(int64_t)(s + 1) * a.pl_part] - Mu);
        float x0[VEC], x1[VEC];
        PartLoad<TP>::load(op + (int64_t)s * a.po_part, x0);
        PartLoad<TP>::load(op + (int64_t)(s + 1) * a.po_part, x1);
        W += w0 + w1;
#pragma unroll
        for (int j = 0; j < VEC; ++j) acc[j] += w0 * x0[j] + w1 * x1[j];
    }
    if (s < a.num_parts) {
        const float w0 = fast_exp2(lp[(int64_t)s * a.pl_part] - Mu);
        float x0[VEC];
        PartLoad<TP>::load(op + (int64_t)s * a.po_part, x0);
        W += w0;
#pragma unroll
        for (int j = 0; j < VEC; ++j) acc[j] += w0 * x0[j];
    }
    const float inv = W > 0.f ? 1.f / W : 0.f;
#pragma unroll
    for (int j = 0; j < VEC; ++j) acc[j] *= inv;
    TO* dst = (TO*)a.out + r0 * a.o_s0 + r1 * a.o_s1 + r2 * a.o_s2 + sub * VEC;
    OutStore<TO, VEC>::store(dst, acc);
    if (sub == 0 && a.lse)
        a.lse[r0 * a.l_s0 + r1 * a.l_s1 + r2 * a.l_s2] = W > 0.f ? M + fast_log2(W) : -INFINITY;
}

template <typename TP, typename TO, int D>
hipError_t launch_merge_t(const MergeArgs& a, hipStream_t st) {
    constexpr int VEC = PartLoad<TP>::VEC;
    constexpr int RPB = 4 * (64 / (D / VEC));  // rows per block
    const int64_t blocks = (a.rows + RPB - 1) / RPB;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((merge_kernel<TP, TO, D>), dim3((unsigned)blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <typename TP, typename TO>
hipError_t launch_merge_d(const MergeArgs& a, int D, hipStream_t st) {
    switch (D) {
        case 64: return launch_merge_t<TP, TO, 64>(a, st);
        case 128: return launch_merge_t<TP, TO, 128>(a, st);
        case 256: return launch_merge_t<TP, TO, 256>(a, st);
        default: return hipErrorInvalidValue;
    }
}

template <typename TP>
hipError_t launch_merge_o(const MergeArgs& a, int out_dtype, int D, hipStream_t st) {
    switch (out_dtype) {
        case 0: return launch_merge_d<TP, __bf16>(a, D, st);
        case 1: return launch_merge_d<TP, _Float16>(a, D, st);
        case 2: return launch_merge_d<TP, float>(a, D, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int parts_dtype, int out_dtype, int D,
                        hipStream_t stream) {
    switch (parts_dtype) {
        case 0: return launch_merge_o<__bf16>(a, out_dtype, D, stream);
        case 1: return launch_merge_o<_Float16>(a, out_dtype, D, stream);
        case 2: return launch_merge_o<float>(a, out_dtype, D, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace skv
