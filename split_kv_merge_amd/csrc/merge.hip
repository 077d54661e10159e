// merge.hip -- stable merge of partial attention states (o_s, lse_s).
//
// Per row: M = max_s lse_s, w_s = 2^(lse_s - M), out = sum_s w_s o_s / sum_s w_s,
// lse = M + log2 sum_s w_s; a part with lse_s = -inf weighs 0 and an all -inf
// row yields (0, -inf).  This is the global-max rescale of ExecuTorch PR #22133
// "Prevent Voxtral NaNs in CUDA split-K attention" (Copilot overview), laid out
// as that PR's reviewer asked for (item 2): the work is spread over the head
// dimension and over part-groups, and the exponentials of a group of parts are
// independent of each other rather than one loop-carried chain.
//
// Layout: a part-group of D/VEC lanes covers one row's head dimension, each lane
// owning VEC contiguous elements (one 16-byte load per part); several part-groups
// share a row so that the parts of one row are read in parallel.  The max is kept
// as a running max (below), which gives the same result as taking it first.
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

// A row's parts are split over P part-groups of LPR = D/VEC lanes each; T = P * LPR
// lanes serve one row (a power of two, at most 256), 256 / T rows per block.
//   1. lane (pg, sub) runs an online merge over parts s = pg, pg + P, ... for its VEC
//      elements, four parts per memory round trip (their LSEs and outputs issued
//      together): it keeps a running max m of the LSEs it has seen, and when a group
//      raises it rescales its sums by 2^(m_old - m_new), so every weight
//      2^(lse_s - m) is at most 1 and no separate max pass (a second round trip) is
//      needed;
//   2. part-group 0 combines the P groups' (m_g, W_g, acc_g) through LDS, rescaling
//      each by 2^(m_g - M) with M the row max.
template <typename TP, typename TO, int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a, int P) {
    constexpr int VEC = PartLoad<TP>::VEC;
    constexpr int LPR = D / VEC;  // lanes per part-group
    constexpr int RS = VEC + 2;   // LDS record per lane: acc, W, m
    __shared__ __attribute__((aligned(16))) float red[256 * RS];

    const int tid = threadIdx.x;
    const int T = LPR * P;        // lanes per row
    const int rib = tid / T, t = tid % T, pg = t / LPR, sub = t % LPR;
    const int64_t row = (int64_t)blockIdx.x * (256 / T) + rib;
    const bool live = row < a.rows;

    // (r0, r1, r2) of this row; 32-bit division whenever the row count allows it (a
    // 64-bit division is a long software sequence, and every lane does three)
    int64_t r0 = 0, r1 = 0, r2 = 0;
    if (live) {
        if (a.rows <= 0xffffffffll) {
            const uint32_t rw = (uint32_t)row, R2 = (uint32_t)a.R2, R1 = (uint32_t)a.R1;
            const uint32_t q2 = rw / R2;
            r2 = rw - q2 * R2;
            r1 = q2 % R1;
            r0 = q2 / R1;
        } else {
            r2 = row % a.R2;
            r1 = (row / a.R2) % a.R1;
            r0 = row / ((int64_t)a.R1 * a.R2);
        }
    }
    const float* lp = a.parts_lse + r0 * a.pl_s0 + r1 * a.pl_s1 + r2 * a.pl_s2;
    const TP* op = (const TP*)a.parts_out + r0 * a.po_s0 + r1 * a.po_s1 + r2 * a.po_s2 + sub * VEC;

    // 1. online merge over this part-group's parts
    float M = -INFINITY, W = 0.f;
    float acc[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) acc[j] = 0.f;
    if (live) {
        const int S = a.num_parts;
        for (int s = pg; s < S; s += 4 * P) {
            float x[4][VEC], l[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int sp = min(s + u * P, S - 1);   // past the end: a real part, weight 0
                l[u] = lp[(int64_t)sp * a.pl_part];
                PartLoad<TP>::load(op + (int64_t)sp * a.po_part, x[u]);
            }
            float mg = -INFINITY;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (s + u * P >= S) l[u] = -INFINITY;
                mg = fmaxf(mg, l[u]);
            }
            const float Mn = fmaxf(M, mg);
            if (Mn == -INFINITY) continue;              // no part with a key so far
            const float sc = fast_exp2(M - Mn);         // 0 while M is still -inf
            W *= sc;
#pragma unroll
            for (int j = 0; j < VEC; ++j) acc[j] *= sc;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float w = fast_exp2(l[u] - Mn);   // -inf parts: 0
                W += w;
#pragma unroll
                for (int j = 0; j < VEC; ++j) acc[j] += w * x[u][j];
            }
            M = Mn;
        }
    }

    // 2. combine the part-groups
    if (P > 1) {
#pragma unroll
        for (int j = 0; j < VEC; ++j) red[tid * RS + j] = acc[j];
        red[tid * RS + VEC] = W;
        red[tid * RS + VEC + 1] = M;
        __syncthreads();
        if (pg != 0) return;
        float Mt = M;
        for (int g = 1; g < P; ++g) Mt = fmaxf(Mt, red[(tid + g * LPR) * RS + VEC + 1]);
        if (Mt != -INFINITY) {
            const float s0 = fast_exp2(M - Mt);
            W *= s0;
#pragma unroll
            for (int j = 0; j < VEC; ++j) acc[j] *= s0;
            for (int g = 1; g < P; ++g) {
                const float* o = &red[(tid + g * LPR) * RS];
                const float sg = fast_exp2(o[VEC + 1] - Mt);
                W += sg * o[VEC];
#pragma unroll
                for (int j = 0; j < VEC; ++j) acc[j] += sg * o[j];
            }
        }
        M = Mt;
    }
    if (!live) return;
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
    constexpr int LPR = D / VEC;
    // Part-groups spread one row's parts over more lanes only when there are too few
    // rows to fill the chip (fewer than ~4 x 256 CUs worth of 256-thread blocks with
    // one lane group per row); then a power of two up to one part per group.
    int P = 1;
    if (a.rows * LPR < (int64_t)4 * 256 * 256)
        while (P < a.num_parts && LPR * P * 2 <= 256) P *= 2;
    const int rows_per_block = 256 / (LPR * P);
    const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((merge_kernel<TP, TO, D>), dim3((unsigned)blocks), dim3(256), 0, st, a, P);
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
