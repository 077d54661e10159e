// splitkv_tail.h -- device pieces both split-KV decode kernels share: the stores that
// publish a work group's partial state, and the merge the last work group of a
// (batch, kv head) runs in the single-launch decode.
#pragma once

#include "device.h"
#include "launch.h"

namespace skv {
namespace dec {

// Cache-policy bits of a buffer load: device-coherent (sc1), nontemporal (nt).
constexpr int kCoherentLoad = 0x10;
constexpr int kNontemporalLoad = 0x2;   // nt: a streaming read

// Device-scope (agent) relaxed atomic stores write through the XCD's L2, so data
// one work group publishes this way reaches memory without the whole-L2 write-back
// a device-scope release fence would issue (once per work group).
__device__ __forceinline__ void store_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Why the last work group sees every partial state, step by step against LLVM's
// AMDGPU memory-model mapping for gfx942/gfx950 (what the compiler emits, checked in
// the assembly of these kernels):
//  1. Partial outputs and LSEs are stored with store_agent: agent-scope relaxed
//     atomic stores, emitted as global_store ... sc1, which write through the XCD's L2
//     to the device coherence point.
//  2. s_waitcnt vmcnt(0), then a work-group barrier: every such store of the work
//     group has completed.  This is the release half of the agent-scope release
//     mapping (buffer_wbl2 sc1; s_waitcnt vmcnt(0)) without the L2 write-back, which
//     only concerns stores that are not already written through.
//  3. One thread takes a ticket with an agent-scope relaxed fetch-add (emitted as
//     global_atomic_add ... sc0, sc0 = return the old value).  The fetch-adds on one
//     ticket are totally ordered, so the work group that draws P - 1 comes after
//     step 2 of every other work group of its (batch, kv head).
//  4. That work group reads the partials with sc1 buffer loads.  The agent-scope
//     acquire mapping's buffer_inv sc1 exists to make later plain loads miss stale
//     L2 lines; sc1 loads miss them by themselves.
// In the source-level (C++/HSA) model a relaxed store followed by a relaxed RMW is no
// release sequence: correctness rests on this instruction-level mapping.  A target
// that maps agent scope to other cache-policy bits needs a release fence before the
// ticket and an acquire fence after it instead (with a device-scope release fence per
// work group, which writes back the whole L2, the same decode took 128 us, not 38 us).
//
// Single-launch decode: once a work group has written its partial state (with
// store_agent) it waits for those stores to complete and takes a ticket for its
// (batch, kv head); the last of the gridDim.x work groups to arrive merges all
// partial states of those rows, writes the output and its LSE, and returns the
// ticket counter to zero for the next call.
//
// The partial outputs of this path are published in the input's 16-bit type (each
// is normalised by its own sum, so it lies in the range of V and the 16-bit type
// holds it; the merge adds them in fp32), half the bytes the merging work group has
// to pull in.  The merge keeps memory latency off serial chains: each thread owns Q
// 4-column groups of one row and reads the partial LSEs and outputs of GS parts per
// round trip (all issued together).  The TPR threads of a row take its groups
// round-robin (thread t: groups t, t + TPR, ...), so each load instruction reads
// TPR * 8 contiguous bytes of every row it touches: whole cache lines, each requested
// once, instead of a quarter of every line of the row.  Across groups of GS it keeps a
// running max M of the part LSEs and rescales its sums by 2^(M_old - M_new) when M
// grows; the result is the stable merge -- out = sum_s 2^(lse_s - M) o_s /
// sum_s 2^(lse_s - M), lse = M + log2 of that sum -- with no exponent above 0.
// Parts with lse = -inf get weight 0; if every part is -inf the row gets (0, -inf).
template <typename T, int D, int NR, int GS>
__device__ __forceinline__ void merge_rows(const SplitArgs& a, int b, int hk, int R, int G,
                                           int P);

template <typename T, int D, int NR>
__device__ __forceinline__ void merge_tail(const SplitArgs& a, int b, int hk, int R, int G) {
    __shared__ int is_last;
    const int tid = threadIdx.x, P = (int)gridDim.x;
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this thread's stores are done
    __syncthreads();                      // ... and every thread's
    int* ticket = a.ticket + (int64_t)b * a.Hkv + hk;
    if (tid == 0)
        is_last = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  P - 1;
    __syncthreads();
    if (!is_last) return;
    if (tid == 0) __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // parts per round trip: the smallest of 4, 8, 16 that covers P, with at most 64
    // loads of 8 bytes per thread in flight
    constexpr int Q = NR * D / 64;
    constexpr int GMAX = 64 / Q < 16 ? 64 / Q : 16;
    if constexpr (GMAX <= 4) {
        merge_rows<T, D, NR, 4>(a, b, hk, R, G, P);
    } else if constexpr (GMAX <= 8) {
        if (P <= 4)
            merge_rows<T, D, NR, 4>(a, b, hk, R, G, P);
        else
            merge_rows<T, D, NR, 8>(a, b, hk, R, G, P);
    } else {
        if (P <= 4)
            merge_rows<T, D, NR, 4>(a, b, hk, R, G, P);
        else if (P <= 8)
            merge_rows<T, D, NR, 8>(a, b, hk, R, G, P);
        else
            merge_rows<T, D, NR, 16>(a, b, hk, R, G, P);
    }
}

template <typename T, int D, int NR, int GS>
__device__ __forceinline__ void merge_rows(const SplitArgs& a, int b, int hk, int R, int G,
                                           int P) {
    using E = Elem<T>;
    constexpr int Q = NR * D / 64;     // 4-column groups per thread: 16 NR rows x D/4 / 256
    constexpr int TPR = 16 / NR;       // threads per row
    static_assert(TPR * Q * 4 == D, "the threads of a row cover its D columns");
    const int tid = threadIdx.x;
    const int r = tid / TPR;           // the row this thread merges
    if (r >= R) return;
    const int t = tid % TPR;           // its groups: t + TPR q, columns 4 (t + TPR q) + [0, 4)
    const int d0 = 4 * t;
    constexpr int DQ = 4 * TPR;        // column step from one of its groups to the next
    // The partials are read with device-coherent (sc1) buffer loads, which miss any
    // stale line this XCD's L2 may hold, so no cache-wide invalidate is needed.
    // Byte offsets stay below 2^31 (checked on the host).
    const __amdgpu_buffer_rsrc_t po_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(a.out_part, (short)0, 0x7fffffff, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t pl_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(a.lse_part, (short)0, 0x7fffffff, kBufferRsrcWord3);
    const int h = hk * G + r / a.Lq, i = r % a.Lq;
    const int64_t row_off = (int64_t)b * a.q_batch + (int64_t)h * a.q_head + (int64_t)i * a.q_row;
    const int64_t lse_row = ((int64_t)b * a.Hq + h) * a.Lq + i;
    const int64_t lse_split = (int64_t)a.B * a.Hq * a.Lq;

    float M = -INFINITY, W = 0.f;
    f32x4 acc[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < P; s0 += GS) {
        float l[GS];
        u32x2 x[GS][Q];
#pragma unroll
        for (int u = 0; u < GS; ++u) {
            const int sp = min(s0 + u, P - 1);   // past P: a real part, weighted 0 below
            l[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                pl_rsrc, (int)((sp * lse_split + lse_row) * 4), 0, kCoherentLoad));
#pragma unroll
            for (int q = 0; q < Q; ++q)
                x[u][q] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                    po_rsrc, (int)((row_off + d0 + DQ * q + sp * a.part_stride) * 2), 0,
                    kCoherentLoad));
        }
        float mg = -INFINITY;
#pragma unroll
        for (int u = 0; u < GS; ++u) {
            if (s0 + u >= P) l[u] = -INFINITY;
            mg = fmaxf(mg, l[u]);
        }
        const float Mn = fmaxf(M, mg);
        if (Mn == -INFINITY) continue;              // no part with a key so far
        const float sc = fast_exp2(M - Mn);         // 0 while M is still -inf
        W *= sc;
#pragma unroll
        for (int q = 0; q < Q; ++q) acc[q] *= sc;
#pragma unroll
        for (int u = 0; u < GS; ++u) {
            const float w = fast_exp2(l[u] - Mn);   // -inf parts: 0
            W += w;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const f32x4 xv = {E::to_float((uint16_t)(x[u][q].x & 0xffff)),
                                  E::to_float((uint16_t)(x[u][q].x >> 16)),
                                  E::to_float((uint16_t)(x[u][q].y & 0xffff)),
                                  E::to_float((uint16_t)(x[u][q].y >> 16))};
                acc[q] += xv * w;
            }
        }
        M = Mn;
    }
    const float inv = W > 0.f ? 1.f / W : 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        u32x2 packed;
        packed.x = E::pack2(acc[q][0] * inv, acc[q][1] * inv);
        packed.y = E::pack2(acc[q][2] * inv, acc[q][3] * inv);
        *reinterpret_cast<u32x2*>((uint16_t*)a.out + row_off + d0 + DQ * q) = packed;
    }
    if (t == 0 && a.lse) a.lse[lse_row] = W > 0.f ? M + fast_log2(W) : -INFINITY;
}

}  // namespace dec
}  // namespace skv
