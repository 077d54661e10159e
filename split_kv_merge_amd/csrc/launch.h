// launch.h -- host-side argument blocks and launchers of the HIP kernels.  Only
// api.cpp calls these, after validating every argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skv {

// Attention forward (dense or packed varlen).  Strides are in elements.
struct FmhaArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;                 // nullable
    const int32_t* cu_q;        // varlen only (device)
    const int32_t* cu_k;
    const float* kbar;          // [B | nseq, Hkv, D] float32 when smoothing, else null
    int Hq, Hkv;
    int Sq, Sk;                 // dense only
    int64_t q_row, q_head, q_batch;     // q and out share strides
    int64_t kv_row, kv_head, kv_batch;  // k and v share strides
    int64_t lse_head, lse_batch;        // lse row stride is 1
    float scale_log2;           // scale * log2(e)
};

// mean(k) over keys per (batch | sequence, kv head): float32 [B | nseq, Hkv, D]
struct KmeanArgs {
    const void* k;
    float* kbar;
    const int32_t* cu_k;        // varlen only
    int Hkv, Sk;
    int64_t kv_row, kv_head, kv_batch;
};

// Split-KV partial states.
struct SplitArgs {
    const void* q;
    const void* k;
    const void* v;
    float* out_part;
    float* lse_part;
    int B, Hq, Hkv, Lq, Lkv, num_splits;
    // filled KV length per batch element (device, nullable: NULL = Lkv for all);
    // read in the kernel and clamped to [0, Lkv]
    const int32_t* kv_len;
    int64_t q_row, q_head, q_batch;
    int64_t kv_row, kv_head, kv_batch;
    int64_t part_stride;        // elements between consecutive splits of out_part
    float scale_log2;
    // single-launch decode only: merged output (q's dtype and strides), its LSE
    // [B, Hq, Lq] (nullable) and one arrival ticket per (batch, kv head)
    void* out;
    float* lse;
    int* ticket;
};

// Merge of partial states over rows (r0, r1, r2).
struct MergeArgs {
    const void* parts_out;
    const float* parts_lse;
    void* out;
    float* lse;                 // nullable
    int num_parts, R1, R2;
    int64_t rows;               // R0 * R1 * R2
    int64_t po_part, po_s0, po_s1, po_s2;
    int64_t pl_part, pl_s0, pl_s1, pl_s2;
    int64_t o_s0, o_s1, o_s2;
    int64_t l_s0, l_s1, l_s2;
};

int fmha_rows_per_block(int D);  // query rows one attention work group covers
hipError_t launch_fmha(const FmhaArgs& a, int dtype, int D, bool causal, bool varlen,
                       int grid_m, int grid_b, hipStream_t stream);
hipError_t launch_kmean(const KmeanArgs& a, int dtype, int D, bool varlen, int grid_b,
                        hipStream_t stream);
constexpr int kMaxDecodeSplits = 256;  // single-launch decode: its merge walks S / 8 round trips
hipError_t launch_splitkv(const SplitArgs& a, int dtype, int D, bool fused, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, int parts_dtype, int out_dtype, int D,
                        hipStream_t stream);

}  // namespace skv
