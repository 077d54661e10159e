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
    // |scale| * log2(e); for a negative scale the kernel negates q (exactly) instead,
    // so that every logit is taken as (-q) . k * |scale|: the max over raw dot
    // products is then the max of the scaled logits for either sign of the scale
    float scale_log2;
    int negate_q;
};

// mean(k) over keys per (batch | sequence, kv head): float32 [B | nseq, Hkv, D].
// nsplit > 1 spreads each (batch, kv head) over nsplit work groups, whose fp64
// column sums go to partial [B | nseq, Hkv, nsplit, D] before a second kernel adds
// them; nsplit == 1 needs no partial buffer.
constexpr int kMaxKmeanSplits = 32;
struct KmeanArgs {
    const void* k;
    float* kbar;
    double* partial;
    const int32_t* cu_k;        // varlen only
    int Hkv, Sk, nsplit;
    int64_t kv_row, kv_head, kv_batch;
};
int kmean_splits(int64_t units, int64_t keys_per_unit, int D);  // nsplit for a launch

// Split-KV partial states.
struct SplitArgs {
    const void* q;
    const void* k;
    const void* v;
    float* out_part;            // float32; the single-launch decode keeps q's 16-bit type
    float* lse_part;
    int B, Hq, Hkv, Lq, Lkv, num_splits;
    // filled KV length per batch element (device, nullable: NULL = Lkv for all);
    // read in the kernel and clamped to [0, Lkv]
    const int32_t* kv_len;
    int64_t q_row, q_head, q_batch;
    int64_t kv_row, kv_head, kv_batch;
    int64_t part_stride;        // elements between consecutive splits of out_part
    // consecutive chunks one work group takes (1 for the partial states; the
    // single-launch decode may group chunks, gridDim.x = ceil(num_splits / group))
    int group;
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

// INT8 quantisation of q and of k - mean(k) (sage_quant.hip).  Strides in elements:
// index 0 is q's, index 1 is k's (and v's).
struct SageQuantArgs {
    const void* q;
    const void* k;
    const void* v;              // read only when v16 is set
    const float* kbar;          // [B, Hkv, D] or null (no smoothing)
    int8_t* q_codes;            // [B, Hq, Sq, D]
    float* q_scale;             // [B, Hq, ceil(Sq/32)]
    float* q_bias;              // [B, Hq, Sq] add-back in log2 units, or null
    int8_t* k_codes;            // [B, Hkv, Sk, D]
    float* k_scale;             // [B, Hkv, ceil(Sk/32)]
    uint16_t* v16;              // [B, Hkv, Sk, D] fp16 copy of v, or null
    int Hq, Hkv, Sq, Sk;
    int64_t q_items, k_items;   // 32-row blocks of q and of k
    int64_t x_row[2], x_head[2], x_batch[2];
    float scale_log2;
};

// INT8 QK^T attention (sage_fwd.hip) on the buffers above.
struct SageFwdArgs {
    const int8_t* q_codes;
    const float* q_scale;
    const float* q_bias;        // nullable
    const int8_t* k_codes;
    const float* k_scale;
    const uint16_t* v;          // fp16
    void* out;                  // q's dtype
    float* lse;                 // [B, Hq, Sq] or null
    int Hq, Hkv, Sq, Sk;
    int64_t v_row, v_head, v_batch;
    int64_t o_row, o_head, o_batch;
    float scale_log2;           // |scale| * log2(e); q's codes are negated when negate_q
    int negate_q;
};

int sage_rows_per_block();     // query rows of one INT8 attention work group
hipError_t launch_sage_quant(const SageQuantArgs& a, int dtype, int D, hipStream_t stream);
hipError_t launch_sage_fwd(const SageFwdArgs& a, int dtype, int D, bool causal, int grid_m,
                           int grid_b, hipStream_t stream);
int fmha_rows_per_block(int D);  // query rows one attention work group covers
hipError_t launch_fmha(const FmhaArgs& a, int dtype, int D, bool causal, bool varlen,
                       int grid_m, int grid_b, hipStream_t stream);
hipError_t launch_kmean(const KmeanArgs& a, int dtype, int D, bool varlen, int grid_b,
                        hipStream_t stream);
constexpr int kMaxDecodeSplits = 256;  // single-launch decode: its merge walks S / 16 round trips
// Single-launch decode: arrival counters for at most this many (batch, kv head) pairs,
// in a block of fixed size at the start of the workspace, so that one zero fill serves
// calls of any shape.
constexpr int kMaxDecodeUnits = 65536;
constexpr size_t kTicketBlockBytes = (size_t)kMaxDecodeUnits * sizeof(int);
hipError_t launch_splitkv(const SplitArgs& a, int dtype, int D, bool fused, hipStream_t stream);
// 17..64 query rows per kv head at D = 64, 128 (splitkv_wide.hip); grid (parts, Hkv, B)
hipError_t launch_splitkv_wide(const SplitArgs& a, int dtype, int D, bool fused, dim3 grid,
                               hipStream_t stream);
int splitkv_max_rows(int D);   // query rows per kv head, (Hq / Hkv) * Lq, the decode serves
// Device-resident scratch of the no-allocation decode (scratch.hip): counters then
// partial states, 16 MiB per device.  noalloc_scratch() returns this device's address
// of it (looked up once per device, counters zeroed on first use).
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
hipError_t noalloc_scratch(void** ptr, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, int parts_dtype, int out_dtype, int D,
                        hipStream_t stream);

}  // namespace skv
