// api.cpp -- the C ABI of include/skv.h: argument validation, stride set-up and
// kernel dispatch.  Every check runs before the first launch, so a rejected call
// neither launches nor writes (SGLang PR #33840 review: check before reshaping;
// SGLang's "Unexpected Ascend TND softmax LSE shape" record: guard shapes).
#include "skv.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "launch.h"

namespace {

thread_local char g_err[512] = "";

skv_status_t fail(skv_status_t st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

void clear_err() { g_err[0] = '\0'; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool is16(int dt) { return dt == SKV_BF16 || dt == SKV_FP16; }
bool valid_dtype(int dt) { return dt == SKV_BF16 || dt == SKV_FP16 || dt == SKV_FP32; }
int dtype_bytes(int dt) { return dt == SKV_FP32 ? 4 : 2; }
bool valid_layout(int l) { return l == SKV_HND || l == SKV_NHD; }
bool supported_D(int D) { return D == 64 || D == 128 || D == 256; }

// product of non-negative factors without int64 overflow
bool mul_ok(int64_t& acc, int64_t f) {
    if (f < 0) return false;
    if (f != 0 && acc > INT64_MAX / f) return false;
    acc *= f;
    return true;
}
bool elems_ok(std::initializer_list<int64_t> dims) {
    int64_t acc = 1;
    for (int64_t d : dims)
        if (!mul_ok(acc, d)) return false;
    return true;
}

skv_status_t launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(SKV_ELAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
    return SKV_OK;
}

// Checks shared by the attention entry points.  Returns SKV_OK or the error.
skv_status_t check_heads_dims(int Hq, int Hkv, int D, int dtype) {
    if (Hq <= 0 || Hkv <= 0) return fail(SKV_EINVAL, "head counts must be positive (Hq=%d, Hkv=%d)", Hq, Hkv);
    if (Hq % Hkv != 0)
        return fail(SKV_EINVAL, "Hq (%d) must be a multiple of Hkv (%d) for grouped-query attention", Hq, Hkv);
    if (Hq > 65535) return fail(SKV_EUNSUPPORTED, "Hq=%d exceeds the 65535 grid limit", Hq);
    if (D <= 0) return fail(SKV_EINVAL, "head dimension D must be positive (D=%d)", D);
    if (!supported_D(D)) return fail(SKV_EUNSUPPORTED, "head dimension D=%d is not built (64, 128, 256)", D);
    if (!valid_dtype(dtype)) return fail(SKV_EINVAL, "unknown dtype code %d", dtype);
    if (!is16(dtype)) return fail(SKV_EUNSUPPORTED, "q/k/v must be bf16 or fp16");
    return SKV_OK;
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// mean(k) buffer: float32 [units, D], padded to 256 bytes.
size_t kbar_bytes(size_t units, int D) { return round256(units * (size_t)D * sizeof(float)); }

// fp64 split sums of the mean(k) kernel for the largest split count it may pick
// for this many (batch | sequence, kv head) units (none when it keeps one split).
size_t kmean_partial_bytes(size_t units, int D) {
    const int s = skv::kmean_splits((int64_t)units, INT64_MAX / 1024, D);
    return s > 1 ? units * (size_t)s * (size_t)D * sizeof(double) : 0;
}

// Launch the mean(k) kernels into kbar, with split sums in `partial` (which must
// hold kmean_partial_bytes) or, when partial is null, one split per unit.
skv_status_t run_kmean_into(const void* k, float* kbar, double* partial, const int32_t* cu_k,
                            int units_b, int Hkv, int Sk, int64_t keys_per_unit, int D, int dtype,
                            int64_t kv_row, int64_t kv_head, int64_t kv_batch, hipStream_t s) {
    skv::KmeanArgs km{};
    km.k = k; km.kbar = kbar; km.partial = partial; km.cu_k = cu_k;
    km.Hkv = Hkv; km.Sk = Sk;
    km.nsplit = partial ? skv::kmean_splits((int64_t)units_b * Hkv, keys_per_unit, D) : 1;
    km.kv_row = kv_row; km.kv_head = kv_head; km.kv_batch = kv_batch;
    return launched(skv::launch_kmean(km, dtype, D, cu_k != nullptr, units_b, s), "kmean");
}

}  // namespace

extern "C" {

const char* skv_status_str(skv_status_t status) {
    switch (status) {
        case SKV_OK: return "ok";
        case SKV_EINVAL: return "invalid argument";
        case SKV_EUNSUPPORTED: return "unsupported configuration";
        case SKV_ELAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

const char* skv_last_error(void) { return g_err; }

size_t skv_workspace_bytes(int B_or_nseq, int Hkv, int D, int smooth_k) {
    if (!smooth_k || B_or_nseq <= 0 || Hkv <= 0 || D <= 0) return 0;
    const size_t units = (size_t)B_or_nseq * (size_t)Hkv;
    return kbar_bytes(units, D) + kmean_partial_bytes(units, D);
}

int skv_pick_num_splits(int B, int Hkv, int rows_per_kv_head, int Lkv, int D) {
    (void)rows_per_kv_head;
    (void)D;
    if (B <= 0 || Hkv <= 0 || Lkv <= 0) return 1;
    // One work group per compute unit (256 CUs) streams best: a launch then needs a
    // single round of work groups (every round pays the latency chain of loading
    // Q, the first blocks, the combine and the partial-state publish), and each wave
    // keeps several blocks in flight; with streaming loads one wave per SIMD keeps
    // HBM busy even for long chunks.  Every chunk keeps at least 256 keys (two
    // 32-key blocks per wave).
    const int64_t units = (int64_t)B * Hkv;
    int64_t s = (256 + units - 1) / units;
    int64_t smax = Lkv / 256;
    if (smax < 1) smax = 1;
    if (s > smax) s = smax;
    if (s > 256) s = 256;
    if (s < 1) s = 1;
    return (int)s;
}

skv_status_t skv_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                          int B, int Hq, int Hkv, int Sq, int Sk, int D, skv_dtype_t dtype,
                          skv_layout_t layout, float scale, int causal, int smooth_k,
                          void* workspace, size_t workspace_bytes, void* stream) {
    clear_err();
    if (!q || !out) return fail(SKV_EINVAL, "q and out must be non-NULL");
    if ((!k || !v) && Sk > 0) return fail(SKV_EINVAL, "k and v must be non-NULL when Sk > 0");
    if (B < 0 || Sq < 0 || Sk < 0)
        return fail(SKV_EINVAL, "sizes must be non-negative (B=%d, Sq=%d, Sk=%d)", B, Sq, Sk);
    skv_status_t st = check_heads_dims(Hq, Hkv, D, dtype);
    if (st != SKV_OK) return st;
    if (!valid_layout(layout)) return fail(SKV_EINVAL, "unknown layout code %d", (int)layout);
    if (!std::isfinite(scale)) return fail(SKV_EINVAL, "scale must be finite");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
        return fail(SKV_EINVAL, "q, k, v and out must be 16-byte aligned");
    if (lse && !aligned(lse, 4)) return fail(SKV_EINVAL, "lse must be 4-byte aligned");
    if (B > 65535) return fail(SKV_EUNSUPPORTED, "B=%d exceeds the 65535 grid limit", B);
    if (!elems_ok({B, Hq, Sq, D}) || !elems_ok({B, Hkv, Sk, D}))
        return fail(SKV_EINVAL, "tensor sizes overflow 64-bit indexing");
    const size_t need = skv_workspace_bytes(B, Hkv, D, smooth_k);
    if (smooth_k && B > 0) {
        if (!workspace || !aligned(workspace, 16))
            return fail(SKV_EINVAL, "smooth_k needs a 16-byte aligned workspace");
        if (workspace_bytes < need)
            return fail(SKV_EINVAL, "workspace has %zu bytes, smooth_k needs %zu", workspace_bytes, need);
    }
    const int bm = skv::fmha_rows_per_block(D);
    const int grid_m = (int)(((int64_t)Sq + bm - 1) / bm);
    if (grid_m > 65535)
        return fail(SKV_EUNSUPPORTED, "Sq=%d needs %d row tiles, over the 65535 grid limit", Sq, grid_m);
    // (The kernels form K/V offsets inside a tile of at most 128 rows in 32 bits:
    // 127 * Hkv * D + D < 2^31 for every Hkv <= Hq <= 65535 and D <= 256.)
    if (B == 0 || Sq == 0) return SKV_OK;

    hipStream_t s = (hipStream_t)stream;
    const bool hnd = layout == SKV_HND;
    skv::FmhaArgs a{};
    a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse;
    a.Hq = Hq; a.Hkv = Hkv; a.Sq = Sq; a.Sk = Sk;
    a.q_row = hnd ? D : (int64_t)Hq * D;
    a.q_head = hnd ? (int64_t)Sq * D : D;
    a.q_batch = (int64_t)Hq * Sq * D;
    a.kv_row = hnd ? D : (int64_t)Hkv * D;
    a.kv_head = hnd ? (int64_t)Sk * D : D;
    a.kv_batch = (int64_t)Hkv * Sk * D;
    a.lse_head = Sq;
    a.lse_batch = (int64_t)Hq * Sq;
    a.scale_log2 = std::fabs(scale) * 1.4426950408889634f;
    a.negate_q = scale < 0.f;
    if (smooth_k) {
        char* ws = (char*)workspace;
        st = run_kmean_into(k, (float*)ws, (double*)(ws + kbar_bytes((size_t)B * Hkv, D)), nullptr,
                            B, Hkv, Sk, Sk, D, dtype, a.kv_row, a.kv_head, a.kv_batch, s);
        if (st != SKV_OK) return st;
        a.kbar = (const float*)workspace;
    }
    return launched(skv::launch_fmha(a, dtype, D, causal != 0, false, grid_m, B, s), "fmha_fwd");
}

skv_status_t skv_attn_fwd_varlen(const void* q, const void* k, const void* v, void* out,
                                 float* lse, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_k, int nseq, int total_q,
                                 int total_k, int max_seqlen_q, int Hq, int Hkv, int D,
                                 skv_dtype_t dtype, float scale, int causal, int smooth_k,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    clear_err();
    if (!q || !out) return fail(SKV_EINVAL, "q and out must be non-NULL");
    if ((!k || !v) && total_k > 0) return fail(SKV_EINVAL, "k and v must be non-NULL when total_k > 0");
    if (nseq < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0)
        return fail(SKV_EINVAL, "sizes must be non-negative (nseq=%d, total_q=%d, total_k=%d, max_seqlen_q=%d)",
                    nseq, total_q, total_k, max_seqlen_q);
    if (nseq > 0 && (!cu_seqlens_q || !cu_seqlens_k))
        return fail(SKV_EINVAL, "cu_seqlens_q and cu_seqlens_k must be non-NULL");
    if (max_seqlen_q > total_q)
        return fail(SKV_EINVAL, "max_seqlen_q (%d) exceeds total_q (%d)", max_seqlen_q, total_q);
    skv_status_t st = check_heads_dims(Hq, Hkv, D, dtype);
    if (st != SKV_OK) return st;
    if (!std::isfinite(scale)) return fail(SKV_EINVAL, "scale must be finite");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
        return fail(SKV_EINVAL, "q, k, v and out must be 16-byte aligned");
    if (lse && !aligned(lse, 4)) return fail(SKV_EINVAL, "lse must be 4-byte aligned");
    if ((cu_seqlens_q && !aligned(cu_seqlens_q, 4)) || (cu_seqlens_k && !aligned(cu_seqlens_k, 4)))
        return fail(SKV_EINVAL, "cu_seqlens must be 4-byte aligned");
    if (nseq > 65535) return fail(SKV_EUNSUPPORTED, "nseq=%d exceeds the 65535 grid limit", nseq);
    if (!elems_ok({total_q, Hq, D}) || !elems_ok({total_k, Hkv, D}))
        return fail(SKV_EINVAL, "tensor sizes overflow 64-bit indexing");
    const size_t need = skv_workspace_bytes(nseq, Hkv, D, smooth_k);
    if (smooth_k && nseq > 0) {
        if (!workspace || !aligned(workspace, 16))
            return fail(SKV_EINVAL, "smooth_k needs a 16-byte aligned workspace");
        if (workspace_bytes < need)
            return fail(SKV_EINVAL, "workspace has %zu bytes, smooth_k needs %zu", workspace_bytes, need);
    }
    const int bm = skv::fmha_rows_per_block(D);
    const int grid_m = (max_seqlen_q + bm - 1) / bm;
    if (grid_m > 65535)
        return fail(SKV_EUNSUPPORTED, "max_seqlen_q=%d needs %d row tiles, over the 65535 grid limit",
                    max_seqlen_q, grid_m);
    if (nseq == 0 || total_q == 0 || max_seqlen_q == 0) return SKV_OK;

    hipStream_t s = (hipStream_t)stream;
    skv::FmhaArgs a{};
    a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse;
    a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k;
    a.Hq = Hq; a.Hkv = Hkv;
    a.q_row = (int64_t)Hq * D; a.q_head = D; a.q_batch = 0;
    a.kv_row = (int64_t)Hkv * D; a.kv_head = D; a.kv_batch = 0;
    a.lse_head = total_q; a.lse_batch = 0;
    a.scale_log2 = std::fabs(scale) * 1.4426950408889634f;
    a.negate_q = scale < 0.f;
    if (smooth_k) {
        char* ws = (char*)workspace;
        st = run_kmean_into(k, (float*)ws, (double*)(ws + kbar_bytes((size_t)nseq * Hkv, D)),
                            cu_seqlens_k, nseq, Hkv, 0, total_k / nseq, D, dtype, a.kv_row,
                            a.kv_head, 0, s);
        if (st != SKV_OK) return st;
        a.kbar = (const float*)workspace;
    }
    return launched(skv::launch_fmha(a, dtype, D, causal != 0, true, grid_m, nseq, s), "fmha_fwd_varlen");
}

}  // extern "C"

namespace {

// Validation and argument block shared by the two split-KV entry points.
skv_status_t prepare_split(const void* q, const void* k, const void* v, int B, int Hq, int Hkv,
                           int Lq, int Lkv, int D, skv_dtype_t dtype, skv_layout_t layout,
                           float scale, int num_splits, const int32_t* kv_len,
                           skv::SplitArgs& a) {
    if (!q) return fail(SKV_EINVAL, "q must be non-NULL");
    if ((!k || !v) && Lkv > 0) return fail(SKV_EINVAL, "k and v must be non-NULL when Lkv > 0");
    if (B < 0 || Lq < 1 || Lkv < 0)
        return fail(SKV_EINVAL, "need B >= 0, Lq >= 1, Lkv >= 0 (B=%d, Lq=%d, Lkv=%d)", B, Lq, Lkv);
    if (num_splits < 1) return fail(SKV_EINVAL, "num_splits must be >= 1 (got %d)", num_splits);
    skv_status_t st = check_heads_dims(Hq, Hkv, D, dtype);
    if (st != SKV_OK) return st;
    if (!valid_layout(layout)) return fail(SKV_EINVAL, "unknown layout code %d", (int)layout);
    if (!std::isfinite(scale)) return fail(SKV_EINVAL, "scale must be finite");
    if ((int64_t)(Hq / Hkv) * Lq > skv::splitkv_max_rows(D))
        return fail(SKV_EUNSUPPORTED, "(Hq/Hkv)*Lq = %lld query rows per kv head exceeds %d at D = %d",
                    (long long)(Hq / Hkv) * Lq, skv::splitkv_max_rows(D), D);
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
        return fail(SKV_EINVAL, "q, k and v must be 16-byte aligned");
    if (kv_len && !aligned(kv_len, 4)) return fail(SKV_EINVAL, "kv_len must be 4-byte aligned");
    if (B > 65535 || Hkv > 65535) return fail(SKV_EUNSUPPORTED, "B or Hkv exceeds the 65535 grid limit");
    if (!elems_ok({num_splits, B, Hq, Lq, D}) || !elems_ok({B, Hkv, Lkv, D}))
        return fail(SKV_EINVAL, "tensor sizes overflow 64-bit indexing");
    const bool hnd = layout == SKV_HND;
    a = skv::SplitArgs{};
    a.q = q; a.k = k; a.v = v;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Lq = Lq; a.Lkv = Lkv; a.num_splits = num_splits;
    a.kv_len = kv_len;
    a.q_row = hnd ? D : (int64_t)Hq * D;
    a.q_head = hnd ? (int64_t)Lq * D : D;
    a.q_batch = (int64_t)Hq * Lq * D;
    a.kv_row = hnd ? D : (int64_t)Hkv * D;
    a.kv_head = hnd ? (int64_t)Lkv * D : D;
    a.kv_batch = (int64_t)Hkv * Lkv * D;
    a.part_stride = (int64_t)B * Hq * Lq * D;
    a.group = 1;
    a.scale_log2 = scale * 1.4426950408889634f;
    return SKV_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

skv_status_t skv_attn_splitkv_partial(const void* q, const void* k, const void* v,
                                      float* out_part, float* lse_part, int B, int Hq,
                                      int Hkv, int Lq, int Lkv, int D, skv_dtype_t dtype,
                                      skv_layout_t layout, float scale, int num_splits,
                                      const int32_t* kv_len, void* stream) {
    clear_err();
    if (!out_part || !lse_part) return fail(SKV_EINVAL, "out_part and lse_part must be non-NULL");
    skv::SplitArgs a;
    skv_status_t st = prepare_split(q, k, v, B, Hq, Hkv, Lq, Lkv, D, dtype, layout, scale,
                                    num_splits, kv_len, a);
    if (st != SKV_OK) return st;
    if (!aligned(out_part, 16)) return fail(SKV_EINVAL, "out_part must be 16-byte aligned");
    if (!aligned(lse_part, 4)) return fail(SKV_EINVAL, "lse_part must be 4-byte aligned");
    if (B == 0) return SKV_OK;
    a.out_part = out_part;
    a.lse_part = lse_part;
    return launched(skv::launch_splitkv(a, dtype, D, false, (hipStream_t)stream), "splitkv_partial");
}

size_t skv_splitkv_workspace_bytes(int B, int Hq, int Lq, int D, int num_splits, int Hkv) {
    if (B <= 0 || Hq <= 0 || Lq <= 0 || D <= 0 || num_splits <= 0 || Hkv <= 0) return 0;
    const size_t rows = (size_t)num_splits * B * Hq * Lq;
    // the counter block (fixed size, first), chunk outputs, chunk LSEs
    return skv::kTicketBlockBytes + align256(rows * D * sizeof(uint16_t)) +
           align256(rows * sizeof(float));
}

}  // extern "C"

namespace {

// Checks of the single-launch decode that do not depend on where its partial states
// live; on success `a` holds the launch arguments without the state pointers.
skv_status_t prepare_decode(const void* q, const void* k, const void* v, void* out, float* lse,
                            int B, int Hq, int Hkv, int Lq, int Lkv, int D, skv_dtype_t dtype,
                            skv_layout_t layout, float scale, int num_splits,
                            const int32_t* kv_len, skv::SplitArgs& a) {
    if (!out) return fail(SKV_EINVAL, "out must be non-NULL");
    skv_status_t st = prepare_split(q, k, v, B, Hq, Hkv, Lq, Lkv, D, dtype, layout, scale,
                                    num_splits, kv_len, a);
    if (st != SKV_OK) return st;
    if (!aligned(out, 16)) return fail(SKV_EINVAL, "out must be 16-byte aligned");
    if (lse && !aligned(lse, 4)) return fail(SKV_EINVAL, "lse must be 4-byte aligned");
    if (num_splits > skv::kMaxDecodeSplits)
        return fail(SKV_EUNSUPPORTED, "the single-launch decode takes at most %d splits (got %d)",
                    skv::kMaxDecodeSplits, num_splits);
    if ((int64_t)B * Hkv > skv::kMaxDecodeUnits)
        return fail(SKV_EUNSUPPORTED, "B*Hkv = %lld exceeds the %d arrival counters of the decode workspace",
                    (long long)B * Hkv, skv::kMaxDecodeUnits);
    const size_t rows = (size_t)num_splits * B * Hq * Lq;
    if (rows * D * sizeof(float) >= ((size_t)1 << 31))
        return fail(SKV_EUNSUPPORTED, "partial states exceed 2 GiB for the single-launch decode");
    a.out = out;
    a.lse = lse;
    return SKV_OK;
}

// Launch the single-launch decode with its counters and partial states in `ws`
// (the layout skv_splitkv_workspace_bytes describes).
skv_status_t launch_decode(skv::SplitArgs& a, int D, skv_dtype_t dtype, void* ws_ptr,
                           hipStream_t stream) {
    // one ticket per (batch, kv head) in the fixed counter block, then the chunk
    // outputs in q's 16-bit type and the float32 chunk LSEs
    const size_t rows = (size_t)a.num_splits * a.B * a.Hq * a.Lq;
    char* ws = (char*)ws_ptr;
    const size_t po_bytes = align256(rows * D * sizeof(uint16_t));
    a.ticket = (int*)ws;
    a.out_part = (float*)(ws + skv::kTicketBlockBytes);
    a.lse_part = (float*)(ws + skv::kTicketBlockBytes + po_bytes);
    // A work group takes `group` consecutive chunks, so that a launch keeps about the
    // work-group count the split heuristic targets whatever num_splits is: its online
    // softmax over those chunks' keys gives the merge of their partial states.
    const int target = skv_pick_num_splits(a.B, a.Hkv, (a.Hq / a.Hkv) * a.Lq, a.Lkv, D);
    a.group = a.num_splits / target > 1 ? a.num_splits / target : 1;
    return launched(skv::launch_splitkv(a, dtype, D, true, stream), "splitkv_decode");
}

}  // namespace

extern "C" {

skv_status_t skv_attn_splitkv_decode(const void* q, const void* k, const void* v, void* out,
                                     float* lse, int B, int Hq, int Hkv, int Lq, int Lkv, int D,
                                     skv_dtype_t dtype, skv_layout_t layout, float scale,
                                     int num_splits, const int32_t* kv_len, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    clear_err();
    skv::SplitArgs a;
    skv_status_t st = prepare_decode(q, k, v, out, lse, B, Hq, Hkv, Lq, Lkv, D, dtype, layout,
                                     scale, num_splits, kv_len, a);
    if (st != SKV_OK) return st;
    const size_t need = skv_splitkv_workspace_bytes(B, Hq, Lq, D, num_splits, Hkv);
    if (B > 0 && (!workspace || !aligned(workspace, 256)))
        return fail(SKV_EINVAL, "the decode workspace must be non-NULL and 256-byte aligned");
    if (workspace_bytes < need)
        return fail(SKV_EINVAL, "workspace has %zu bytes, the decode needs %zu", workspace_bytes, need);
    if (B == 0) return SKV_OK;
    return launch_decode(a, D, dtype, workspace, (hipStream_t)stream);
}

size_t skv_splitkv_decode_noalloc_max_bytes(void) { return skv::kNoAllocScratchBytes; }

skv_status_t skv_attn_splitkv_decode_noalloc(const void* q, const void* k, const void* v,
                                             void* out, float* lse, int B, int Hq, int Hkv, int Lq,
                                             int Lkv, int D, skv_dtype_t dtype,
                                             skv_layout_t layout, float scale, int num_splits,
                                             const int32_t* kv_len, void* stream) {
    clear_err();
    skv::SplitArgs a;
    skv_status_t st = prepare_decode(q, k, v, out, lse, B, Hq, Hkv, Lq, Lkv, D, dtype, layout,
                                     scale, num_splits, kv_len, a);
    if (st != SKV_OK) return st;
    const size_t need = skv_splitkv_workspace_bytes(B, Hq, Lq, D, num_splits, Hkv);
    if (need > skv::kNoAllocScratchBytes)
        return fail(SKV_EUNSUPPORTED,
                    "the no-allocation decode needs %zu bytes of partial states and counters, over "
                    "its fixed %zu-byte device scratch (use skv_attn_splitkv_decode with a workspace)",
                    need, skv::kNoAllocScratchBytes);
    if (B == 0) return SKV_OK;
    hipStream_t s = (hipStream_t)stream;
    void* ws = nullptr;
    hipError_t e = skv::noalloc_scratch(&ws, s);
    if (e != hipSuccess)
        return fail(SKV_ELAUNCH, "device scratch set-up failed: %s", hipGetErrorString(e));
    return launch_decode(a, D, dtype, ws, s);
}

skv_status_t skv_merge_state(int num_parts, int R0, int R1, int R2, int D,
                             const void* parts_out, skv_dtype_t parts_dtype,
                             int64_t parts_out_part_stride, const int64_t parts_out_strides[3],
                             const float* parts_lse, int64_t parts_lse_part_stride,
                             const int64_t parts_lse_strides[3],
                             void* out, skv_dtype_t out_dtype, const int64_t out_strides[3],
                             float* lse, const int64_t lse_strides[3], void* stream) {
    clear_err();
    if (!parts_out || !parts_lse || !out)
        return fail(SKV_EINVAL, "parts_out, parts_lse and out must be non-NULL");
    if (!parts_out_strides || !parts_lse_strides || !out_strides || (lse && !lse_strides))
        return fail(SKV_EINVAL, "stride arrays must be non-NULL");
    if (num_parts < 1) return fail(SKV_EINVAL, "num_parts must be >= 1 (got %d)", num_parts);
    if (R0 < 0 || R1 < 0 || R2 < 0) return fail(SKV_EINVAL, "row extents must be non-negative");
    if (D <= 0) return fail(SKV_EINVAL, "D must be positive (D=%d)", D);
    if (!supported_D(D)) return fail(SKV_EUNSUPPORTED, "D=%d is not built (64, 128, 256)", D);
    if (!valid_dtype(parts_dtype) || !valid_dtype(out_dtype))
        return fail(SKV_EINVAL, "unknown dtype code (parts %d, out %d)", (int)parts_dtype, (int)out_dtype);
    const int pb = dtype_bytes(parts_dtype), ob = dtype_bytes(out_dtype);
    if (!aligned(parts_out, 16) || !aligned(out, 16))
        return fail(SKV_EINVAL, "parts_out and out must be 16-byte aligned");
    if (!aligned(parts_lse, 4) || (lse && !aligned(lse, 4)))
        return fail(SKV_EINVAL, "LSE buffers must be 4-byte aligned");
    if ((parts_out_part_stride * pb) % 16 != 0)
        return fail(SKV_EINVAL, "parts_out part stride must be a multiple of 16 bytes");
    for (int i = 0; i < 3; ++i) {
        if ((parts_out_strides[i] * pb) % 16 != 0 || (out_strides[i] * ob) % 16 != 0)
            return fail(SKV_EINVAL, "row strides of parts_out and out must be multiples of 16 bytes");
    }
    int64_t rows = 1;
    if (!mul_ok(rows, R0) || !mul_ok(rows, R1) || !mul_ok(rows, R2))
        return fail(SKV_EINVAL, "row count overflows");
    if (rows == 0) return SKV_OK;
    if (rows > (int64_t)1 << 40) return fail(SKV_EUNSUPPORTED, "too many rows (%lld)", (long long)rows);

    skv::MergeArgs a{};
    a.parts_out = parts_out; a.parts_lse = parts_lse; a.out = out; a.lse = lse;
    a.num_parts = num_parts; a.R1 = R1; a.R2 = R2; a.rows = rows;
    a.po_part = parts_out_part_stride;
    a.po_s0 = parts_out_strides[0]; a.po_s1 = parts_out_strides[1]; a.po_s2 = parts_out_strides[2];
    a.pl_part = parts_lse_part_stride;
    a.pl_s0 = parts_lse_strides[0]; a.pl_s1 = parts_lse_strides[1]; a.pl_s2 = parts_lse_strides[2];
    a.o_s0 = out_strides[0]; a.o_s1 = out_strides[1]; a.o_s2 = out_strides[2];
    if (lse) { a.l_s0 = lse_strides[0]; a.l_s1 = lse_strides[1]; a.l_s2 = lse_strides[2]; }
    return launched(skv::launch_merge(a, parts_dtype, out_dtype, D, (hipStream_t)stream), "merge_state");
}

}  // extern "C"

// ------------------------------------------------------- INT8 QK^T (skv_sage_*)

namespace {

// Byte offsets of the INT8 path's buffers inside one workspace, each 256-byte
// aligned: mean(k), q codes, q scales, q add-back, k codes, k scales, fp16 V.
struct SageLayout {
    size_t kbar, part, qc, qs, qb, kc, ks, v16, total;
};

SageLayout sage_layout(int B, int Hq, int Hkv, int Sq, int Sk, int D, int dtype, int smooth) {
    SageLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += round256(bytes);
        return o;
    };
    const size_t nq = ((size_t)Sq + 31) / 32, nk = ((size_t)Sk + 31) / 32;
    L.kbar = take(smooth ? (size_t)B * Hkv * D * 4 : 0);
    L.part = take(smooth ? kmean_partial_bytes((size_t)B * Hkv, D) : 0);
    L.qc = take((size_t)B * Hq * Sq * D);
    L.qs = take((size_t)B * Hq * nq * 4);
    L.qb = take(smooth ? (size_t)B * Hq * Sq * 4 : 0);
    L.kc = take((size_t)B * Hkv * Sk * D);
    L.ks = take((size_t)B * Hkv * nk * 4);
    L.v16 = take(dtype == SKV_BF16 ? (size_t)B * Hkv * Sk * D * 2 : 0);
    L.total = off;
    return L;
}

// Checks shared by skv_sage_quant and skv_sage_fwd.
skv_status_t check_sage(const void* q, const void* k, int B, int Hq, int Hkv, int Sq, int Sk,
                        int D, int dtype, int layout) {
    if (!q) return fail(SKV_EINVAL, "q must be non-NULL");
    if (!k && Sk > 0) return fail(SKV_EINVAL, "k must be non-NULL when Sk > 0");
    if (B < 0 || Sq < 0 || Sk < 0)
        return fail(SKV_EINVAL, "sizes must be non-negative (B=%d, Sq=%d, Sk=%d)", B, Sq, Sk);
    skv_status_t st = check_heads_dims(Hq, Hkv, D, dtype);
    if (st != SKV_OK) return st;
    if (D != 64 && D != 128)
        return fail(SKV_EUNSUPPORTED, "the INT8 path is built for D = 64 and 128 (D=%d)", D);
    if (!valid_layout(layout)) return fail(SKV_EINVAL, "unknown layout code %d", layout);
    if (!aligned(q, 16) || !aligned(k, 16)) return fail(SKV_EINVAL, "q and k must be 16-byte aligned");
    if (B > 65535) return fail(SKV_EUNSUPPORTED, "B=%d exceeds the 65535 grid limit", B);
    if (!elems_ok({B, Hq, Sq, D}) || !elems_ok({B, Hkv, Sk, D}))
        return fail(SKV_EINVAL, "tensor sizes overflow 64-bit indexing");
    const int64_t items = (int64_t)B * Hq * ((Sq + 31) / 32) + (int64_t)B * Hkv * ((Sk + 31) / 32);
    if ((items + 3) / 4 > INT32_MAX)
        return fail(SKV_EUNSUPPORTED, "%lld quantisation blocks exceed the grid limit", (long long)items);
    return SKV_OK;
}

// Quantisation launch arguments for q / k in `layout`.
skv::SageQuantArgs quant_args(const void* q, const void* k, int B, int Hq, int Hkv, int Sq,
                              int Sk, int D, int layout) {
    const bool hnd = layout == SKV_HND;
    skv::SageQuantArgs a{};
    a.q = q; a.k = k;
    a.Hq = Hq; a.Hkv = Hkv; a.Sq = Sq; a.Sk = Sk;
    a.q_items = (int64_t)B * Hq * ((Sq + 31) / 32);
    a.k_items = (int64_t)B * Hkv * ((Sk + 31) / 32);
    a.x_row[0] = hnd ? D : (int64_t)Hq * D;
    a.x_head[0] = hnd ? (int64_t)Sq * D : D;
    a.x_batch[0] = (int64_t)Hq * Sq * D;
    a.x_row[1] = hnd ? D : (int64_t)Hkv * D;
    a.x_head[1] = hnd ? (int64_t)Sk * D : D;
    a.x_batch[1] = (int64_t)Hkv * Sk * D;
    return a;
}

skv_status_t run_kmean(const void* k, float* kbar, double* partial, int B, int Hkv, int Sk, int D,
                       int dtype, const skv::SageQuantArgs& qa, hipStream_t s) {
    return run_kmean_into(k, kbar, partial, nullptr, B, Hkv, Sk, Sk, D, dtype, qa.x_row[1],
                          qa.x_head[1], qa.x_batch[1], s);
}

}  // namespace

extern "C" {

size_t skv_sage_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D,
                                skv_dtype_t dtype, int smooth_k) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Sk < 0 || D <= 0) return 0;
    return sage_layout(B, Hq, Hkv, Sq, Sk, D, dtype, smooth_k != 0).total;
}

skv_status_t skv_sage_quant(const void* q, const void* k, int B, int Hq, int Hkv, int Sq,
                            int Sk, int D, skv_dtype_t dtype, skv_layout_t layout, int smooth_k,
                            int8_t* q_codes, float* q_scale, int8_t* k_codes, float* k_scale,
                            float* kbar, void* stream) {
    clear_err();
    skv_status_t st = check_sage(q, k, B, Hq, Hkv, Sq, Sk, D, dtype, layout);
    if (st != SKV_OK) return st;
    if (!q_codes || !q_scale || (Sk > 0 && (!k_codes || !k_scale)))
        return fail(SKV_EINVAL, "q_codes, q_scale, k_codes and k_scale must be non-NULL");
    if (smooth_k && !kbar) return fail(SKV_EINVAL, "smooth_k needs the kbar output");
    if (!aligned(q_codes, 16) || !aligned(k_codes, 16) || !aligned(q_scale, 4) ||
        !aligned(k_scale, 4) || (kbar && !aligned(kbar, 4)))
        return fail(SKV_EINVAL, "code buffers must be 16-byte and scale buffers 4-byte aligned");
    if (B == 0 || (Sq == 0 && Sk == 0)) return SKV_OK;
    hipStream_t s = (hipStream_t)stream;
    skv::SageQuantArgs a = quant_args(q, k, B, Hq, Hkv, Sq, Sk, D, layout);
    a.q_codes = q_codes; a.q_scale = q_scale; a.k_codes = k_codes; a.k_scale = k_scale;
    if (smooth_k) {
        st = run_kmean(k, kbar, nullptr, B, Hkv, Sk, D, dtype, a, s);
        if (st != SKV_OK) return st;
        a.kbar = kbar;
    }
    return launched(skv::launch_sage_quant(a, dtype, D, s), "sage_quant");
}

skv_status_t skv_sage_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                          int B, int Hq, int Hkv, int Sq, int Sk, int D, skv_dtype_t dtype,
                          skv_layout_t layout, float scale, int causal, int smooth_k,
                          void* workspace, size_t workspace_bytes, void* stream) {
    clear_err();
    skv_status_t st = check_sage(q, k, B, Hq, Hkv, Sq, Sk, D, dtype, layout);
    if (st != SKV_OK) return st;
    if (!out) return fail(SKV_EINVAL, "out must be non-NULL");
    if (!v && Sk > 0) return fail(SKV_EINVAL, "v must be non-NULL when Sk > 0");
    if (!aligned(v, 16) || !aligned(out, 16)) return fail(SKV_EINVAL, "v and out must be 16-byte aligned");
    if (lse && !aligned(lse, 4)) return fail(SKV_EINVAL, "lse must be 4-byte aligned");
    if (!std::isfinite(scale)) return fail(SKV_EINVAL, "scale must be finite");
    const int grid_m = (int)(((int64_t)Sq + skv::sage_rows_per_block() - 1) / skv::sage_rows_per_block());
    if (grid_m > 65535)
        return fail(SKV_EUNSUPPORTED, "Sq=%d needs %d row tiles, over the 65535 grid limit", Sq, grid_m);
    if (B == 0 || Sq == 0) return SKV_OK;
    const SageLayout L = sage_layout(B, Hq, Hkv, Sq, Sk, D, dtype, smooth_k != 0);
    if (!workspace || !aligned(workspace, 256))
        return fail(SKV_EINVAL, "the INT8 path needs a 256-byte aligned workspace");
    if (workspace_bytes < L.total)
        return fail(SKV_EINVAL, "workspace has %zu bytes, the INT8 path needs %zu", workspace_bytes, L.total);

    hipStream_t s = (hipStream_t)stream;
    char* ws = (char*)workspace;
    const float scale_log2 = scale * 1.4426950408889634f;
    skv::SageQuantArgs a = quant_args(q, k, B, Hq, Hkv, Sq, Sk, D, layout);
    a.v = v;
    a.q_codes = (int8_t*)(ws + L.qc);
    a.q_scale = (float*)(ws + L.qs);
    a.k_codes = (int8_t*)(ws + L.kc);
    a.k_scale = (float*)(ws + L.ks);
    a.scale_log2 = scale_log2;
    if (dtype == SKV_BF16) a.v16 = (uint16_t*)(ws + L.v16);
    if (smooth_k) {
        st = run_kmean(k, (float*)(ws + L.kbar), (double*)(ws + L.part), B, Hkv, Sk, D, dtype, a, s);
        if (st != SKV_OK) return st;
        a.kbar = (const float*)(ws + L.kbar);
        a.q_bias = (float*)(ws + L.qb);
    }
    st = launched(skv::launch_sage_quant(a, dtype, D, s), "sage_quant");
    if (st != SKV_OK) return st;

    const bool hnd = layout == SKV_HND;
    skv::SageFwdArgs f{};
    f.q_codes = a.q_codes; f.q_scale = a.q_scale; f.q_bias = a.q_bias;
    f.k_codes = a.k_codes; f.k_scale = a.k_scale;
    if (a.v16) {
        f.v = a.v16;
        f.v_row = D; f.v_head = (int64_t)Sk * D; f.v_batch = (int64_t)Hkv * Sk * D;
    } else {
        f.v = (const uint16_t*)v;
        f.v_row = a.x_row[1]; f.v_head = a.x_head[1]; f.v_batch = a.x_batch[1];
    }
    f.out = out; f.lse = lse;
    f.Hq = Hq; f.Hkv = Hkv; f.Sq = Sq; f.Sk = Sk;
    f.o_row = a.x_row[0]; f.o_head = a.x_head[0]; f.o_batch = a.x_batch[0];
    f.scale_log2 = std::fabs(scale_log2);
    f.negate_q = scale < 0.f;
    return launched(skv::launch_sage_fwd(f, dtype, D, causal != 0, grid_m, B, s), "sage_fwd");
}

}  // extern "C"
