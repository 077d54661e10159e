/*
 * skv.h -- C ABI of the split-KV attention library for MI355X (gfx950).
 *
 * Attention forward that returns its output plus one log-sum-exp per query row,
 * the split-KV decode step that produces per-chunk partial (out, LSE) states, and
 * the stable merge of such states.
 *
 * Sources (page title, then section):
 *   [ARK]  auto-round issue #2556, "ARK return_lse gives the same LSE for every 16
 *          query rows (sdpa, sagev1, sageattn) on XPU" -- task statement, Problem
 *          Description, Reproduction Steps.
 *   [SGL]  SGLang PR #33840, "[XPU] Support softmax_lse in sgl_kernel::fwd API" --
 *          Modifications, review thread.
 *   [ET]   ExecuTorch PR #22133, "Prevent Voxtral NaNs in CUDA split-K attention" --
 *          description, Copilot overview, reviewer comments 1-3.
 *   [ASC]  SGLang error record "Unexpected Ascend TND softmax LSE shape".
 *
 * Conventions shared by every call
 *   - LSE means log2( sum_j exp(scale * q_i . k_j) ) over the keys row i sees, on the
 *     original unsmoothed logits, one value per query row [ARK task statement and
 *     Problem Description].  It is float32.  A row that sees no key gets LSE = -inf
 *     and an all-zero output row.
 *   - Outputs are written in place into caller memory; a call returns only a status
 *     and an optional LSE pointer may be NULL, meaning "not wanted" [SGL
 *     Modifications; review thread on has_value()].
 *   - All tensor pointers are DEVICE pointers (k and v may be NULL when there is no
 *     key to read), contiguous in the named layout, with
 *     the head dimension D innermost; q/k/v/out must be 16-byte aligned, LSE
 *     buffers 4-byte aligned.  The caller owns every buffer; the library keeps no
 *     state (apart from the fixed device scratch of skv_attn_splitkv_decode_noalloc),
 *     allocates nothing and never synchronises: each call only enqueues
 *     kernels on `stream` (a hipStream_t; NULL = the default stream), so calls can
 *     be captured into a HIP graph.
 *   - Shapes are checked before anything is launched or written [SGL review:
 *     check before reshaping; ASC record: shape guard]; a rejected call returns
 *     SKV_EINVAL (malformed) or SKV_EUNSUPPORTED (valid but not built, e.g.
 *     D = 96) and touches no memory.  A launch failure returns SKV_ELAUNCH.
 *     skv_last_error() then describes the reason.  No C++ exception crosses the ABI.
 *   - GQA: Hq must be a multiple of Hkv; q head h reads kv head h / (Hq / Hkv).
 *   - Supported: D in {64, 128, 256} (the INT8 calls: 64, 128); q/k/v in bf16 or
 *     fp16.
 *   - Layouts: SKV_HND = [B, H, S, D], SKV_NHD = [B, S, H, D] [ARK Problem
 *     Description: both tensor_layout values].
 */
#ifndef SKV_H_
#define SKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SKV_OK = 0,
    SKV_EINVAL = 1,        /* malformed arguments: nothing launched, nothing written */
    SKV_EUNSUPPORTED = 2,  /* well-formed but outside what is built (D, dtype, rows) */
    SKV_ELAUNCH = 3        /* the HIP runtime refused a launch */
} skv_status_t;

typedef enum { SKV_BF16 = 0, SKV_FP16 = 1, SKV_FP32 = 2 } skv_dtype_t;
typedef enum { SKV_HND = 0, SKV_NHD = 1 } skv_layout_t;

/*
 * Dense attention forward with an optional per-row LSE.
 *
 *   q   [B, Hq, Sq, D] (HND) or [B, Sq, Hq, D] (NHD), dtype
 *   k,v [B, Hkv, Sk, D] or [B, Sk, Hkv, D], dtype
 *   out same shape and layout as q, dtype (round to nearest even)
 *   lse float32 [B, Hq, Sq] or NULL
 *
 * out_i = sum_j softmax_j(scale * q_i . k_j) v_j.  causal != 0 masks keys with
 * j > i + Sk - Sq (bottom-right aligned; j <= i when Sq == Sk).
 *
 * smooth_k != 0 computes the logits against k - mean(k), the mean taken over this
 * call's Sk keys per (batch, kv head), and adds scale * q_i . mean(k) back into
 * the LSE, so the LSE still refers to the unsmoothed logits [ARK Problem
 * Description, second issue; Reproduction Steps part 3].  The output is
 * unchanged by smoothing.  It needs a workspace of skv_workspace_bytes(B, Hkv, D, 1)
 * bytes (device memory, 16-byte aligned, no initialisation required; it holds
 * mean(k) and its partial sums, so calls that may run at the same time need separate
 * workspaces); without smoothing `workspace` may be NULL.
 *
 * Sizes: B, Sq, Sk >= 0 (zero-sized problems return SKV_OK without launching,
 * except Sk == 0 with Sq > 0, which writes zero outputs and -inf LSEs).  Grid
 * limits: B <= 65535 and at most 65535 row tiles (Sq <= 65535 * 256 at D <= 128,
 * 65535 * 128 at D = 256); SKV_EUNSUPPORTED beyond.
 */
skv_status_t skv_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                          int B, int Hq, int Hkv, int Sq, int Sk, int D, skv_dtype_t dtype,
                          skv_layout_t layout, float scale, int causal, int smooth_k,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Packed variable-length attention forward [SGL review thread; ASC record].
 *
 *   q, out [total_q, Hq, D] and k, v [total_k, Hkv, D], dtype, token-major packed.
 *   cu_seqlens_q, cu_seqlens_k: DEVICE int32 [nseq + 1], non-decreasing, starting
 *     at 0 and ending at total_q / total_k; sequence b owns query tokens
 *     [cu_q[b], cu_q[b+1]) and key tokens [cu_k[b], cu_k[b+1]).  Their contents are
 *     not validated on the host (that would need a synchronisation); malformed
 *     values are undefined behaviour.
 *   max_seqlen_q: an upper bound on every query length (sizes the grid).
 *   lse: float32 [Hq, total_q] (2-D: head-major, token index as in q) or NULL.
 *
 * causal and smooth_k act per sequence as in skv_attn_fwd (mean(k) per sequence
 * and kv head; workspace of skv_workspace_bytes(nseq, Hkv, D, 1) bytes).  Grid
 * limits as in skv_attn_fwd, with nseq for B and max_seqlen_q for Sq.
 */
skv_status_t skv_attn_fwd_varlen(const void* q, const void* k, const void* v, void* out,
                                 float* lse, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_k, int nseq, int total_q,
                                 int total_k, int max_seqlen_q, int Hq, int Hkv, int D,
                                 skv_dtype_t dtype, float scale, int causal, int smooth_k,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Split-KV decode step: per-chunk partial attention states [ET description and
 * Copilot overview: per-split online softmax with its own running max].
 *
 *   q   [B, Hq, Lq, D] (HND) or [B, Lq, Hq, D] (NHD), dtype; every query row sees
 *       every key (no causal mask).
 *   k,v [B, Hkv, Lkv, D] or [B, Lkv, Hkv, D], dtype
 *   out_part float32 [num_splits, <q's shape>]: chunk s's output normalised by its
 *       own softmax sum.
 *   lse_part float32 [num_splits, B, Hq, Lq]: chunk s's LSE (log2).
 *
 *   kv_len DEVICE int32 [B] or NULL: the filled length of each batch element's KV
 *       cache [ET docstring diff: only the filled positions are swept, O(context)
 *       instead of O(max_seq_len), read on the device and graph-safe; NULL sweeps
 *       the full Lkv].  Keys at or past kv_len[b] are never read (they may hold
 *       anything, NaN included).  Values are read in the kernel, not validated on
 *       the host; each is clamped to [0, Lkv].
 *
 * With N_b = Lkv (or the clamped kv_len[b]), chunk s of batch element b covers keys
 * [s*C_b, min((s+1)*C_b, N_b)) with C_b = ceil(N_b / num_splits): the chunks split
 * the filled length evenly.  Every slot of both buffers is written, including
 * chunks that hold no key, which get (0, -inf) [ET reviewer item 3: no early exit
 * for empty splits], so neither buffer needs initialising.  Merge the states with
 * skv_merge_state.
 * Limits: Lq >= 1, Lkv >= 0, num_splits >= 1; query rows per kv head
 * (Hq / Hkv) * Lq <= 64 at D <= 128 and <= 16 at D = 256 (SKV_EUNSUPPORTED beyond).
 * Every K/V byte of a chunk is read once for all of that kv head's query rows [ET
 * reviewer item 1: the small-query range, Lq 2 to 4 with grouped heads].
 */
skv_status_t skv_attn_splitkv_partial(const void* q, const void* k, const void* v,
                                      float* out_part, float* lse_part, int B, int Hq,
                                      int Hkv, int Lq, int Lkv, int D, skv_dtype_t dtype,
                                      skv_layout_t layout, float scale, int num_splits,
                                      const int32_t* kv_len, void* stream);

/*
 * Split-KV decode in one launch: the partial states of skv_attn_splitkv_partial
 * followed by their stable merge (as skv_merge_state computes it), done by the
 * last work group of each (batch, kv head) to finish [ET description: stable
 * per-split softmax and global-max rescale; reviewer item 2: keep the reduce off
 * a separate serial path].
 *
 *   q, k, v, layout, num_splits, kv_len: as skv_attn_splitkv_partial; num_splits <= 256
 *       and num_splits*B*Hq*Lq*D*4 < 2^31 bytes of partial states (SKV_EUNSUPPORTED
 *       beyond).
 *   out  q's shape, layout and dtype: the merged output.
 *   lse  float32 [B, Hq, Lq] (log2) or NULL.
 *   workspace: device memory of skv_splitkv_workspace_bytes(B, Hq, Lq, D,
 *       num_splits, Hkv) bytes, 256-byte aligned: a fixed block of arrival counters
 *       at its start (one per (batch, kv head), room for 65536, the same bytes for
 *       every shape), then the partial states (chunk outputs in q's 16-bit type --
 *       each is normalised by its own sum, so it lies in the range of V -- and
 *       float32 chunk LSEs).  It must be ZERO-FILLED before its first use; every call
 *       returns its counters to zero, so one zero fill serves any number of later
 *       calls of any shape that fits (including HIP graph replays).  Two calls that
 *       may run at the same time must not share a workspace.  B*Hkv > 65536:
 *       SKV_EUNSUPPORTED.
 */
skv_status_t skv_attn_splitkv_decode(const void* q, const void* k, const void* v, void* out,
                                     float* lse, int B, int Hq, int Hkv, int Lq, int Lkv, int D,
                                     skv_dtype_t dtype, skv_layout_t layout, float scale,
                                     int num_splits, const int32_t* kv_len, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Workspace bytes of skv_attn_splitkv_decode (0 for non-positive sizes). */
size_t skv_splitkv_workspace_bytes(int B, int Hq, int Lq, int D, int num_splits, int Hkv);

/*
 * The single-launch decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It computes exactly what skv_attn_splitkv_decode computes (the same kernels),
 * but keeps its arrival counters and partial states in a fixed device scratch that
 * the library holds, instead of a caller workspace; the caller still passes q, k,
 * v, out and lse.  The call allocates nothing and calls no allocating routine.
 *
 *   Arguments, limits and results: as skv_attn_splitkv_decode without the workspace.
 *   Scratch: skv_splitkv_decode_noalloc_max_bytes() bytes (16 MiB) per device,
 *       taken on the first call on a device and held until the process ends.  A call
 *       whose skv_splitkv_workspace_bytes(B, Hq, Lq, D, num_splits, Hkv) exceeds it
 *       returns SKV_EUNSUPPORTED before any launch (a decode of 8 x 32 query rows at
 *       D = 128 fits with up to 128 splits).
 *   The first call on a device also enqueues one small kernel that zeroes the
 *       counters; every call leaves them at zero again.
 *   Concurrency: all calls on one device share that device's scratch, so calls that
 *       may overlap on one GPU (other streams, other threads) race and give wrong
 *       results; serialise them, or use skv_attn_splitkv_decode with one workspace
 *       per concurrent call.
 */
skv_status_t skv_attn_splitkv_decode_noalloc(const void* q, const void* k, const void* v,
                                             void* out, float* lse, int B, int Hq, int Hkv, int Lq,
                                             int Lkv, int D, skv_dtype_t dtype,
                                             skv_layout_t layout, float scale, int num_splits,
                                             const int32_t* kv_len, void* stream);

/* Bytes of the device scratch of skv_attn_splitkv_decode_noalloc (its size limit). */
size_t skv_splitkv_decode_noalloc_max_bytes(void);

/*
 * Stable merge of num_parts partial states (o_s, lse_s) per row [ET Copilot
 * overview: global max over splits, rescale each split, reduce all together;
 * reviewer item 2: keep the exponentials off a serial chain, parallelise over D].
 *
 * For each row:  M = max_s lse_s;  w_s = 2^(lse_s - M);
 *                out = sum_s w_s o_s / sum_s w_s;  lse = M + log2(sum_s w_s).
 * Parts with lse_s = -inf get weight 0; if all are -inf the row gets out = 0 and
 * lse = -inf.
 *
 * Rows are addressed by a 3-D index (r0, r1, r2) in [R0) x [R1) x [R2); strides are
 * in ELEMENTS of the pointed-to type, D is contiguous.  Element d of part s of row
 * (r0, r1, r2) is parts_out[s * part_stride + r0 * strides[0] + r1 * strides[1] +
 * r2 * strides[2] + d]; likewise for parts_lse, out and lse.  One call thus serves
 * HND, NHD and the varlen [Hq, total_q] LSE.
 *
 *   parts_out  dtype parts_dtype (SKV_FP32, SKV_BF16 or SKV_FP16)
 *   parts_lse  float32
 *   out        dtype out_dtype (SKV_FP32, SKV_BF16 or SKV_FP16)
 *   lse        float32, or NULL
 * Vector access requires parts_out / out 16-byte aligned and their row strides and
 * part stride multiples of 16 bytes.  num_parts >= 1; D in {64, 128, 256}.
 */
skv_status_t skv_merge_state(int num_parts, int R0, int R1, int R2, int D,
                             const void* parts_out, skv_dtype_t parts_dtype,
                             int64_t parts_out_part_stride, const int64_t parts_out_strides[3],
                             const float* parts_lse, int64_t parts_lse_part_stride,
                             const int64_t parts_lse_strides[3],
                             void* out, skv_dtype_t out_dtype, const int64_t out_strides[3],
                             float* lse, const int64_t lse_strides[3], void* stream);

/* Workspace bytes skv_attn_fwd / skv_attn_fwd_varlen need when smooth_k != 0 (else
 * 0): the float32 mean(k) buffer [B_or_nseq, Hkv, D] padded to 256 bytes, then, when
 * U = B_or_nseq * Hkv < 512, the fp64 column sums of the S = min(32, ceil(512 / U))
 * key ranges each (batch | sequence, kv head) is split into: U * S * D * 8 bytes. */
size_t skv_workspace_bytes(int B_or_nseq, int Hkv, int D, int smooth_k);

/* A split count for the split-KV calls: about one (batch, kv head, chunk) work
 * group per compute unit (256 CUs), with chunks of at least 256 keys (D and
 * rows_per_kv_head do not change it at present).  Pure host arithmetic; returns >= 1. */
int skv_pick_num_splits(int B, int Hkv, int rows_per_kv_head, int Lkv, int D);

/*
 * INT8 QK^T attention with smoothing [ARK task statement and Reproduction Steps,
 * the apis table: ark.sagev1 and ark.sageattn(kernel="v1_pvhalf"); Problem
 * Description, second issue: smooth_k on by default, the LSE must still be that of
 * the unsmoothed logits].  The pages name these variants without spelling out the
 * quantisation; this library reads it as follows (one fixed scheme):
 *
 *   mean(k)  per (batch, kv head) over the call's Sk keys: the exact mean rounded
 *            once to float32 (accumulated in fp64); zero without smoothing.
 *   blocks   32 consecutive rows (query rows of q, or keys of k - mean(k) taken in
 *            float32) per (batch, head), all D columns; the last block may be short.
 *   codes    for a block with a = max |x|:  delta = a / 127 and
 *            code = rint(x * (127 / a)) (0 when a = 0), each a correctly rounded
 *            float32 operation, round half to even, codes in [-127, 127].
 *
 * Quantisation only.  Outputs (device memory, written in full, any alignment the
 * element type needs):
 *   q_codes  int8 [B, Hq, Sq, D] and k_codes int8 [B, Hkv, Sk, D], HND order
 *            whatever the input layout;
 *   q_scale  float32 [B, Hq, ceil(Sq/32)] and k_scale float32 [B, Hkv, ceil(Sk/32)]
 *            (the deltas);
 *   kbar     float32 [B, Hkv, D]: mean(k); required when smooth_k != 0, ignored
 *            (may be NULL) otherwise.
 * q, k: as skv_attn_fwd (bf16 or fp16, HND or NHD, 16-byte aligned).  D in {64, 128}.
 */
skv_status_t skv_sage_quant(const void* q, const void* k, int B, int Hq, int Hkv, int Sq,
                            int Sk, int D, skv_dtype_t dtype, skv_layout_t layout, int smooth_k,
                            int8_t* q_codes, float* q_scale, int8_t* k_codes, float* k_scale,
                            float* kbar, void* stream);

/*
 * Attention forward on the INT8 logits of skv_sage_quant's scheme, with P.V in
 * half precision (P and V rounded to fp16, float32 accumulation) [ARK apis table:
 * kernel "v1_pvhalf"]:
 *     t_ij = scale * dQ(i) * dK(j) * (q^_i . k^_j)    (exact integer dot product)
 *     out_i = sum_j softmax_j(t_ij) v_j
 *     lse_i = log2 sum_j exp(t_ij) + scale * q_i . mean(k) / ln 2
 * so with smooth_k the LSE refers to the unsmoothed logits [ARK Reproduction Steps
 * part 3]; it approximates skv_attn_fwd's LSE to the quantisation error.
 *
 * Arguments as skv_attn_fwd (q, k, v, out, lse, sizes, dtype, layout, scale,
 * causal, smooth_k), with D in {64, 128}.  The workspace (device memory, 256-byte
 * aligned, no initialisation required) holds the codes, scales, mean(k), the per-row
 * add-back and, for bf16 inputs, an fp16 copy of V: skv_sage_workspace_bytes(...)
 * bytes.  V values outside the fp16 range overflow to +-inf in that copy.  Grid
 * limits as skv_attn_fwd (256 query rows per row tile).
 */
skv_status_t skv_sage_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                          int B, int Hq, int Hkv, int Sq, int Sk, int D, skv_dtype_t dtype,
                          skv_layout_t layout, float scale, int causal, int smooth_k,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of skv_sage_fwd (0 for empty problems). */
size_t skv_sage_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D,
                                skv_dtype_t dtype, int smooth_k);

/* Static description of a status code. */
const char* skv_status_str(skv_status_t status);

/* Description of the last error returned on the calling thread ("" if none). */
const char* skv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SKV_H_ */
