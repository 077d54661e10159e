// splitkv.hip -- split-KV decode: per-chunk partial attention states.
//
// Each work group owns one (batch, kv head, chunk) and ALL query rows that read
// that kv head (G = Hq/Hkv heads x Lq rows: up to 64 at D <= 128 as one, two or four
// blocks of 16 rows on the MFMA N axis, up to 16 at D = 256), so every K/V byte of
// the chunk is read from HBM exactly once.
// Within the chunk, each wave keeps its own online-softmax state (running max in
// log2 units, running sum, unnormalised output) over an interleaved subset of 32-key
// blocks; the waves' states are then merged through LDS and the chunk's (out
// normalised by its own sum, log2 LSE) is written.  This is the stable per-split
// online softmax of ExecuTorch PR #22133 "Prevent Voxtral NaNs in CUDA split-K
// attention" (description and Copilot overview); a chunk with no key still writes
// (0, -inf), so the partial buffers need no initialisation (reviewer item 3 of that
// PR).
//
// Per 32-key block and wave: S^T = K Q^T on v_mfma_f32_16x16x32 tiles (keys on M,
// query rows on N), K fed straight from global memory in the operand layout
// (k-step kk takes head-dim elements [32kk, 32kk + 32) of 16 key rows, the four
// lanes of a row reading 64 contiguous bytes) and each K operand used by every
// 16-row block; O^T += V^T P^T with V staged in a per-wave LDS slice and read back
// with ds_read_b64_tr_b16 (each V^T operand also used by every row block), the key
// order of P matching the C layout of S^T.
#include "device.h"
#include "launch.h"

namespace skv {

namespace {

constexpr int kWaves = 4;
constexpr float kTau = 8.f;   // lazy-rescale threshold of the running max (log2 units)
// Keys per block: 32, or 16 where two 32-key blocks in flight per wave (K and V)
// would not fit in the register file beside the rest of the wave's state: at
// D = 256, and with more than 16 query rows (their Q operands and outputs).
template <int D, int NR> constexpr int keys_per_block() { return (D == 256 || NR > 1) ? 16 : 32; }

// Q operands live in registers for the whole key loop, except where they would not
// fit beside the outputs (more than 256 head-dim elements x 16-row blocks): there the
// work group stages its rows of Q once in LDS and each block re-reads its operands.
template <int D, int NR> constexpr bool q_in_lds() { return NR * D > 256; }

template <int D, int NR> struct SplitLds {
    static constexpr int VLD = D + 16;  // V pitch (elements) in the staging slice
    static constexpr int OLD = D + 4;   // pitch (floats) of the combine buffer
    static constexpr int QLD = D + 8;   // Q row pitch (elements) when Q is staged in LDS
    static constexpr int ROWS = 16 * NR;
    static constexpr int STAGE = kWaves * keys_per_block<D, NR>() * VLD * 2;
    static constexpr int QOFF = STAGE;  // byte offset of the staged Q rows
    static constexpr int QBYTES = q_in_lds<D, NR>() ? ROWS * QLD * 2 : 0;
    static constexpr int LOOP = STAGE + QBYTES;
    static constexpr int COMB = kWaves * (ROWS * OLD + 2 * ROWS) * 4;
    static constexpr int BYTES = LOOP > COMB ? LOOP : COMB;
};

// Buffer resource word 3 for raw (untyped) buffer access on gfx950, and the
// cache-policy bit that makes a buffer load device-coherent (sc1).
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kCoherentLoad = 0x10;

// Device-scope (agent) relaxed atomic stores write through the XCD's L2, so data
// one work group publishes this way reaches memory without the whole-L2 write-back
// a device-scope release fence would issue (once per work group).
__device__ __forceinline__ void store_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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
// adjacent 4-column groups of one row and reads the partial LSEs and outputs of GS
// parts per round trip (all issued together).  Across groups of GS it keeps a
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
    const int tid = threadIdx.x;
    const int r = tid * Q / (D / 4);   // the row this thread merges
    if (r >= R) return;
    const int d0 = (tid * Q % (D / 4)) * 4;
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
                    po_rsrc, (int)((row_off + d0 + 4 * q + sp * a.part_stride) * 2), 0,
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
        *reinterpret_cast<u32x2*>((uint16_t*)a.out + row_off + d0 + 4 * q) = packed;
    }
    if (d0 == 0 && a.lse) a.lse[lse_row] = W > 0.f ? M + fast_log2(W) : -INFINITY;
}

// Waves per SIMD: two where the state fits in half the register file (so launches
// with more work groups than compute units still fill the chip; the usual split
// count gives one work group per CU), one where it does not (D = 256, or more than
// 16 rows at D = 128).
template <int D, int NR> constexpr int split_waves_per_eu() {
    return (D == 256 || NR * D >= 256) ? 1 : 2;
}

template <typename T, int D, int NR, bool FUSED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(split_waves_per_eu<D, NR>())))
void splitkv_kernel(SplitArgs a) {
    using E = Elem<T>;
    typedef SplitLds<D, NR> L;
    constexpr int NKK = D / 32;          // 16x16x32 k-steps over D
    constexpr int NDB = D / 16;          // 16-wide blocks of O^T
    constexpr int CPR = D / 8;           // 16-byte chunks per V row
    constexpr int KPB = keys_per_block<D, NR>();      // keys per block
    constexpr int NHF = KPB / 16;                 // 16-key halves per block
    constexpr int VCH = KPB * CPR / 64;           // V chunks per lane per block
    constexpr int VLD = L::VLD, OLD = L::OLD, ROWS = L::ROWS;

    __shared__ __attribute__((aligned(16))) unsigned char smem[L::BYTES];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, g4 = lane >> 4;
    const int s = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    const int G = a.Hq / a.Hkv, R = G * a.Lq;

    // Key range [j0, j1) of this work group.  The keys this batch element holds are
    // Lkv, or its filled length kv_len[b] (read on the device, so a captured graph
    // follows the length from replay to replay); the num_splits chunks split that
    // length evenly (chunk c = [cC, (c + 1)C), C = ceil(nkeys / num_splits)), and work
    // group s takes the `group` consecutive chunks [s group, (s + 1) group).
    int nkeys = a.Lkv;
    if (a.kv_len) nkeys = min(max(a.kv_len[b], 0), a.Lkv);
    const int64_t C = ((int64_t)nkeys + a.num_splits - 1) / a.num_splits;
    const int64_t j0l = min((int64_t)s * a.group * C, (int64_t)nkeys);
    const int j0 = (int)j0l;
    const int j1 = (int)min(j0l + a.group * C, (int64_t)nkeys);
    const int nblk = (j1 - j0 + KPB - 1) / KPB;

    // Query row rb*16 + n of this kv head: head hk*G + r / Lq, position r % Lq.  Rows
    // past R are zero (their results are never stored).
    constexpr bool QL = q_in_lds<D, NR>();
    constexpr int QLD = L::QLD;
    uint16_t* const qlds = (uint16_t*)(smem + L::QOFF);
    typename E::vec8 qf[QL ? 1 : NR][NKK];
    if constexpr (QL) {
        // the work group's ROWS x D rows of Q, 16-byte chunk c of row r by thread
        for (int it = tid; it < ROWS * (D / 8); it += 256) {
            const int r = it / (D / 8), c = it % (D / 8);
            u32x4 raw = {0u, 0u, 0u, 0u};
            if (r < R) {
                const int hq = hk * G + r / a.Lq, iq = r % a.Lq;
                raw = load16((const uint16_t*)a.q + (int64_t)b * a.q_batch +
                             (int64_t)hq * a.q_head + (int64_t)iq * a.q_row + c * 8);
            }
            store16(qlds + r * QLD + c * 8, raw);
        }
        __syncthreads();
    } else {
#pragma unroll
        for (int rb = 0; rb < NR; ++rb) {
            const int r = rb * 16 + n;
            const bool r_ok = r < R;
            const int hq = hk * G + (r_ok ? r / a.Lq : 0), iq = r_ok ? r % a.Lq : 0;
            const uint16_t* qr = (const uint16_t*)a.q + (int64_t)b * a.q_batch +
                                 (int64_t)hq * a.q_head + (int64_t)iq * a.q_row + g4 * 8;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                u32x4 raw = {0u, 0u, 0u, 0u};
                if (r_ok) raw = load16(qr + kk * 32);
                qf[QL ? 0 : rb][kk] = as_vec8<T>(raw);
            }
        }
    }
    // Q operand of k-step kk for row block rb
    auto q_operand = [&](int rb, int kk) -> typename E::vec8 {
        if constexpr (QL)
            return as_vec8<T>(load16(qlds + (rb * 16 + n) * QLD + kk * 32 + g4 * 8));
        else
            return qf[rb][kk];
    };

    const uint16_t* kp = (const uint16_t*)a.k + (int64_t)b * a.kv_batch + (int64_t)hk * a.kv_head;
    const uint16_t* vp = (const uint16_t*)a.v + (int64_t)b * a.kv_batch + (int64_t)hk * a.kv_head;

    // Loads of one block into a register buffer, as streaming (nontemporal) loads:
    // every K/V byte is read once.  Rows past the range end are clamped to its last
    // key (real, finite data; the range is non-empty whenever a block exists) and
    // masked out of the softmax, so no load needs a branch.  A prefetch past the
    // wave's last block (`idle`) reads only the range's first key row: the same
    // instructions, so the wait counts stay the same, but no second pass over a block.
    typedef u32x4 KBuf[NHF][NKK];
    typedef u32x4 VBuf[VCH];
    auto load_block = [&](KBuf& kb_, VBuf& vb_, int blk, bool idle) {
        const int kb = j0 + blk * KPB;
#pragma unroll
        for (int hf = 0; hf < NHF; ++hf) {
            const int j = idle ? j0 : min(kb + hf * 16 + n, j1 - 1);
            const uint16_t* kr = kp + (int64_t)j * a.kv_row + g4 * 8;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) kb_[hf][kk] = load16_stream(kr + kk * 32);
        }
#pragma unroll
        for (int u = 0; u < VCH; ++u) {
            const int c = lane + 64 * u;
            const int j = idle ? j0 : min(kb + c / CPR, j1 - 1);
            vb_[u] = load16_stream(vp + (int64_t)j * a.kv_row + (c % CPR) * 8);
        }
    };

    f32x4 o[NR][NDB];
#pragma unroll
    for (int rb = 0; rb < NR; ++rb)
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[rb][db] = f32x4{};
    float m_run[NR], l_run[NR];
#pragma unroll
    for (int rb = 0; rb < NR; ++rb) {
        m_run[rb] = -INFINITY;
        l_run[rb] = 0.f;
    }

    uint16_t* vl = (uint16_t*)smem + wave * KPB * VLD;
    const int e4 = (lane & 15) >> 2, q4 = lane & 3;

    auto compute_block = [&](const KBuf& kc, const VBuf& vc, int blk) {
        const int kb = j0 + blk * KPB;
        // stage V (KPB keys x D) in this wave's LDS slice; V^T operands are read back
        // by transpose reads: slot 4h + e of lane (d, g4) is V[16h + 4g4 + e][d] (with
        // 16-key blocks the upper slots repeat the lower keys, finite and weighted 0)
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int u = 0; u < VCH; ++u) {
            const int c = lane + 64 * u;
            store16(vl + (c / CPR) * VLD + (c % CPR) * 8, vc[u]);
        }
        lds_wave_sync();
        // One 16-row block at a time (its logits, softmax and P.V), so that only one
        // block's scores are live; the V^T operands are re-read from LDS per block.
#pragma unroll
        for (int rb = 0; rb < NR; ++rb) {
            // S^T for keys [16hf, 16hf + 16) of the block: lane holds keys 16hf + 4g4 + i.
            f32x4 sv[NHF];
#pragma unroll
            for (int hf = 0; hf < NHF; ++hf) {
                sv[hf] = f32x4{};
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk)
                    sv[hf] = E::mfma16(as_vec8<T>(kc[hf][kk]), q_operand(rb, kk), sv[hf]);
            }
            float mx = -INFINITY;
#pragma unroll
            for (int hf = 0; hf < NHF; ++hf)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int j = kb + hf * 16 + 4 * g4 + i;
                    const float x = j < j1 ? sv[hf][i] * a.scale_log2 : -INFINITY;
                    sv[hf][i] = x;
                    mx = fmaxf(mx, x);
                }
            mx = fmaxf(mx, xor_shfl(mx, 16));
            mx = fmaxf(mx, xor_shfl(mx, 32));
            // The reference max m_run moves lazily, only when a block's max exceeds it
            // by more than kTau (so every p = 2^(s - m_run) <= 2^kTau): most blocks then
            // leave O and l as they are.
            const bool rescale = __any(mx > m_run[rb] + kTau);
            float alpha = 1.f;
            if (rescale) {
                const float m_new = mx > m_run[rb] + kTau ? mx : m_run[rb];
                alpha = m_run[rb] == -INFINITY ? 0.f : fast_exp2(m_run[rb] - m_new);
                m_run[rb] = m_new;
                l_run[rb] *= alpha;
            }
            const float m_use = m_run[rb] == -INFINITY ? 0.f : m_run[rb];
            // B operand: slot j <-> key 16(j/4) + 4g4 + j%4; with 16-key blocks the
            // upper four slots hold 0, so the 32-key MFMA step adds nothing for them.
            float p[8];
            float psum = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                p[j] = (j >> 2) < NHF ? fast_exp2(sv[(j >> 2) % NHF][j & 3] - m_use) : 0.f;
                psum += p[j];
            }
            l_run[rb] += psum;
            const u32x4 pb = {E::pack2(p[0], p[1]), E::pack2(p[2], p[3]), E::pack2(p[4], p[5]),
                              E::pack2(p[6], p[7])};
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int key0 = 4 * g4 + e4, col = db * 16 + 4 * q4;
                const u32x2 lo = lds_read_tr16(vl + key0 * VLD + col);
                u32x4 av = {lo.x, lo.y, lo.x, lo.y};
                if constexpr (NHF == 2) {
                    const u32x2 hi = lds_read_tr16(vl + (key0 + 16) * VLD + col);
                    av = u32x4{lo.x, lo.y, hi.x, hi.y};
                }
                if (rescale) o[rb][db] *= alpha;
                o[rb][db] = E::mfma16(as_vec8<T>(av), as_vec8<T>(pb), o[rb][db]);
            }
        }
        lds_wave_sync();
    };

    // Ping-pong between two register buffers: the loads of the wave's next block
    // are in flight while the current one is computed.  The prefetch is issued
    // unconditionally (past the wave's last block it reads one key row) and never
    // copied between registers, so the compiler's wait counts only cover the older
    // group of loads.
    KBuf ka, kb2;
    VBuf va, vb2;
    if (wave < nblk) load_block(ka, va, wave, false);
    for (int blk = wave; blk < nblk; blk += 2 * kWaves) {
        const int nxt = blk + kWaves;
        load_block(kb2, vb2, nxt, nxt >= nblk);
        compute_block(ka, va, blk);
        if (nxt >= nblk) break;
        load_block(ka, va, nxt + kWaves, nxt + kWaves >= nblk);
        compute_block(kb2, vb2, nxt);
    }

    // Merge the waves' states through LDS.  The four lanes of a row hold disjoint
    // keys: total their sums first.
    __syncthreads();
    float* cm = (float*)smem;            // [kWaves][ROWS] running max
    float* cl = cm + kWaves * ROWS;      // [kWaves][ROWS] running sum
    float* co = cl + kWaves * ROWS;      // [kWaves][ROWS][OLD] unnormalised output
#pragma unroll
    for (int rb = 0; rb < NR; ++rb) {
        float l = l_run[rb];
        l += xor_shfl(l, 16);
        l += xor_shfl(l, 32);
        const int r = rb * 16 + n;
        if (g4 == 0) {
            cm[wave * ROWS + r] = m_run[rb];
            cl[wave * ROWS + r] = l;
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            *reinterpret_cast<f32x4*>(&co[(wave * ROWS + r) * OLD + db * 16 + g4 * 4]) = o[rb][db];
    }
    __syncthreads();

    for (int it = tid; it < ROWS * (D / 4); it += 256) {
        const int r = it / (D / 4), d = (it % (D / 4)) * 4;
        if (r >= R) break;  // rows are the slow index: every later item is padding too
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, cm[w * ROWS + r]);
        const float Mu = M == -INFINITY ? 0.f : M;
        float Ls = 0.f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float wt = fast_exp2(cm[w * ROWS + r] - Mu);
            Ls += cl[w * ROWS + r] * wt;
            acc += *reinterpret_cast<const f32x4*>(&co[(w * ROWS + r) * OLD + d]) * wt;
        }
        const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
        const int h = hk * G + r / a.Lq, i = r % a.Lq;
        const int64_t po = (int64_t)s * a.part_stride + (int64_t)b * a.q_batch +
                           (int64_t)h * a.q_head + (int64_t)i * a.q_row + d;
        float* lp = a.lse_part + (((int64_t)s * a.B + b) * a.Hq + h) * a.Lq + i;
        const float lse_s = Ls > 0.f ? M + fast_log2(Ls) : -INFINITY;
        if constexpr (FUSED) {
            // 16-bit partial output (workspace), published with one 8-byte store
            const uint64_t w = (uint64_t)E::pack2(acc[0] * inv, acc[1] * inv) |
                               ((uint64_t)E::pack2(acc[2] * inv, acc[3] * inv) << 32);
            store_agent(reinterpret_cast<uint64_t*>((uint16_t*)a.out_part + po), w);
            if (d == 0) store_agent(lp, lse_s);
        } else {
            *reinterpret_cast<f32x4*>(a.out_part + po) = acc * inv;
            if (d == 0) *lp = lse_s;
        }
    }
    if constexpr (FUSED) merge_tail<T, D, NR>(a, b, hk, R, G);
}

template <typename T, int D, int NR>
hipError_t launch_splitkv_r(const SplitArgs& a, bool fused, dim3 grid, hipStream_t st) {
    if (fused)
        hipLaunchKernelGGL((splitkv_kernel<T, D, NR, true>), grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((splitkv_kernel<T, D, NR, false>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_splitkv_f(const SplitArgs& a, bool fused, dim3 grid, hipStream_t st) {
    const int R = (a.Hq / a.Hkv) * a.Lq;
    if (R <= 16) return launch_splitkv_r<T, D, 1>(a, fused, grid, st);
    if constexpr (D != 256) {   // (at D = 256 more rows would spill registers)
        if (R <= 32) return launch_splitkv_r<T, D, 2>(a, fused, grid, st);
        if (R <= 64) return launch_splitkv_r<T, D, 4>(a, fused, grid, st);
    }
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_splitkv_t(const SplitArgs& a, int D, bool fused, hipStream_t st) {
    // fused: one work group per group of `group` consecutive chunks
    const int parts = (a.num_splits + a.group - 1) / a.group;
    const dim3 grid((unsigned)parts, (unsigned)a.Hkv, (unsigned)a.B);
    switch (D) {
        case 64: return launch_splitkv_f<T, 64>(a, fused, grid, st);
        case 128: return launch_splitkv_f<T, 128>(a, fused, grid, st);
        case 256: return launch_splitkv_f<T, 256>(a, fused, grid, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int splitkv_max_rows(int D) { return D == 256 ? 16 : 64; }

hipError_t launch_splitkv(const SplitArgs& a, int dtype, int D, bool fused, hipStream_t stream) {
    if (dtype == 0) return launch_splitkv_t<__bf16>(a, D, fused, stream);
    return launch_splitkv_t<_Float16>(a, D, fused, stream);
}

}  // namespace skv
