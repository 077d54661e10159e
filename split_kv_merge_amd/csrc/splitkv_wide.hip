// splitkv_wide.hip -- split-KV decode for 17..64 query rows per kv head (D = 64, 128).
//
// Same operation as splitkv.hip -- per (batch, kv head, chunk) the partial attention
// state (out normalised by the chunk's own sum, log2 LSE) of every query row that
// reads the kv head, the stable per-split online softmax of ExecuTorch PR #22133
// "Prevent Voxtral NaNs in CUDA split-K attention" (description and Copilot overview)
// -- for the small-query range of that PR's reviewer item 1 (G query heads per kv
// head times Lq rows, above 16).
//
// Design (gfx950, wave64, one wave per SIMD):
//   * work group = 4 waves over one chunk; each wave takes every fourth 32-key block
//     and keeps its own online-softmax state; the waves' states merge through LDS.
//   * S^T = K Q^T on v_mfma_f32_32x32x16: 32 keys on M, 32 query rows on N, in one or
//     two 32-row blocks (NB); every K operand and every V^T operand feeds the MFMAs of
//     all row blocks, so K and V are read from HBM once per chunk whatever the row
//     count.  K and V are loaded in whole rows (16 lanes per 256-byte row: a 32-byte
//     piece per row per instruction, as the MFMA operand layout would have it, doubles
//     the L1-to-L2 requests and makes the loads the bottleneck) and staged in per-wave
//     LDS slices; K operands are read back with ds_read_b128 (k-step kk, lane half h:
//     head-dim elements 16 kk + 8 h .. + 8 of the lane's key row), V^T operands with
//     ds_read_b64_tr_b16.  Q (all rows) sits in LDS, shared by the four waves.
//   * The C layout of S^T is the B operand of O^T += V^T P^T (the key order inside P
//     permuted to match, as in the prefill kernel).  The output accumulators, 64 or 128
//     registers, are pinned in AGPRs: those MFMAs are written as asm with "+a", and the
//     builtin S^T MFMAs are compiled in VGPR form (-amdgpu-mfma-vgpr-form for this
//     file), so no accumulator moves between register files in the key loop.
//   * Every lane holds one row's keys with its partner lane l ^ 32: row max and sum
//     take one v_permlane32_swap.
#include "device.h"
#include "launch.h"
#include "splitkv_tail.h"

namespace skv {

namespace {

using namespace dec;

template <bool B> struct BoolC {
    static constexpr bool value = B;
};


constexpr int kWideWaves = 4;
constexpr int kWideKeys = 32;       // keys per block
constexpr float kWideTau = 8.f;     // lazy-rescale threshold of the running max (log2 units)

template <int D, int NB> struct WideLds {
    static constexpr int ROWS = 32 * NB;
    static constexpr int QLD = D + 8;    // Q row pitch (elements): conflict-free operand reads
    static constexpr int KLD = D + 8;    // K row pitch (elements): conflict-free operand reads
    static constexpr int VLD = D + 32;   // V row pitch (elements): conflict-free transpose reads
    static constexpr int OLD = D + 4;    // combine-buffer pitch (floats)
    static constexpr int QBYTES = ROWS * QLD * 2;
    static constexpr int KOFF = QBYTES;  // byte offset of the waves' K slices
    static constexpr int VOFF = KOFF + kWideWaves * kWideKeys * KLD * 2;  // ... and V slices
    static constexpr int LOOP = VOFF + kWideWaves * kWideKeys * VLD * 2;
    static constexpr int COMB = kWideWaves * (ROWS * OLD + 2 * ROWS) * 4;
    static constexpr int BYTES = LOOP > COMB ? LOOP : COMB;
};

// O^T += V^T P^T with the accumulator in AGPRs.  The hazard recognizer does not look
// inside asm, so the kernel adds the wait states itself: p_fence between the VALU
// writes of P and the first MFMA reading it, o_fence between the last MFMA writing
// O and any other read of O, including the register copies the compiler may place at
// control-flow joins (a 16-pass MFMA needs at most 20; 24 given).
template <typename T> struct WideMfma;
template <> struct WideMfma<__bf16> {
    static __device__ __forceinline__ void acc(f32x16& c, u32x4 a, u32x4 b) {
        asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    }
};
template <> struct WideMfma<_Float16> {
    static __device__ __forceinline__ void acc(f32x16& c, u32x4 a, u32x4 b) {
        asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    }
};
__device__ __forceinline__ void p_fence(u32x4 (&p)[1][2]) {
    asm volatile("s_nop 2" : "+v"(p[0][0]), "+v"(p[0][1]));
}
__device__ __forceinline__ void p_fence(u32x4 (&p)[2][2]) {
    asm volatile("s_nop 2" : "+v"(p[0][0]), "+v"(p[0][1]), "+v"(p[1][0]), "+v"(p[1][1]));
}
__device__ __forceinline__ void o_fence(f32x16 (&o)[1][2]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(o[0][0]), "+a"(o[0][1]));
}
__device__ __forceinline__ void o_fence(f32x16 (&o)[2][2]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[1][0]), "+a"(o[1][1]));
}
__device__ __forceinline__ void o_fence(f32x16 (&o)[1][4]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]));
}
__device__ __forceinline__ void o_fence(f32x16 (&o)[2][4]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]), "+a"(o[1][0]),
                   "+a"(o[1][1]), "+a"(o[1][2]), "+a"(o[1][3]));
}

template <typename T, int D, int NB, bool FUSED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void splitkv_wide_kernel(SplitArgs a) {
    using E = Elem<T>;
    typedef WideLds<D, NB> L;
    constexpr int NKK = D / 16;                  // 32x32x16 k-steps over D
    constexpr int NDB = D / 32;                  // 32-wide blocks of O^T
    constexpr int CPR = D / 8;                   // 16-byte chunks per row
    constexpr int VCH = kWideKeys * CPR / 64;    // V chunks per lane per block
    constexpr int ROWS = L::ROWS, QLD = L::QLD, KLD = L::KLD, VLD = L::VLD, OLD = L::OLD;

    __shared__ __attribute__((aligned(16))) unsigned char smem[L::BYTES];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 31, hg = lane >> 5;
    const int s = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    const int G = a.Hq / a.Hkv, R = G * a.Lq;

    // Key range [j0, j1) of this work group: the keys this batch element holds (Lkv,
    // or its filled length kv_len[b], read on the device) split evenly into
    // num_splits chunks, of which the work group takes `group` consecutive ones.
    int nkeys = a.Lkv;
    if (a.kv_len) nkeys = min(max(a.kv_len[b], 0), a.Lkv);
    const int64_t C = ((int64_t)nkeys + a.num_splits - 1) / a.num_splits;
    const int64_t j0l = min((int64_t)s * a.group * C, (int64_t)nkeys);
    const int j0 = (int)j0l;
    const int j1 = (int)min(j0l + a.group * C, (int64_t)nkeys);
    const int nblk = (j1 - j0 + kWideKeys - 1) / kWideKeys;

    // Q rows of this kv head into LDS: row r is head hk*G + r / Lq, position r % Lq;
    // rows past R are zero (their results are never stored).  With a negative scale
    // the rows are stored negated (a sign flip, exact) and the logit scale is |scale|,
    // so the maximum of the raw dot products is the maximum of the scaled logits.  The
    // rows are loaded first, then the wave's first K/V blocks are requested, and only
    // then are the rows written to LDS: the K/V requests do not wait for Q.
    const uint32_t qsign = a.scale_log2 < 0.f ? 0x80008000u : 0u;
    const float c = fabsf(a.scale_log2);
    uint16_t* const qlds = (uint16_t*)smem;
    constexpr int QPT = ROWS * CPR / 256;  // 16-byte chunks of Q per thread
    u32x4 qraw[QPT];
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
        // rows past R load row R - 1 and are zeroed after the load, so the loads carry
        // no branch and go out together
        const int it = tid + 256 * u, r = it / CPR, cc = it % CPR, rc = min(r, R - 1);
        const int hq = hk * G + rc / a.Lq, iq = rc % a.Lq;
        const u32x4 raw = load16((const uint16_t*)a.q + (int64_t)b * a.q_batch +
                                 (int64_t)hq * a.q_head + (int64_t)iq * a.q_row + cc * 8);
        qraw[u] = r < R ? (raw ^ qsign) : u32x4{0u, 0u, 0u, 0u};
    }

    const uint16_t* kp = (const uint16_t*)a.k + (int64_t)b * a.kv_batch + (int64_t)hk * a.kv_head;
    const uint16_t* vp = (const uint16_t*)a.v + (int64_t)b * a.kv_batch + (int64_t)hk * a.kv_head;

    // Loads of one block into a register buffer: buffer loads over a descriptor that
    // starts at the block's first key and ends after its last key in the range, so
    // chunks of keys past the range end read as zero (and are masked out of the
    // softmax), and the per-lane offsets are loop invariants.  A prefetch past the
    // wave's last block (`idle`) covers one key row: the same instructions, so the wait
    // counts stay the same, with no second pass over a block.  Nontemporal (nt): every
    // K/V byte is read once.
    int voff[VCH];  // byte offset of chunk c = lane + 64u: key c / CPR, columns (c % CPR) * 8
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
        const int ch = lane + 64 * u;
        voff[u] = (ch / CPR) * (int)a.kv_row * 2 + (ch % CPR) * 16;
    }
    typedef u32x4 KBuf[VCH];
    typedef u32x4 VBuf[VCH];
    // The block's first key and key count are the same in every lane of the wave; read
    // into scalar registers, they make the descriptors scalar, so each load is one
    // instruction rather than a loop over the distinct descriptors of the lanes.
    auto load_block = [&](KBuf& kb_, VBuf& vb_, int blk, bool idle) {
        const int kb = __builtin_amdgcn_readfirstlane(idle ? j0 : j0 + blk * kWideKeys);
        const int nk = __builtin_amdgcn_readfirstlane(idle ? 1 : min(kWideKeys, j1 - kb));
        // a chunk with no key reads nothing: num_records 0 makes every lane read zero
        // without a memory access
        const uint32_t nrec = nblk == 0 ? 0u : (uint32_t)((nk - 1) * a.kv_row * 2 + D * 2);
        const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(kp + (int64_t)kb * a.kv_row), (short)0, (int)nrec, kBufferRsrcWord3);
        const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(vp + (int64_t)kb * a.kv_row), (short)0, (int)nrec, kBufferRsrcWord3);
#pragma unroll
        for (int u = 0; u < VCH; ++u) {
            kb_[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   kr, voff[u], 0, kNontemporalLoad));
            vb_[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   vr, voff[u], 0, kNontemporalLoad));
        }
    };

    f32x16 o[NB][NDB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[nb][db] = f32x16{};
    float m_run[NB], l_run[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        m_run[nb] = -INFINITY;
        l_run[nb] = 0.f;
    }

    uint16_t* const kl = (uint16_t*)(smem + L::KOFF) + wave * kWideKeys * KLD;
    uint16_t* const vl = (uint16_t*)(smem + L::VOFF) + wave * kWideKeys * VLD;
    // lane roles of the V^T transpose reads
    const int g16 = lane >> 4, e4 = (lane & 15) >> 2, q4 = lane & 3;

    // One block: S^T, the online softmax, O^T += V^T P^T.  MASK (the range's last
    // block, when it ends inside it) masks the keys past the range end; other blocks
    // carry no mask arithmetic.
    auto block_body = [&](const KBuf& kc, const VBuf& vc, int kb, auto mask_c) {
        constexpr bool MASK = decltype(mask_c)::value;
        // stage K and V (32 keys x D each) in this wave's LDS slices
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int u = 0; u < VCH; ++u) {
            const int ch = lane + 64 * u;
            store16(kl + (ch / CPR) * KLD + (ch % CPR) * 8, kc[u]);
            store16(vl + (ch / CPR) * VLD + (ch % CPR) * 8, vc[u]);
        }
        // S^T = K Q^T for every row block; lane holds keys 8(i/4) + 4hg + i%4 of row n
        f32x16 sv[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sv[nb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const u32x4 kv = load16(kl + n * KLD + kk * 16 + hg * 8);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const u32x4 qv = load16(qlds + (nb * 32 + n) * QLD + kk * 16 + hg * 8);
                sv[nb] = E::mfma32(as_vec8<T>(kv), as_vec8<T>(qv), sv[nb]);
            }
        }
        // online softmax per row block on the raw dot products (c >= 0), with the lazily
        // moved reference max m_run: it moves only when a block's max exceeds it by more
        // than kWideTau, so every p = 2^(s c - m_run) <= 2^kWideTau and most blocks leave
        // O and l as they are.  Every block holds a key of the range, so after the first
        // block m_run is finite.
        u32x4 pb[NB][2];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            if constexpr (MASK) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (kb + 8 * (i >> 2) + 4 * hg + (i & 3) >= j1) sv[nb][i] = -INFINITY;
            }
            float mx = sv[nb][0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sv[nb][i]);
            const float m_tile = pair_max(mx) * c;
            if (__any(m_tile > m_run[nb] + kWideTau)) {
                const float m_new = m_tile > m_run[nb] + kWideTau ? m_tile : m_run[nb];
                const float alpha = m_run[nb] == -INFINITY ? 0.f : fast_exp2(m_run[nb] - m_new);
                m_run[nb] = m_new;
                l_run[nb] *= alpha;
                o_fence(o);
#pragma unroll
                for (int db = 0; db < NDB; ++db) o[nb][db] *= alpha;
            }
            const float nm = -m_run[nb];
            // packed P pairs; the row sum adds the packed (rounded) values the P.V product
            // uses.  A masked key gives p = 0 also when c = 0.
            auto logit = [&](float x) {
                const float y = fmaf(x, c, nm);
                return (MASK && x == -INFINITY) ? -INFINITY : y;
            };
            float psum = 0.f;
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t w = E::pack2(fast_exp2(logit(sv[nb][8 * st + 2 * j])),
                                                fast_exp2(logit(sv[nb][8 * st + 2 * j + 1])));
                    pb[nb][st][j] = w;
                    psum = E::sum2(w, psum);
                }
            l_run[nb] += psum;
        }
        lds_wave_sync();  // the V slice is written (and K read)
        p_fence(pb);
        // O^T += V^T P^T: k-step st covers keys 16 st + 8 h + 4 (lane / 32) + e for
        // operand slots 4 h + e, the order the C layout of S^T leaves P in
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const int key0 = 16 * st + 4 * (g16 >> 1) + e4;
                const int col = db * 32 + (g16 & 1) * 16 + 4 * q4;
                const u32x2 lo = lds_read_tr16(vl + key0 * VLD + col);
                const u32x2 hi = lds_read_tr16(vl + (key0 + 8) * VLD + col);
                const u32x4 vf = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) WideMfma<T>::acc(o[nb][db], vf, pb[nb][st]);
            }
        // The wait states after the block's last MFMA, here rather than at the next read
        // of O: at the loop's back edge and exits the compiler may copy O between
        // registers, and it cannot tell that the asm MFMAs are still writing it.
        o_fence(o);
        lds_wave_sync();  // the slices are read before the next block overwrites them
    };
    auto compute_block = [&](const KBuf& kc, const VBuf& vc, int blk) {
        const int kb = j0 + blk * kWideKeys;
        if (kb + kWideKeys <= j1)
            block_body(kc, vc, kb, BoolC<false>{});
        else
            block_body(kc, vc, kb, BoolC<true>{});
    };

    // Register buffers: the loads of the wave's next blocks are in flight while the
    // current one is computed -- three blocks with one row block, two with two (where
    // a fourth buffer would not fit beside the outputs).  With one wave per SIMD the
    // memory latency outlasts the compute of two blocks.  Loads past the wave's last
    // block cover one key row (`idle`), so every iteration waits for the same count.
    constexpr int W = kWideWaves;
    KBuf k0, k1, k2, k3;
    VBuf v0, v1, v2, v3;
    // Issued on every path (idle loads for a wave with no block), so the compiler's
    // count of loads in flight is the same on all of them and the wait for Q below
    // leaves the K/V requests in flight.
    load_block(k0, v0, wave, wave >= nblk);
    load_block(k1, v1, wave + W, wave + W >= nblk);
    if constexpr (NB == 1) load_block(k2, v2, wave + 2 * W, wave + 2 * W >= nblk);
    // Q rows to LDS (the compiler waits for the Q loads only), then a barrier that
    // waits for LDS writes alone: __syncthreads would also wait for the K/V requests.
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
        const int it = tid + 256 * u;
        store16(qlds + (it / CPR) * QLD + (it % CPR) * 8, qraw[u]);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    if constexpr (NB == 1) {
        for (int blk = wave; blk < nblk; blk += 4 * W) {
            load_block(k3, v3, blk + 3 * W, blk + 3 * W >= nblk);
            compute_block(k0, v0, blk);
            if (blk + W >= nblk) break;
            load_block(k0, v0, blk + 4 * W, blk + 4 * W >= nblk);
            compute_block(k1, v1, blk + W);
            if (blk + 2 * W >= nblk) break;
            load_block(k1, v1, blk + 5 * W, blk + 5 * W >= nblk);
            compute_block(k2, v2, blk + 2 * W);
            if (blk + 3 * W >= nblk) break;
            load_block(k2, v2, blk + 6 * W, blk + 6 * W >= nblk);
            compute_block(k3, v3, blk + 3 * W);
        }
    } else {
        for (int blk = wave; blk < nblk; blk += 3 * W) {
            load_block(k2, v2, blk + 2 * W, blk + 2 * W >= nblk);
            compute_block(k0, v0, blk);
            if (blk + W >= nblk) break;
            load_block(k0, v0, blk + 3 * W, blk + 3 * W >= nblk);
            compute_block(k1, v1, blk + W);
            if (blk + 2 * W >= nblk) break;
            load_block(k1, v1, blk + 4 * W, blk + 4 * W >= nblk);
            compute_block(k2, v2, blk + 2 * W);
        }
    }

    // Merge the waves' states through LDS (over the Q rows and V slices: every wave is
    // past its last block).  The two lanes of a row hold disjoint keys: total their sums.
    __syncthreads();
    o_fence(o);
    float* cm = (float*)smem;              // [kWideWaves][ROWS] running max
    float* cl = cm + kWideWaves * ROWS;    // [kWideWaves][ROWS] running sum
    float* co = cl + kWideWaves * ROWS;    // [kWideWaves][ROWS][OLD] unnormalised output
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const float l = pair_sum(l_run[nb]);
        const int r = nb * 32 + n;
        if (hg == 0) {
            cm[wave * ROWS + r] = m_run[nb];
            cl[wave * ROWS + r] = l;
        }
        // lane holds output columns db*32 + 8 a4 + 4 hg + e of row r
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const f32x4 v4 = {o[nb][db][4 * a4], o[nb][db][4 * a4 + 1], o[nb][db][4 * a4 + 2],
                                  o[nb][db][4 * a4 + 3]};
                *reinterpret_cast<f32x4*>(&co[(wave * ROWS + r) * OLD + db * 32 + 8 * a4 + 4 * hg]) =
                    v4;
            }
    }
    __syncthreads();

    for (int it = tid; it < ROWS * (D / 4); it += 256) {
        const int r = it / (D / 4), d = (it % (D / 4)) * 4;
        if (r >= R) break;  // rows are the slow index: every later item is padding too
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWideWaves; ++w) M = fmaxf(M, cm[w * ROWS + r]);
        const float Mu = M == -INFINITY ? 0.f : M;
        float Ls = 0.f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kWideWaves; ++w) {
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
    if constexpr (FUSED) merge_tail<T, D, 2 * NB>(a, b, hk, R, G);
}

template <typename T, int D, int NB>
hipError_t launch_wide_nb(const SplitArgs& a, bool fused, dim3 grid, hipStream_t st) {
    if (fused)
        hipLaunchKernelGGL((splitkv_wide_kernel<T, D, NB, true>), grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((splitkv_wide_kernel<T, D, NB, false>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_wide_d(const SplitArgs& a, bool fused, dim3 grid, hipStream_t st) {
    const int R = (a.Hq / a.Hkv) * a.Lq;
    if (R <= 32) return launch_wide_nb<T, D, 1>(a, fused, grid, st);
    if (R <= 64) return launch_wide_nb<T, D, 2>(a, fused, grid, st);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_splitkv_wide(const SplitArgs& a, int dtype, int D, bool fused, dim3 grid,
                               hipStream_t stream) {
    if (dtype == 0) {
        if (D == 64) return launch_wide_d<__bf16, 64>(a, fused, grid, stream);
        if (D == 128) return launch_wide_d<__bf16, 128>(a, fused, grid, stream);
    } else {
        if (D == 64) return launch_wide_d<_Float16, 64>(a, fused, grid, stream);
        if (D == 128) return launch_wide_d<_Float16, 128>(a, fused, grid, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace skv
