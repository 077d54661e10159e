// splitkv.hip -- split-KV decode: per-chunk partial attention states.
//
// Each work group owns one (batch, kv head, chunk) and ALL query rows that read
// that kv head (G = Hq/Hkv heads x Lq rows, up to 16: one block of 16 rows on the
// MFMA N axis; more rows go to splitkv_wide.hip), so every K/V byte of the chunk is
// read from HBM exactly once.
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
// query rows on N), K fed straight from global memory in the operand layout at
// D <= 128 (k-step kk takes head-dim elements [32kk, 32kk + 32) of 16 key rows, the
// four lanes of a row reading 64 contiguous bytes) and, at D = 256, loaded in whole
// rows and staged in a per-wave LDS slice like V; O^T += V^T P^T with V staged in a
// per-wave LDS slice and read back with ds_read_b64_tr_b16, the key order of P
// matching the C layout of S^T.
#include "device.h"
#include "launch.h"
#include "splitkv_tail.h"

namespace skv {

namespace {

using namespace dec;

constexpr int kWaves = 4;
constexpr float kTau = 8.f;   // lazy-rescale threshold of the running max (log2 units)
// Keys per block: 32, or 16 at D = 256, where two 32-key blocks in flight per wave
// (K and V) would not fit in the register file beside the rest of the wave's state.
template <int D> constexpr int keys_per_block() { return D == 256 ? 16 : 32; }

// K is staged through LDS at D = 256 only (see the kernel).
template <int D> constexpr bool stage_k() { return D == 256; }

template <int D> struct SplitLds {
    static constexpr int VLD = D + 16;  // V pitch (elements) in the staging slice
    static constexpr int KLD = D + 8;   // K pitch (elements) in the staging slice
    static constexpr int OLD = D + 4;   // pitch (floats) of the combine buffer
    static constexpr int ROWS = 16;
    static constexpr int KOFF = kWaves * keys_per_block<D>() * VLD * 2;   // K slices (bytes)
    static constexpr int STAGE =
        KOFF + (stage_k<D>() ? kWaves * keys_per_block<D>() * KLD * 2 : 0);
    static constexpr int COMB = kWaves * (ROWS * OLD + 2 * ROWS) * 4;
    static constexpr int BYTES = STAGE > COMB ? STAGE : COMB;
};

// Waves per SIMD: two where the state fits in half the register file (so launches
// with more work groups than compute units still fill the chip; the usual split
// count gives one work group per CU), one at D = 256.
template <int D> constexpr int split_waves_per_eu() { return D == 256 ? 1 : 2; }

template <typename T, int D, bool FUSED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(split_waves_per_eu<D>())))
void splitkv_kernel(SplitArgs a) {
    using E = Elem<T>;
    typedef SplitLds<D> L;
    constexpr int NKK = D / 32;          // 16x16x32 k-steps over D
    constexpr int NDB = D / 16;          // 16-wide blocks of O^T
    constexpr int CPR = D / 8;           // 16-byte chunks per V row
    constexpr int KPB = keys_per_block<D>();      // keys per block
    constexpr int NHF = KPB / 16;                 // 16-key halves per block
    constexpr int VCH = KPB * CPR / 64;           // V chunks per lane per block
    constexpr int VLD = L::VLD, KLD = L::KLD, OLD = L::OLD, ROWS = L::ROWS;
    constexpr bool KST = stage_k<D>();
    static_assert(NHF * NKK == VCH, "K and V buffers hold the same number of chunks");
    static_assert(ROWS == 16, "one 16-row block on the MFMA N axis");

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

    // Query row n of this kv head: head hk*G + n / Lq, position n % Lq, as the B
    // operand of k-step kk (head-dim elements 32kk + 8g4 .. + 8).  Rows past R are zero
    // (their results are never stored).
    typename E::vec8 qf[NKK];
    {
        const bool r_ok = n < R;
        const int hq = hk * G + (r_ok ? n / a.Lq : 0), iq = r_ok ? n % a.Lq : 0;
        const uint16_t* qr = (const uint16_t*)a.q + (int64_t)b * a.q_batch +
                             (int64_t)hq * a.q_head + (int64_t)iq * a.q_row + g4 * 8;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            u32x4 raw = {0u, 0u, 0u, 0u};
            if (r_ok) raw = load16(qr + kk * 32);
            qf[kk] = as_vec8<T>(raw);
        }
    }

    const uint16_t* kp = (const uint16_t*)a.k + (int64_t)b * a.kv_batch + (int64_t)hk * a.kv_head;
    const uint16_t* vp = (const uint16_t*)a.v + (int64_t)b * a.kv_batch + (int64_t)hk * a.kv_head;

    // Loads of one block into a register buffer, as streaming (nontemporal) loads:
    // every K/V byte is read once.  Rows past the range end are clamped to its last
    // key (real, finite data; the range is non-empty whenever a block exists) and
    // masked out of the softmax, so no load needs a branch.  A prefetch past the
    // wave's last block (`idle`) reads only the range's first key row: the same
    // instructions, so the wait counts stay the same, but no second pass over a block.
    typedef u32x4 KBuf[VCH];
    typedef u32x4 VBuf[VCH];
    auto load_block = [&](KBuf& kb_, VBuf& vb_, int blk, bool idle) {
        const int kb = j0 + blk * KPB;
        if constexpr (!KST) {
            // K in the operand layout: chunk hf*NKK + kk is k-step kk of keys 16hf + n
#pragma unroll
            for (int hf = 0; hf < NHF; ++hf) {
                const int j = idle ? j0 : min(kb + hf * 16 + n, j1 - 1);
                const uint16_t* kr = kp + (int64_t)j * a.kv_row + g4 * 8;
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) kb_[hf * NKK + kk] = load16_stream(kr + kk * 32);
            }
        }
#pragma unroll
        for (int u = 0; u < VCH; ++u) {
            const int c = lane + 64 * u;
            const int j = idle ? j0 : min(kb + c / CPR, j1 - 1);
            if constexpr (KST) kb_[u] = load16_stream(kp + (int64_t)j * a.kv_row + (c % CPR) * 8);
            vb_[u] = load16_stream(vp + (int64_t)j * a.kv_row + (c % CPR) * 8);
        }
    };

    f32x4 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x4{};
    float m_run = -INFINITY, l_run = 0.f;

    uint16_t* vl = (uint16_t*)smem + wave * KPB * VLD;
    uint16_t* kl = (uint16_t*)(smem + L::KOFF) + wave * KPB * KLD;  // used when KST
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
            if constexpr (KST) store16(kl + (c / CPR) * KLD + (c % CPR) * 8, kc[u]);
            store16(vl + (c / CPR) * VLD + (c % CPR) * 8, vc[u]);
        }
        lds_wave_sync();
        // S^T for keys [16hf, 16hf + 16) of the block: lane holds keys 16hf + 4g4 + i.
        f32x4 sv[NHF];
#pragma unroll
        for (int hf = 0; hf < NHF; ++hf) {
            sv[hf] = f32x4{};
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const u32x4 kop = KST ? load16(kl + (hf * 16 + n) * KLD + kk * 32 + g4 * 8)
                                      : kc[hf * NKK + kk];
                sv[hf] = E::mfma16(as_vec8<T>(kop), qf[kk], sv[hf]);
            }
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
        // The reference max m_run moves lazily, only when a block's max exceeds it by
        // more than kTau (so every p = 2^(s - m_run) <= 2^kTau): most blocks then leave
        // O and l as they are.
        const bool rescale = __any(mx > m_run + kTau);
        float alpha = 1.f;
        if (rescale) {
            const float m_new = mx > m_run + kTau ? mx : m_run;
            alpha = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
        }
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        // B operand: slot j <-> key 16(j/4) + 4g4 + j%4; with 16-key blocks the upper
        // four slots hold 0, so the 32-key MFMA step adds nothing for them.
        float p[8];
        float psum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[j] = (j >> 2) < NHF ? fast_exp2(sv[(j >> 2) % NHF][j & 3] - m_use) : 0.f;
            psum += p[j];
        }
        l_run += psum;
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
            if (rescale) o[db] *= alpha;
            o[db] = E::mfma16(as_vec8<T>(av), as_vec8<T>(pb), o[db]);
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
    {
        float l = l_run;
        l += xor_shfl(l, 16);
        l += xor_shfl(l, 32);
        if (g4 == 0) {
            cm[wave * ROWS + n] = m_run;
            cl[wave * ROWS + n] = l;
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            *reinterpret_cast<f32x4*>(&co[(wave * ROWS + n) * OLD + db * 16 + g4 * 4]) = o[db];
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
    if constexpr (FUSED) merge_tail<T, D, 1>(a, b, hk, R, G);
}

template <typename T, int D>
hipError_t launch_splitkv_d(const SplitArgs& a, bool fused, dim3 grid, hipStream_t st) {
    if (fused)
        hipLaunchKernelGGL((splitkv_kernel<T, D, true>), grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((splitkv_kernel<T, D, false>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_splitkv_t(const SplitArgs& a, int D, bool fused, dim3 grid, hipStream_t st) {
    switch (D) {
        case 64: return launch_splitkv_d<T, 64>(a, fused, grid, st);
        case 128: return launch_splitkv_d<T, 128>(a, fused, grid, st);
        case 256: return launch_splitkv_d<T, 256>(a, fused, grid, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int splitkv_max_rows(int D) { return D == 256 ? 16 : 64; }

hipError_t launch_splitkv(const SplitArgs& a, int dtype, int D, bool fused, hipStream_t stream) {
    // one work group per group of `group` consecutive chunks (group = 1 unless fused)
    const int parts = (a.num_splits + a.group - 1) / a.group;
    const dim3 grid((unsigned)parts, (unsigned)a.Hkv, (unsigned)a.B);
    // more than 16 query rows per kv head (D <= 128): the 32-row-block kernel
    if ((a.Hq / a.Hkv) * a.Lq > 16) return launch_splitkv_wide(a, dtype, D, fused, grid, stream);
    if (dtype == 0) return launch_splitkv_t<__bf16>(a, D, fused, grid, stream);
    return launch_splitkv_t<_Float16>(a, D, fused, grid, stream);
}

}  // namespace skv
