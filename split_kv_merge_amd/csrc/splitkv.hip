// splitkv.hip -- split-KV decode: per-chunk partial attention states.
//
// Each work group owns one (batch, kv head, chunk) and ALL query rows that read
// that kv head (G = Hq/Hkv heads x Lq rows, at most 16), so every K/V byte of the
// chunk is read from HBM exactly once.  Within the chunk, each wave keeps its own
// online-softmax state (running max in log2 units, running sum, unnormalised
// output) over an interleaved subset of 32-key blocks; the waves' states are then
// merged through LDS and the chunk's (out normalised by its own sum, log2 LSE) is
// written.  This is the stable per-split online softmax of ExecuTorch PR #22133
// "Prevent Voxtral NaNs in CUDA split-K attention" (description and Copilot
// overview); a chunk with no key still writes (0, -inf), so the partial buffers
// need no initialisation (reviewer item 3 of that PR).
//
// Per 32-key block and wave: S^T = K Q^T on two v_mfma_f32_16x16x32 tiles (keys on
// M, query rows on N), K fed straight from global memory in the operand layout
// (each lane loads D/4 contiguous elements of one key row); O^T += V^T P^T with
// V staged in a per-wave LDS slice and read back with ds_read_b64_tr_b16, the key
// order of P matching the C layout of S^T.
#include "device.h"
#include "launch.h"

namespace skv {

namespace {

constexpr int kWaves = 4;
constexpr int kKeysPerBlock = 32;

template <int D> struct SplitLds {
    static constexpr int VLD = D + 16;  // V pitch (elements) in the staging slice
    static constexpr int OLD = D + 4;   // pitch (floats) of the combine buffer
    static constexpr int STAGE = kWaves * kKeysPerBlock * VLD * 2;
    static constexpr int COMB = kWaves * (16 * OLD + 32) * 4;
    static constexpr int BYTES = STAGE > COMB ? STAGE : COMB;
};

template <typename T, int D>
__global__ __launch_bounds__(256) void splitkv_kernel(SplitArgs a) {
    using E = Elem<T>;
    typedef SplitLds<D> L;
    constexpr int NKK = D / 32;          // 16x16x32 k-steps over D
    constexpr int NDB = D / 16;          // 16-wide blocks of O^T
    constexpr int CPR = D / 8;           // 16-byte chunks per V row
    constexpr int VCH = kKeysPerBlock * CPR / 64;  // V chunks per lane per block
    constexpr int VLD = L::VLD, OLD = L::OLD;

    __shared__ __attribute__((aligned(16))) unsigned char smem[L::BYTES];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, g4 = lane >> 4;
    const int s = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    const int G = a.Hq / a.Hkv, R = G * a.Lq;

    // chunk [j0, j1) of this split
    const int64_t C = ((int64_t)a.Lkv + a.num_splits - 1) / a.num_splits;
    const int64_t j0l = min((int64_t)s * C, (int64_t)a.Lkv);
    const int j0 = (int)j0l;
    const int j1 = (int)min(j0l + C, (int64_t)a.Lkv);
    const int nblk = (j1 - j0 + kKeysPerBlock - 1) / kKeysPerBlock;

    // Query row n of this kv head: head hk*G + n / Lq, position n % Lq.
    const bool r_ok = n < R;
    const int hq = hk * G + (r_ok ? n / a.Lq : 0), iq = r_ok ? n % a.Lq : 0;
    typename E::vec8 qf[NKK];
    {
        const uint16_t* qr = (const uint16_t*)a.q + (int64_t)b * a.q_batch +
                             (int64_t)hq * a.q_head + (int64_t)iq * a.q_row + g4 * (D / 4);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            u32x4 raw = {0u, 0u, 0u, 0u};
            if (r_ok) raw = load16(qr + kk * 8);
            qf[kk] = as_vec8<T>(raw);
        }
    }

    const uint16_t* kp = (const uint16_t*)a.k + (int64_t)b * a.kv_batch + (int64_t)hk * a.kv_head;
    const uint16_t* vp = (const uint16_t*)a.v + (int64_t)b * a.kv_batch + (int64_t)hk * a.kv_head;

    u32x4 kreg[2][NKK], vreg[VCH];
    auto load_block = [&](int blk) {
        const int kb = j0 + blk * kKeysPerBlock;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int j = kb + hf * 16 + n;
            const uint16_t* kr = kp + (int64_t)j * a.kv_row + g4 * (D / 4);
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                u32x4 z = {0u, 0u, 0u, 0u};
                if (j < j1) z = load16(kr + kk * 8);
                kreg[hf][kk] = z;
            }
        }
#pragma unroll
        for (int u = 0; u < VCH; ++u) {
            const int c = lane + 64 * u;
            const int j = kb + c / CPR;
            u32x4 z = {0u, 0u, 0u, 0u};
            if (j < j1) z = load16(vp + (int64_t)j * a.kv_row + (c % CPR) * 8);
            vreg[u] = z;
        }
    };

    f32x4 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x4{};
    float m_run = -INFINITY, l_run = 0.f;

    uint16_t* vl = (uint16_t*)smem + wave * kKeysPerBlock * VLD;
    const int e4 = (lane & 15) >> 2, q4 = lane & 3;

    if (wave < nblk) load_block(wave);
    for (int blk = wave; blk < nblk; blk += kWaves) {
        u32x4 kc[2][NKK], vc[VCH];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) kc[hf][kk] = kreg[hf][kk];
#pragma unroll
        for (int u = 0; u < VCH; ++u) vc[u] = vreg[u];
        if (blk + kWaves < nblk) load_block(blk + kWaves);

        // S^T for keys [16hf, 16hf + 16) of the block: lane holds keys 16hf + 4g4 + i.
        f32x4 sv[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            sv[hf] = f32x4{};
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
                sv[hf] = E::mfma16(as_vec8<T>(kc[hf][kk]), qf[kk], sv[hf]);
        }
        const int kb = j0 + blk * kKeysPerBlock;
        float mx = -INFINITY;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = kb + hf * 16 + 4 * g4 + i;
                const float x = j < j1 ? sv[hf][i] * a.scale_log2 : -INFINITY;
                sv[hf][i] = x;
                mx = fmaxf(mx, x);
            }
        mx = fmaxf(mx, xor_shfl(mx, 16));
        mx = fmaxf(mx, xor_shfl(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        m_run = m_new;
        float p[8];
        float psum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[j] = fast_exp2(sv[j >> 2][j & 3] - m_use);
            psum += p[j];
        }
        l_run = l_run * alpha + psum;
        // B operand: slot j <-> key 16(j/4) + 4g4 + j%4
        const u32x4 pb = {E::pack2(p[0], p[1]), E::pack2(p[2], p[3]), E::pack2(p[4], p[5]),
                          E::pack2(p[6], p[7])};

        // stage V (32 keys x D) in this wave's LDS slice, then V^T operands by
        // transpose reads: slot 4h + e of lane (d, g4) is V[16h + 4g4 + e][d].
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int u = 0; u < VCH; ++u) {
            const int c = lane + 64 * u;
            store16(vl + (c / CPR) * VLD + (c % CPR) * 8, vc[u]);
        }
        lds_wave_sync();
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            o[db] *= alpha;
            const int key0 = 4 * g4 + e4, col = db * 16 + 4 * q4;
            const u32x2 lo = lds_read_tr16(vl + key0 * VLD + col);
            const u32x2 hi = lds_read_tr16(vl + (key0 + 16) * VLD + col);
            const u32x4 av = {lo.x, lo.y, hi.x, hi.y};
            o[db] = E::mfma16(as_vec8<T>(av), as_vec8<T>(pb), o[db]);
        }
        lds_wave_sync();
    }

    // The four lanes of a row hold disjoint keys: total their sums.
    l_run += xor_shfl(l_run, 16);
    l_run += xor_shfl(l_run, 32);

    // Merge the waves' states through LDS.
    __syncthreads();
    float* cm = (float*)smem;           // [kWaves][16] running max
    float* cl = cm + kWaves * 16;       // [kWaves][16] running sum
    float* co = cl + kWaves * 16;       // [kWaves][16][OLD] unnormalised output
    if (g4 == 0) {
        cm[wave * 16 + n] = m_run;
        cl[wave * 16 + n] = l_run;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
        *reinterpret_cast<f32x4*>(&co[(wave * 16 + n) * OLD + db * 16 + g4 * 4]) = o[db];
    __syncthreads();

    for (int it = tid; it < 16 * (D / 4); it += 256) {
        const int r = it / (D / 4), d = (it % (D / 4)) * 4;
        if (r >= R) break;  // rows are the slow index: every later item is padding too
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, cm[w * 16 + r]);
        const float Mu = M == -INFINITY ? 0.f : M;
        float Ls = 0.f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float wt = fast_exp2(cm[w * 16 + r] - Mu);
            Ls += cl[w * 16 + r] * wt;
            acc += *reinterpret_cast<const f32x4*>(&co[(w * 16 + r) * OLD + d]) * wt;
        }
        const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
        const int h = hk * G + r / a.Lq, i = r % a.Lq;
        float* op = a.out_part + (int64_t)s * a.part_stride + (int64_t)b * a.q_batch +
                    (int64_t)h * a.q_head + (int64_t)i * a.q_row + d;
        *reinterpret_cast<f32x4*>(op) = acc * inv;
        if (d == 0)
            a.lse_part[(((int64_t)s * a.B + b) * a.Hq + h) * a.Lq + i] =
                Ls > 0.f ? M + fast_log2(Ls) : -INFINITY;
    }
}

template <typename T>
hipError_t launch_splitkv_t(const SplitArgs& a, int D, hipStream_t st) {
    const dim3 grid((unsigned)a.num_splits, (unsigned)a.Hkv, (unsigned)a.B), block(256);
    switch (D) {
        case 64: hipLaunchKernelGGL((splitkv_kernel<T, 64>), grid, block, 0, st, a); break;
        case 128: hipLaunchKernelGGL((splitkv_kernel<T, 128>), grid, block, 0, st, a); break;
        case 256: hipLaunchKernelGGL((splitkv_kernel<T, 256>), grid, block, 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_splitkv(const SplitArgs& a, int dtype, int D, hipStream_t stream) {
    if (dtype == 0) return launch_splitkv_t<__bf16>(a, D, stream);
    return launch_splitkv_t<_Float16>(a, D, stream);
}

}  // namespace skv
