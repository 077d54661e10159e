// sage_fwd.hip -- attention forward with INT8 QK^T and half-precision P.V, one log2
// LSE per query row on the unsmoothed logits.
//
// The INT8 variants of the ARK return_lse report (auto-round #2556, task statement;
// Reproduction Steps, the apis table: ark.sagev1 and
// ark.sageattn(kernel="v1_pvhalf")) must return the LSE of the original logits
// log2 sum_j exp(scale q_i . k_j), also with smooth_k on, where the term
// scale * q_i . mean(k) removed by smoothing is added back (Problem Description,
// second issue; Reproduction Steps part 3).  Inputs come from sage_quant.hip:
// per-block INT8 codes of q and of k - mean(k), their float32 scales, the per-row
// add-back in log2 units and V in fp16.
//
// Design (gfx950, wave64), the structure of fmha_fwd.hip with INT8 logits:
//   * work group = 8 waves = 256 query rows; wave w owns one 32-row block, which is
//     exactly one quantisation block of Q, so its scale is one scalar per wave.
//   * S^T = K Q^T on v_mfma_i32_32x32x32_i8 (keys on M, query rows on the lane
//     axis): D / 32 MFMAs per 32 x 32 block, half the count of the 16-bit path.
//     Each 32-key block of a tile is one quantisation block of K.
//   * The int32 accumulators start at 0x4B400000 (the float 1.5 * 2^23), so the
//     finished sum x reads as the float 1.5 * 2^23 + x exactly (|x| <= 127^2 D <
//     2^22): no conversion instruction per logit.  The constant and both scales
//     fold into the exp2 argument, fma(f, c_j, nb_j) with
//     c_j = scale log2(e) dQ dK_j and nb_j = -(1.5 * 2^23 c_j + m_ref); the add-back
//     c q . mean(k) enters only the LSE.
//   * Online softmax, lazy rescale, P packed to fp16 as the B operand of
//     O^T += V^T P^T on v_mfma_f32_32x32x16_f16 (V^T by ds_read_b64_tr_b16), the row
//     sum taken on the packed P, exactly as in the 16-bit kernel.
#include "device.h"
#include "launch.h"

namespace skv {

namespace {

template <bool B> struct BoolC {
    static constexpr bool value = B;
};

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

template <int D> struct SageTile {
    static constexpr int NW = 8;
    static constexpr int NT = 64 * NW;
    static constexpr int BM = 32 * NW;
    static constexpr int BN = D == 64 ? 128 : 64;
    static constexpr int KLD = D + 16;             // K row pitch in LDS (bytes)
    static constexpr int VLD = D + 32;             // V row pitch in LDS (fp16 elements)
    static constexpr int KCH = BN * D / 16 / NT;   // 16-byte K chunks per thread per tile
    static constexpr int VCH = BN * D / 8 / NT;    // 16-byte V chunks per thread per tile
    static constexpr int OLD = D + 8;              // O row pitch in a wave's slice (elements)
};

constexpr int kMagic = 0x4B400000;                 // bit pattern of 1.5 * 2^23
constexpr float kMagicF = 12582912.f;

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(SageTile<D>::NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sage_fwd_kernel(SageFwdArgs a) {
    using EO = Elem<T>;            // output type
    using EV = Elem<_Float16>;     // P and V
    typedef SageTile<D> Tl;
    constexpr int BM = Tl::BM, BN = Tl::BN, KLD = Tl::KLD, VLD = Tl::VLD;
    constexpr int NKK = D / 32;    // INT8 MFMA k-steps over the head dimension
    constexpr int NJB = BN / 32;   // 32-key blocks per tile
    constexpr int NDB = D / 32;    // 32-wide blocks of the output head dimension
    constexpr int KCPR = D / 16;   // 16-byte chunks per K row (int8)
    constexpr int VCPR = D / 8;    // 16-byte chunks per V row (fp16)

    __shared__ __attribute__((aligned(16))) int8_t k_lds[2][BN * KLD];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][BN * VLD];
    // One slice per wave: its 32 rows of Q codes on the way in (pitch KLD bytes, the
    // conflict-free pattern of the K reads), of O on the way out (pitch OLD).
    __shared__ __attribute__((aligned(16))) uint16_t qo_lds[Tl::NW][32 * Tl::OLD];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int n = lane & 31, hg = lane >> 5;
    // grid (head, batch, row tile), head-fastest, causal row tiles last-first; with
    // Hq a multiple of 8 each XCD takes a contiguous block of Hq/8 heads, so the query
    // heads of one K/V head share an L2
    const int h = (a.Hq & 7) ? (int)blockIdx.x
                             : (int)(blockIdx.x & 7) * (a.Hq >> 3) + (int)(blockIdx.x >> 3);
    const int b = blockIdx.y;
    const int mt = CAUSAL ? (int)(gridDim.z - 1 - blockIdx.z) : (int)blockIdx.z;
    const int Lq = a.Sq, Lk = a.Sk;
    const int m0 = mt * BM;
    if (m0 >= Lq) return;

    const int g = h / (a.Hq / a.Hkv);
    const int64_t bh = (int64_t)b * a.Hq + h, bg = (int64_t)b * a.Hkv + g;
    const int nq = (Lq + 31) / 32, nk = (Lk + 31) / 32;
    const int8_t* kc = a.k_codes + bg * Lk * D;
    const float* ksc = a.k_scale + bg * nk;
    const uint16_t* vp = a.v + (int64_t)b * a.v_batch + (int64_t)g * a.v_head;

    const int rblk = wave >= 4 ? 11 - wave : wave;   // mirrored blocks per SIMD
    const int wrow0 = m0 + rblk * 32;
    const int row = wrow0 + n;
    const bool row_ok = row < Lq;

    // The wave's 32 rows of Q codes come in, and its 32 rows of O go out, in whole
    // rows through its LDS slice: consecutive lanes take consecutive 16-byte chunks
    // of a row, so each instruction covers 1 KB of rows.  Rows past the end read the
    // last row (finite codes whose results are never stored).
    uint16_t* qs = qo_lds[wave];
    int8_t* qsb = reinterpret_cast<int8_t*>(qs);
    constexpr int QCPR = D / 16, QRPC = 64 / QCPR, QCH = 32 / QRPC;  // Q code chunks
    {
        const int lr = lane / QCPR, lc = (lane % QCPR) * 16;
        const int8_t* qb = a.q_codes + bh * Lq * D + lc;
        u32x4 qraw[QCH];
#pragma unroll
        for (int c = 0; c < QCH; ++c)
            qraw[c] = load16(qb + (int64_t)min(wrow0 + c * QRPC + lr, Lq - 1) * D);
#pragma unroll
        for (int c = 0; c < QCH; ++c) store16(qsb + (c * QRPC + lr) * KLD + lc, qraw[c]);
    }
    // Q codes as the B operand: lane holds q^[row][hg*D/2 + 16kk .. +16) per k-step
    // (a wave's LDS accesses complete in order).
    // With a negative scale the operand is -q^ (codes lie in [-127, 127], so each
    // byte negates exactly) and the logit scale |scale|: the raw integer dot products
    // keep the order of the logits.
    i32x4 qf[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        u32x4 w = load16(qsb + n * KLD + hg * (D / 2) + kk * 16);
        if (a.negate_q) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // bytewise 0 - x: ~x + 1 per byte, the carry kept inside each byte
                const uint32_t nx = ~w[e];
                w[e] = ((nx & 0x7f7f7f7fu) + 0x01010101u) ^ (nx & 0x80808080u);
            }
        }
        qf[kk] = __builtin_bit_cast(i32x4, w);
    }
    const float cq = wrow0 < Lq ? a.scale_log2 * a.q_scale[bh * nq + wrow0 / 32] : 0.f;
    const float bias = (a.q_bias && row_ok) ? a.q_bias[bh * Lq + row] : 0.f;

    int kv_end = Lk;
    if (CAUSAL) kv_end = min(Lk, m0 + BM + Lk - Lq);
    const int ntiles = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
    const int diag = Lk - Lq;
    int first_masked = Lk / BN;
    if (CAUSAL) first_masked = min(first_masked, max(0, (m0 + diag + 1) / BN));
    int wave_tiles = ntiles;
    if (wrow0 >= Lq)
        wave_tiles = 0;
    else if (CAUSAL)
        wave_tiles = min(ntiles, max(0, (min(wrow0 + 31, Lq - 1) + diag + BN) / BN));

    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
    constexpr float kTau = 8.f;
    float m_ref = -INFINITY, l_run = 0.f;

    // Tile staging: K chunk ci of this thread is key ch / KCPR, byte (ch % KCPR) * 16;
    // V chunk likewise with VCPR.  Rows past the last key are clamped to it in masked
    // tiles (finite data, masked out of the softmax).
    u32x4 kr[Tl::KCH], vr[Tl::VCH];
    auto load_tile = [&](int t, bool clamp) {
        const int kb0 = t * BN;
#pragma unroll
        for (int ci = 0; ci < Tl::KCH; ++ci) {
            const int ch = tid + ci * Tl::NT;
            int key = ch / KCPR;
            if (clamp) key = min(key, Lk - 1 - kb0);
            kr[ci] = load16(kc + (int64_t)(kb0 + key) * D + (ch % KCPR) * 16);
        }
        const uint16_t* vt = vp + (int64_t)kb0 * a.v_row;
#pragma unroll
        for (int ci = 0; ci < Tl::VCH; ++ci) {
            const int ch = tid + ci * Tl::NT;
            int key = ch / VCPR;
            if (clamp) key = min(key, Lk - 1 - kb0);
            vr[ci] = load16(vt + (int64_t)key * a.v_row + (ch % VCPR) * 8);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int ci = 0; ci < Tl::KCH; ++ci) {
            const int ch = tid + ci * Tl::NT;
            store16(&k_lds[buf][(ch / KCPR) * KLD + (ch % KCPR) * 16], kr[ci]);
        }
#pragma unroll
        for (int ci = 0; ci < Tl::VCH; ++ci) {
            const int ch = tid + ci * Tl::NT;
            store16(&v_lds[buf][(ch / VCPR) * VLD + (ch % VCPR) * 8], vr[ci]);
        }
    };
    const int full_tiles = Lk / BN;
    const int g16 = lane >> 4, e4 = (lane & 15) >> 2, q4 = lane & 3;

    auto process = [&](int t, auto mask_c) {
        constexpr bool MASK = decltype(mask_c)::value;
        const int buf = t & 1;
        if (!MASK || t < wave_tiles) {
            u32x4 kop[NJB][NKK];
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                const int8_t* kr0 = &k_lds[buf][(jb * 32 + n) * KLD + hg * (D / 2)];
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) kop[jb][kk] = load16(kr0 + kk * 16);
            }
            // dequantisation factor of each 32-key block (uniform over the wave)
            float cj[NJB];
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
                cj[jb] = fmaxf(cq * ksc[min(t * NJB + jb, nk - 1)], 1.17549435e-38f);
            i32x16 si[NJB];
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                for (int i = 0; i < 16; ++i) si[jb][i] = kMagic;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb)
                    si[jb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                        __builtin_bit_cast(i32x4, kop[jb][kk]), qf[kk], si[jb], 0, 0, 0);
            u32x4 vop[NDB][NJB][2];
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
                        const int key0 = jb * 32 + 16 * st + 4 * (g16 >> 1) + e4;
                        const int col = db * 32 + (g16 & 1) * 16 + 4 * q4;
                        const u32x2 lo = lds_read_tr16(&v_lds[buf][key0 * VLD + col]);
                        const u32x2 hi = lds_read_tr16(&v_lds[buf][(key0 + 8) * VLD + col]);
                        vop[db][jb][st] = u32x4{lo.x, lo.y, hi.x, hi.y};
                    }
            __builtin_amdgcn_sched_group_barrier(0x100, NJB * NKK, 0);  // K reads
#pragma unroll
            for (int i = 0; i < NJB * NKK; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // one QK MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * NDB * NJB * 2 / (NJB * NKK), 0);
            }
            f32x16 s[NJB];
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) s[jb] = __builtin_bit_cast(f32x16, si[jb]);
            if constexpr (MASK) {
                const int kbase = t * BN;
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = kbase + jb * 32 + 8 * (i >> 2) + hg * 4 + (i & 3);
                        bool ok = key < Lk;
                        if (CAUSAL) ok = ok && key <= row + diag;
                        s[jb][i] = ok ? s[jb][i] : -INFINITY;
                    }
            }
            // tile max in log2 units: max over blocks of (max f - 1.5*2^23) * c_j
            float mx = -INFINITY;
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                float mj = -INFINITY;
#pragma unroll
                for (int i = 0; i < 16; ++i) mj = fmaxf(mj, s[jb][i]);
                // (c_j = 0 for an all-zero K block: its logits are 0, not NaN)
                mx = fmaxf(mx, mj == -INFINITY ? -INFINITY : (mj - kMagicF) * cj[jb]);
            }
            mx = fmaxf(mx, xor_shfl(mx, 32));
            // (the codes are of k - mean(k): these logits are already the smoothed ones)
            const float m_tile = mx;
            if (__any(m_tile > m_ref + kTau)) {
                const float m_new = m_tile > m_ref + kTau ? m_tile : m_ref;
                const float alpha = m_ref == -INFINITY ? 0.f : fast_exp2(m_ref - m_new);
                m_ref = m_new;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db) o[db] *= alpha;
            }
            const float nb0 = m_ref == -INFINITY ? 0.f : -m_ref;

            uint32_t pk[NJB][2][4];
            float psum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                const float nb = fmaf(-kMagicF, cj[jb], nb0);
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        // masked logits give p = 0 also when c_j = 0 (an all-zero K
                        // block, or scale 0)
                        const float x0 = s[jb][8 * st + 2 * j], x1 = s[jb][8 * st + 2 * j + 1];
                        float y0 = fmaf(x0, cj[jb], nb), y1 = fmaf(x1, cj[jb], nb);
                        if (MASK) {
                            y0 = x0 == -INFINITY ? -INFINITY : y0;
                            y1 = x1 == -INFINITY ? -INFINITY : y1;
                        }
                        const float p0 = fast_exp2(y0);
                        const float p1 = fast_exp2(y1);
                        pk[jb][st][j] = EV::pack2(p0, p1);
                        psum[j] = EV::sum2(pk[jb][st][j], psum[j]);
                    }
            }
            l_run += (psum[0] + psum[1]) + (psum[2] + psum[3]);

#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
                        const u32x4 bv = {pk[jb][st][0], pk[jb][st][1], pk[jb][st][2],
                                          pk[jb][st][3]};
                        o[db] = EV::mfma32(as_vec8<_Float16>(vop[db][jb][st]),
                                           as_vec8<_Float16>(bv), o[db]);
                    }
        }
        if (t + 1 < ntiles) {
            store_tile(buf ^ 1);
            if (t + 2 < ntiles) load_tile(t + 2, t + 2 >= full_tiles);
        }
        __syncthreads();
    };

    if (ntiles > 0) {
        load_tile(0, 0 >= full_tiles);
        store_tile(0);
    }
    // Every load so far has landed on every path into the loop, so the compiler's
    // wait counts inside it cover only the tile loads in flight.
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    if (ntiles > 1) load_tile(1, 1 >= full_tiles);
    __syncthreads();
    const int nfree = min(first_masked, ntiles);
    int t = 0;
    for (; t < nfree; ++t) process(t, BoolC<false>{});
    for (; t < ntiles; ++t) process(t, BoolC<true>{});

    const float l_tot = l_run + xor_shfl(l_run, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    // O^T columns into the slice as rows, then out in whole rows.
    constexpr int OLD = Tl::OLD, OCPR = D / 8, ORPC = 64 / OCPR, OCH = 32 / ORPC;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
            const int d = db * 32 + 8 * a4 + hg * 4;
            u32x2 w;
            w.x = EO::pack2(o[db][4 * a4 + 0] * inv, o[db][4 * a4 + 1] * inv);
            w.y = EO::pack2(o[db][4 * a4 + 2] * inv, o[db][4 * a4 + 3] * inv);
            *reinterpret_cast<u32x2*>(&qs[n * OLD + d]) = w;
        }
    const int lr = lane / OCPR, lc = (lane % OCPR) * 8;
    uint16_t* const op = (uint16_t*)a.out + (int64_t)b * a.o_batch + (int64_t)h * a.o_head +
                         (int64_t)(wrow0 + lr) * a.o_row + lc;
    const int rows_left = Lq - wrow0 - lr;  // this lane's rows c * ORPC below it exist
#pragma unroll
    for (int c = 0; c < OCH; ++c) {
        const u32x4 w = load16(qs + (c * ORPC + lr) * OLD + lc);
        if (c * ORPC < rows_left) store16(op + (int64_t)c * ORPC * a.o_row, w);
    }
    if (row_ok && hg == 0 && a.lse)
        a.lse[bh * Lq + row] = l_tot > 0.f ? m_ref + fast_log2(l_tot) + bias : -INFINITY;
}

template <typename T, int D>
hipError_t launch_sage_t(const SageFwdArgs& a, bool causal, dim3 grid, hipStream_t st) {
    const dim3 block(SageTile<D>::NT);
    if (causal)
        hipLaunchKernelGGL((sage_fwd_kernel<T, D, true>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((sage_fwd_kernel<T, D, false>), grid, block, 0, st, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_sage_d(const SageFwdArgs& a, int D, bool causal, dim3 grid, hipStream_t st) {
    switch (D) {
        case 64: return launch_sage_t<T, 64>(a, causal, grid, st);
        case 128: return launch_sage_t<T, 128>(a, causal, grid, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int sage_rows_per_block() { return SageTile<128>::BM; }

hipError_t launch_sage_fwd(const SageFwdArgs& a, int dtype, int D, bool causal, int grid_m,
                           int grid_b, hipStream_t stream) {
    const dim3 grid((unsigned)a.Hq, (unsigned)grid_b, (unsigned)grid_m);
    if (dtype == 0) return launch_sage_d<__bf16>(a, D, causal, grid, stream);
    return launch_sage_d<_Float16>(a, D, causal, grid, stream);
}

}  // namespace skv
