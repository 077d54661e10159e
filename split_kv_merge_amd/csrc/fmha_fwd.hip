// fmha_fwd.hip -- fused attention forward with one log2 LSE per query row.
//
// Computes, per query row i, out_i = softmax_j(scale q_i . k_j) V and
// LSE_i = log2 sum_j exp(scale q_i . k_j) on the unsmoothed logits (auto-round
// #2556 "ARK return_lse gives the same LSE for every 16 query rows", task
// statement and Problem Description).  Optional smoothing subtracts
// scale * q_i . mean(k) from every logit of row i and adds it back in the LSE
// (same report, second issue; Reproduction Steps part 3).
//
// Design (gfx950, wave64):
//   * work group = 8 waves = 256 query rows (4 waves = 128 rows for D = 256);
//     each wave owns one block of 32 rows.  All waves of a compute unit share one
//     staged K/V tile, so each tile is loaded and written to LDS once per 256
//     rows rather than once per 128.
//   * S^T = K Q^T on v_mfma_f32_32x32x16 with keys on the M axis and query rows on
//     the N (lane) axis, so every lane owns exactly one query row: its running
//     max and sum live in that lane (plus its partner lane^32), and the LSE
//     epilogue stores one value per row from one lane -- the per-row ownership the
//     report's 16-row-block bug lacked.
//   * Q stays in registers as the B operand for the whole key loop; it arrives, and
//     the output leaves, through a 32-row LDS slice per wave, so that global loads
//     and stores cover whole rows.  K and V tiles are staged global -> registers ->
//     LDS (the next tile's loads are in flight while the current one is computed).
//   * The C layout of S^T is reused directly as the B operand of O^T += V^T P^T;
//     the key order inside P is permuted and V^T is read from LDS with
//     ds_read_b64_tr_b16 in the matching permuted order (a sum over keys does not
//     care about their order).
//   * Online softmax in base 2: logits are scaled by scale*log2(e) with one
//     multiply, p = exp2(s - m) (v_exp_f32), all statistics in fp32 registers.
#include "device.h"
#include "launch.h"

namespace skv {

namespace {

template <bool B> struct BoolC {
    static constexpr bool value = B;
};

template <int D> struct FmhaTile {
    // Waves per work group: two per SIMD.  At D = 256 a wave needs the whole
    // 512-register file, so only one fits per SIMD.
    static constexpr int NW = D == 256 ? 4 : 8;
    static constexpr int NT = 64 * NW;             // threads per work group
    static constexpr int BM = 32 * NW;             // query rows per work group
    // keys per tile: 128 at D = 64, where the softmax work per key is largest
    // relative to the MFMA work and fewer, longer tiles give it more independence
    static constexpr int BN = D == 256 ? 32 : (D == 64 ? 128 : 64);
    static constexpr int KLD = D + 8;              // K row pitch in LDS (elements)
    // V row pitch in LDS (elements): 16 dwords past a multiple of 64 banks, so each
    // 32-lane pass of the transpose read (4 rows x 2 column groups x 4 lanes x 2
    // dwords) touches all 64 banks once.
    static constexpr int VLD = D + 32;
    static constexpr int NCH = BN * D / 8 / NT;    // 16-byte chunks per thread per tile
    // Row pitch (elements) of each wave's Q / O staging slice: the operand reads of
    // Q use the conflict-free pattern of the K reads.
    static constexpr int QLD = D + 8;
};

template <typename T, int D, bool CAUSAL, bool VARLEN>
// One work group per compute unit (two waves per SIMD, one at D = 256); telling the
// compiler so lets it spend up to 256 (512) registers on keeping loads ahead of the
// MFMAs instead of squeezing for an occupancy the work-group size cannot reach.
__global__ __launch_bounds__(FmhaTile<D>::NT) __attribute__((amdgpu_waves_per_eu(D == 256 ? 1 : 2, D == 256 ? 1 : 2)))
void fmha_fwd_kernel(FmhaArgs a) {
    using E = Elem<T>;
    typedef typename E::vec8 V8;
    typedef FmhaTile<D> Tl;
    constexpr int BM = Tl::BM, BN = Tl::BN, KLD = Tl::KLD, VLD = Tl::VLD, NCH = Tl::NCH;
    constexpr int QLD = Tl::QLD;
    constexpr int NKK = D / 16;   // MFMA k-steps over the head dimension
    constexpr int NJB = BN / 32;  // 32-key blocks per tile
    constexpr int NDB = D / 32;   // 32-wide blocks of the output head dimension
    constexpr int CPR = D / 8;    // 16-byte chunks per K/V row

    __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][BN * KLD];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][BN * VLD];
    // One slice per wave: its 32 rows of Q on the way in, of O on the way out.
    __shared__ __attribute__((aligned(16))) uint16_t qo_lds[Tl::NW][32 * QLD];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int n = lane & 31, hg = lane >> 5;
    // Grid (head, batch | sequence, row tile), dispatched head-fastest: with causal
    // masking the row tiles run last-first, so the work groups go out in order of
    // decreasing work (a row tile's key count grows with its index) across every
    // head and sequence, and none of the long ones trails the grid.  Work groups are
    // dealt to the 8 XCDs round-robin, so head slot x lands on XCD x % 8; when Hq is
    // a multiple of 8, XCD x takes the contiguous heads x Hq/8 .. (x + 1) Hq/8 - 1,
    // and the query heads that share a K/V head (GQA) share one L2, where they read
    // the same tiles at about the same time (varlen causal prefill: -2 %).
    const int h = (a.Hq & 7) ? (int)blockIdx.x
                             : (int)(blockIdx.x & 7) * (a.Hq >> 3) + (int)(blockIdx.x >> 3);
    const int b = blockIdx.y;
    const int mt = CAUSAL ? (int)(gridDim.z - 1 - blockIdx.z) : (int)blockIdx.z;

    int Lq, Lk;
    int64_t q_off, kv_off, lse_off;
    if (VARLEN) {
        const int q0 = a.cu_q[b], k0 = a.cu_k[b];
        Lq = a.cu_q[b + 1] - q0;
        Lk = a.cu_k[b + 1] - k0;
        q_off = (int64_t)q0 * a.q_row;
        kv_off = (int64_t)k0 * a.kv_row;
        lse_off = q0;
    } else {
        Lq = a.Sq;
        Lk = a.Sk;
        q_off = (int64_t)b * a.q_batch;
        kv_off = (int64_t)b * a.kv_batch;
        lse_off = (int64_t)b * a.lse_batch;
    }
    const int m0 = mt * BM;
    if (m0 >= Lq) return;  // uniform across the work group

    const int g = h / (a.Hq / a.Hkv);
    const uint16_t* qp = (const uint16_t*)a.q + q_off + (int64_t)h * a.q_head;
    const uint16_t* kp = (const uint16_t*)a.k + kv_off + (int64_t)g * a.kv_head;
    const uint16_t* vp = (const uint16_t*)a.v + kv_off + (int64_t)g * a.kv_head;

    // Row block of this wave.  The two waves sharing a SIMD (w and w + 4) take
    // mirrored blocks (w and 7 - w), so in the causal diagonal band, where later
    // blocks see more keys, every SIMD carries about the same work.
    const int rblk = (Tl::NW == 8 && wave >= 4) ? 11 - wave : wave;
    const int wrow0 = m0 + rblk * 32;
    const int row = wrow0 + n;
    const bool row_ok = row < Lq;

    // The wave's 32 rows of Q and O move between global memory and its LDS slice
    // in whole rows: chunk c of a lane is the 16-byte chunk c * 64 + lane of the
    // slice, so consecutive lanes cover consecutive bytes of a row (one load or store
    // instruction spans 1 KB of rows instead of 64 scattered pieces).
    constexpr int QCH = 32 * CPR / 64;  // 16-byte chunks per lane
    constexpr int RPC = 64 / CPR;       // rows per chunk step
    const int lrow = lane / CPR, lcol = (lane % CPR) * 8;
    uint16_t* qs = qo_lds[wave];
    uint16_t* const qsl = qs + lrow * QLD + lcol;  // chunk c of this lane: qsl + c * RPC * QLD
    // mean(k) of this (batch | sequence, kv head) for the smoothing bias, this lane's
    // half of D, requested together with Q so the prologue waits for one memory round
    // trip.  Without smoothing the descriptor has length 0: the loads return zeros
    // without a memory access, and the bias below is 0.
    f32x4 kbv[NKK * 2];
    {
        const bool sm = a.kbar != nullptr;
        const __amdgpu_buffer_rsrc_t kbr = __builtin_amdgcn_make_buffer_rsrc(
            sm ? (void*)(a.kbar + ((int64_t)b * a.Hkv + g) * D) : (void*)a.q, (short)0,
            sm ? D * 4 : 0, kBufferRsrcWord3);
#pragma unroll
        for (int i = 0; i < NKK * 2; ++i)
            kbv[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   kbr, (hg * (D / 2) + 4 * i) * 4, 0, 0));
    }
    // Q rows past the end read the last row: finite data whose results are never stored.
    u32x4 qraw[QCH];
#pragma unroll
    for (int c = 0; c < QCH; ++c)
        qraw[c] = load16(qp + (int64_t)min(wrow0 + c * RPC + lrow, Lq - 1) * a.q_row + lcol);

    // Keys this tile of rows can see.
    int kv_end = Lk;
    if (CAUSAL) kv_end = min(Lk, m0 + BM + Lk - Lq);
    const int ntiles = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
    const int diag = Lk - Lq;  // row i sees keys j <= i + diag
    // Tiles from this index on need a mask (the key tail, or the causal diagonal of
    // the work group's first row); the ones before it are used whole.
    int first_masked = Lk / BN;
    if (CAUSAL) first_masked = min(first_masked, max(0, (m0 + diag + 1) / BN));
    // Masked tiles this wave computes.  A tile entirely past the causal diagonal of
    // the wave's last row, or any tile of a wave whose rows all lie past Lq, would
    // only add masked (-inf) logits -- exactly nothing -- so the wave skips its math
    // there (it still stages tiles and joins every barrier).
    const bool wave_live = wrow0 < Lq;
    int wave_tiles = ntiles;
    if (wrow0 >= Lq)
        wave_tiles = 0;
    else if (CAUSAL)
        wave_tiles = min(ntiles, max(0, (min(wrow0 + 31, Lq - 1) + diag + BN) / BN));

    // K/V tile loads: chunk ci of this thread is key ch / CPR, column (ch % CPR) * 8,
    // ch = tid + NT ci; its offset inside a tile is a 32-bit constant and the tile
    // base is uniform.  In masked tiles, rows past the last key are clamped to it
    // (real, finite data; a tile exists only when Lk > 0) and masked out of the
    // softmax, so no load needs a branch.
    int koff[NCH];
#pragma unroll
    for (int ci = 0; ci < NCH; ++ci) {
        const int ch = tid + ci * Tl::NT;
        koff[ci] = (ch / CPR) * (int)a.kv_row + (ch % CPR) * 8;
    }
    u32x4 kr[NCH], vr[NCH];
    auto load_tile = [&](int t, bool clamp) {
        const int64_t tb = (int64_t)t * BN * a.kv_row;
        const uint16_t* kt = kp + tb;
        const uint16_t* vt = vp + tb;
#pragma unroll
        for (int ci = 0; ci < NCH; ++ci) {
            int off = koff[ci];
            if (clamp) {
                const int ch = tid + ci * Tl::NT;
                const int key = min(ch / CPR, Lk - 1 - t * BN);
                off = key * (int)a.kv_row + (ch % CPR) * 8;
            }
            kr[ci] = load16(kt + off);
            vr[ci] = load16(vt + off);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int ci = 0; ci < NCH; ++ci) {
            const int ch = tid + ci * Tl::NT;
            const int key = ch / CPR, col = (ch % CPR) * 8;
            store16(&k_lds[buf][key * KLD + col], kr[ci]);
            store16(&v_lds[buf][key * VLD + col], vr[ci]);
        }
    };
    const int full_tiles = Lk / BN;  // tiles with no key past the end

    // The first tile's loads go out while Q is still in flight.
    if (ntiles > 0) load_tile(0, 0 >= full_tiles);

    // Q as the B operand: this lane holds q[row][hg*D/2 + 8kk .. +8) for each k-step,
    // read back from the slice (a wave's LDS accesses complete in order).
#pragma unroll
    for (int c = 0; c < QCH; ++c) store16(qsl + c * RPC * QLD, qraw[c]);
    // With a negative scale the operand is -q (a sign flip per element, exact) and the
    // logit scale |scale|, so the raw dot products keep the order of the logits.
    const uint32_t qsign = a.negate_q ? 0x80008000u : 0u;
    V8 qf[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
        qf[kk] = as_vec8<T>(load16(&qs[n * QLD + hg * (D / 2) + kk * 8]) ^ qsign);

    // Smoothing bias in log2 units: scale*log2(e) * (q_row . mean(k)) (0 without
    // smoothing: the mean reads as zeros).
    float bias;
    {
        float acc = 0.f;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            u32x4 raw = __builtin_bit_cast(u32x4, qf[kk]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = kk * 8 + 2 * j;   // element of this lane's half of D
                acc += E::to_float((uint16_t)(raw[j] & 0xffff)) * kbv[e / 4][e % 4];
                acc += E::to_float((uint16_t)(raw[j] >> 16)) * kbv[(e + 1) / 4][(e + 1) % 4];
            }
        }
        acc += xor_shfl(acc, 32);
        bias = acc * a.scale_log2;
    }

    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
    // Online softmax with a lazily moved reference max m_ref (log2 units, smoothed
    // logits): it only moves when a tile's max exceeds it by more than kTau, so most
    // tiles skip rescaling O and l.  Every p = 2^(s - m_ref) stays <= 2^kTau.
    constexpr float kTau = 8.f;
    float m_ref = -INFINITY, l_run = 0.f;
    // Logit scale, at least the smallest normal float: with scale 0 (or a denormal one)
    // s * c then shifts no logit by a representable amount (|s| * 2^-126 is far below
    // half an ulp of any logit that is not itself below 2^-100, whose 2^x rounds to 1
    // either way), and -inf * c is -inf, never NaN.
    const float c = fmaxf(a.scale_log2, 1.17549435e-38f);

    // Lane roles for the transpose read of V^T operands.
    const int g16 = lane >> 4, e4 = (lane & 15) >> 2, q4 = lane & 3;

    // One key tile: S^T = K Q^T, (mask,) online softmax, O^T += V^T P^T, then stage
    // the next tile.  MASK is a compile-time switch so unmasked tiles carry no mask
    // arithmetic.
    auto process = [&](int t, auto mask_c) {
        constexpr bool MASK = decltype(mask_c)::value;
        const int buf = t & 1;
        // (a wave whose rows all lie past the sequence end skips unmasked tiles too:
        // their results are never stored; the branch is uniform per wave.  Not at
        // D = 256, where the branch makes the instantiation spill.)
        if (MASK ? t < wave_tiles : (D > 128 || wave_live)) {
            // Operands from LDS, issued ahead of their MFMAs: the 16-byte K rows of
            // every k-step first, then the V^T transpose reads interleaved with the QK
            // MFMAs, so their latency hides behind the QK product and the softmax.
            u32x4 kop[NJB][NKK];
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                const uint16_t* kr0 = &k_lds[buf][(jb * 32 + n) * KLD + hg * (D / 2)];
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) kop[jb][kk] = load16(kr0 + kk * 8);
            }
            f32x16 s[NJB];
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) s[jb] = f32x16{};
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb)
                    s[jb] = E::mfma32(as_vec8<T>(kop[jb][kk]), qf[kk], s[jb]);
            // V^T operands: k-step st of block jb covers keys 16st + 8h + 4(lane/32) + e
            // for operand slots 4h + e (the order the C layout of S^T leaves P in).
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
            if constexpr (MASK && D <= 128) {
                // lane holds keys t*BN + 4hg + off, off = 32jb + 8(i/4) + i%4, of the
                // tile; the visible ones are those up to the row's last key (the key
                // tail and, causal, the diagonal), i.e. off <= lim: one compare with a
                // constant per logit
                int last = Lk - 1;
                if (CAUSAL) last = min(last, row + diag);
                const int lim = last - (t * BN + hg * 4);
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        s[jb][i] = jb * 32 + 8 * (i >> 2) + (i & 3) <= lim ? s[jb][i] : -INFINITY;
            }
            if constexpr (MASK && D > 128) {
                // (per-key indexes: the bound form above makes this instantiation spill)
                // lane holds keys 8(i/4) + 4hg + i%4 of each 32-key block
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
            float mx = -INFINITY;
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[jb][i]);
            mx = fmaxf(mx, xor_shfl(mx, 32));
            const float m_tile = mx == -INFINITY ? -INFINITY : mx * c - bias;
            if (__any(m_tile > m_ref + kTau)) {
                const float m_new = m_tile > m_ref + kTau ? m_tile : m_ref;
                const float alpha = m_ref == -INFINITY ? 0.f : fast_exp2(m_ref - m_new);
                m_ref = m_new;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db) o[db] *= alpha;
            }
            const float nb = -(bias + (m_ref == -INFINITY ? 0.f : m_ref));

            // p = 2^(s*c - bias - m_ref), packed to 16-bit as the B operand of PV.  The
            // row sum adds the packed (rounded) pairs with one dot2 against (1, 1): the
            // normaliser then sums exactly the P values the PV product uses.  Four
            // partial sums keep the dependent chains short.  c > 0, so a masked logit
            // (-inf) stays -inf and gives p = 0.
            auto logit = [&](float x) { return fmaf(x, c, nb); };
            uint32_t pk[NJB][2][4];
            float psum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float p0 = fast_exp2(logit(s[jb][8 * st + 2 * j]));
                        const float p1 = fast_exp2(logit(s[jb][8 * st + 2 * j + 1]));
                        pk[jb][st][j] = E::pack2(p0, p1);
                        psum[j] = E::sum2(pk[jb][st][j], psum[j]);
                    }
            l_run += (psum[0] + psum[1]) + (psum[2] + psum[3]);

            // O^T[d, row] += V^T[d, keys] P^T[keys, row]
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                    for (int st = 0; st < 2; ++st) {
                        const u32x4 bv = {pk[jb][st][0], pk[jb][st][1], pk[jb][st][2],
                                          pk[jb][st][3]};
                        o[db] = E::mfma32(as_vec8<T>(vop[db][jb][st]), as_vec8<T>(bv), o[db]);
                    }
        }
        if (t + 1 < ntiles) {
            store_tile(buf ^ 1);
            if (t + 2 < ntiles) load_tile(t + 2, t + 2 >= full_tiles);
        }
        __syncthreads();
    };

    // Two LDS buffers: tile t is computed from buffer t&1 while tile t+1 is stored
    // into the other one and tile t+2 is being loaded; one barrier per tile.
    if (ntiles > 0) store_tile(0);
    // Every load so far (Q, tile 0) has landed on every path into the loop, so the
    // compiler's wait counts inside it cover only the tile loads in flight.
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    if (ntiles > 1) load_tile(1, 1 >= full_tiles);
    __syncthreads();
    const int nfree = min(first_masked, ntiles);
    int t = 0;
    for (; t < nfree; ++t) process(t, BoolC<false>{});
    for (; t < ntiles; ++t) process(t, BoolC<true>{});

    // Epilogue: out = O / l; LSE = m_ref + log2(l) (+ smoothing bias), one store per row.
    const float l_tot = l_run + xor_shfl(l_run, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    // O^T columns into the slice as rows, then out in whole rows.
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
            const int d = db * 32 + 8 * a4 + hg * 4;
            u32x2 w;
            w.x = E::pack2(o[db][4 * a4 + 0] * inv, o[db][4 * a4 + 1] * inv);
            w.y = E::pack2(o[db][4 * a4 + 2] * inv, o[db][4 * a4 + 3] * inv);
            *reinterpret_cast<u32x2*>(&qs[n * QLD + d]) = w;
        }
    uint16_t* const op = (uint16_t*)a.out + q_off + (int64_t)h * a.q_head +
                         (int64_t)(wrow0 + lrow) * a.q_row + lcol;
    const int rows_left = Lq - wrow0 - lrow;  // this lane's rows c * RPC below it exist
#pragma unroll
    for (int c = 0; c < QCH; ++c) {
        const u32x4 w = load16(qsl + c * RPC * QLD);
        if (c * RPC < rows_left) store16(op + (int64_t)c * RPC * a.q_row, w);
    }
    if (row_ok && hg == 0 && a.lse)
        a.lse[lse_off + (int64_t)h * a.lse_head + row] =
            l_tot > 0.f ? m_ref + fast_log2(l_tot) + bias : -INFINITY;
}

template <typename T, int D>
hipError_t launch_fmha_t(const FmhaArgs& a, bool causal, bool varlen, dim3 grid, hipStream_t st) {
    const dim3 block(FmhaTile<D>::NT);
    if (causal) {
        if (varlen)
            hipLaunchKernelGGL((fmha_fwd_kernel<T, D, true, true>), grid, block, 0, st, a);
        else
            hipLaunchKernelGGL((fmha_fwd_kernel<T, D, true, false>), grid, block, 0, st, a);
    } else {
        if (varlen)
            hipLaunchKernelGGL((fmha_fwd_kernel<T, D, false, true>), grid, block, 0, st, a);
        else
            hipLaunchKernelGGL((fmha_fwd_kernel<T, D, false, false>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_fmha_d(const FmhaArgs& a, int D, bool causal, bool varlen, dim3 grid,
                         hipStream_t st) {
    switch (D) {
        case 64: return launch_fmha_t<T, 64>(a, causal, varlen, grid, st);
        case 128: return launch_fmha_t<T, 128>(a, causal, varlen, grid, st);
        case 256: return launch_fmha_t<T, 256>(a, causal, varlen, grid, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int fmha_rows_per_block(int D) {
    switch (D) {
        case 64: return FmhaTile<64>::BM;
        case 128: return FmhaTile<128>::BM;
        default: return FmhaTile<256>::BM;
    }
}

hipError_t launch_fmha(const FmhaArgs& a, int dtype, int D, bool causal, bool varlen, int grid_m,
                       int grid_b, hipStream_t stream) {
    const dim3 grid((unsigned)a.Hq, (unsigned)grid_b, (unsigned)grid_m);
    if (dtype == 0) return launch_fmha_d<__bf16>(a, D, causal, varlen, grid, stream);
    return launch_fmha_d<_Float16>(a, D, causal, varlen, grid, stream);
}

}  // namespace skv
