// kda_prepare.hip -- stage 1 of the chunk method: one "update card" per
// (batch row, head, chunk), all chunks in parallel.
//
// The pages name the card's contents -- forget gate, query/key
// normalisation, decay, intra-chunk correction matrix -- and say they are
// prepared ahead of the ordered stage [zuoshipin.com/article/18261 §四,
// FlashKDA paragraph].  The algebra is derived from the recurrence:
//
//   lambda = max(log_alpha, floor); gamma = inclusive cumsum of lambda over
//   the chunk, per key channel (the floor keeps e^{-gamma} <= e^{64|floor|},
//   the bf16-range argument of zuoshipin §二)
//   Qt = q^ e^gamma,  Kt = k^ e^gamma,  Kh = k^ e^-gamma,  Ke = k^ e^(gamma_C - gamma)
//   L  = strict_lower(Kt Kh^T) (the intra-chunk correction matrix),
//   P  = lower_incl(Qt Kh^T)
//   T  = (I + diag(beta) L)^-1,  M = T diag(beta),  Wk = M Kt,  Wv = M V
//
// One workgroup (4 waves) per chunk-head.  Phases:
//   A  coalesced loads (one wave-instruction = one token row), floored
//      log-decay, per-channel cumulative sum (serial in registers, then a
//      cross-group offset through LDS), q/k norms (wave reductions), decay
//      folding; Kt/Kh/Qt to LDS, Ke^T and e^gamma_C straight to the card
//   B  L and P on MFMA (10 lower tiles each)
//   C  Qt and P (staged in LDS) to the card; diag(beta) L to LDS in fp32
//   D  T by blocked substitution in fp32: 16x16 diagonal blocks by forward
//      substitution, off-diagonal blocks with fp32 MFMA; M = T diag(beta)
//   E  Wk and Wv on MFMA (block-lower-triangular T); Wv to the card in
//      accumulator order, Wk through LDS to the card in fragment order
// Qt, Ke^T, P and Wk leave in MFMA A-fragment order (Card, kda_common.hpp).
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

namespace {

__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// One transpose-reduce exchange over lanes l and l ^ (4*HALF): the lane with
// that bit clear keeps (and sums) values [0, HALF), the other [HALF, 2*HALF),
// each sending the half it gives up.  Values end in x[0..HALF).
template <int HALF>
__device__ __forceinline__ void tr_halve(float* x, float* y, int lane) {
    constexpr int m = 4 * HALF;
    const bool hi = (lane & m) != 0;
#pragma unroll
    for (int j = 0; j < HALF; ++j) {
        const float sx = hi ? x[j] : x[j + HALF], kx = hi ? x[j + HALF] : x[j];
        const float sy = hi ? y[j] : y[j + HALF], ky = hi ? y[j + HALF] : y[j];
        x[j] = kx + __shfl_xor(sx, m);
        y[j] = ky + __shfl_xor(sy, m);
    }
}

template <typename E, int DK>
struct PrepLds {
    static constexpr int C = kChunk;
    static constexpr int PAD = 16 / (int)sizeof(E);
    static constexpr int LDR = DK + PAD;   // row-major [C][DK] tiles
    static constexpr int LDT = C + PAD;    // transposed [DK][C] tiles and T
    static constexpr int LDA = C + 4;      // fp32 [C][C] correction matrix / T
    static constexpr size_t R0 = 0;
    static constexpr size_t R_ROWMAJOR = (size_t)C * LDR * sizeof(E);
    static constexpr size_t R_TRANS = (size_t)DK * LDT * sizeof(E);
    static constexpr size_t RSZ = R_ROWMAJOR > R_TRANS ? R_ROWMAJOR : R_TRANS;
    static constexpr size_t R1 = R0 + RSZ;
    static constexpr size_t R2 = R1 + RSZ;
    static constexpr size_t R2SZ = R_ROWMAJOR > (size_t)C * LDA * 4 ? R_ROWMAJOR : (size_t)C * LDA * 4;
    static constexpr size_t R4 = R2 + R2SZ;
    static constexpr size_t R4SZ = (size_t)C * LDT * sizeof(E);
    static constexpr int NG = kThreads / (DK / 2);
    static constexpr size_t TOT = R4 + R4SZ;                    // fp32 [NG][DK]
    static constexpr size_t BETA = TOT + (size_t)NG * DK * 4;   // fp32 [C]
    static constexpr size_t RQ = BETA + (size_t)C * 4;          // fp32 [C] 1/|q|
    static constexpr size_t RK = RQ + (size_t)C * 4;            // fp32 [C] 1/|k|
    static constexpr size_t BYTES = RK + (size_t)C * 4;
};

// two workgroups per CU with bf16 cards; the fp32 variant's LDS allows one
template <typename E, int DK>
__global__ __launch_bounds__(kThreads, sizeof(E) == 2 ? 2 : 1) void kda_prepare_kernel(PrepareArgs a) {
    using M = MM<E>;
    using CL = Card<E, DK>;
    using LY = PrepLds<E, DK>;
    constexpr int C = kChunk, KS = M::KS;
    constexpr int CP = DK / 2;          // channel pairs: one lane per pair
    constexpr int NG = kThreads / CP;   // token groups
    constexpr int TPG = C / NG;         // tokens per group
    constexpr int LDR = LY::LDR, LDT = LY::LDT, LDA = LY::LDA;
    constexpr int NT = DK / 16;         // 16-wide column tiles
    constexpr float kLog2e = 1.4426950408889634f;

    __shared__ __attribute__((aligned(16))) char lds[LY::BYTES];
    E* sKt = reinterpret_cast<E*>(lds + LY::R0);     // phase A-B: Kt row-major
    E* sKh = reinterpret_cast<E*>(lds + LY::R1);     // phase A-B: Kh row-major
    E* sQt = reinterpret_cast<E*>(lds + LY::R2);     // phase A-C: Qt row-major
    E* sKtT = reinterpret_cast<E*>(lds + LY::R0);    // phase C-E: Kt^T
    E* sVT = reinterpret_cast<E*>(lds + LY::R1);     // phase C-E: V^T
    float* sA = reinterpret_cast<float*>(lds + LY::R2);   // phase C-D: diag(beta) L -> T (fp32)
    E* sP = reinterpret_cast<E*>(lds + LY::R4);      // phase C: P staging (row-major, ld LDT)
    E* sTb = reinterpret_cast<E*>(lds + LY::R4);     // phase D-E: T diag(beta) as MFMA operand
    E* sWk = reinterpret_cast<E*>(lds + LY::R0);     // phase E: Wk staging
    float* sTot = reinterpret_cast<float*>(lds + LY::TOT);
    float* sBeta = reinterpret_cast<float*>(lds + LY::BETA);
    float* sRq = reinterpret_cast<float*>(lds + LY::RQ);
    float* sRk = reinterpret_cast<float*>(lds + LY::RK);

    const int t = threadIdx.x;
    const int lane = t & 63, g = lane >> 4, n = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // wave index (uniform)

    // block -> (b, chunk, h): heads fastest, so neighbouring workgroups read
    // neighbouring pieces of the same token rows.  Packed variable-length
    // batches number chunks across all sequences (chunk_off and chunk_seq,
    // written by the plan kernel); workgroups past the last chunk have
    // nothing to do.
    const int H = a.H;
    const int64_t wg = blockIdx.x;
    const int h = (int)(wg % H);
    const int64_t rest = wg / H;
    int64_t b;
    int c;
    if (a.cu_seqlens) {
        if (rest >= a.chunk_off[a.B]) return;
        b = a.chunk_seq[rest];   // the sequence holding global chunk `rest`
        c = (int)(rest - a.chunk_off[b]);
    } else {
        c = (int)(rest % a.NC);
        b = rest / a.NC;
    }
    // the plan kernel wrote the chunk offsets just before, in the same call
    const SeqSpan sp = seq_span<false>(a.cu_seqlens, a.chunk_off, a.T, a.row_stride, a.NC, a.B, b, h, H);
    const int64_t tok0 = (int64_t)c * C;
    char* card = a.ws + (size_t)(sp.card0 + c) * CL::BYTES;

    // ---------------- phase A ----------------
    // Log-decay is carried in base-2 units (lambda * log2 e) so every
    // exponential is a single v_exp_f32; e^-gamma comes from v_rcp_f32.
    const int cp = t % CP, c0 = 2 * cp;
    const int grp = (CP == 64) ? w : t / CP;   // at d_k = 128 a token group is a wave
    const size_t row0 = (size_t)(sp.tok0 + tok0) * H + h;
    const size_t tstride = (size_t)H * DK;
    const float* la_b = a.log_alpha + row0 * DK;
    const E* q_b = reinterpret_cast<const E*>(a.q) + row0 * DK;
    const E* k_b = reinterpret_cast<const E*>(a.k) + row0 * DK;
    const E* v_b = reinterpret_cast<const E*>(a.v) + row0 * DK;
    const int nvalid = (int)((sp.len - tok0) < C ? (sp.len - tok0) : C);
    // Loads are unconditional: a padded token re-reads the last valid row (a
    // load under a branch would be followed by a wait on every outstanding
    // load).  Padding is an exact identity step as long as its beta and
    // lambda are zero: then its rows of Wk, Wv and U vanish and its q, k, v
    // never reach an output.
    // per-token row pointers are uniform within a wave at d_k = 128 (scalar
    // registers); the lane's channel pair is a 32-bit byte offset
    const uint32_t lo_a = (uint32_t)c0 * 4u, lo_e = (uint32_t)c0 * (uint32_t)sizeof(E);
    float lam[TPG][2], qv[TPG][2], kv[TPG][2], vv[TPG][2];
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
        const int tl = grp * TPG + i;
        const size_t toff = (size_t)(tl < nvalid ? tl : nvalid - 1) * tstride;
        const f32x2 l2 = *reinterpret_cast<const f32x2*>(reinterpret_cast<const char*>(la_b + toff) + lo_a);
        const f32x2 q2 = ld2(reinterpret_cast<const E*>(reinterpret_cast<const char*>(q_b + toff) + lo_e));
        const f32x2 k2 = ld2(reinterpret_cast<const E*>(reinterpret_cast<const char*>(k_b + toff) + lo_e));
        const f32x2 v2 = ld2(reinterpret_cast<const E*>(reinterpret_cast<const char*>(v_b + toff) + lo_e));
        const bool ok = tl < nvalid;
        lam[i][0] = ok ? fmaxf(l2[0], a.floor_) * kLog2e : 0.f;
        lam[i][1] = ok ? fmaxf(l2[1], a.floor_) * kLog2e : 0.f;
        qv[i][0] = q2[0]; qv[i][1] = q2[1];
        kv[i][0] = k2[0]; kv[i][1] = k2[1];
        vv[i][0] = v2[0]; vv[i][1] = v2[1];
    }
    {   // no branch around the load: every thread loads the beta of token t % C
        // (clamped) and stores it; the threads sharing a token store the same value
        const int tb = t % C;
        const float bv = a.beta[row0 + (size_t)(tb < nvalid ? tb : nvalid - 1) * H];
        sBeta[tb] = (tb < nvalid) ? bv : 0.f;
    }
    // inclusive cumulative log-decay inside the group
    float run0 = 0.f, run1 = 0.f;
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
        run0 += lam[i][0]; lam[i][0] = run0;
        run1 += lam[i][1]; lam[i][1] = run1;
    }
    sTot[grp * DK + c0] = run0;
    sTot[grp * DK + c0 + 1] = run1;
    {   // q/k squared norms of the group's TPG tokens, summed over its CP lanes.
        // Transpose-reduce: each exchange halves the number of values a lane
        // carries, so lane l ends with the full sum of token (l >> 2) % TPG.
        float sq[TPG], sk[TPG];
#pragma unroll
        for (int i = 0; i < TPG; ++i) {
            sq[i] = qv[i][0] * qv[i][0] + qv[i][1] * qv[i][1];
            sk[i] = kv[i][0] * kv[i][0] + kv[i][1] * kv[i][1];
        }
        if constexpr (TPG >= 16) tr_halve<8>(sq, sk, lane);
        if constexpr (TPG >= 8) tr_halve<4>(sq, sk, lane);
        tr_halve<2>(sq, sk, lane);
        tr_halve<1>(sq, sk, lane);
        sq[0] += __shfl_xor(sq[0], 2);
        sk[0] += __shfl_xor(sk[0], 2);
        sq[0] += __shfl_xor(sq[0], 1);
        sk[0] += __shfl_xor(sk[0], 1);
        if ((lane & 3) == 0) {
            const int tl = grp * TPG + ((lane >> 2) & (TPG - 1));
            sRq[tl] = 1.0f / fmaxf(sqrtf(sq[0]), 1e-6f);
            sRk[tl] = 1.0f / fmaxf(sqrtf(sk[0]), 1e-6f);
        }
    }
    __syncthreads();

    float off0 = 0.f, off1 = 0.f, tot0 = 0.f, tot1 = 0.f;
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) {
        const float x0 = sTot[gg * DK + c0], x1 = sTot[gg * DK + c0 + 1];
        if (gg < grp) { off0 += x0; off1 += x1; }
        tot0 += x0; tot1 += x1;
    }
    // e^gamma_C per key channel: Ke = k^ e^(gamma_C - gamma) = Kh * e^gamma_C
    const float gc0 = __builtin_amdgcn_exp2f(tot0), gc1 = __builtin_amdgcn_exp2f(tot1);
    float kt[TPG][2], ke[TPG][2];
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
        const int tl = grp * TPG + i;
        const float rq = sRq[tl], rk = sRk[tl];
        const float e0 = __builtin_amdgcn_exp2f(lam[i][0] + off0), e1 = __builtin_amdgcn_exp2f(lam[i][1] + off1);
        const float ei0 = __builtin_amdgcn_rcpf(e0), ei1 = __builtin_amdgcn_rcpf(e1);
        const float kn0 = kv[i][0] * rk, kn1 = kv[i][1] * rk;
        const float qn0 = qv[i][0] * rq, qn1 = qv[i][1] * rq;
        kt[i][0] = kn0 * e0;
        kt[i][1] = kn1 * e1;
        const float kh0 = kn0 * ei0, kh1 = kn1 * ei1;
        st2(sKt + tl * LDR + c0, kt[i][0], kt[i][1]);
        st2(sKh + tl * LDR + c0, kh0, kh1);
        st2(sQt + tl * LDR + c0, qn0 * e0, qn1 * e1);
        ke[i][0] = kh0 * gc0;
        ke[i][1] = kh1 * gc1;
    }
    {   // Ke^T rows c0, c0+1 (key channels), columns = this group's TPG tokens,
        // written in fragment order
        E* keT = reinterpret_cast<E*>(card + CL::KET);
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
            if constexpr (M::KF == 8) {
#pragma unroll
                for (int j = 0; j < TPG; j += 8) {
                    bf16x8 x;
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = (__bf16)ke[j + e][ch];
                    *reinterpret_cast<bf16x8*>(keT + frag_index<E>(c0 + ch, grp * TPG + j, C)) = x;
                }
            } else {
#pragma unroll
                for (int j = 0; j < TPG; ++j) keT[frag_index<E>(c0 + ch, grp * TPG + j, C)] = from_f32<E>(ke[j][ch]);
            }
        }
        if (grp == 0) *reinterpret_cast<f32x2*>(reinterpret_cast<float*>(card + CL::GC) + c0) = f32x2{gc0, gc1};
    }
    __syncthreads();

    // ---------------- phase B: L = Kt Kh^T, P = Qt Kh^T (lower tiles) ----------------
    // diag(beta) L needs no mask: the inversion reads only strictly-lower
    // entries of the diagonal tiles.  P is masked on its diagonal tiles.
    f32x4 acc[5];
#pragma unroll
    for (int r = 0; r < 5; ++r) {
        const int tau = w + 4 * r;
        const bool isP = tau >= 10;
        const int id = isP ? tau - 10 : tau;
        const int ti = (id >= 1) + (id >= 3) + (id >= 6);
        const int tj = id - ti * (ti + 1) / 2;
        const E* src = isP ? sQt : sKt;
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DK / KS; ++s)
            x = M::mma(ld_frag(src, LDR, 16 * ti + n, s * KS, g), ld_frag(sKh, LDR, 16 * tj + n, s * KS, g), x);
        if (isP) {
            if (ti == tj) {
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = (n <= 4 * g + e) ? x[e] : 0.f;
            }
        } else {
            const f32x4 bt = *reinterpret_cast<const f32x4*>(sBeta + 16 * ti + 4 * g);
            x *= bt;
        }
        acc[r] = x;
    }
    __syncthreads();

    // ---------------- phase C ----------------
#pragma unroll
    for (int i = 0; i < TPG; i += 4) {   // Kt^T and V^T, TPG tokens per row
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
            st4(sKtT + (c0 + ch) * LDT + grp * TPG + i, f32x4{kt[i][ch], kt[i + 1][ch], kt[i + 2][ch], kt[i + 3][ch]});
            st4(sVT + (c0 + ch) * LDT + grp * TPG + i, f32x4{vv[i][ch], vv[i + 1][ch], vv[i + 2][ch], vv[i + 3][ch]});
        }
    }
#pragma unroll
    for (int r = 0; r < 5; ++r) {   // P -> LDS staging: the 10 lower tiles ...
        const int tau = w + 4 * r;
        if (tau >= 10) {
            const int id = tau - 10;
            const int ti = (id >= 1) + (id >= 3) + (id >= 6);
            const int tj = id - ti * (ti + 1) / 2;
#pragma unroll
            for (int e = 0; e < 4; ++e) sP[(16 * ti + 4 * g + e) * LDT + 16 * tj + n] = from_f32<E>(acc[r][e]);
        }
    }
    for (int idx = t; idx < 6 * 64; idx += kThreads) {   // ... and zeros for the 6 upper tiles
        const int ut = idx >> 6, el = (idx & 63) * 4;     // 4 elements per item
        // upper tiles (ti, tj), tj > ti: (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
        const int ti = (ut >= 3) + (ut >= 5);
        const int tj = ut - (ti == 0 ? 0 : (ti == 1 ? 3 : 5)) + ti + 1;
        st4(sP + (16 * ti + (el >> 4)) * LDT + 16 * tj + (el & 15), f32x4{0.f, 0.f, 0.f, 0.f});
    }
    store_frag_order<E, C, DK>(card + CL::QT, sQt, LDR, t);   // Qt -> card
    __syncthreads();
    store_frag_order<E, C, C>(card + CL::P, sP, LDT, t);      // P -> card
#pragma unroll
    for (int r = 0; r < 5; ++r) {   // diag(beta) L -> sA (fp32; overwrites Qt)
        const int tau = w + 4 * r;
        if (tau < 10) {
            const int ti = (tau >= 1) + (tau >= 3) + (tau >= 6);
            const int tj = tau - ti * (ti + 1) / 2;
#pragma unroll
            for (int e = 0; e < 4; ++e) sA[(16 * ti + 4 * g + e) * LDA + 16 * tj + n] = acc[r][e];
        }
    }
    __syncthreads();

    // ---------------- phase D: T = (I + A)^-1, in place in sA ----------------
    {   // D1: diagonal 16x16 blocks by forward substitution; lane n owns column n
        float x[16];
        if (g == 0) {
            const float* Ab = sA + (16 * w) * LDA + 16 * w;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s = (i == n) ? 1.f : 0.f;
#pragma unroll
                for (int kk = 0; kk < i; ++kk) s -= Ab[i * LDA + kk] * x[kk];
                x[i] = s;
            }
        }
        __syncthreads();
        if (g == 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sA[(16 * w + i) * LDA + 16 * w + n] = x[i];
        }
        __syncthreads();
    }
    // D2: block row i: T_ij = -D_i * sum_{kb=j}^{i-1} A_{i,kb} T_{kb,j}; wave j computes T_ij
#pragma unroll
    for (int i = 1; i < 4; ++i) {
        f32x4 tij = {0.f, 0.f, 0.f, 0.f};
        if (w < i) {
            const int j = w;
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            for (int kb = j; kb < i; ++kb) {
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    x = mma_f32(sA[(16 * i + n) * LDA + 16 * kb + 4 * s + g],
                                sA[(16 * kb + 4 * s + g) * LDA + 16 * j + n], x);
            }
            // D_i * X with X taken straight from the accumulator: at step s,
            // lane group g holds X[4g + s][n], so A supplies D_i[m][4g + s]
#pragma unroll
            for (int s = 0; s < 4; ++s)
                tij = mma_f32(sA[(16 * i + n) * LDA + 16 * i + 4 * g + s], x[s], tij);
        }
        __syncthreads();
        if (w < i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) sA[(16 * i + 4 * g + e) * LDA + 16 * w + n] = -tij[e];
        }
        __syncthreads();
    }
    // D3: M = T diag(beta) -> MFMA operand type, zero above the diagonal
    // (a thread's LDS reads all issued before its writes)
    {
        constexpr int ND = C * C / 4 / kThreads;
        static_assert((C * C / 4) % kThreads == 0 && LDA % 4 == 0, "whole 4-element pieces");
        f32x4 av[ND], bt[ND];
#pragma unroll
        for (int j = 0; j < ND; ++j) {
            const int idx = t + j * kThreads, row = idx / (C / 4), col = (idx % (C / 4)) * 4;
            av[j] = *reinterpret_cast<const f32x4*>(sA + row * LDA + col);
            bt[j] = *reinterpret_cast<const f32x4*>(sBeta + col);
        }
#pragma unroll
        for (int j = 0; j < ND; ++j) {
            const int idx = t + j * kThreads, row = idx / (C / 4), col = (idx % (C / 4)) * 4;
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (col + e <= row) ? av[j][e] * bt[j][e] : 0.f;
            st4(sTb + row * LDT + col, x);
        }
    }
    __syncthreads();

    // ---------------- phase E: Wk = M Kt, Wv = M V ----------------
    constexpr int NTW = NT / 4;   // column tiles per wave
    f32x4 wk[NTW][4];
#pragma unroll
    for (int jt = 0; jt < NTW; ++jt) {
        const int ni = w * NTW + jt;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            f32x4 xk = {0.f, 0.f, 0.f, 0.f}, xv = {0.f, 0.f, 0.f, 0.f};
            const int nks = (16 * (mi + 1) + KS - 1) / KS;
#pragma unroll
            for (int s = 0; s < (C / KS); ++s) {
                if (s < nks) {
                    const auto af = ld_frag(sTb, LDT, 16 * mi + n, s * KS, g);
                    xk = M::mma(af, ld_frag(sKtT, LDT, 16 * ni + n, s * KS, g), xk);
                    xv = M::mma(af, ld_frag(sVT, LDT, 16 * ni + n, s * KS, g), xv);
                }
            }
            st4(reinterpret_cast<E*>(card + CL::WV) + ((size_t)(ni * 4 + mi) * 64 + lane) * 4, xv);
            wk[jt][mi] = xk;
        }
    }
    __syncthreads();
#pragma unroll
    for (int jt = 0; jt < NTW; ++jt)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sWk[(16 * mi + 4 * g + e) * LDR + 16 * (w * NTW + jt) + n] = from_f32<E>(wk[jt][mi][e]);
    __syncthreads();
    store_frag_order<E, C, DK>(card + CL::WK, sWk, LDR, t);   // Wk -> card
}

// Chunk offsets of a packed variable-length batch: chunk_off[s] = sum of
// ceil(len/C) over the sequences before s (one workgroup, a block-wide scan
// per 256 sequences), and chunk_seq[j] = the sequence that global chunk j
// belongs to, so a prepare workgroup finds its sequence with one load.  The
// offsets are clamped to maxc = ceil(T/C) + nseq, the chunks the workspace
// holds: only offsets that decrease somewhere (overlapping sequences) can
// reach it, and then the later sequences lose chunks instead of sending
// accesses past the workspace.
__global__ __launch_bounds__(kThreads) void kda_varlen_plan_kernel(const int32_t* cu, int64_t nseq, int64_t T,
                                                                  int64_t maxc, int64_t* chunk_off,
                                                                  int32_t* chunk_seq) {
    __shared__ int64_t part[kThreads];
    const int t = threadIdx.x;
    if (t == 0) chunk_off[0] = 0;
    int64_t carry = 0;
    for (int64_t base = 0; base < nseq; base += kThreads) {
        const int64_t s = base + t;
        int64_t ncs = 0;
        if (s < nseq) {
            int64_t st, en;
            seq_bounds(cu, s, T, st, en);
            ncs = (en - st + kChunk - 1) / kChunk;
        }
        part[t] = ncs;
        __syncthreads();
        for (int d = 1; d < kThreads; d <<= 1) {
            const int64_t x = t >= d ? part[t - d] : 0;
            __syncthreads();
            part[t] += x;
            __syncthreads();
        }
        if (s < nseq) {
            const int64_t end = carry + part[t] < maxc ? carry + part[t] : maxc;
            const int64_t first = carry + part[t] - ncs < maxc ? carry + part[t] - ncs : maxc;
            chunk_off[s + 1] = end;
            for (int64_t j = first; j < end; ++j) chunk_seq[j] = (int32_t)s;
        }
        carry += part[kThreads - 1];
        __syncthreads();
    }
}

template <typename E, int DK>
hipError_t launch_prepare_t(const PrepareArgs& a, hipStream_t s) {
    if (a.cu_seqlens) {
        if (a.B == 0) return hipSuccess;
        const int64_t maxc = (a.T + kChunk - 1) / kChunk + a.B;   // chunks the workspace holds
        hipLaunchKernelGGL(kda_varlen_plan_kernel, dim3(1), dim3(kThreads), 0, s, a.cu_seqlens, a.B, a.T, maxc,
                           a.chunk_off, a.chunk_seq);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // packed batches: an upper bound on the chunk count (sum of ceil(len/C) <= ceil(T/C) + B for
    // non-decreasing offsets; the plan kernel clamps the offsets to it otherwise)
    const int64_t chunks = a.cu_seqlens ? (a.T + kChunk - 1) / kChunk + a.B : a.B * (int64_t)a.NC;
    const int64_t blocks = chunks * a.H;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((kda_prepare_kernel<E, DK>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

size_t card_bytes(bool bf16, int dk) {
    if (bf16) return dk == 128 ? Card<__bf16, 128>::BYTES : Card<__bf16, 64>::BYTES;
    return dk == 128 ? Card<float, 128>::BYTES : Card<float, 64>::BYTES;
}

hipError_t launch_prepare(bool bf16, int dk, const PrepareArgs& a, hipStream_t s) {
    if (bf16) return dk == 128 ? launch_prepare_t<__bf16, 128>(a, s) : launch_prepare_t<__bf16, 64>(a, s);
    return dk == 128 ? launch_prepare_t<float, 128>(a, s) : launch_prepare_t<float, 64>(a, s);
}

}  // namespace kda
