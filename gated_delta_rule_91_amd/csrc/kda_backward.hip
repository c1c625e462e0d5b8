// kda_backward.hip -- gradients of the KDA token mixer for training, by the
// chunk method run in reverse (the pages say the fused chunk kernels serve
// training throughput [zuoshipin.com/article/18261 §四, FlashKDA paragraph];
// the recurrence is the one of the forward path, §二).
//
// With L = <d_out, out> + <d_state, S_T>, inside one chunk (C = 64 tokens,
// S0 the state entering it, dS the gradient of the state leaving it) the
// forward is
//   A  = strict_lower(Kt Kh^T),  P = lower_incl(Qt Kh^T),  T = (I + diag(beta) A)^-1
//   R  = V - Kt S0,  U = T diag(beta) R,  O = Qt S0 + P U,  out = O * sigmoid(g)
//   S_C = G S0 + Ke^T U,  G = diag(e^gamma_C)
// (Kt, Kh, Qt, Ke: k^ and q^ with the per-channel decay folded in, as in the
// prepare kernel), so its adjoint is
//   dO = d_out * sigmoid(g),  dg = d_out * out * (1 - sigmoid(g))
//   dU = Ke dS + P^T dO,  dU~ = T^T dU,  dv = diag(beta) dU~
//   dM = -dU~ U^T,  dbeta_i = dU~_i . R_i + sum_j dM_ij A_ij,  dA = strict_lower(diag(beta) dM)
//   dP = lower_incl(dO U^T)
//   dQt = dO S0^T + dP Kh,  dKt = -(diag(beta) dU~) S0^T + dA Kh,  dKh = dP^T Qt + dA^T Kt,
//   dKe = U dS^T,  dgamma_C += rowsum(S0 * dS) e^gamma_C + sum_i dKe_i * Ke_i
//   dS0 = G dS + Qt^T dO - Wk^T dU        (Wk = T diag(beta) Kt)
// and dgamma_i, dk^, dq^ follow from the decay folding; dlog_alpha is the
// reverse cumulative sum of dgamma over the chunk (zero where the floor
// binds), and dk, dq come through the L2 normalisation.
//
// Kernels, in order (the first two are the forward path's own):
//   1. kda_prepare_kernel     forward update cards
//   2. kda_scan_kernel        forward hand-off, also storing the state that
//                             enters every chunk, tiled (tiled_state_index),
//                             and out, for dg
//   3. kda_bwd_card_kernel    per chunk, in parallel: the operands of the
//                             reverse hand-off -- Ke, Qt^T, -Wk^T, dO in MFMA
//                             operand order and P^T dO in accumulator order
//   4. kda_bwd_scan_kernel    the reverse hand-off dS <- G dS + Qt^T dO - Wk^T dU
//                             over the chunks in reverse, one workgroup per
//                             16-column slice; stores the dS leaving every
//                             chunk, tiled
//   5. kda_bwd_grad_kernel    per chunk, in parallel (eight waves): every token
//                             gradient from S0, dS and the chunk's inputs
//                             (bf16 MFMA for most products with bf16 I/O,
//                             fp32 MFMA otherwise)
#include <type_traits>

#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

namespace {

constexpr int kXcds = 8;

__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// bf16 16x16x16: lane (n, g) supplies A[n][4g..4g+3] and B[4g..4g+3][n]
__device__ __forceinline__ f32x4 mma_bf16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) {
    return bf16x4{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
}
// bf16 16x16x32 (the same matrix-pipe cycles as 16x16x16 for twice the
// work): lane (n, g) supplies A[n][8g..8g+7] and B[8g..8g+7][n]
__device__ __forceinline__ f32x4 mma_bf16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 to_bf16x8(f32x4 lo, f32x4 hi) {
    return bf16x8{(__bf16)lo[0], (__bf16)lo[1], (__bf16)lo[2], (__bf16)lo[3],
                  (__bf16)hi[0], (__bf16)hi[1], (__bf16)hi[2], (__bf16)hi[3]};
}
// eight consecutive rows of one column of an fp32 LDS tile (row stride ld)
__device__ __forceinline__ bf16x8 col8(const float* p, int ld) {
    return bf16x8{(__bf16)p[0], (__bf16)p[ld], (__bf16)p[2 * ld], (__bf16)p[3 * ld],
                  (__bf16)p[4 * ld], (__bf16)p[5 * ld], (__bf16)p[6 * ld], (__bf16)p[7 * ld]};
}
__device__ __forceinline__ f32x4 ld4s(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 rcp4(f32x4 x) {
    return f32x4{__builtin_amdgcn_rcpf(x[0]), __builtin_amdgcn_rcpf(x[1]), __builtin_amdgcn_rcpf(x[2]),
                 __builtin_amdgcn_rcpf(x[3])};
}

// The operands of the reverse hand-off for one (batch row, head, chunk):
//   KEA [C x DK]  Ke in A-fragment order          (dU = Ke dS + ...)
//   QTT [DK x C]  Qt^T in A-fragment order        (dS += Qt^T dO)
//   WKT [DK x C]  -Wk^T in A-fragment order       (dS += -Wk^T dU)
//   DOT [DV x C]  dO^T in A-fragment order, which is dO in B-fragment order
//   DUL [C x DV]  P^T dO in accumulator order (the layout of Wv in Card)
//   G   [DK]      e^gamma_C, fp32
template <typename E, int DK>
struct BCard {
    static constexpr int C = kChunk;
    static constexpr size_t KEA = 0;
    static constexpr size_t QTT = KEA + (size_t)C * DK * sizeof(E);
    static constexpr size_t WKT = QTT + (size_t)DK * C * sizeof(E);
    static constexpr size_t DOT = WKT + (size_t)DK * C * sizeof(E);
    static constexpr size_t DUL = DOT + (size_t)DK * C * sizeof(E);
    static constexpr size_t G = DUL + (size_t)C * DK * sizeof(E);
    static constexpr size_t BYTES = ((G + (size_t)DK * sizeof(float)) + 255) / 256 * 256;
};

// Workspace of one backward call, in this order, each region 256-byte aligned.
// A uniform batch keeps NC + 1 entering-state slots per (b, h) (the last one
// unused).  A packed batch (varlen: B sequences over T tokens) starts with the
// chunk offsets and the chunk -> sequence map, sizes every per-chunk region
// for the most chunks B sequences can have (ceil(T / C) + B per head), and
// indexes the entering states like the cards: one slot per chunk-head.
struct BwdLayout {
    size_t offs, seqmap, cards, bcards, out, states, dstates, total;
    __host__ __device__ BwdLayout(bool bf16, int64_t B, int64_t T, int H, int dk, bool varlen = false) {
        const int64_t NC = (T + kChunk - 1) / kChunk;
        const size_t chunks = varlen ? (size_t)(NC + B) * H : (size_t)B * H * NC;
        const size_t tokens = varlen ? (size_t)T : (size_t)B * T;
        const size_t esz = bf16 ? 2 : 4;
        const size_t card = bf16 ? (dk == 128 ? Card<__bf16, 128>::BYTES : Card<__bf16, 64>::BYTES)
                                 : (dk == 128 ? Card<float, 128>::BYTES : Card<float, 64>::BYTES);
        const size_t bcard = bf16 ? (dk == 128 ? BCard<__bf16, 128>::BYTES : BCard<__bf16, 64>::BYTES)
                                  : (dk == 128 ? BCard<float, 128>::BYTES : BCard<float, 64>::BYTES);
        offs = 0;
        seqmap = varlen ? up((size_t)(B + 1) * 8) : 0;
        cards = varlen ? seqmap + up((size_t)(NC + B) * 4) : 0;
        bcards = cards + up(chunks * card);
        out = bcards + up(chunks * bcard);
        states = out + up(tokens * H * dk * esz);
        dstates = states + up((chunks + (varlen ? 0 : (size_t)B * H)) * (size_t)dk * dk * 4);
        total = dstates + up(chunks * (size_t)dk * dk * 4);
    }
    __host__ __device__ static size_t up(size_t x) { return (x + 255) / 256 * 256; }
};

// The chunk-head of a workgroup of the reverse-card and gradient kernels (one
// per chunk-head, heads fastest): its (row, head), the chunk's index in its
// sequence, its tokens inside the sequence, the row of its first token along
// the token axis (times H, plus the head), and its slots in the per-chunk
// regions.  A packed batch numbers chunks across all sequences (chunk_off,
// chunk_seq); workgroups past the last chunk have nothing to do.
struct BwdChunk {
    bool live;
    int h, c, nvalid;
    int64_t b, bh;
    size_t row0;    // token row of the chunk's first token, times H, plus h
    size_t cidx;    // card, reverse card and state gradient slot
    size_t sidx;    // entering-state slot
};
template <bool VL>
__device__ __forceinline__ BwdChunk bwd_chunk(const BackwardArgs& a, int64_t wg) {
    BwdChunk r;
    const int H = a.H;
    r.h = (int)(wg % H);
    const int64_t rest = wg / H;
    if constexpr (VL) {
        r.live = rest < a.chunk_off[a.B];
        if (!r.live) return r;
        const int32_t sq = a.chunk_seq[rest];
        r.b = sq < 0 ? 0 : (sq >= a.B ? a.B - 1 : sq);
        const SeqSpan sp = seq_span(a.cu_seqlens, a.chunk_off, a.T, 0, 0, a.B, r.b, r.h, H);
        const int64_t cc = rest - sp.chunk0;
        r.live = cc >= 0 && cc < sp.nc;   // a chunk outside its sequence's (clamped) span has nothing to do
        if (!r.live) return r;
        r.c = (int)cc;
        const int64_t t0 = (int64_t)r.c * kChunk;
        r.nvalid = (int)(sp.len - t0 < kChunk ? sp.len - t0 : kChunk);
        r.row0 = (size_t)(sp.tok0 + t0) * H + r.h;
        r.cidx = (size_t)sp.card0 + r.c;
        r.sidx = r.cidx;
        r.bh = r.b * H + r.h;
    } else {
        r.live = true;
        const int NC = a.NC;
        r.c = (int)(rest % NC);
        r.b = rest / NC;
        r.bh = r.b * H + r.h;
        const int64_t t0 = (int64_t)r.c * kChunk;
        r.nvalid = (int)(a.T - t0 < kChunk ? a.T - t0 : kChunk);
        r.row0 = ((size_t)r.b * a.T + t0) * H + r.h;
        r.cidx = (size_t)r.bh * NC + r.c;
        r.sidx = (size_t)r.bh * (NC + 1) + r.c;
    }
    return r;
}

// one element of a lane fragment
__device__ __forceinline__ float frag_elem(float v, int) { return v; }
__device__ __forceinline__ float frag_elem(bf16x8 v, int e) { return (float)v[e]; }

// Visit an R x K matrix stored in A-fragment order: f(row, k, value) for
// every element, each lane fragment read with one load (a thread's loads are
// all requested before the first is used).
template <typename E, int R, int K, typename F>
__device__ __forceinline__ void for_each_frag(const char* src, int t, F f) {
    constexpr int KF = MM<E>::KF, KS = MM<E>::KS, NF = R * K / KF / kThreads;
    static_assert((R * K / KF) % kThreads == 0, "whole fragments per thread");
    typedef typename MM<E>::frag Fr;
    Fr v[NF];
#pragma unroll
    for (int j = 0; j < NF; ++j) v[j] = reinterpret_cast<const Fr*>(src)[t + j * kThreads];
#pragma unroll
    for (int j = 0; j < NF; ++j) {
        const int idx = t + j * kThreads, blk = idx >> 6, lane = idx & 63;
        const int row = 16 * (blk / (K / KS)) + (lane & 15);
        const int k = (blk % (K / KS)) * KS + (lane >> 4) * KF;
#pragma unroll
        for (int e = 0; e < KF; ++e) f(row, k + e, frag_elem(v[j], e));
    }
}

// ---------------------------------------------------------------------------
// 3. operands of the reverse hand-off (one workgroup per chunk-head)
template <typename E, int DK, bool VL>
__global__ __launch_bounds__(kThreads) void kda_bwd_card_kernel(BackwardArgs a) {
    using M = MM<E>;
    using CL = Card<E, DK>;
    using BC = BCard<E, DK>;
    constexpr int C = kChunk, KS = M::KS, DV = DK;
    constexpr int PAD = 16 / (int)sizeof(E);
    constexpr int LDC = C + PAD;    // rows of C elements
    constexpr int LDD = DK + PAD;   // rows of DK elements
    constexpr int STAGE = DK * LDC > C * LDD ? DK * LDC : C * LDD;
    __shared__ __attribute__((aligned(16))) E sStage[STAGE];
    __shared__ __attribute__((aligned(16))) E sPT[C * LDC];    // P^T, row-major
    __shared__ __attribute__((aligned(16))) E sDOT[DV * LDC];  // dO^T, row-major

    const int t = threadIdx.x, lane = t & 63, g = lane >> 4, n = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const BwdChunk ck = bwd_chunk<VL>(a, blockIdx.x);
    if (!ck.live) return;
    const int H = a.H, nvalid = ck.nvalid;
    const BwdLayout L(sizeof(E) == 2, a.B, a.T, a.H, DK, VL);
    const char* card = a.ws + L.cards + ck.cidx * CL::BYTES;
    char* bcard = a.ws + L.bcards + ck.cidx * BC::BYTES;

    // Ke (from Ke^T) -> row-major -> fragment order
    for_each_frag<E, DK, C>(card + CL::KET, t, [&](int r, int k, float x) { sStage[k * LDD + r] = from_f32<E>(x); });
    __syncthreads();
    store_frag_order<E, C, DK>(bcard + BC::KEA, sStage, LDD, t);
    __syncthreads();
    // Qt^T
    for_each_frag<E, C, DK>(card + CL::QT, t, [&](int r, int k, float x) { sStage[k * LDC + r] = from_f32<E>(x); });
    __syncthreads();
    store_frag_order<E, DK, C>(bcard + BC::QTT, sStage, LDC, t);
    __syncthreads();
    // -Wk^T
    for_each_frag<E, C, DK>(card + CL::WK, t, [&](int r, int k, float x) { sStage[k * LDC + r] = from_f32<E>(-x); });
    // P^T, and dO = d_out * sigmoid(g) transposed (zero on padded tokens)
    for_each_frag<E, C, C>(card + CL::P, t, [&](int r, int k, float x) { sPT[k * LDC + r] = from_f32<E>(x); });
    {
        const size_t row0 = ck.row0;
        const E* dop = reinterpret_cast<const E*>(a.d_out);
        const E* gp = reinterpret_cast<const E*>(a.g);
        const E* dsrc = dop ? dop : gp;   // loaded unconditionally, zeroed after when d_out is absent
        constexpr int NP = C * DV / 4 / kThreads;   // four-column pieces per thread
        static_assert((C * DV / 4) % kThreads == 0, "whole pieces per thread");
        f32x4 dl[NP], gg[NP];
#pragma unroll
        for (int jj = 0; jj < NP; ++jj) {   // every piece requested before the first is used
            const int idx = t + jj * kThreads;
            const int i = idx / (DV / 4), v4 = (idx % (DV / 4)) * 4;
            const size_t r = (row0 + (size_t)(i < nvalid ? i : nvalid - 1) * H) * DV + v4;
            dl[jj] = ld4(dsrc + r);
            gg[jj] = ld4(gp + r);
        }
#pragma unroll
        for (int jj = 0; jj < NP; ++jj) {
            const int idx = t + jj * kThreads;
            const int i = idx / (DV / 4), v4 = (idx % (DV / 4)) * 4;
            const f32x4 dy = dop ? dl[jj] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) sDOT[(v4 + e) * LDC + i] = from_f32<E>(i < nvalid ? dy[e] * sigmoidf_(gg[jj][e]) : 0.f);
        }
    }
    if (t < DK) reinterpret_cast<float*>(bcard + BC::G)[t] = reinterpret_cast<const float*>(card + CL::GC)[t];
    __syncthreads();
    store_frag_order<E, DK, C>(bcard + BC::WKT, sStage, LDC, t);
    store_frag_order<E, DV, C>(bcard + BC::DOT, sDOT, LDC, t);
    // P^T dO: wave w takes column tiles [w*NT/4, (w+1)*NT/4), all token tiles
    constexpr int NT = DV / 16, NTW = NT / 4;
#pragma unroll
    for (int jt = 0; jt < NTW; ++jt) {
        const int ni = w * NTW + jt;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < C / KS; ++s)
                x = M::mma(ld_frag(sPT, LDC, 16 * mi + n, s * KS, g), ld_frag(sDOT, LDC, 16 * ni + n, s * KS, g), x);
            st4(reinterpret_cast<E*>(bcard + BC::DUL) + ((size_t)(ni * 4 + mi) * 64 + lane) * 4, x);
        }
    }
}

// ---------------------------------------------------------------------------
// 4. reverse hand-off: one workgroup per (batch row, head, 16-column slice),
// chunks in reverse.  Wave w owns dU rows (tokens) 16w..16w+15 and dS rows
// w*DK/4 .. (w+1)*DK/4 - 1; dS^T and dU^T cross waves through LDS.
template <typename E, int DK, bool VL>
__global__ __launch_bounds__(kThreads) void kda_bwd_scan_kernel(BackwardArgs a) {
    using M = MM<E>;
    using BC = BCard<E, DK>;
    typedef typename M::frag F;
    constexpr int C = kChunk, KS = M::KS, KF = M::KF, DV = DK;
    constexpr int NT = DV / 16, MTS = DK / 64, NKD = DK / KS, NKC = C / KS;
    constexpr int PADE = 16 / (int)sizeof(E);
    constexpr int LDS_S = DK + PADE, LDS_U = C + PADE;
    constexpr uint32_t FB = KF * sizeof(E), KSB = 64 * FB;
    __shared__ __attribute__((aligned(16))) E sS[16 * LDS_S];
    __shared__ __attribute__((aligned(16))) E sU[16 * LDS_U];

    const int t = threadIdx.x, lane = t & 63, w = t >> 6, g = lane >> 4, n = lane & 15;
    const int64_t BH = a.B * (int64_t)a.H;
    const int64_t x = blockIdx.x;
    const int xcd = (int)(x % kXcds);
    const int64_t slot = x / kXcds;
    const int tile = (int)(slot % NT);
    const int64_t bh = (slot / NT) * kXcds + xcd;
    if (bh >= BH) return;
    const int col0 = 16 * tile;
    const BwdLayout L(sizeof(E) == 2, a.B, a.T, a.H, DK, VL);
    // this chain's chunks and its first chunk's slot in the per-chunk regions
    int NC;
    size_t cbase;
    if constexpr (VL) {
        const SeqSpan sp = seq_span(a.cu_seqlens, a.chunk_off, a.T, 0, 0, a.B, bh / a.H, (int)(bh % a.H), a.H);
        NC = sp.nc;
        cbase = (size_t)sp.card0;
    } else {
        NC = a.NC;
        cbase = (size_t)bh * NC;
    }

    f32x4 dS[MTS];
#pragma unroll
    for (int mt = 0; mt < MTS; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = (DK / 4) * w + 16 * mt + 4 * g + e;
            dS[mt][e] = a.d_state ? a.d_state[((size_t)bh * DK + r) * DV + col0 + n] : 0.f;
        }
#pragma unroll
    for (int mt = 0; mt < MTS; ++mt) st4(sS + n * LDS_S + (DK / 4) * w + 16 * mt + 4 * g, dS[mt]);
    __syncthreads();

    const char* bcards = a.ws + L.bcards + cbase * BC::BYTES;
    float* dstates = reinterpret_cast<float*>(a.ws + L.dstates) + cbase * DK * DV;
    // one chunk's operands in registers: a two-slot ring loads chunk c - 1
    // while chunk c computes (loads are unconditional: past chunk 0 the ring
    // re-reads chunk 0)
    struct Ops {
        F kea[NKD], qtt[MTS][NKC], wkt[MTS][NKC], dot[NKC];
        f32x4 gv[MTS];
        f32x4 dul;
    };
    auto load = [&](Ops& o, int c) {
        const char* bc = bcards + (size_t)(c > 0 ? c : 0) * BC::BYTES;
        o.dul = ld4(reinterpret_cast<const E*>(bc + BC::DUL) + ((size_t)(tile * 4 + w) * 64 + lane) * 4);
#pragma unroll
        for (int s = 0; s < NKD; ++s) o.kea[s] = *reinterpret_cast<const F*>(bc + BC::KEA + (w * NKD + s) * KSB + lane * FB);
#pragma unroll
        for (int s = 0; s < NKC; ++s) o.dot[s] = *reinterpret_cast<const F*>(bc + BC::DOT + (tile * NKC + s) * KSB + lane * FB);
#pragma unroll
        for (int mt = 0; mt < MTS; ++mt) {
            const int rb = (DK / 64) * w + mt;
            o.gv[mt] = *reinterpret_cast<const f32x4*>(bc + BC::G + ((DK / 4) * w + 16 * mt + 4 * g) * 4);
#pragma unroll
            for (int s = 0; s < NKC; ++s) {
                o.qtt[mt][s] = *reinterpret_cast<const F*>(bc + BC::QTT + (rb * NKC + s) * KSB + lane * FB);
                o.wkt[mt][s] = *reinterpret_cast<const F*>(bc + BC::WKT + (rb * NKC + s) * KSB + lane * FB);
            }
        }
    };
    auto step = [&](const Ops& o, int c) {
        float* dst = dstates + (size_t)c * DK * DV;   // gradient of the state leaving chunk c, tiled
#pragma unroll
        for (int mt = 0; mt < MTS; ++mt)
            *reinterpret_cast<f32x4*>(dst + tiled_state_index(DK, tile, (DK / 16) * w + 4 * mt + g, n)) = dS[mt];
        // dU rows 16w..16w+15 = P^T dO + Ke dS
        f32x4 du = o.dul;
#pragma unroll
        for (int s = 0; s < NKD; ++s) du = M::mma(o.kea[s], ld_frag(sS, LDS_S, n, s * KS, g), du);
        st4(sU + n * LDS_U + 16 * w + 4 * g, du);
        __syncthreads();
        // dS <- G dS + Qt^T dO - Wk^T dU
        F ub[NKC];
#pragma unroll
        for (int s = 0; s < NKC; ++s) ub[s] = ld_frag(sU, LDS_U, n, s * KS, g);
#pragma unroll
        for (int mt = 0; mt < MTS; ++mt) {
            f32x4 acc = dS[mt] * o.gv[mt];
#pragma unroll
            for (int s = 0; s < NKC; ++s) acc = M::mma(o.qtt[mt][s], o.dot[s], acc);
#pragma unroll
            for (int s = 0; s < NKC; ++s) acc = M::mma(o.wkt[mt][s], ub[s], acc);
            dS[mt] = acc;
        }
#pragma unroll
        for (int mt = 0; mt < MTS; ++mt) st4(sS + n * LDS_S + (DK / 4) * w + 16 * mt + 4 * g, dS[mt]);
        __syncthreads();
    };
    if (NC > 0) {
        Ops o0, o1;
        load(o0, NC - 1);
        int c = NC - 1;
        for (; c >= 1; c -= 2) {
            load(o1, c - 1);
            step(o0, c);
            load(o0, c - 2);
            step(o1, c - 1);
        }
        if (c == 0) step(o0, 0);
    }
    if (a.d_state_in) {
#pragma unroll
        for (int mt = 0; mt < MTS; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = (DK / 4) * w + 16 * mt + 4 * g + e;
                a.d_state_in[((size_t)bh * DK + r) * DV + col0 + n] = dS[mt][e];
            }
    }
}

// ---------------------------------------------------------------------------
// 5. token gradients: one workgroup of eight waves per chunk-head, fp32 LDS
// tiles of the chunk's k^, q^, e^gamma, P and T.  The value-side quantities (R, U, dO, dU)
// go through in 16-column blocks; the products that contract over the value
// columns accumulate in registers across the blocks.  Wave w works on token
// tile w % 4; the two halves of the workgroup (w / 4) run independent
// products side by side (R | dO, dg and Ke dS;  U | + P^T dO;  dU~ | dO U^T;
// dU~ U^T) and split the d_k-wide outputs by channel tile, so two waves share
// each SIMD and either can issue while the other waits.  Triangular products
// run over all four 16-token blocks (the blocks past the diagonal are zero in
// LDS), and no global load sits under a branch, so loads stay in flight
// across the phases.  With bf16 I/O the
// Gram matrices, R, U, Ke dS + P^T dO, dU~, dM, dP and the three products
// that contract over the value columns take bf16 operands (16x16x32 and
// 16x16x16 MFMA, fp32 accumulation), the operand precision of the forward
// cards; at d_k = 128 the column loop reads them from bf16 copies laid out so
// that each fragment is one LDS read.  The products after the column loop
// stay on fp32 MFMA (dgamma takes their differences), as does all of fp32 I/O.
constexpr int kGradThreads = 512;

template <int DK>
struct GradLds {
    static constexpr int C = kChunk, NB = 16;
    static constexpr int LDK = DK + 4;   // [C][DK] rows
    static constexpr int LDC = C + 4;    // [C][C] rows
    static constexpr int LDB = NB + 4;   // [C][NB] rows
    static constexpr int LDSB = NB + 4;  // [DK][NB] rows of the staged state blocks
    static constexpr size_t K = 0;                          // k^ (zero on padded tokens)
    static constexpr size_t Q = K + (size_t)C * LDK * 4;    // q^; during the column loop, the block of S0 and dS
    static constexpr size_t EG = Q + (size_t)C * LDK * 4;   // e^gamma
    static constexpr size_t P = EG + (size_t)C * LDK * 4;   // P, then dP, then dgamma (spans P and T)
    static constexpr size_t T = P + (size_t)C * LDC * 4;    // diag(beta) A -> T, then dA
    static constexpr size_t R = T + (size_t)C * LDC * 4;      // R, then dU~
    static constexpr size_t U = R + (size_t)C * LDB * 4;
    static constexpr size_t DO = U + (size_t)C * LDB * 4;
    static constexpr size_t DU = DO + (size_t)C * LDB * 4;  // dU
    static constexpr size_t BETA = DU + (size_t)C * LDB * 4;
    static constexpr size_t NK = BETA + (size_t)C * 4;      // |k|
    static constexpr size_t NQ = NK + (size_t)C * 4;        // |q|
    static constexpr size_t RK = NQ + (size_t)C * 4;        // 1 / max(|k|, 1e-6)
    static constexpr size_t RQ = RK + (size_t)C * 4;        // 1 / max(|q|, 1e-6)
    static constexpr size_t DGC = RQ + (size_t)C * 4;       // [5][DK]: per-token-tile sum dKe*Ke, rowsum(S0*dS)
    static constexpr size_t XD = DGC + (size_t)5 * DK * 4;  // [2 halves][k, q][C]: partial x^ . dx^
    static constexpr size_t BYTES = XD + (size_t)4 * C * 4;
    static_assert(2 * DK * LDSB <= C * LDK, "state blocks fit over q^");
    static_assert((size_t)C * LDK <= 2 * (size_t)C * LDC, "dgamma fits over P and T");
};

template <typename E, int DK, bool VL>
__global__ __launch_bounds__(kGradThreads, 1) void kda_bwd_grad_kernel(BackwardArgs a) {
    using LY = GradLds<DK>;
    constexpr int C = kChunk, NB = LY::NB, DV = DK, NTH = kGradThreads;
    constexpr int LDK = LY::LDK, LDC = LY::LDC, LDB = LY::LDB, LDSB = LY::LDSB;
    constexpr int NT = DK / 16;     // channel tiles
    constexpr int NTH2 = NT / 2;    // ... per half
    constexpr int NKD = DK / 4;     // fp32 MFMA k-steps over the channels
    constexpr int NKC = C / 4;      // ... over the tokens
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr bool BF = sizeof(E) == 2;   // bf16 operands for the big products

    __shared__ __attribute__((aligned(16))) char lds[LY::BYTES];
    float* sK = reinterpret_cast<float*>(lds + LY::K);
    float* sQ = reinterpret_cast<float*>(lds + LY::Q);
    float* sEG = reinterpret_cast<float*>(lds + LY::EG);
    float* sP = reinterpret_cast<float*>(lds + LY::P);
    float* sT = reinterpret_cast<float*>(lds + LY::T);
    float* sR = reinterpret_cast<float*>(lds + LY::R);
    float* sU = reinterpret_cast<float*>(lds + LY::U);
    float* sDO = reinterpret_cast<float*>(lds + LY::DO);
    float* sDU = reinterpret_cast<float*>(lds + LY::DU);
    float* sBeta = reinterpret_cast<float*>(lds + LY::BETA);
    float* sNk = reinterpret_cast<float*>(lds + LY::NK);
    float* sNq = reinterpret_cast<float*>(lds + LY::NQ);
    float* sRk = reinterpret_cast<float*>(lds + LY::RK);
    float* sRq = reinterpret_cast<float*>(lds + LY::RQ);
    float* sDGC = reinterpret_cast<float*>(lds + LY::DGC);
    float* sXD = reinterpret_cast<float*>(lds + LY::XD);
    static_assert(LDK % 4 == 0 && LDB % 4 == 0 && LY::LDSB % 4 == 0, "16-byte rows for the bf16 operand reads");
    float* sDG = sP;
    float* sS0 = sQ;                   // [DK][LDSB]: S0, this block's columns
    float* sDS = sQ + DK * LDSB;       // [DK][LDSB]: dS, this block's columns

    const int t = threadIdx.x, lane = t & 63, g = lane >> 4, n = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int w4 = w & 3, half = w >> 2;   // token tile; which half of the workgroup
    const int ct0 = half * NTH2;           // this wave's first channel tile
    const BwdChunk ck = bwd_chunk<VL>(a, blockIdx.x);
    if (!ck.live) return;
    const int H = a.H;
    const int nvalid = ck.nvalid;
    const size_t row0 = ck.row0;
    // token row of chunk token i (padded tokens re-read the last valid row)
    auto rowi = [&](int i) { return row0 + (size_t)(i < nvalid ? i : nvalid - 1) * H; };
    const BwdLayout L(sizeof(E) == 2, a.B, a.T, a.H, DK, VL);
    const float* S0 = reinterpret_cast<const float*>(a.ws + L.states) + ck.sidx * DK * DV;
    const float* dSo = reinterpret_cast<const float*>(a.ws + L.dstates) + ck.cidx * DK * DV;
    const E* qp = reinterpret_cast<const E*>(a.q);
    const E* kp = reinterpret_cast<const E*>(a.k);

    // ---- 1: norms, k^, q^, e^gamma, beta ----
    // Every global input of the phase is requested first (one memory round
    // trip).  Thread t holds the four-channel pieces jj of tokens
    // (t + jj * NTH) / (DK / 4); the DK / 4 pieces of a token sit in adjacent
    // lanes, which sum its squared norms with shuffles.
    constexpr int TPL = DK / 4;               // lanes per token
    constexpr int NPC = C * TPL / NTH;        // pieces per thread
    static_assert(NTH % TPL == 0 && (C * TPL) % NTH == 0, "piece layout");
    f32x4 kx[NPC], qx[NPC], lx[NPC];
#pragma unroll
    for (int jj = 0; jj < NPC; ++jj) {
        const int idx = t + jj * NTH, i = idx / TPL, ch = (idx % TPL) * 4;
        const size_t r = rowi(i) * DK + ch;
        kx[jj] = ld4(kp + r);
        qx[jj] = ld4(qp + r);
        lx[jj] = *reinterpret_cast<const f32x4*>(a.log_alpha + r);
    }
    // no branch around the beta load: every thread loads the beta of token
    // t % C (clamped) and stores it; the threads sharing a token store the same value
    const float bv = a.beta[rowi(t % C)];
    for (int idx = t; idx < C * LDC; idx += NTH) sT[idx] = 0.f;   // T's upper tiles stay zero
    sBeta[t % C] = t % C < nvalid ? bv : 0.f;
#pragma unroll
    for (int jj = 0; jj < NPC; ++jj) {
        const int idx = t + jj * NTH, i = idx / TPL, ch = (idx % TPL) * 4;
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sk += kx[jj][e] * kx[jj][e];
            sq += qx[jj][e] * qx[jj][e];
        }
#pragma unroll
        for (int off = 1; off < TPL; off <<= 1) {
            sk += __shfl_xor(sk, off);
            sq += __shfl_xor(sq, off);
        }
        const float nk = sqrtf(sk), nq = sqrtf(sq);
        const float rk = 1.f / fmaxf(nk, 1e-6f), rq = 1.f / fmaxf(nq, 1e-6f);
        if (idx % TPL == 0) {
            sNk[i] = nk;
            sNq[i] = nq;
            sRk[i] = rk;
            sRq[i] = rq;
        }
        const bool ok = i < nvalid;   // padded tokens: k^ = q^ = 0, no decay
        st4(sK + i * LDK + ch, ok ? kx[jj] * rk : f32x4{0.f, 0.f, 0.f, 0.f});
        st4(sQ + i * LDK + ch, ok ? qx[jj] * rq : f32x4{0.f, 0.f, 0.f, 0.f});
        f32x4 lam;   // floored log-decay in base 2
#pragma unroll
        for (int e = 0; e < 4; ++e) lam[e] = ok ? fmaxf(lx[jj][e], a.floor_) * kLog2e : 0.f;
        st4(sEG + i * LDK + ch, lam);
    }
    __syncthreads();
    // q^ again after the column loop: its LDS rows hold the state blocks
    // meanwhile.  Recomputed from the input and the stored reciprocal norms,
    // so the values are the same.  The loads are issued first and the
    // products stored later, so that other work covers their latency.
    typedef typename Raw4<E>::type RawPiece;
    auto issue_hat = [&](const E* xp, RawPiece* raw) {
#pragma unroll
        for (int jj = 0; jj < NPC; ++jj) {
            int i = (t + jj * NTH) / TPL;
            // recomputed here rather than kept live from the input phase (that spills)
            asm volatile("" : "+v"(i));
            raw[jj] = *reinterpret_cast<const RawPiece*>(xp + rowi(i) * DK + ((t + jj * NTH) % TPL) * 4);
        }
    };
    auto store_hat = [&](const RawPiece* raw, float* dst, const float* rn) {
#pragma unroll
        for (int jj = 0; jj < NPC; ++jj) {
            const int idx = t + jj * NTH;
            const int i = idx / TPL, ch = (idx % TPL) * 4;
            st4(dst + i * LDK + ch, i < nvalid ? widen4(raw[jj]) * rn[i] : f32x4{0.f, 0.f, 0.f, 0.f});
        }
    };
    if (t < DK) {   // e^gamma: cumulative log-decay of channel t (the column read first, then summed)
        float col[C];
#pragma unroll
        for (int i = 0; i < C; ++i) col[i] = sEG[i * LDK + t];
        float run = 0.f;
#pragma unroll
        for (int i = 0; i < C; ++i) {
            run += col[i];
            sEG[i * LDK + t] = __builtin_amdgcn_exp2f(run);
        }
    }
    __syncthreads();

    auto Kt = [&](int i, int ch) { return sK[i * LDK + ch] * sEG[i * LDK + ch]; };
    auto Kh = [&](int i, int ch) { return sK[i * LDK + ch] * __builtin_amdgcn_rcpf(sEG[i * LDK + ch]); };
    auto Qt = [&](int i, int ch) { return sQ[i * LDK + ch] * sEG[i * LDK + ch]; };
    auto Ke = [&](int i, int ch) { return Kh(i, ch) * sEG[(C - 1) * LDK + ch]; };

    // ---- 2: half 0: A = Kt Kh^T (kept in registers, strictly lower) and
    // diag(beta) A -> sT; half 1: P = Qt Kh^T -> sP ----
    // With bf16 operands, Kh = k^ e^-gamma is formed once as bf16 rows (over
    // the value tiles, unused until the column loop), so each B fragment is
    // one 16-byte read, and each wave's A fragments (rows of Kt or Qt) are
    // formed once for its four products.
    constexpr int LDH = DK + 8;
    static_assert(C * LDH * 2 <= 4 * C * LDB * 4, "Kh fits over the value tiles");
    const __bf16* bKh = reinterpret_cast<const __bf16*>(sR);
    bf16x8 ag[BF ? DK / 32 : 1];
    if constexpr (BF) {
        for (int idx = t; idx < C * DK / 4; idx += NTH) {   // four channels of one token per step
            const int i = idx / (DK / 4), ch = (idx % (DK / 4)) * 4;
            *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(sR) + i * LDH + ch) =
                to_bf16x4(ld4s(sK + i * LDK + ch) * rcp4(ld4s(sEG + i * LDK + ch)));
        }
        const float* xa = (half == 0 ? sK : sQ) + (16 * w4 + n) * LDK;
        const float* ea = sEG + (16 * w4 + n) * LDK;
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) {
            const int c0 = 32 * s + 8 * g;
            ag[s] = to_bf16x8(ld4s(xa + c0) * ld4s(ea + c0), ld4s(xa + c0 + 4) * ld4s(ea + c0 + 4));
        }
        __syncthreads();
    }
    f32x4 As[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {   // tiles right of the diagonal come out masked to zero
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if constexpr (BF) {   // rows of Kt (or Qt) against rows of Kh, 32 channels per step
#pragma unroll
            for (int s = 0; s < DK / 32; ++s)
                x = mma_bf16x32(ag[s], *reinterpret_cast<const bf16x8*>(bKh + (16 * j + n) * LDH + 32 * s + 8 * g), x);
        } else if (half == 0) {
#pragma unroll 8
            for (int s = 0; s < NKD; ++s) x = mma_f32(Kt(16 * w4 + n, 4 * s + g), Kh(16 * j + n, 4 * s + g), x);
        } else {
#pragma unroll 8
            for (int s = 0; s < NKD; ++s) x = mma_f32(Qt(16 * w4 + n, 4 * s + g), Kh(16 * j + n, 4 * s + g), x);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * w4 + 4 * g + e, jj = 16 * j + n;
            if (half == 0) {
                As[j][e] = jj < i ? x[e] : 0.f;
                sT[i * LDC + jj] = jj < i ? sBeta[i] * x[e] : 0.f;
            } else {
                sP[i * LDC + jj] = jj <= i ? x[e] : 0.f;
            }
        }
    }
    __syncthreads();

    // ---- 3: T = (I + diag(beta) A)^-1 in place (blocked substitution, half 0) ----
    {   // diagonal 16x16 blocks by forward substitution; lane n of wave w4 owns column n of block w4
        float x[16];
        if (half == 0 && g == 0) {
            const float* Ab = sT + (16 * w4) * LDC + 16 * w4;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s = (i == n) ? 1.f : 0.f;
#pragma unroll
                for (int kk = 0; kk < i; ++kk) s -= Ab[i * LDC + kk] * x[kk];
                x[i] = s;
            }
        }
        __syncthreads();
        if (half == 0 && g == 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sT[(16 * w4 + i) * LDC + 16 * w4 + n] = x[i];
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 1; i < 4; ++i) {   // block row i: T_ij = -D_i sum_{kb=j}^{i-1} A_{i,kb} T_{kb,j}, wave j
        f32x4 tij = {0.f, 0.f, 0.f, 0.f};
        if (half == 0 && w4 < i) {
            const int j = w4;
            f32x4 xx = {0.f, 0.f, 0.f, 0.f};
            for (int kb = j; kb < i; ++kb) {
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    xx = mma_f32(sT[(16 * i + n) * LDC + 16 * kb + 4 * s + g], sT[(16 * kb + 4 * s + g) * LDC + 16 * j + n],
                                 xx);
            }
            // D_i X with X straight from the accumulator: at step s lane group g
            // holds X[4g + s][n], so A supplies D_i[m][4g + s]
#pragma unroll
            for (int s = 0; s < 4; ++s) tij = mma_f32(sT[(16 * i + n) * LDC + 16 * i + 4 * g + s], xx[s], tij);
        }
        __syncthreads();
        if (half == 0 && w4 < i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) sT[(16 * i + 4 * g + e) * LDC + 16 * w4 + n] = -tij[e];
        }
        __syncthreads();
    }

    // ---- 4: value columns in blocks of NB ----
    const E* vp = reinterpret_cast<const E*>(a.v);
    const E* gp = reinterpret_cast<const E*>(a.g);
    const E* op = reinterpret_cast<const E*>(a.out);
    const E* dop = reinterpret_cast<const E*>(a.d_out);
    E* dvp = reinterpret_cast<E*>(a.dv);
    E* dgp = reinterpret_cast<E*>(a.dg);
    // channel tiles ct0 .. ct0 + NTH2 - 1: dQt, dKt, dKe (then dKh in phase 6)
    f32x4 aQ[NTH2], aK[NTH2], aE[NTH2], dMP[4];   // dMP: dM tiles (half 0) or dP tiles (half 1), (w4, j)
#pragma unroll
    for (int c2 = 0; c2 < NTH2; ++c2) aQ[c2] = aK[c2] = aE[c2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) dMP[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 dbp = {0.f, 0.f, 0.f, 0.f};
    // The states are stored tiled (tiled_state_index): a block of NB = 16
    // columns is one contiguous tile, and piece idx of it holds rows
    // 4 (idx / 16) .. + 3 of column idx % 16.
    static_assert(NB == 16 && NTH % 16 == 0, "one tile per column block; a row group's 16 pieces in 16 adjacent lanes");
    constexpr int NSI = (DK * NB / 4 + NTH - 1) / NTH;   // staged 4-float pieces per thread
    f32x4 rowp[NSI];   // rowsum(S0 * dS) over the blocks so far: rows 4 (idx / 16) + e, column idx % 16
#pragma unroll
    for (int j = 0; j < NSI; ++j) rowp[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the global inputs of a column block, fetched one block ahead into
    // registers (every load unconditional: addresses are clamped, the block
    // after the last re-reads the last)
    struct Pre {
        f32x4 s[NSI], d[NSI];   // S0 and dS pieces
        f32x4 a, b, c;          // V (half 0), or d_out, g, out (half 1)
    };
    auto fetch = [&](int vb) {
        Pre p;
        const int tb = vb < DV / NB ? vb : DV / NB - 1;
        const int col0 = NB * tb;
#pragma unroll
        for (int j = 0; j < NSI; ++j) {
            const int idx = t + j * NTH < DK * NB / 4 ? t + j * NTH : DK * NB / 4 - 1;
            const int o = tiled_state_index(DK, tb, idx / 16, idx % 16);
            p.s[j] = *reinterpret_cast<const f32x4*>(S0 + o);
            p.d[j] = *reinterpret_cast<const f32x4*>(dSo + o);
        }
        // both halves load three values per element (the V pointer twice on
        // half 0), so no load sits under a branch
        const E* pa = half == 0 ? vp : (dop ? dop : gp);
        const E* pb = half == 0 ? vp : gp;
        const E* pc = half == 0 ? vp : op;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const size_t ri = rowi(16 * w4 + 4 * g + e) * DV + col0 + n;
            const float xa = to_f32(pa[ri]);   // loaded unconditionally (pa is never null)
            p.a[e] = (half == 0 || dop) ? xa : 0.f;
            p.b[e] = to_f32(pb[ri]);
            p.c[e] = to_f32(pc[ri]);
        }
        return p;
    };
    // the A operands that stay the same in every column block, as bf16
    // fragments: -Kt rows 16 w4 .. for R on half 0, K_end rows for K_end dS on half 1
    constexpr int NKF = BF ? DK / 32 : 1;
    bf16x8 afr[NKF];
    if constexpr (BF) {
        const float* xa = sK + (16 * w4 + n) * LDK;
        const float* ea = sEG + (16 * w4 + n) * LDK;
        const float* ec = sEG + (C - 1) * LDK;
#pragma unroll
        for (int s = 0; s < NKF; ++s) {
            const int c0 = 32 * s + 8 * g;
            const f32x4 xl = ld4s(xa + c0), xh = ld4s(xa + c0 + 4), el = ld4s(ea + c0), eh = ld4s(ea + c0 + 4);
            afr[s] = half == 0 ? to_bf16x8(-(xl * el), -(xh * eh))
                               : to_bf16x8(xl * rcp4(el) * ld4s(ec + c0), xh * rcp4(eh) * ld4s(ec + c0 + 4));
        }
    }
    Pre pre = fetch(0);
    if constexpr (BF && DK == 128) {
        // bf16 operand copies laid out so that every MFMA fragment is one
        // 8- or 16-byte LDS read (the fp32 tiles were read one element at a
        // time down their columns): over q^ the state blocks, transposed for
        // the products that contract over channels and as they are for the
        // ones that contract over the block's columns; over the fp32 P and T
        // (not read again before phase 5 writes dP and dA there) T, P^T and
        // T^T; over the fp32 value tiles the value-side operands.  Every value
        // is the bf16 rounding the fp32 version used.
        constexpr int LDT = DK + 8;    // [NB][DK] transposed state blocks
        constexpr int LDN = NB + 8;    // [rows][NB] blocks as they are
        constexpr int LDM = C + 8;     // [C][C] matrices and [NB][C] transposed value blocks
        static_assert(2 * NB * LDT * 2 + 2 * DK * LDN * 2 <= C * LDK * 4, "state blocks fit over q^");
        static_assert(3 * C * LDM * 2 <= 2 * C * LDC * 4 && LY::T == LY::P + (size_t)C * LDC * 4, "T, P^T, T^T fit over P and T");
        static_assert(3 * NB * LDM * 2 + 4 * C * LDN * 2 <= 4 * C * LDB * 4, "value blocks fit over the fp32 value tiles");
        __bf16* bS0T = reinterpret_cast<__bf16*>(sQ);          // [NB][LDT]: S0 block, transposed
        __bf16* bDST = bS0T + NB * LDT;                        // [NB][LDT]: dS block, transposed
        __bf16* bS0 = bDST + NB * LDT;                         // [DK][LDN]
        __bf16* bDS = bS0 + DK * LDN;                          // [DK][LDN]
        __bf16* bT = reinterpret_cast<__bf16*>(sP);            // [C][LDM]: T
        __bf16* bPT = bT + C * LDM;                            // [C][LDM]: P^T
        __bf16* bTT = bPT + C * LDM;                           // [C][LDM]: T^T
        __bf16* bBRT = reinterpret_cast<__bf16*>(sR);          // [NB][LDM]: (diag(beta) R)^T
        __bf16* bDOT = bBRT + NB * LDM;                        // [NB][LDM]: dO^T
        __bf16* bDUT = bDOT + NB * LDM;                        // [NB][LDM]: dU^T
        __bf16* bU = bDUT + NB * LDM;                          // [C][LDN]: U
        __bf16* bDO = bU + C * LDN;                            // [C][LDN]: dO
        __bf16* bDUt = bDO + C * LDN;                          // [C][LDN]: dU~
        __bf16* bBDUt = bDUt + C * LDN;                        // [C][LDN]: -diag(beta) dU~
        auto rd8 = [](const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); };
        auto rd4 = [](const __bf16* p) { return *reinterpret_cast<const bf16x4*>(p); };
        auto neg4 = [](bf16x4 x) {   // exact sign flip
            typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
            return __builtin_bit_cast(bf16x4, __builtin_bit_cast(u16x4, x) ^ (uint16_t)0x8000);
        };
        {   // read every source element first, then overwrite P and T
            constexpr int NEL = C * C / NTH;
            static_assert(C * C % NTH == 0, "whole elements per thread");
            __bf16 xt[NEL], xp[NEL], xtt[NEL];
#pragma unroll
            for (int k = 0; k < NEL; ++k) {
                const int idx = t + k * NTH, i = idx / C, j = idx % C;
                xt[k] = (__bf16)sT[i * LDC + j];
                xp[k] = (__bf16)sP[j * LDC + i];
                xtt[k] = (__bf16)sT[j * LDC + i];
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < NEL; ++k) {
                const int idx = t + k * NTH, i = idx / C, j = idx % C;
                bT[i * LDM + j] = xt[k];
                bPT[i * LDM + j] = xp[k];
                bTT[i * LDM + j] = xtt[k];
            }
        }
        // FULL: the chunk holds C tokens, so the dv and dg stores are
        // unconditional (a store under a branch leaves the compiler unsure how
        // many accesses are in flight, and its later waits then also wait for
        // those stores and for the next block's inputs)
        auto column_loop = [&](auto full) {
            constexpr bool FULL = decltype(full)::value;
            for (int vb = 0; vb < DV / NB; ++vb) {
                const int col0 = NB * vb;
                // S0 and dS, this block's columns: rows 4 (idx / 16) .. + 3 of column idx % 16 per piece
#pragma unroll
                for (int j = 0; j < NSI; ++j) {
                    const int idx = t + j * NTH;
                    if (idx < DK * NB / 4) {
                        const int r0 = 4 * (idx / 16), c = idx % 16;
                        const f32x4 x = pre.s[j], y = pre.d[j];
                        *reinterpret_cast<bf16x4*>(bS0T + c * LDT + r0) = to_bf16x4(x);
                        *reinterpret_cast<bf16x4*>(bDST + c * LDT + r0) = to_bf16x4(y);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            bS0[(r0 + e) * LDN + c] = (__bf16)x[e];
                            bDS[(r0 + e) * LDN + c] = (__bf16)y[e];
                        }
                        rowp[j] += x * y;
                    }
                }
                const f32x4 cA = pre.a, cB = pre.b, cC = pre.c;
                pre = fetch(vb + 1);
                __syncthreads();
                f32x4 rr = {0.f, 0.f, 0.f, 0.f};   // half 0: R, kept for dbeta
                f32x4 du = {0.f, 0.f, 0.f, 0.f};   // half 1: Ke dS, then + P^T dO
                if (half == 0) {   // R = V - Kt S0 (rows 16 w4 ..)
#pragma unroll
                    for (int e = 0; e < 4; ++e) rr[e] = 16 * w4 + 4 * g + e < nvalid ? cA[e] : 0.f;
#pragma unroll
                    for (int s = 0; s < NKF; ++s) rr = mma_bf16x32(afr[s], rd8(bS0T + n * LDT + 32 * s + 8 * g), rr);
                    f32x4 br;
#pragma unroll
                    for (int e = 0; e < 4; ++e) br[e] = sBeta[16 * w4 + 4 * g + e] * rr[e];
                    *reinterpret_cast<bf16x4*>(bBRT + n * LDM + 16 * w4 + 4 * g) = to_bf16x4(br);
                } else {           // dO = d_out * sigmoid(g); dg = d_out * out * (1 - sigmoid(g)); Ke dS
                    f32x4 dov;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 16 * w4 + 4 * g + e;
                        const size_t ri = rowi(i) * DV + col0 + n;
                        const float dy = cA[e];
                        const float sg = sigmoidf_(cB[e]);
                        dov[e] = i < nvalid ? dy * sg : 0.f;
                        bDO[i * LDN + n] = (__bf16)dov[e];
                        if (FULL || i < nvalid) dgp[ri] = from_f32<E>(dy * cC[e] * (1.f - sg));
                    }
                    *reinterpret_cast<bf16x4*>(bDOT + n * LDM + 16 * w4 + 4 * g) = to_bf16x4(dov);
#pragma unroll
                    for (int s = 0; s < NKF; ++s) du = mma_bf16x32(afr[s], rd8(bDST + n * LDT + 32 * s + 8 * g), du);
                }
                __syncthreads();
                if (half == 0) {   // U = T diag(beta) R (T lower triangular: its tiles past block w4 are zero)
                    f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 2; ++s)
                        u = mma_bf16x32(rd8(bT + (16 * w4 + n) * LDM + 32 * s + 8 * g), rd8(bBRT + n * LDM + 32 * s + 8 * g), u);
#pragma unroll
                    for (int e = 0; e < 4; ++e) bU[(16 * w4 + 4 * g + e) * LDN + n] = (__bf16)u[e];
                } else {           // dU = (Ke dS, from the previous phase) + P^T dO (P^T upper triangular)
#pragma unroll
                    for (int s = 0; s < 2; ++s)
                        du = mma_bf16x32(rd8(bPT + (16 * w4 + n) * LDM + 32 * s + 8 * g), rd8(bDOT + n * LDM + 32 * s + 8 * g), du);
                    *reinterpret_cast<bf16x4*>(bDUT + n * LDM + 16 * w4 + 4 * g) = to_bf16x4(du);
                }
                __syncthreads();
                if (half == 0) {   // dU~ = T^T dU (T^T upper triangular); dv = diag(beta) dU~; dbeta += dU~ . R
                    f32x4 dut = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 2; ++s)
                        dut = mma_bf16x32(rd8(bTT + (16 * w4 + n) * LDM + 32 * s + 8 * g), rd8(bDUT + n * LDM + 32 * s + 8 * g), dut);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 16 * w4 + 4 * g + e;
                        if (FULL || i < nvalid) dvp[rowi(i) * DV + col0 + n] = from_f32<E>(sBeta[i] * dut[e]);
                        dbp[e] += dut[e] * rr[e];
                        bDUt[i * LDN + n] = (__bf16)dut[e];
                        bBDUt[i * LDN + n] = (__bf16)(-sBeta[i] * dut[e]);
                    }
                } else {           // dP += dO U^T (all column tiles; those above the diagonal are discarded)
                    const bf16x4 ao = rd4(bDO + (16 * w4 + n) * LDN + 4 * g);
#pragma unroll
                    for (int j = 0; j < 4; ++j) dMP[j] = mma_bf16(ao, rd4(bU + (16 * j + n) * LDN + 4 * g), dMP[j]);
                }
                __syncthreads();
                if (half == 0) {   // dM -= dU~ U^T (all column tiles; those above the diagonal are discarded)
                    const bf16x4 am = neg4(rd4(bDUt + (16 * w4 + n) * LDN + 4 * g));
#pragma unroll
                    for (int j = 0; j < 4; ++j) dMP[j] = mma_bf16(am, rd4(bU + (16 * j + n) * LDN + 4 * g), dMP[j]);
                }
                // dQt += dO S0^T, dKt -= (diag(beta) dU~) S0^T, dKe += U dS^T (this half's channel tiles; the
                // block's 16 value columns are one bf16 k-step)
                const int ra = (16 * w4 + n) * LDN + 4 * g;
                const bf16x4 ao = rd4(bDO + ra), ar = rd4(bBDUt + ra), au = rd4(bU + ra);
#pragma unroll
                for (int c2 = 0; c2 < NTH2; ++c2) {
                    const int si = (16 * (ct0 + c2) + n) * LDN + 4 * g;
                    const bf16x4 b0 = rd4(bS0 + si), b1 = rd4(bDS + si);
                    aQ[c2] = mma_bf16(ao, b0, aQ[c2]);
                    aK[c2] = mma_bf16(ar, b0, aK[c2]);
                    aE[c2] = mma_bf16(au, b1, aE[c2]);
                }
                __syncthreads();
            }
        };
        if (nvalid == C) column_loop(std::true_type{});
        else column_loop(std::false_type{});
    } else {
        for (int vb = 0; vb < DV / NB; ++vb) {
            const int col0 = NB * vb;
            // S0 and dS, this block's columns, to LDS (q^ is reloaded after the loop)
#pragma unroll
            for (int j = 0; j < NSI; ++j) {
                const int idx = t + j * NTH;
                if (idx < DK * NB / 4) {
                    const int r0 = 4 * (idx / 16), c = idx % 16;
                    const f32x4 x = pre.s[j], y = pre.d[j];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        sS0[(r0 + e) * LDSB + c] = x[e];
                        sDS[(r0 + e) * LDSB + c] = y[e];
                    }
                    rowp[j] += x * y;
                }
            }
            const f32x4 cA = pre.a, cB = pre.b, cC = pre.c;
            pre = fetch(vb + 1);
            __syncthreads();
            f32x4 du = {0.f, 0.f, 0.f, 0.f};   // half 1: Ke dS, then + P^T dO
            if (half == 0) {   // R = V - Kt S0 (rows 16 w4 ..)
                f32x4 r;
#pragma unroll
                for (int e = 0; e < 4; ++e) r[e] = 16 * w4 + 4 * g + e < nvalid ? cA[e] : 0.f;
                if constexpr (BF) {
#pragma unroll
                    for (int s = 0; s < NKF; ++s) r = mma_bf16x32(afr[s], col8(sS0 + (32 * s + 8 * g) * LDSB + n, LDSB), r);
                } else {
#pragma unroll 8
                    for (int s = 0; s < NKD; ++s) r = mma_f32(-Kt(16 * w4 + n, 4 * s + g), sS0[(4 * s + g) * LDSB + n], r);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) sR[(16 * w4 + 4 * g + e) * LDB + n] = r[e];
            } else {           // dO = d_out * sigmoid(g); dg = d_out * out * (1 - sigmoid(g)); Ke dS
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 16 * w4 + 4 * g + e;
                    const size_t ri = rowi(i) * DV + col0 + n;
                    const float dy = cA[e];
                    const float sg = sigmoidf_(cB[e]);
                    sDO[i * LDB + n] = i < nvalid ? dy * sg : 0.f;
                    if (i < nvalid) dgp[ri] = from_f32<E>(dy * cC[e] * (1.f - sg));
                }
                if constexpr (BF) {
#pragma unroll
                    for (int s = 0; s < NKF; ++s) du = mma_bf16x32(afr[s], col8(sDS + (32 * s + 8 * g) * LDSB + n, LDSB), du);
                } else {
#pragma unroll 8
                    for (int s = 0; s < NKD; ++s) du = mma_f32(Ke(16 * w4 + n, 4 * s + g), sDS[(4 * s + g) * LDSB + n], du);
                }
            }
            __syncthreads();
            if (half == 0) {   // U = T diag(beta) R (T lower triangular)
                f32x4 u = {0.f, 0.f, 0.f, 0.f};
                if constexpr (BF) {   // 32-token k-blocks 0, 1 (T's tiles above block w4 are zero)
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const int j0 = 32 * s + 8 * g;
                        bf16x8 bb;
#pragma unroll
                        for (int e = 0; e < 8; ++e) bb[e] = (__bf16)(sBeta[j0 + e] * sR[(j0 + e) * LDB + n]);
                        const float* ta = sT + (16 * w4 + n) * LDC + j0;
                        u = mma_bf16x32(to_bf16x8(ld4s(ta), ld4s(ta + 4)), bb, u);
                    }
                } else {
                    for (int s = 0; s < 4 * (w4 + 1); ++s)
                        u = mma_f32(sT[(16 * w4 + n) * LDC + 4 * s + g], sBeta[4 * s + g] * sR[(4 * s + g) * LDB + n], u);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) sU[(16 * w4 + 4 * g + e) * LDB + n] = u[e];
            } else {           // dU = (Ke dS, from the previous phase) + P^T dO (P^T upper triangular)
                if constexpr (BF) {   // 32-token k-blocks 0, 1 (P^T's tiles below block w4 are zero)
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const int j0 = 32 * s + 8 * g, ci = 16 * w4 + n;
                        du = mma_bf16x32(col8(sP + j0 * LDC + ci, LDC), col8(sDO + j0 * LDB + n, LDB), du);
                    }
                } else {
                    for (int s = 4 * w4; s < NKC; ++s)
                        du = mma_f32(sP[(4 * s + g) * LDC + 16 * w4 + n], sDO[(4 * s + g) * LDB + n], du);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) sDU[(16 * w4 + 4 * g + e) * LDB + n] = du[e];
            }
            __syncthreads();
            f32x4 dut = {0.f, 0.f, 0.f, 0.f};
            if (half == 0) {   // dU~ = T^T dU (T^T upper triangular); dv = diag(beta) dU~; dbeta += dU~ . R
                if constexpr (BF) {   // 32-token k-blocks 0, 1 (T^T's tiles below block w4 are zero)
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const int j0 = 32 * s + 8 * g, ci = 16 * w4 + n;
                        dut = mma_bf16x32(col8(sT + j0 * LDC + ci, LDC), col8(sDU + j0 * LDB + n, LDB), dut);
                    }
                } else {
                    for (int s = 4 * w4; s < NKC; ++s)
                        dut = mma_f32(sT[(4 * s + g) * LDC + 16 * w4 + n], sDU[(4 * s + g) * LDB + n], dut);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {   // dU~ replaces R in LDS (each element by the lane that read it)
                    const int i = 16 * w4 + 4 * g + e;
                    if (i < nvalid) dvp[rowi(i) * DV + col0 + n] = from_f32<E>(sBeta[i] * dut[e]);
                    dbp[e] += dut[e] * sR[i * LDB + n];
                    sR[i * LDB + n] = dut[e];
                }
            } else {           // dP += dO U^T (all column tiles; those above the diagonal are discarded)
                const bf16x4 ao = to_bf16x4(ld4s(sDO + (16 * w4 + n) * LDB + 4 * g));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    {
                        if constexpr (BF) {
                            dMP[j] = mma_bf16(ao, to_bf16x4(ld4s(sU + (16 * j + n) * LDB + 4 * g)), dMP[j]);
                        } else {
#pragma unroll
                            for (int s = 0; s < NB / 4; ++s)
                                dMP[j] = mma_f32(sDO[(16 * w4 + n) * LDB + 4 * s + g], sU[(16 * j + n) * LDB + 4 * s + g],
                                                 dMP[j]);
                        }
                    }
                }
            }
            __syncthreads();
            if (half == 0) {   // dM -= dU~ U^T (all column tiles; those above the diagonal are discarded)
                const bf16x4 am = to_bf16x4(-ld4s(sR + (16 * w4 + n) * LDB + 4 * g));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    {
                        if constexpr (BF) {
                            dMP[j] = mma_bf16(am, to_bf16x4(ld4s(sU + (16 * j + n) * LDB + 4 * g)), dMP[j]);
                        } else {
#pragma unroll
                            for (int s = 0; s < NB / 4; ++s)
                                dMP[j] = mma_f32(-sR[(16 * w4 + n) * LDB + 4 * s + g], sU[(16 * j + n) * LDB + 4 * s + g],
                                                 dMP[j]);
                        }
                    }
                }
            }
            // dQt += dO S0^T, dKt -= (diag(beta) dU~) S0^T, dKe += U dS^T (this half's channel tiles)
            if constexpr (BF) {   // the block's 16 value columns are one bf16 k-step
                const int ra = (16 * w4 + n) * LDB + 4 * g;
                const bf16x4 ao = to_bf16x4(ld4s(sDO + ra));
                const bf16x4 ar = to_bf16x4(-sBeta[16 * w4 + n] * ld4s(sR + ra));
                const bf16x4 au = to_bf16x4(ld4s(sU + ra));
#pragma unroll
                for (int c2 = 0; c2 < NTH2; ++c2) {
                    const int si = (16 * (ct0 + c2) + n) * LDSB + 4 * g;
                    const bf16x4 b0 = to_bf16x4(ld4s(sS0 + si)), b1 = to_bf16x4(ld4s(sDS + si));
                    aQ[c2] = mma_bf16(ao, b0, aQ[c2]);
                    aK[c2] = mma_bf16(ar, b0, aK[c2]);
                    aE[c2] = mma_bf16(au, b1, aE[c2]);
                }
            } else
#pragma unroll
            for (int s = 0; s < NB / 4; ++s) {
                const float ao = sDO[(16 * w4 + n) * LDB + 4 * s + g];
                const float ar = -sBeta[16 * w4 + n] * sR[(16 * w4 + n) * LDB + 4 * s + g];
                const float au = sU[(16 * w4 + n) * LDB + 4 * s + g];
#pragma unroll
                for (int c2 = 0; c2 < NTH2; ++c2) {
                    const int si = (16 * (ct0 + c2) + n) * LDSB + 4 * s + g;
                    const float b0 = sS0[si], b1 = sDS[si];
                    aQ[c2] = mma_f32(ao, b0, aQ[c2]);
                    aK[c2] = mma_f32(ar, b0, aK[c2]);
                    aE[c2] = mma_f32(au, b1, aE[c2]);
                }
            }
            __syncthreads();
        }
    }

    // q^ back over the state blocks: the loads now, the stores after phase 5
    RawPiece qraw[NPC];
    issue_hat(qp, qraw);
    // rowsum(S0 * dS): the 16 columns of a row group sit in 16 adjacent lanes
#pragma unroll
    for (int j = 0; j < NSI; ++j) {
        f32x4 x = rowp[j];
#pragma unroll
        for (int m = 1; m < 16; m <<= 1)
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] += __shfl_xor(x[e], m);
        const int idx = t + j * NTH;
        if (idx < DK * NB / 4 && (idx & 15) == 0) st4(sDGC + 4 * DK + 4 * (idx / 16), x);
    }

    // ---- 5: dbeta, dA -> sT (half 0); dP -> sP (half 1) ----
    if (half == 0) {
        f32x4 db = dbp;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) db[e] += dMP[j][e] * As[j][e];   // As: strictly lower, zero for j > w4
#pragma unroll
        for (int m = 1; m < 16; m <<= 1)
#pragma unroll
            for (int e = 0; e < 4; ++e) db[e] += __shfl_xor(db[e], m);
        if (n == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * w4 + 4 * g + e;
                if (i < nvalid) a.dbeta[rowi(i)] = db[e];
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * w4 + 4 * g + e, jj = 16 * j + n;
            if (half == 0) sT[i * LDC + jj] = (j <= w4 && jj < i) ? sBeta[i] * dMP[j][e] : 0.f;   // dA
            else sP[i * LDC + jj] = (j <= w4 && jj <= i) ? dMP[j][e] : 0.f;                      // dP
        }
    store_hat(qraw, sQ, sRq);
    __syncthreads();

    // ---- 6: dQt += dP Kh, dKt += dA Kh, dKh = dP^T Qt + dA^T Kt ----
    f32x4 aH[NTH2];
#pragma unroll
    for (int c2 = 0; c2 < NTH2; ++c2) aH[c2] = f32x4{0.f, 0.f, 0.f, 0.f};
    // fp32 for every I/O type: dgamma takes differences of these products
    // (dKt Kt - dKh Kh), and bf16 operands here doubled its error
    {
        for (int s4 = 0; s4 <= w4; ++s4)
#pragma unroll
        for (int s = 4 * s4; s < 4 * s4 + 4; ++s) {
            const float ap = sP[(16 * w4 + n) * LDC + 4 * s + g], aa = sT[(16 * w4 + n) * LDC + 4 * s + g];
#pragma unroll
            for (int c2 = 0; c2 < NTH2; ++c2) {
                const float kh = Kh(4 * s + g, 16 * (ct0 + c2) + n);
                aQ[c2] = mma_f32(ap, kh, aQ[c2]);
                aK[c2] = mma_f32(aa, kh, aK[c2]);
            }
        }
        for (int s4 = w4; s4 < 4; ++s4)
#pragma unroll
        for (int s = 4 * s4; s < 4 * s4 + 4; ++s) {
            const float ap = sP[(4 * s + g) * LDC + 16 * w4 + n], aa = sT[(4 * s + g) * LDC + 16 * w4 + n];
#pragma unroll
            for (int c2 = 0; c2 < NTH2; ++c2) {
                const int ch = 16 * (ct0 + c2) + n;
                aH[c2] = mma_f32(ap, Qt(4 * s + g, ch), aH[c2]);
                aH[c2] = mma_f32(aa, Kt(4 * s + g, ch), aH[c2]);
            }
        }
    }

    // ---- 7: through the decay folding: dq^ (aQ), dk^ (aK), dgamma (aH), in place ----
#pragma unroll
    for (int c2 = 0; c2 < NTH2; ++c2) {
        const int ch = 16 * (ct0 + c2) + n;
        const float egc = sEG[(C - 1) * LDK + ch];
        float gsum = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * w4 + 4 * g + e;
            const float kh = sK[i * LDK + ch], qh = sQ[i * LDK + ch], eg = sEG[i * LDK + ch];
            const float ieg = __builtin_amdgcn_rcpf(eg);
            const float ktv = kh * eg, khv = kh * ieg, qtv = qh * eg, kev = khv * egc;
            const float dqt = aQ[c2][e], dkt = aK[c2][e], dkhv = aH[c2][e], dke = aE[c2][e];
            aQ[c2][e] = dqt * eg;                                           // dq^
            aK[c2][e] = dkt * eg + dkhv * ieg + dke * egc * ieg;            // dk^
            aH[c2][e] = dkt * ktv - dkhv * khv + dqt * qtv - dke * kev;     // dgamma
            gsum += dke * kev;
        }
        gsum += __shfl_xor(gsum, 16);
        gsum += __shfl_xor(gsum, 32);
        if (g == 0) sDGC[w4 * DK + ch] = gsum;
    }
    // ---- 8: L2 normalisation: dx = (dx^ - x^ (x^ . dx^)) / |x| (constant divisor below 1e-6) ----
    {
        f32x4 kd = {0.f, 0.f, 0.f, 0.f}, qd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c2 = 0; c2 < NTH2; ++c2)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * w4 + 4 * g + e, ch = 16 * (ct0 + c2) + n;
                kd[e] += sK[i * LDK + ch] * aK[c2][e];
                qd[e] += sQ[i * LDK + ch] * aQ[c2][e];
            }
#pragma unroll
        for (int m = 1; m < 16; m <<= 1)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kd[e] += __shfl_xor(kd[e], m);
                qd[e] += __shfl_xor(qd[e], m);
            }
        if (n == 0) {   // this half's share of the per-token dot products
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sXD[(2 * half) * C + 16 * w4 + 4 * g + e] = kd[e];
                sXD[(2 * half + 1) * C + 16 * w4 + 4 * g + e] = qd[e];
            }
        }
        __syncthreads();
        // a lane holds four tokens of one channel: dk and dq replace k^ and q^
        // in LDS (each element by the lane that read it), then go out as
        // whole 8-channel pieces of a token
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * w4 + 4 * g + e;
            const float nk = sNk[i], nq = sNq[i], rk = sRk[i], rq = sRq[i];
            const float kdi = sXD[i] + sXD[2 * C + i], qdi = sXD[C + i] + sXD[3 * C + i];
#pragma unroll
            for (int c2 = 0; c2 < NTH2; ++c2) {
                const int ch = 16 * (ct0 + c2) + n;
                float* kk = sK + i * LDK + ch;
                float* qq = sQ + i * LDK + ch;
                // rk = 1 / max(|k|, 1e-6): below the floor the normaliser is the constant 1e6
                const float dkx = (nk < 1e-6f ? aK[c2][e] : aK[c2][e] - *kk * kdi) * rk;
                const float dqx = (nq < 1e-6f ? aQ[c2][e] : aQ[c2][e] - *qq * qdi) * rq;
                *kk = dkx;
                *qq = dqx;
            }
        }
        __syncthreads();
        E* dkp = reinterpret_cast<E*>(a.dk);
        E* dqp = reinterpret_cast<E*>(a.dq);
        for (int idx = t; idx < nvalid * (DK / 8); idx += NTH) {
            const int i = idx / (DK / 8), ch = (idx % (DK / 8)) * 8;
            const size_t ri = rowi(i) * DK + ch;
            st4(dkp + ri, ld4s(sK + i * LDK + ch));
            st4(dkp + ri + 4, ld4s(sK + i * LDK + ch + 4));
            st4(dqp + ri, ld4s(sQ + i * LDK + ch));
            st4(dqp + ri + 4, ld4s(sQ + i * LDK + ch + 4));
        }
    }
    // ---- 9: dgamma to LDS (over dP and dA, read for the last time in phase 6) ----
#pragma unroll
    for (int c2 = 0; c2 < NTH2; ++c2)
#pragma unroll
        for (int e = 0; e < 4; ++e) sDG[(16 * w4 + 4 * g + e) * LDK + 16 * (ct0 + c2) + n] = aH[c2][e];
    __syncthreads();
    // ---- 10: dlog_alpha = reverse cumulative sum of dgamma (zero where the floor binds) ----
    if (t < DK) {   // in place, channel t
        float acc = sDGC[t] + sDGC[DK + t] + sDGC[2 * DK + t] + sDGC[3 * DK + t] +
                    sEG[(C - 1) * LDK + t] * sDGC[4 * DK + t];
        for (int i = nvalid - 1; i >= 0; --i) {
            acc += sDG[i * LDK + t];
            sDG[i * LDK + t] = acc;
        }
    }
    __syncthreads();
    for (int idx = t; idx < nvalid * (DK / 4); idx += NTH) {
        const int i = idx / (DK / 4), ch = (idx % (DK / 4)) * 4;
        const size_t r = rowi(i) * DK + ch;
        const f32x4 la = *reinterpret_cast<const f32x4*>(a.log_alpha + r);
        const f32x4 acc = *reinterpret_cast<const f32x4*>(sDG + i * LDK + ch);
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = la[e] > a.floor_ ? acc[e] : 0.f;
        *reinterpret_cast<f32x4*>(a.dlog_alpha + r) = y;
    }
}

template <typename E, int DK, bool VL>
hipError_t launch_backward_t(const BackwardArgs& a, hipStream_t s) {
    const int64_t BH = a.B * (int64_t)a.H;
    if (BH == 0) return hipSuccess;
    // one workgroup per chunk-head; a packed batch launches as many as its
    // sequences can have chunks, and those past the last chunk return
    const int64_t chunks = VL ? ((a.T + kChunk - 1) / kChunk + a.B) * a.H : BH * a.NC;
    if (chunks > 0) {
        hipLaunchKernelGGL((kda_bwd_card_kernel<E, DK, VL>), dim3((unsigned)chunks), dim3(kThreads), 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t groups = (BH + kXcds - 1) / kXcds;
    hipLaunchKernelGGL((kda_bwd_scan_kernel<E, DK, VL>), dim3((unsigned)(groups * kXcds * (DK / 16))), dim3(kThreads),
                       0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || chunks == 0) return e;
    hipLaunchKernelGGL((kda_bwd_grad_kernel<E, DK, VL>), dim3((unsigned)chunks), dim3(kGradThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(bool bf16, int64_t B, int64_t T, int H, int dk, bool varlen) {
    return T == 0 ? 0 : BwdLayout(bf16, B, T, H, dk, varlen).total;
}

hipError_t launch_backward_forward(bool bf16, int dk, const BackwardArgs& a, void* out, float* state_out,
                                   hipStream_t s) {
    const bool vl = a.cu_seqlens != nullptr;
    if (a.B == 0 || (vl ? a.T == 0 : a.NC == 0)) return hipSuccess;
    const BwdLayout L(bf16, a.B, a.T, a.H, dk, vl);
    PrepareArgs p = {};
    p.q = a.q; p.k = a.k; p.v = a.v; p.log_alpha = a.log_alpha; p.beta = a.beta;
    p.ws = a.ws + L.cards;
    p.B = a.B; p.T = a.T; p.H = a.H; p.NC = a.NC; p.floor_ = a.floor_;
    if (vl) {   // the plan kernel writes the chunk offsets and the chunk -> sequence map first
        p.cu_seqlens = a.cu_seqlens;
        p.chunk_off = reinterpret_cast<int64_t*>(a.ws + L.offs);
        p.chunk_seq = reinterpret_cast<int32_t*>(a.ws + L.seqmap);
    }
    hipError_t e = launch_prepare(bf16, dk, p, s);
    if (e != hipSuccess) return e;
    ScanArgs f = {};
    f.ws = a.ws + L.cards;
    f.g = a.g; f.state_in = a.state_in; f.out = out; f.state_out = state_out;
    f.states = reinterpret_cast<float*>(a.ws + L.states);
    f.ckpt_every = 1;
    f.states_tiled = true;
    f.B = a.B; f.T = a.T; f.H = a.H; f.NC = a.NC;
    if (vl) {
        f.cu_seqlens = a.cu_seqlens;
        f.chunk_off = p.chunk_off;
    }
    return launch_scan(bf16, dk, false, f, s);
}

hipError_t launch_backward(bool bf16, int dk, const BackwardArgs& a, bool recompute, hipStream_t s) {
    BackwardArgs b = a;
    const bool vl = a.cu_seqlens != nullptr;
    const BwdLayout L(bf16, a.B, a.T, a.H, dk, vl);
    if (recompute) {   // forward cards, then the forward hand-off keeping every chunk's entering state
        b.out = a.ws + L.out;
        const hipError_t e = launch_backward_forward(bf16, dk, b, a.ws + L.out, nullptr, s);
        if (e != hipSuccess) return e;
    }
    if (vl) {
        b.chunk_off = reinterpret_cast<const int64_t*>(a.ws + L.offs);
        b.chunk_seq = reinterpret_cast<const int32_t*>(a.ws + L.seqmap);
        if (bf16) return dk == 128 ? launch_backward_t<__bf16, 128, true>(b, s) : launch_backward_t<__bf16, 64, true>(b, s);
        return dk == 128 ? launch_backward_t<float, 128, true>(b, s) : launch_backward_t<float, 64, true>(b, s);
    }
    if (bf16) return dk == 128 ? launch_backward_t<__bf16, 128, false>(b, s) : launch_backward_t<__bf16, 64, false>(b, s);
    return dk == 128 ? launch_backward_t<float, 128, false>(b, s) : launch_backward_t<float, 64, false>(b, s);
}

}  // namespace kda
