// kda_scan.hip -- stage 2 of the chunk method: the ordered state hand-off and
// the gated read-out [zuoshipin.com/article/18261 §四, FlashKDA paragraph:
// only the state hand-off and the output read-out stay sequential], and the
// per-segment summary of the context-parallel scheme [same page, §三,
// "KDA 上下文并行" paragraph].
//
// Per chunk, with the card written by the prepare kernel and S the state
// entering the chunk (fp32, d_k x d_v):
//   U  = Wv - Wk S                      (the chunk's corrected writes)
//   O  = Qt S + P U;  out = O * sigmoid(g)
//   S <- diag(e^gamma_C) S + Ke^T U
//
// The columns of S never interact, so the chain of one (batch row, head) is
// split into d_v/16 independent 16-column chains, one workgroup each; the
// state slice (d_k x 16, fp32) lives in accumulator registers for the whole
// sequence.  Four waves share a chain: wave w owns U/O rows 16w..16w+15 and
// state rows w*d_k/4 .. (w+1)*d_k/4 - 1.  U and the operand copy of S cross
// waves through LDS (two barriers per chunk); the chunk's card operands are
// prefetched from global memory one chunk ahead, straight into registers in
// MFMA operand layout.
//
// Summary mode runs the same hand-off on the augmented state [Bz | A] from
// [0 | I]: the first d_v/16 chains carry value columns (from 0), the next
// d_k/16 chains carry transition columns (from the identity, with no value
// input).  No outputs; the final slices are the summary pair.
//
// Workgroup -> chain mapping is XCD-aware: workgroups are dealt round-robin
// to the 8 XCDs, so the tiles of one head are given ids that are congruent
// mod 8 and share one XCD's L2, where the head's cards are read by all of
// its chains.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

namespace {

constexpr int kXcds = 8;

template <typename E, int DK>
struct ChunkOps {
    using M = MM<E>;
    static constexpr int NKD = DK / M::KS;      // k-steps over d_k
    static constexpr int NKC = kChunk / M::KS;  // k-steps over the chunk's tokens
    static constexpr int MTS = DK / 64;         // 16-row state tiles per wave
    typename M::frag wk[NKD];                   // -Wk rows 16w..16w+15
    typename M::frag qt[NKD];                   // Qt rows 16w..16w+15
    typename M::frag ke[MTS][NKC];              // Ke^T rows of this wave's state tiles
    typename M::frag p[NKC];                    // P rows 16w..16w+15
    f32x4 wv;                                   // Wv tile (accumulator order)
    f32x4 gc[MTS];                              // e^gamma_C for the lane's state rows
};

template <typename E, int DK, bool SUMMARY>
__device__ __forceinline__ void load_ops(ChunkOps<E, DK>& o, const char* card, int w, int g, int n, int lane,
                                         int tile, bool vcols) {
    using M = MM<E>;
    using CL = Card<E, DK>;
    using O = ChunkOps<E, DK>;
    constexpr int KS = M::KS;
    const E* wk = reinterpret_cast<const E*>(card + CL::WK);
    const E* ket = reinterpret_cast<const E*>(card + CL::KET);
#pragma unroll
    for (int s = 0; s < O::NKD; ++s) o.wk[s] = M::neg(ld_frag(wk, DK, 16 * w + n, s * KS, g));
#pragma unroll
    for (int mt = 0; mt < O::MTS; ++mt)
#pragma unroll
        for (int s = 0; s < O::NKC; ++s)
            o.ke[mt][s] = ld_frag(ket, kChunk, (DK / 4) * w + 16 * mt + n, s * KS, g);
#pragma unroll
    for (int mt = 0; mt < O::MTS; ++mt)
        o.gc[mt] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(card + CL::GC) +
                                                   (DK / 4) * w + 16 * mt + 4 * g);
    if (vcols)
        o.wv = ld4(reinterpret_cast<const E*>(card + CL::WV) + ((size_t)(tile * 4 + w) * 64 + lane) * 4);
    else
        o.wv = f32x4{0.f, 0.f, 0.f, 0.f};
    if (!SUMMARY) {
        const E* qt = reinterpret_cast<const E*>(card + CL::QT);
        const E* p = reinterpret_cast<const E*>(card + CL::P);
#pragma unroll
        for (int s = 0; s < O::NKD; ++s) o.qt[s] = ld_frag(qt, DK, 16 * w + n, s * KS, g);
#pragma unroll
        for (int s = 0; s < O::NKC; ++s) o.p[s] = ld_frag(p, kChunk, 16 * w + n, s * KS, g);
    }
}

template <typename E, int DK, bool SUMMARY>
__global__ __launch_bounds__(kThreads, 1) void kda_scan_kernel(ScanArgs a) {
    using M = MM<E>;
    using CL = Card<E, DK>;
    using O = ChunkOps<E, DK>;
    constexpr int C = kChunk, KS = M::KS;
    constexpr int NT = DK / 16;                         // value-column tiles
    constexpr int NTALL = SUMMARY ? 2 * NT : NT;        // + transition-column tiles
    constexpr int PADE = 16 / (int)sizeof(E);
    constexpr int LDS_S = DK + PADE;                    // sS[16][LDS_S]: S^T operand copy
    constexpr int LDS_U = C + PADE;                     // sU[16][LDS_U]: U^T
    constexpr int MTS = O::MTS;

    __shared__ __attribute__((aligned(16))) E sS[16 * LDS_S];
    __shared__ __attribute__((aligned(16))) E sU[16 * LDS_U];

    const int t = threadIdx.x, lane = t & 63, w = t >> 6, g = lane >> 4, n = lane & 15;

    // XCD-aware chain decode
    const int H = a.H, NC = a.NC;
    const int64_t BH = a.B * (int64_t)H;
    const int64_t x = blockIdx.x;
    const int xcd = (int)(x % kXcds);
    const int64_t slot = x / kXcds;
    const int tile = (int)(slot % NTALL);
    const int64_t bh = (slot / NTALL) * kXcds + xcd;
    if (bh >= BH) return;
    const int64_t b = bh / H;
    const int h = (int)(bh % H);
    const bool vcols = tile < NT;                       // value columns (else transition columns)
    const int col0 = (vcols ? tile : tile - NT) * 16;   // first column of this slice

    // ---- initial state slice: rows (DK/4)*w + 16*mt + 4g + e, column col0 + n ----
    f32x4 S[MTS];
#pragma unroll
    for (int mt = 0; mt < MTS; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = (DK / 4) * w + 16 * mt + 4 * g + e;
            float s0 = 0.f;
            if (SUMMARY) {
                if (!vcols) s0 = (r == col0 + n) ? 1.f : 0.f;
            } else if (a.state_in) {
                s0 = a.state_in[((size_t)bh * DK + r) * DK + col0 + n];
            }
            S[mt][e] = s0;
        }
#pragma unroll
    for (int mt = 0; mt < MTS; ++mt) st4(sS + n * LDS_S + (DK / 4) * w + 16 * mt + 4 * g, S[mt]);

    const char* cards = a.ws + (size_t)bh * NC * CL::BYTES;
    const E* gin = reinterpret_cast<const E*>(a.g);
    E* out = reinterpret_cast<E*>(a.out);

    O cur;
    if (NC > 0) load_ops<E, DK, SUMMARY>(cur, cards, w, g, n, lane, tile, vcols);
    __syncthreads();

    for (int c = 0; c < NC; ++c) {
        O nxt;
        const bool more = c + 1 < NC;
        if (more) load_ops<E, DK, SUMMARY>(nxt, cards + (size_t)(c + 1) * CL::BYTES, w, g, n, lane, tile, vcols);

        // gate values for this wave's 16 output rows (issued early)
        const int64_t tbase = (int64_t)c * C + 16 * w + 4 * g;
        float gv[4];
        if (!SUMMARY) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t tt = tbase + e;
                gv[e] = (tt < a.T) ? to_f32(gin[(((size_t)b * a.T + tt) * H + h) * DK + col0 + n]) : 0.f;
            }
        }

        // S operand (B fragments) from the shared copy
        typename M::frag sb[O::NKD];
#pragma unroll
        for (int s = 0; s < O::NKD; ++s) sb[s] = ld_frag(sS, LDS_S, n, s * KS, g);

        // U rows 16w..16w+15 = Wv - Wk S
        f32x4 u = cur.wv;
#pragma unroll
        for (int s = 0; s < O::NKD; ++s) u = M::mma(cur.wk[s], sb[s], u);
        st4(sU + n * LDS_U + 16 * w + 4 * g, u);
        __syncthreads();

        typename M::frag ub[O::NKC];
#pragma unroll
        for (int s = 0; s < O::NKC; ++s) ub[s] = ld_frag(sU, LDS_U, n, s * KS, g);

        // S <- diag(e^gamma_C) S + Ke^T U
#pragma unroll
        for (int mt = 0; mt < MTS; ++mt) {
            f32x4 acc = S[mt] * cur.gc[mt];
#pragma unroll
            for (int s = 0; s < O::NKC; ++s) acc = M::mma(cur.ke[mt][s], ub[s], acc);
            S[mt] = acc;
        }
#pragma unroll
        for (int mt = 0; mt < MTS; ++mt) st4(sS + n * LDS_S + (DK / 4) * w + 16 * mt + 4 * g, S[mt]);

        if (!SUMMARY) {
            // O rows 16w..16w+15 = Qt S_old + P U (P is zero above the diagonal)
            f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < O::NKD; ++s) o = M::mma(cur.qt[s], sb[s], o);
#pragma unroll
            for (int s = 0; s < O::NKC; ++s)
                if (s * KS < 16 * (w + 1)) o = M::mma(cur.p[s], ub[s], o);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t tt = tbase + e;
                if (tt < a.T)
                    out[(((size_t)b * a.T + tt) * H + h) * DK + col0 + n] = from_f32<E>(o[e] * sigmoidf_(gv[e]));
            }
        }
        __syncthreads();
        if (more) cur = nxt;
    }

    // ---- final state slice ----
#pragma unroll
    for (int mt = 0; mt < MTS; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = (DK / 4) * w + 16 * mt + 4 * g + e;
            if (SUMMARY) {
                if (vcols) a.zero_state[((size_t)bh * DK + r) * DK + col0 + n] = S[mt][e];
                else a.transition[((size_t)bh * DK + r) * DK + col0 + n] = S[mt][e];
            } else if (a.state_out) {
                a.state_out[((size_t)bh * DK + r) * DK + col0 + n] = S[mt][e];
            }
        }
}

template <typename E, int DK, bool SUMMARY>
hipError_t launch_scan_t(const ScanArgs& a, hipStream_t s) {
    constexpr int NTALL = SUMMARY ? 2 * (DK / 16) : DK / 16;
    const int64_t BH = a.B * (int64_t)a.H;
    if (BH == 0) return hipSuccess;
    const int64_t groups = (BH + kXcds - 1) / kXcds;
    const int64_t blocks = groups * kXcds * NTALL;
    hipLaunchKernelGGL((kda_scan_kernel<E, DK, SUMMARY>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_scan(bool bf16, int dk, bool summary, const ScanArgs& a, hipStream_t s) {
    if (bf16) {
        if (dk == 128) return summary ? launch_scan_t<__bf16, 128, true>(a, s) : launch_scan_t<__bf16, 128, false>(a, s);
        return summary ? launch_scan_t<__bf16, 64, true>(a, s) : launch_scan_t<__bf16, 64, false>(a, s);
    }
    if (dk == 128) return summary ? launch_scan_t<float, 128, true>(a, s) : launch_scan_t<float, 128, false>(a, s);
    return summary ? launch_scan_t<float, 64, true>(a, s) : launch_scan_t<float, 64, false>(a, s);
}

}  // namespace kda
