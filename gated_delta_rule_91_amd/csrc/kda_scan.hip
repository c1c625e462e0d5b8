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
// split into independent 16-column slices; a workgroup runs one, two or four
// of them, and its state slices (d_k x 16 fp32 each) live in accumulator
// registers for the whole sequence.  (Summaries of bf16 d_k = 128 cards with
// many (row, head) pairs run in kda_scan_wave.hip instead.)  Four waves share a chain: wave w owns
// U/O rows 16w..16w+15 and state rows w*d_k/4 .. (w+1)*d_k/4 - 1.  U and the
// operand copy of S cross waves through LDS (two barriers per chunk); the
// card operands and the gate values are prefetched from global memory four
// chunks ahead (three with four or more slices), straight into registers in MFMA
// operand layout (a register ring, so the dependent chunk loop does not wait
// on memory latency).  Every global load is unconditional: the load counter
// retires in order, so a load under a branch makes the compiler wait for ALL
// outstanding loads, which would drain the ring.  A wave can have at most 63
// vector-memory operations in flight and a chunk costs it 18 loads, so the
// ring is as deep as that allows.
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
#include <type_traits>

#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

namespace {

constexpr int kXcds = 8;

template <typename E, int DK, int NTW>
struct ChunkOps {
    using M = MM<E>;
    static constexpr int NKD = DK / M::KS;      // k-steps over d_k
    static constexpr int NKC = kChunk / M::KS;  // k-steps over the chunk's tokens
    static constexpr int MTS = DK / 64;         // 16-row state tiles per wave
    typename M::frag wk[NKD];                   // Wk rows 16w..16w+15
    typename M::frag qt[NKD];                   // Qt rows 16w..16w+15
    typename M::frag ke[MTS][NKC];              // Ke^T rows of this wave's state tiles
    typename M::frag p[NKC];                    // P rows 16w..16w+15
    float gc;                                   // e^gamma_C of state row (d_k/4)w + (lane mod d_k/4)
    typename Raw4<E>::type wv[NTW];             // Wv tiles (accumulator order), raw
    typename Raw4<E>::type graw[NTW];           // gate pre-activations: token n, columns 4g..4g+3 (raw)
    uint32_t pf;                                // L2 prefetch of a later card (value unused)
};

// Byte offsets of this lane's operand fragments inside a card: the same for
// every chunk, so each load is (uniform card base) + (32-bit lane offset) +
// (immediate), which the compiler issues in the scalar-base form.
template <typename E, int DK, int NTW>
struct LaneOff {
    static constexpr int MTS = DK / 64;
    uint32_t wk, qt, p;
    uint32_t ke[MTS], gc, wv[NTW];
    uint32_t gcol;   // byte offset of this lane's 4 gate/output columns (4g..4g+3) in slice 0
    int grow;        // this lane's gate/output row inside the chunk (16w + n)

    __device__ LaneOff(int w, int g, int n, int lane, int tile0, bool vcols) {
        using M = MM<E>;
        using CL = Card<E, DK>;
        constexpr int FB = M::KF * (int)sizeof(E);          // bytes of one lane fragment
        constexpr int NKD = DK / M::KS, NKC = kChunk / M::KS, SZ = (int)sizeof(E);
        // A operands are in fragment order: block (row block, k step) is 64
        // consecutive lane fragments
        wk = (uint32_t)(CL::WK + (w * NKD * 64 + lane) * FB);
        qt = (uint32_t)(CL::QT + (w * NKD * 64 + lane) * FB);
        p = (uint32_t)(CL::P + (w * NKC * 64 + lane) * FB);
#pragma unroll
        for (int j = 0; j < NTW; ++j)   // transition columns read tile 0 and discard it
            wv[j] = (uint32_t)(CL::WV + (((vcols ? tile0 + j : 0) * 4 + w) * 64 + lane) * 4 * SZ);
#pragma unroll
        for (int mt = 0; mt < MTS; ++mt) {
            ke[mt] = (uint32_t)(CL::KET + ((((DK / 64) * w + mt) * NKC) * 64 + lane) * FB);
        }
        // one dword per lane: the wave's d_k/4 state rows (repeated across lanes)
        gc = (uint32_t)(CL::GC + ((DK / 4) * w + lane % (DK / 4)) * 4);
        gcol = (uint32_t)(4 * g * SZ);
        grow = 16 * w + n;
    }
};

template <typename T>
__device__ __forceinline__ T ldc(const char* base, uint32_t off) {
    return *reinterpret_cast<const T*>(base + off);
}

// card: this chunk's card (uniform); gbase: the chunk's first token row of g
// at column col0 (uniform); rsb: bytes between tokens; nvalid: tokens of
// this chunk inside the sequence (rows past it re-read the last one)
template <typename E, int DK, int NTW, bool SUMMARY>
__device__ __forceinline__ void load_ops(ChunkOps<E, DK, NTW>& o, const char* card, const LaneOff<E, DK, NTW>& lo,
                                         const char* gbase, uint32_t rsb, int nvalid) {
    using M = MM<E>;
    using O = ChunkOps<E, DK, NTW>;
    typedef typename M::frag F;
    constexpr int KSB = 64 * M::KF * (int)sizeof(E);   // bytes per fragment block (one k-step)
#pragma unroll
    for (int s = 0; s < O::NKD; ++s) o.wk[s] = ldc<F>(card, lo.wk + s * KSB);
#pragma unroll
    for (int mt = 0; mt < O::MTS; ++mt)
#pragma unroll
        for (int s = 0; s < O::NKC; ++s) o.ke[mt][s] = ldc<F>(card, lo.ke[mt] + s * KSB);
    o.gc = ldc<float>(card, lo.gc);
#pragma unroll
    for (int j = 0; j < NTW; ++j) o.wv[j] = ldc<typename Raw4<E>::type>(card, lo.wv[j]);
    if (!SUMMARY) {
#pragma unroll
        for (int s = 0; s < O::NKD; ++s) o.qt[s] = ldc<F>(card, lo.qt + s * KSB);
#pragma unroll
        for (int s = 0; s < O::NKC; ++s) o.p[s] = ldc<F>(card, lo.p + s * KSB);
        const int r = lo.grow < nvalid ? lo.grow : nvalid - 1;
#pragma unroll
        for (int j = 0; j < NTW; ++j)
            o.graw[j] = ldc<typename Raw4<E>::type>(gbase, (uint32_t)r * rsb + lo.gcol + 16 * j * (int)sizeof(E));
    }
}

// One workgroup = NTW adjacent 16-column slices of one (batch row, head):
// the card fragments a wave loads serve all NTW slices.
// Depth of the operand ring (chunks of card fragments in flight per wave):
// four, or three for four or more slices per workgroup, or two for fp32 at d_k = 128 (register file), and how far
// past the chunk a ring load fetches the L2 prefetch runs.
constexpr int kRing4 = 4;
constexpr int kPrefetch = kRing4 + 1;
// With two or more slices per workgroup an XCD's L2 serves two to four times
// as many (row, head) chains, each pulling about 74 KB per chunk: a line
// pulled kPrefetch chunks past the ring load (about nine chunks before its
// use) has then left the 4 MB L2 before the ring reads it.  Measured: pulling
// the chunk one past the ring load is 7% faster on the medium workload's
// two-slice scan and 2-3% on the 1M-token segmented summaries and recompute.
constexpr int kPrefetchMulti = 1;

// CKPT: 0 no checkpoints; 1 the state entering every chunk (unconditional
// stores); 2 every ckpt_every chunks (a branch around the stores: the cheaper
// choice when checkpoints are sparse); 3 the state entering every chunk in
// the backward's tiled layout (one 16-byte store per lane and 16-row tile),
// no final-state slot; NC + 1 slots per (row, head), or for a packed batch
// one slot per chunk-head, indexed like the cards
template <typename E, int DK, int NTW, bool SUMMARY, int CKPT>
__global__ __launch_bounds__(kThreads, 1) void kda_scan_kernel(ScanArgs a) {
    using M = MM<E>;
    using CL = Card<E, DK>;
    using O = ChunkOps<E, DK, NTW>;
    constexpr int C = kChunk, KS = M::KS;
    constexpr int NT = DK / 16;                         // value-column tiles
    constexpr int NTALL = SUMMARY ? 2 * NT : NT;        // + transition-column tiles
    constexpr int NWG = NTALL / NTW;                    // workgroups per (batch row, head)
    constexpr int PADE = 16 / (int)sizeof(E);
    constexpr int LDS_S = DK + PADE;                    // sS[16*NTW][LDS_S]: S^T operand copy
    constexpr int LDS_U = C + PADE;                     // sU[16*NTW][LDS_U]: U^T
    constexpr int MTS = O::MTS;
    static_assert(NT % NTW == 0, "slices of one workgroup never straddle value/transition columns");

    __shared__ __attribute__((aligned(16))) E sS[16 * NTW * LDS_S];
    __shared__ __attribute__((aligned(16))) E sU[16 * NTW * LDS_U];

    const int t = threadIdx.x, lane = t & 63, w = t >> 6, g = lane >> 4, n = lane & 15;

    // XCD-aware chain decode
    const int H = a.H;
    const int64_t BH = a.B * (int64_t)H;
    const int64_t x = blockIdx.x;
    const int xcd = (int)(x % kXcds);
    const int64_t slot = x / kXcds;
    const int tile0 = (int)(slot % NWG) * NTW;
    const int64_t bh = (slot / NWG) * kXcds + xcd;
    if (bh >= BH) return;
    const int64_t b = bh / H;
    const int h = (int)(bh % H);
    const SeqSpan sp = seq_span(a.cu_seqlens, a.chunk_off, a.T, a.row_stride, a.NC, a.B, b, h, H);
    const int NC = sp.nc;
    const int64_t Tl = sp.len;   // this sequence's tokens
    const bool vcols = tile0 < NT;                        // value columns (else transition columns)
    const int col0 = (vcols ? tile0 : tile0 - NT) * 16;   // first column of this workgroup

    // ---- initial state: slice j, rows (DK/4)*w + 16*mt + 4g + e, column col0 + 16j + n ----
    f32x4 S[NTW][MTS];
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int mt = 0; mt < MTS; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = (DK / 4) * w + 16 * mt + 4 * g + e;
                const int col = col0 + 16 * j + n;
                float s0 = 0.f;
                if (SUMMARY) {
                    if (!vcols) s0 = (r == col) ? 1.f : 0.f;
                } else if (a.state_in) {
                    s0 = a.state_in[((size_t)bh * DK + r) * DK + col];
                }
                S[j][mt][e] = s0;
            }
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int mt = 0; mt < MTS; ++mt) st4(sS + (16 * j + n) * LDS_S + (DK / 4) * w + 16 * mt + 4 * g, S[j][mt]);

    const char* cards = a.ws + (size_t)sp.card0 * CL::BYTES;
    const LaneOff<E, DK, NTW> lo(w, g, n, lane, tile0, vcols);
    const uint32_t rsb = (uint32_t)(H * DK * (int)sizeof(E));              // bytes between tokens
    // first token row of this (b, h) at column col0, as bytes, for g and out
    const size_t head0 = (((size_t)sp.tok0 * H + h) * DK + col0) * sizeof(E);
    const char* gseq = reinterpret_cast<const char*>(a.g) + head0;
    char* oseq = reinterpret_cast<char*>(a.out) + head0;

    // prefetches past the last chunk re-read the last card (never used), so
    // the steady-state loop has no branches around its loads
    // The workgroups of one (row, head) read the same cards; each also pulls
    // its share of the card kPrefetch (one slice per workgroup) or
    // kPrefetchMulti chunks past the ring into L2 (one dword
    // per 128-byte line), so the ring loads of all of them hit in L2 instead of
    // all waiting on the same HBM misses.  Summaries, which have no read-out,
    // pull only what all their slices share, Wk and Ke^T.  (The read-out scan
    // measured slower with only its shared operands pulled, so it pulls the
    // whole card, Wv and e^gamma_C included.)
    constexpr size_t RA = SUMMARY ? CL::QT : CL::BYTES;                       // [0, RA): Wk (or all)
    constexpr size_t RB0 = SUMMARY ? CL::KET : 0, RB1 = SUMMARY ? CL::P : 0;  // Ke^T
    constexpr int NLA = (int)(RA / 128);
    constexpr int NL = NLA + (int)((RB1 - RB0) / 128);         // lines pulled per card
    constexpr int LPW = (NL + NWG - 1) / NWG;                  // lines per workgroup
    const int pline = (int)(slot % NWG) * LPW + (w * 64 + lane < LPW ? w * 64 + lane : LPW - 1);
    const int pl = pline < NL ? pline : NL - 1;
    const uint32_t poff = (uint32_t)(pl < NLA ? (size_t)pl * 128 : RB0 + (size_t)(pl - NLA) * 128);
    auto load = [&](O& o, int c) {
        const int cc = c < NC ? c : NC - 1;
        const int64_t t0 = (int64_t)cc * C;
        const int nvalid = (int)(Tl - t0 < C ? Tl - t0 : C);
        load_ops<E, DK, NTW, SUMMARY>(o, cards + (size_t)cc * CL::BYTES, lo, gseq + (size_t)t0 * rsb, rsb, nvalid);
        constexpr int PFD = NTW == 1 ? kPrefetch : kPrefetchMulti;
        const int cp = c + PFD < NC ? c + PFD : NC - 1;
        o.pf = ldc<uint32_t>(cards + (size_t)cp * CL::BYTES, poff);
    };

    // FULL: the chunk holds C tokens, so its output stores are unconditional
    // (a store under a branch leaves the compiler unsure how many accesses are
    // in flight, and every later wait would tighten by one)
    auto step = [&](auto full, const O& cur, int c) {
        constexpr bool FULL = decltype(full)::value;
        asm volatile("" ::"v"(cur.pf));   // the prefetch retires with the slot
        if constexpr (CKPT == 3) {   // the state entering chunk c, tiled (a packed batch: at the card's slot)
            float* dst = a.states + (a.cu_seqlens ? (size_t)sp.card0 + c : (size_t)bh * (NC + 1) + c) * DK * DK;
#pragma unroll
            for (int j = 0; j < NTW; ++j)
#pragma unroll
                for (int mt = 0; mt < MTS; ++mt)
                    *reinterpret_cast<f32x4*>(dst + tiled_state_index(DK, tile0 + j, (DK / 16) * w + 4 * mt + g, n)) =
                        S[j][mt];
        } else if constexpr (CKPT != 0) {   // the state entering chunk c, to slot c / every
            const int every = CKPT == 1 ? 1 : a.ckpt_every;
            const int64_t nslot = ((int64_t)NC + every - 1) / every + 1;
            if (CKPT == 1 || c % every == 0) {
                float* dst = a.states + ((size_t)bh * nslot + c / every) * DK * DK + col0 + n;
#pragma unroll
                for (int j = 0; j < NTW; ++j)
#pragma unroll
                    for (int mt = 0; mt < MTS; ++mt)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            dst[(size_t)((DK / 4) * w + 16 * mt + 4 * g + e) * DK + 16 * j] = S[j][mt][e];
            }
        }
        // S operand (B fragments) from the shared copy
        typename M::frag sb[NTW][O::NKD];
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int s = 0; s < O::NKD; ++s) sb[j][s] = ld_frag(sS + 16 * j * LDS_S, LDS_S, n, s * KS, g);

        // U rows 16w..16w+15 = Wv - Wk S = -((-Wv) + Wk S)
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            f32x4 u = vcols ? -widen4(cur.wv[j]) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < O::NKD; ++s) u = M::mma(cur.wk[s], sb[j][s], u);
            st4(sU + (16 * j + n) * LDS_U + 16 * w + 4 * g, -u);
        }
        __syncthreads();

        typename M::frag ub[NTW][O::NKC];
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int s = 0; s < O::NKC; ++s) ub[j][s] = ld_frag(sU + 16 * j * LDS_U, LDS_U, n, s * KS, g);

        // S <- diag(e^gamma_C) S + Ke^T U; lane (g, n) takes e^gamma_C of its
        // rows 16mt + 4g + e from the lanes that loaded them
        f32x4 gcv[MTS];
#pragma unroll
        for (int mt = 0; mt < MTS; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                gcv[mt][e] = __int_as_float(
                    __builtin_amdgcn_ds_bpermute((16 * mt + 4 * g + e) * 4, __float_as_int(cur.gc)));
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int mt = 0; mt < MTS; ++mt) {
                f32x4 acc = S[j][mt] * gcv[mt];
#pragma unroll
                for (int s = 0; s < O::NKC; ++s) acc = M::mma(cur.ke[mt][s], ub[j][s], acc);
                S[j][mt] = acc;
            }
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int mt = 0; mt < MTS; ++mt) st4(sS + (16 * j + n) * LDS_S + (DK / 4) * w + 16 * mt + 4 * g, S[j][mt]);

        if (!SUMMARY) {
            char* ochunk = oseq + (size_t)c * C * rsb;
            const int nvalid = (int)(Tl - (int64_t)c * C < C ? Tl - (int64_t)c * C : C);
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                // O^T (16 columns x this wave's 16 tokens) = S_old^T Qt^T + U^T P^T.
                // A 16x16 A fragment and B fragment share one lane layout, so
                // the S/U B fragments serve as the A operands and the Qt/P A
                // fragments as the B operands.  Lane (g, n) then holds token
                // 16w + n, columns 4g..4g+3: one 4-element gate load and one
                // 4-element output store.  (P is zero above the diagonal, so
                // the full k range is exact.)
                f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < O::NKD; ++s) o = M::mma(sb[j][s], cur.qt[s], o);
#pragma unroll
                for (int s = 0; s < O::NKC; ++s) o = M::mma(ub[j][s], cur.p[s], o);
                const f32x4 gg = widen4(cur.graw[j]);
                f32x4 y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = o[e] * sigmoidf_(gg[e]);
                // keep the gate math out of the store branch below: inside a
                // branch the compiler would wait for every outstanding load
                if (!FULL) asm volatile("" ::"v"(y[0]), "v"(y[1]), "v"(y[2]), "v"(y[3]));
                if (FULL || lo.grow < nvalid)
                    st4(reinterpret_cast<E*>(ochunk + (uint32_t)lo.grow * rsb + lo.gcol + 16 * j * (int)sizeof(E)), y);
            }
        }
        __syncthreads();
    };

    // kRing chunks of operands in flight: chunk c + kRing is requested as soon
    // as chunk c's registers are free.  The loop body is branch-free so the
    // load-counter waits stay exact.  It runs over full chunks only; the
    // rest (fewer than kRing full chunks, then a partial one) finish in the
    // tail from the slots already loaded.  (Named ring slots: an array of
    // them allocates worse.)  fp32 operands at d_k = 128 take twice the
    // registers per chunk: a two-deep ring keeps them out of scratch memory
    // (measured 1.96 -> 0.48 ms on 8K tokens x 32 heads with one slice per
    // workgroup, 1.55 -> 0.39 ms with two, 1.61 -> 0.80 ms with four).
    constexpr int kRing = (sizeof(E) == 4 && DK == 128) ? 2 : (NTW >= 4 ? 3 : kRing4);
    static_assert(kRing >= 2 && kRing <= 4, "ring depth");
    if (NC > 0) {
        using Full = std::integral_constant<bool, true>;
        using Part = std::integral_constant<bool, false>;
        const int NCF = (int64_t)NC * C > Tl ? NC - 1 : NC;   // full chunks
        O o0, o1, o2, o3;
        load(o0, 0);
        load(o1, 1);
        if (kRing > 2) load(o2, 2);
        if (kRing > 3) load(o3, 3);
        __syncthreads();
        int c = 0;
        for (; c + kRing <= NCF; c += kRing) {
            step(Full{}, o0, c);
            load(o0, c + kRing);
            step(Full{}, o1, c + 1);
            load(o1, c + kRing + 1);
            if (kRing > 2) {
                step(Full{}, o2, c + 2);
                load(o2, c + kRing + 2);
            }
            if (kRing > 3) {
                step(Full{}, o3, c + 3);
                load(o3, c + kRing + 3);
            }
        }
        if (c < NC) step(Part{}, o0, c);
        if (c + 1 < NC) step(Part{}, o1, c + 1);
        if (kRing > 2 && c + 2 < NC) step(Part{}, o2, c + 2);
        if (kRing > 3 && c + 3 < NC) step(Part{}, o3, c + 3);
    }

    // ---- final state ----
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int mt = 0; mt < MTS; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = (DK / 4) * w + 16 * mt + 4 * g + e;
                const size_t idx = ((size_t)bh * DK + r) * DK + col0 + 16 * j + n;
                if (SUMMARY) {
                    if (vcols) a.zero_state[idx] = S[j][mt][e];
                    else a.transition[idx] = S[j][mt][e];
                } else if (a.state_out) {
                    a.state_out[idx] = S[j][mt][e];
                }
            }
    if constexpr (CKPT == 1 || CKPT == 2) {   // the final state in the last checkpoint slot
        const int every = CKPT == 1 ? 1 : a.ckpt_every;
        const int64_t nslot = ((int64_t)NC + every - 1) / every + 1;
        float* dst = a.states + ((size_t)bh * nslot + nslot - 1) * DK * DK + col0 + n;
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int mt = 0; mt < MTS; ++mt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    dst[(size_t)((DK / 4) * w + 16 * mt + 4 * g + e) * DK + 16 * j] = S[j][mt][e];
    }
}

// Slices per workgroup: two or four slices share each card fragment (more
// work per compute-unit cycle) but divide the workgroup count, so the most
// slices that still leave at least one workgroup per compute unit are used.
// Four slices fit the register file only with a three-deep ring.
constexpr int kCUs = 256;
inline int pick_ntw(int64_t BH, int NTALL) {
    if (NTALL % 4 == 0 && BH * (NTALL / 4) >= kCUs) return 4;
    return (NTALL % 2 == 0 && BH * (NTALL / 2) >= kCUs) ? 2 : 1;
}

template <typename E, int DK, int NTW, bool SUMMARY, int CKPT>
hipError_t launch_scan_n(const ScanArgs& a, hipStream_t s) {
    constexpr int NTALL = SUMMARY ? 2 * (DK / 16) : DK / 16;
    const int64_t BH = a.B * (int64_t)a.H;
    const int64_t groups = (BH + kXcds - 1) / kXcds;
    const int64_t blocks = groups * kXcds * (NTALL / NTW);
    hipLaunchKernelGGL((kda_scan_kernel<E, DK, NTW, SUMMARY, CKPT>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <typename E, int DK, bool SUMMARY, int CKPT = 0>
hipError_t launch_scan_t(const ScanArgs& a, hipStream_t s) {
    constexpr int NTALL = SUMMARY ? 2 * (DK / 16) : DK / 16;
    const int64_t BH = a.B * (int64_t)a.H;
    if (BH == 0) return hipSuccess;
    // summaries of bf16 d_k = 128 cards with enough (b, h) pairs to give
    // every workgroup four or eight slices run one whole slice per wave (or
    // two): no exchange of the state between waves, operands shared through
    // an LDS ring.  Measured on 16K-token segments: 0.23 against 0.28 ms at
    // 32 pairs, 0.49 against 0.72 ms at 128; slower below 32 pairs.
    if constexpr (SUMMARY && sizeof(E) == 2 && DK == 128)
        if (BH * 4 >= kCUs / 2) return launch_summary_wave(BH * 2 >= kCUs ? 2 : 1, a, s);
    // the backward's hand-off, which stores every chunk's state, runs at most
    // two slices per workgroup: measured on 64 (row, head) pairs and on a
    // 24-sequence packed batch (384 pairs), two beat one and four
    if constexpr (CKPT == 3) {
        if (pick_ntw(BH, NTALL) >= 2) return launch_scan_n<E, DK, 2, SUMMARY, CKPT>(a, s);
        return launch_scan_n<E, DK, 1, SUMMARY, CKPT>(a, s);
    } else {
        switch (pick_ntw(BH, NTALL)) {
        case 4: return launch_scan_n<E, DK, 4, SUMMARY, CKPT>(a, s);
        case 2: return launch_scan_n<E, DK, 2, SUMMARY, CKPT>(a, s);
        default: return launch_scan_n<E, DK, 1, SUMMARY, CKPT>(a, s);
        }
    }
}

}  // namespace

hipError_t launch_scan(bool bf16, int dk, bool summary, const ScanArgs& a, hipStream_t s) {
    if (a.states && a.states_tiled) {   // the state entering every chunk, for the backward pass
        if (bf16) return dk == 128 ? launch_scan_t<__bf16, 128, false, 3>(a, s) : launch_scan_t<__bf16, 64, false, 3>(a, s);
        return dk == 128 ? launch_scan_t<float, 128, false, 3>(a, s) : launch_scan_t<float, 64, false, 3>(a, s);
    }
    if (a.states && a.ckpt_every == 1) {   // checkpoints at every chunk
        if (bf16) return dk == 128 ? launch_scan_t<__bf16, 128, false, 1>(a, s) : launch_scan_t<__bf16, 64, false, 1>(a, s);
        return dk == 128 ? launch_scan_t<float, 128, false, 1>(a, s) : launch_scan_t<float, 64, false, 1>(a, s);
    }
    if (a.states) {   // checkpoints every ckpt_every chunks
        if (bf16) return dk == 128 ? launch_scan_t<__bf16, 128, false, 2>(a, s) : launch_scan_t<__bf16, 64, false, 2>(a, s);
        return dk == 128 ? launch_scan_t<float, 128, false, 2>(a, s) : launch_scan_t<float, 64, false, 2>(a, s);
    }
    if (bf16) {
        if (dk == 128) return summary ? launch_scan_t<__bf16, 128, true>(a, s) : launch_scan_t<__bf16, 128, false>(a, s);
        return summary ? launch_scan_t<__bf16, 64, true>(a, s) : launch_scan_t<__bf16, 64, false>(a, s);
    }
    if (dk == 128) return summary ? launch_scan_t<float, 128, true>(a, s) : launch_scan_t<float, 128, false>(a, s);
    return summary ? launch_scan_t<float, 64, true>(a, s) : launch_scan_t<float, 64, false>(a, s);
}

}  // namespace kda
