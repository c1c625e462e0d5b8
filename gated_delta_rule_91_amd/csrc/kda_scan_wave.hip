// kda_scan_wave.hip -- the segment summaries of the context-parallel scheme
// [zuoshipin.com/article/18261 §三, "KDA 上下文并行" paragraph] with one
// or two 16-column slices of the augmented state per wave (bf16 cards): the hand-off
// of [Bz | A] from [0 | I] over a segment's cards, with the same per-chunk
// arithmetic as kda_scan_kernel [same page, §四, FlashKDA paragraph: only the
// hand-off stays sequential]:
//   U = Wv - Wk X,   X <- diag(e^gamma_C) X + Ke^T U
// where X is a slice of [Bz | A] (value columns start at zero and read Wv;
// transition columns start at the identity and have no value input).
// Summaries have no read-out, so a wave can carry one or two whole slices.
//
// Layout.  A wave keeps its whole slice -- all d_k state rows of 16 columns --
// in MFMA accumulators, so no part of the chain crosses waves: no LDS
// exchange of X or U and a single barrier per chunk (the hand-off of the
// operand ring).  The trick is the row order of the accumulator tiles.  An
// accumulator tile gives lane (g, n) rows 4g..4g+3 of column n; tiles are
// taken in pairs (2p, 2p+1) and lane (g, n) of tile 2p+h holds rows
// 32p + 8g + 4h + e (e < 4).  Lane (g, n) then holds rows 32p + 8g .. +7 of
// column n across the pair, which is exactly its B fragment of the k-block
// p of a 16x16x32 product.  So
//   * X (key rows in that order) is the B operand of Wk X straight from its
//     accumulators, and
//   * U (token rows in that order) is the B operand of Ke^T U,
// while the A operands that produce these tiles (Wk rows for U, Ke^T rows
// for X) are read from LDS with the same row order, one 16-byte piece per
// lane at its own address.
//
// Operands.  Two loader waves copy each chunk's shared operands -- Wk, Ke^T
// and e^gamma_C -- from the card into a three-slot LDS ring with direct
// global-to-LDS loads, two chunks ahead; every compute wave reads them from
// there.  1 KB fragment blocks are stored 64 bytes apart so that the gathered
// row reads do not collide in LDS banks.  The Wv rows of a wave's slices come
// through a small register ring.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

namespace {

constexpr int kXcdsW = 8;
constexpr int kComputeW = 4;                           // compute waves
constexpr int kLoadersW = 2;                           // loader waves
constexpr int kThreadsW = 64 * (kComputeW + kLoadersW);
constexpr int kBlkPitch = 1024 + 64;                   // LDS bytes per 1 KB fragment block
constexpr int kPullAheadW = 1;                         // L2 pull: chunks past the last ring load

typedef __attribute__((address_space(3))) char lds_c;

template <int DK>
struct WaveRing {
    static constexpr int C = kChunk;
    // shared operand blocks per chunk (1 KB each): Wk, then Ke^T
    static constexpr int NB_WK = C * DK * 2 / 1024;
    static constexpr int NB_KE = DK * C * 2 / 1024;
    static constexpr int NBLK = NB_WK + NB_KE;
    // slot layout (block index b at b * kBlkPitch): Wk, Ke^T, then e^gamma_C
    static constexpr int B_WK = 0, B_KE = NB_WK;
    static constexpr size_t GC_OFF = (size_t)NBLK * kBlkPitch;
    static constexpr size_t SLOT = GC_OFF + DK * 4;
    static constexpr int SLOTS = 3;
    static constexpr size_t BYTES = SLOTS * SLOT;
};

// byte offset, inside a ring slot, of lane (g, m)'s 16-byte piece of the
// fragment (row r, k-block kb) of an A operand with NKB k-blocks starting at
// slot block b0 (fragment order: block (r/16, kb), lane position g*16 + r%16)
__device__ __forceinline__ uint32_t frag_at(int b0, int nkb, int r, int kb, int g) {
    const int blk = b0 + (r >> 4) * nkb + kb;
    return (uint32_t)(blk * kBlkPitch + (g * 16 + (r & 15)) * 16);
}

__device__ __forceinline__ bf16x8 ld_lds8(const lds_c* base, uint32_t off) {
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(base + off);
}
__device__ __forceinline__ f32x4 ld_lds4f(const lds_c* base, uint32_t off) {
    return *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(base + off);
}
__device__ __forceinline__ f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// the B fragment of k-block p from the accumulator pair (2p, 2p+1)
__device__ __forceinline__ bf16x8 pack_pair(f32x4 lo, f32x4 hi) {
    return bf16x8{(__bf16)lo[0], (__bf16)lo[1], (__bf16)lo[2], (__bf16)lo[3],
                   (__bf16)hi[0], (__bf16)hi[1], (__bf16)hi[2], (__bf16)hi[3]};
}

// Wv of one chunk for one wave's slices, U-tile order [slice][tile (q, h) = 2q + h]
template <int SPW>
struct WaveOps {
    bf16x4 wv[SPW][4];
};

// SPW: slices per wave; a workgroup covers 4 * SPW adjacent slices of the
// augmented state [Bz | A] of one (row, head): value columns (from zero) or
// transition columns (from the identity).
template <int DK, int SPW>
__global__ __launch_bounds__(kThreadsW, 1) void kda_summary_wave_kernel(ScanArgs a) {
    using CL = Card<__bf16, DK>;
    using WR = WaveRing<DK>;
    using R = WaveOps<SPW>;
    constexpr int NKB = DK / 32;                   // key k-blocks (pairs of key tiles)
    constexpr int NT = DK / 16;                    // value-column slices
    constexpr int NTALL = 2 * NT;                  // + transition-column slices
    constexpr int SPG = kComputeW * SPW;           // slices per workgroup
    constexpr int NWG = NTALL / SPG;               // workgroups per chain
    static_assert(NTALL % SPG == 0 && NT % SPG == 0, "a workgroup's slices never straddle value/transition");
    constexpr int L = WR::SLOTS - 1;               // chunks the loaders run ahead

    __shared__ __attribute__((aligned(1024))) char ring[WR::BYTES];
    __shared__ __attribute__((aligned(16))) uint32_t dump[64 * kLoadersW];

    const int t = threadIdx.x, lane = t & 63, g = lane >> 4, n = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);

    // XCD-aware chain decode (as kda_scan_kernel): the workgroups of one
    // (row, head) get ids congruent mod 8, so they share one XCD's L2
    const int H = a.H;
    const int64_t BH = a.B * (int64_t)H;
    const int64_t x = blockIdx.x;
    const int xcd = (int)(x % kXcdsW);
    const int64_t slotid = x / kXcdsW;
    const int wgi = (int)(slotid % NWG);
    const int64_t bh = (slotid / NWG) * kXcdsW + xcd;
    if (bh >= BH) return;
    const int64_t b = bh / H;
    const int h = (int)(bh % H);
    const SeqSpan sp = seq_span(a.cu_seqlens, a.chunk_off, a.T, a.row_stride, a.NC, a.B, b, h, H);
    const int NC = sp.nc;
    const char* cards = a.ws + (size_t)sp.card0 * CL::BYTES;
    lds_c* const ring_l = (lds_c*)ring;

    if (w >= kComputeW) {
        // ---------------- loader waves ----------------
        const int lw = w - kComputeW;
        // lines of the card the summaries read: Wk, Ke^T, then Wv and e^gamma_C
        // (Qt and P, between them, are only read by the read-out scan)
        constexpr int NL_WK = (int)((CL::QT - CL::WK) / 128), NL_KE = (int)((CL::P - CL::KET) / 128);
        constexpr int NL = NL_WK + NL_KE + (int)((CL::BYTES - CL::WV) / 128);
        static_assert(CL::WK % 128 == 0 && CL::KET % 128 == 0 && CL::WV % 128 == 0 && CL::BYTES % 128 == 0, "line map");
        auto line_off = [](int li) -> size_t {
            return li < NL_WK ? CL::WK + (size_t)li * 128
                 : li < NL_WK + NL_KE ? CL::KET + (size_t)(li - NL_WK) * 128
                 : CL::WV + (size_t)(li - NL_WK - NL_KE) * 128;
        };
        constexpr int LPW = (NL + NWG - 1) / NWG;
        constexpr int PPL = (LPW + 64 * kLoadersW - 1) / (64 * kLoadersW);
        lds_c* const dump_l = (lds_c*)dump + lw * 256;
        static_assert(WR::NBLK % kLoadersW == 0, "loader split");
        constexpr int BPL = WR::NBLK / kLoadersW;             // 1 KB blocks per loader wave and chunk
        // e^gamma_C moves as 256-byte pieces (a dword per lane: the narrower
        // direct loads do not pack lanes densely in LDS); a loader without a
        // piece pulls the first one into its dump, so both count the same loads
        constexpr int NGC = DK * 4 / 256;
        static_assert(NGC >= 1 && NGC <= kLoadersW, "e^gamma_C pieces");
        const bool gc_mine = lw < NGC;
        auto issue = [&](int c) {   // chunk c -> slot c % SLOTS (past the end: the last card again)
            const int cc = c < NC ? c : NC - 1;
            const char* card = cards + (size_t)cc * CL::BYTES + lane * 16;
            lds_c* dst = ring_l + (size_t)(c % WR::SLOTS) * WR::SLOT;
#pragma unroll
            for (int i = 0; i < BPL; ++i) {
                const int blk = i * kLoadersW + lw;
                // card offset of slot block blk (Wk, then Ke^T; the card's Qt sits between them)
                const size_t cb = blk >= WR::NB_WK ? CL::KET + (size_t)(blk - WR::NB_WK) * 1024 : (size_t)blk * 1024;
                __builtin_amdgcn_global_load_lds(card + cb, dst + blk * kBlkPitch, 16, 0, 0);
            }
            // e^gamma_C (DK floats)
            __builtin_amdgcn_global_load_lds(cards + (size_t)cc * CL::BYTES + CL::GC + (gc_mine ? lw * 256 : 0) + lane * 4,
                                             gc_mine ? dst + WR::GC_OFF + lw * 256 : dump_l, 4, 0, 0);
            // L2 pull of a later card's lines that are read here: each workgroup
            // of the chain a disjoint share
            const int cp = c + kPullAheadW < NC ? c + kPullAheadW : NC - 1;
            const char* pbase = cards + (size_t)cp * CL::BYTES;
#pragma unroll
            for (int i = 0; i < PPL; ++i) {
                int line = wgi * LPW + (i * kLoadersW + lw) * 64 + lane;
                line = line < (wgi + 1) * LPW ? line : (wgi + 1) * LPW - 1;
                line = line < NL ? line : NL - 1;
                __builtin_amdgcn_global_load_lds(pbase + line_off(line), dump_l, 4, 0, 0);
            }
        };
        // loads per chunk and loader wave, and the s_waitcnt encoding (gfx9:
        // vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at their maxima)
        // that leaves L-1 chunks' loads in flight
        constexpr int G = BPL + 1 + PPL;
        constexpr int KEEP = (L - 1) * G;
        static_assert(L * G <= 63, "vmcnt range");
        constexpr int kWait = (KEEP & 15) | ((KEEP >> 4) << 14) | (7 << 4) | (15 << 8);
        // The loaders meet the compute waves at the bare barrier: a
        // workgroup fence would wait for every load in flight (the direct
        // loads count as LDS writes), which would cut the run-ahead to
        // one chunk.  The explicit wait before it is what publishes a slot.
        auto barrier = [] {
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        if (NC > 0) {
#pragma unroll
            for (int c = 0; c < L; ++c) issue(c);
            __builtin_amdgcn_s_waitcnt(kWait);             // chunk 0 has landed
        }
        barrier();                                         // chunk 0 is in its slot
        for (int c = 0; c < NC; ++c) {
            issue(c + L);                                  // into the slot chunk c-1 used
            __builtin_amdgcn_s_waitcnt(kWait);             // chunk c+1 has landed
            barrier();                                     // chunk c done, chunk c+1 in its slot
        }
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }

    // ---------------- compute waves ----------------
    const int slice0 = wgi * SPG + w * SPW;                      // first slice of this wave (of NTALL)
    const bool vcols = slice0 < NT;                             // value columns (else transition columns)
    const int colbase = (vcols ? slice0 : slice0 - NT) * 16;    // first column of this wave's slices

    // X: [slice][key tile pair p][h]; lane (g, n) holds rows 32p + 8g + 4h + e of column colbase + 16s + n
    f32x4 X[SPW][NKB][2];
#pragma unroll
    for (int s = 0; s < SPW; ++s)
#pragma unroll
        for (int p = 0; p < NKB; ++p)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 32 * p + 8 * g + 4 * hh + e;
                    X[s][p][hh][e] = (!vcols && r == colbase + 16 * s + n) ? 1.f : 0.f;
                }

    // this lane's Wv pieces: U-tile (q, hh) row 32q + 8g + 4hh + e sits in card
    // tile mi = 2q + ((2g + hh) >> 2), lane group (2g + hh) & 3
    auto load = [&](R& o, int c) {
        const int cc = c < NC ? c : NC - 1;
        const char* card = cards + (size_t)cc * CL::BYTES;
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
            // (transition columns have no value input: they read the first
            // value slice and discard it, so no load sits under a branch)
            const int nv = vcols ? colbase / 16 + s : 0;
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int mi = 2 * q + ((2 * g + hh) >> 2), gl = (2 * g + hh) & 3;
                    const size_t off = CL::WV + ((size_t)((nv * 4 + mi) * 64 + gl * 16 + n) * 4) * 2;
                    o.wv[s][2 * q + hh] = *reinterpret_cast<const bf16x4*>(card + off);
                }
        }
    };

    auto step = [&](R& cur, int c) {
        // the slot's registers are taken here, after the previous chunk's
        // barrier (else the compiler hoists their use and waits early)
#pragma unroll
        for (int s = 0; s < SPW; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(cur.wv[s][i]));
        const lds_c* sl = ring_l + (size_t)(c % WR::SLOTS) * WR::SLOT;

        // X (entering the chunk) as bf16 B fragments of Wk X
        bf16x8 xF[SPW][NKB];
#pragma unroll
        for (int s = 0; s < SPW; ++s)
#pragma unroll
            for (int p = 0; p < NKB; ++p) xF[s][p] = pack_pair(X[s][p][0], X[s][p][1]);

        // U tiles (q, hh): rows (tokens) 32q + 8g + 4hh + e.  acc = Wk X - Wv = -U
        f32x4 U[SPW][2][2];
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                // A: Wk rows tau(m) = 32q + 8(m/4) + 4hh + m%4 for this lane's m = n
                const int tau = 32 * q + 8 * (n >> 2) + 4 * hh + (n & 3);
                bf16x8 wk[NKB];
#pragma unroll
                for (int p = 0; p < NKB; ++p) wk[p] = ld_lds8(sl, frag_at(WR::B_WK, NKB, tau, p, g));
#pragma unroll
                for (int s = 0; s < SPW; ++s) {
                    const bf16x4 v = cur.wv[s][2 * q + hh];
                    f32x4 acc = vcols ? f32x4{-(float)v[0], -(float)v[1], -(float)v[2], -(float)v[3]}
                                      : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int p = 0; p < NKB; ++p) acc = mma16(wk[p], xF[s][p], acc);
                    U[s][q][hh] = -acc;
                }
            }
        bf16x8 uF[SPW][2];   // U as B operand (token k-block q)
#pragma unroll
        for (int s = 0; s < SPW; ++s)
#pragma unroll
            for (int q = 0; q < 2; ++q) uF[s][q] = pack_pair(U[s][q][0], U[s][q][1]);

        // X <- diag(e^gamma_C) X + Ke^T U, tiles (p, hh) with key rows 32p + 8g + 4hh + e
#pragma unroll
        for (int p = 0; p < NKB; ++p)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const f32x4 gc = ld_lds4f(sl, (uint32_t)(WR::GC_OFF + (32 * p + 8 * g + 4 * hh) * 4));
                const int kap = 32 * p + 8 * (n >> 2) + 4 * hh + (n & 3);
                const bf16x8 ke0 = ld_lds8(sl, frag_at(WR::B_KE, 2, kap, 0, g));
                const bf16x8 ke1 = ld_lds8(sl, frag_at(WR::B_KE, 2, kap, 1, g));
#pragma unroll
                for (int s = 0; s < SPW; ++s) {
                    f32x4 acc = X[s][p][hh] * gc;
                    acc = mma16(ke0, uF[s][0], acc);
                    acc = mma16(ke1, uF[s][1], acc);
                    X[s][p][hh] = acc;
                }
            }
        __syncthreads();   // this slot is free; the next chunk's is in place
    };

    // register ring of Wv, two chunks deep
    if (NC > 0) {
        R o0, o1;
        load(o0, 0);
        asm volatile("" ::: "memory");
        load(o1, 1);
        asm volatile("" ::: "memory");
        __syncthreads();   // chunk 0 is in its slot
        int c = 0;
        for (; c + 2 <= NC; c += 2) {
            step(o0, c);
            load(o0, c + 2);
            asm volatile("" ::: "memory");
            step(o1, c + 1);
            load(o1, c + 3);
            asm volatile("" ::: "memory");
        }
        if (c < NC) step(o0, c);
    } else {
        __syncthreads();
    }

    // the summary pair: value columns -> Bz, transition columns -> A
    float* const dst = vcols ? a.zero_state : a.transition;
#pragma unroll
    for (int s = 0; s < SPW; ++s)
#pragma unroll
        for (int p = 0; p < NKB; ++p)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 32 * p + 8 * g + 4 * hh + e;
                    dst[((size_t)bh * DK + r) * DK + colbase + 16 * s + n] = X[s][p][hh][e];
                }
}

template <int DK, int SPW>
hipError_t launch_summary_wave_n(const ScanArgs& a, hipStream_t s) {
    constexpr int NWG = 2 * (DK / 16) / (kComputeW * SPW);
    const int64_t BH = a.B * (int64_t)a.H;
    const int64_t groups = (BH + kXcdsW - 1) / kXcdsW;
    const int64_t blocks = groups * kXcdsW * NWG;
    hipLaunchKernelGGL((kda_summary_wave_kernel<DK, SPW>), dim3((unsigned)blocks), dim3(kThreadsW), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_summary_wave(int spw, const ScanArgs& a, hipStream_t s) {
    return spw == 2 ? launch_summary_wave_n<128, 2>(a, s) : launch_summary_wave_n<128, 1>(a, s);
}

}  // namespace kda
