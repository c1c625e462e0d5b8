// kda_common.hpp -- device-side building blocks shared by the KDA kernels
// (gfx950 / CDNA4, wave64).
//
//  * bf16 <-> fp32 conversion (round to nearest even, NaN kept NaN)
//  * the MFMA operand policy: bf16 operands use v_mfma_f32_16x16x32_bf16,
//    fp32 operands use v_mfma_f32_16x16x4_f32; both accumulate in fp32
//  * the layout of one "update card" (the per-chunk bundle the prepare
//    kernel writes and the ordered hand-off kernel reads)
//
// MFMA 16x16 register layout (one wave, lane l, g = l / 16, n = l % 16):
//   A operand : A[m = n][k = k0 + KF*g + e],  e < KF
//   B operand : B[k = k0 + KF*g + e][n]
//   C/D       : acc[v] = D[4*g + v][n],      v < 4
// with KF = 8 (bf16, K step 32) or KF = 1 (fp32, K step 4).  A and B use the
// same k assignment, so any consistent permutation of k is harmless.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kChunk = 64;      // tokens per chunk
constexpr int kThreads = 256;   // four waves per workgroup

// ---- scalar conversions ---------------------------------------------------
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// The backward's per-chunk fp32 states (the state entering every chunk and
// the state gradient leaving it) are stored in 16-column tiles, and inside a
// tile four consecutive rows of one column are contiguous: element (row, col)
// of a d_k x d_v state sits at tiled_state_index(d_k, col / 16, row / 4,
// col % 16) + row % 4.  A lane that holds rows 4i..4i+3 of one column (the
// accumulator layout of the hand-off kernels) writes them with one 16-byte
// store, a wave's 64 lanes one contiguous kilobyte, and one 16-column block
// of the state is a contiguous d_k x 16 region.
__host__ __device__ constexpr int tiled_state_index(int dk, int tile, int row4, int n) {
    return ((tile * (dk / 4) + row4) * 16 + n) * 4;
}

// ---- MFMA policy ------------------------------------------------------------
template <typename E> struct MM;

template <> struct MM<__bf16> {
    static constexpr int KF = 8;      // k values per lane per step
    static constexpr int KS = 32;     // k per MFMA
    typedef bf16x8 frag;
    __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static frag neg(frag a) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        u32x4 u = __builtin_bit_cast(u32x4, a);
        u ^= 0x80008000u;
        return __builtin_bit_cast(frag, u);
    }
};

template <> struct MM<float> {
    static constexpr int KF = 1;
    static constexpr int KS = 4;
    typedef float frag;
    __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static frag neg(frag a) { return -a; }
};

// Fragment at row `row`, k range [k0 + KF*g, k0 + KF*g + KF) of a row-major
// matrix with leading dimension `ld` (elements).  Works for LDS and global
// pointers; the address must be aligned to the fragment size.
template <typename E>
__device__ __forceinline__ typename MM<E>::frag ld_frag(const E* base, int ld, int row, int k0, int g) {
    return *reinterpret_cast<const typename MM<E>::frag*>(base + (size_t)row * ld + k0 + MM<E>::KF * g);
}

// Four consecutive elements (8 B for bf16, 16 B for fp32) <-> fp32x4.
// Four consecutive elements kept as loaded; widened to fp32 only where used,
// so no conversion sits right behind its load.
template <typename E> struct Raw4 { typedef f32x4 type; };
template <> struct Raw4<__bf16> { typedef bf16x4 type; };
__device__ __forceinline__ f32x4 widen4(bf16x4 x) { return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]}; }
__device__ __forceinline__ f32x4 widen4(f32x4 x) { return x; }

__device__ __forceinline__ f32x4 ld4(const __bf16* p) {
    bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
    return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(__bf16* p, f32x4 v) {
    *reinterpret_cast<bf16x4*>(p) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
}
__device__ __forceinline__ void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

// Two consecutive elements <-> fp32x2.
__device__ __forceinline__ f32x2 ld2(const __bf16* p) {
    bf16x2 x = *reinterpret_cast<const bf16x2*>(p);
    return f32x2{(float)x[0], (float)x[1]};
}
__device__ __forceinline__ f32x2 ld2(const float* p) { return *reinterpret_cast<const f32x2*>(p); }
__device__ __forceinline__ void st2(__bf16* p, float a, float b) {
    *reinterpret_cast<bf16x2*>(p) = bf16x2{(__bf16)a, (__bf16)b};
}
__device__ __forceinline__ void st2(float* p, float a, float b) { *reinterpret_cast<f32x2*>(p) = f32x2{a, b}; }

// sigmoid(x) = 1 / (1 + 2^(-x log2 e)) with the hardware exp2 and reciprocal
// (about 1 ulp each); saturates cleanly to 0 and 1
__device__ __forceinline__ float sigmoidf_(float x) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

// ---- update card --------------------------------------------------------------
// One card per (batch row, head, chunk), for chunk length C = 64 and
// d_k = d_v = DK.  E is the operand type of the ordered stage (bf16 or fp32).
//   Wk  [C x DK]   Wk = T diag(beta) Kt          (A operand of U = Wv - Wk S)
//   Qt  [C x DK]   q^ * e^gamma                   (A operand of O = Qt S + P U)
//   KeT [DK x C]   (k^ * e^(gamma_C - gamma))^T   (A operand of S' = G S + Ke^T U)
//   P   [C x C]    lower_incl(Qt Kh^T)            (A operand of P U)
// are stored in MFMA A-fragment order: the matrix is cut into blocks of 16
// rows x KS columns, blocks row-block-major, and inside a block lane l's
// fragment (row l % 16, columns KF*(l/16) .. +KF-1) sits at l * KF elements.
// One wave-wide fragment load is then a single contiguous 64*KF-element run.
//   Wv  [DK/16][C/16][64][4] in accumulator order: the 16x16 tile (token tile
//       mi, column tile ni) sits at ((ni*4 + mi)*64 + lane)*4, lane holding
//       rows 4g..4g+3 of column n -- exactly the C operand of U's MFMA.
//   GC  [DK] fp32            e^gamma_C, the chunk's total retention per key channel
template <typename E, int DK>
struct Card {
    static constexpr int C = kChunk;
    static constexpr size_t WK = 0;
    static constexpr size_t QT = WK + (size_t)C * DK * sizeof(E);
    static constexpr size_t KET = QT + (size_t)C * DK * sizeof(E);
    static constexpr size_t P = KET + (size_t)DK * C * sizeof(E);
    static constexpr size_t WV = P + (size_t)C * C * sizeof(E);
    static constexpr size_t GC = WV + (size_t)C * DK * sizeof(E);
    static constexpr size_t BYTES = ((GC + (size_t)DK * sizeof(float)) + 255) / 256 * 256;
};

// Where one (sequence, head)'s tokens and cards are.
//  * Uniform batch: row b holds T tokens starting at token b*rs (rs = the
//    arrays' row stride, T unless a call works on a token range of longer
//    rows); its chunks' cards start at card (b*H + h)*NC.
//  * Packed variable-length batch: sequence s holds tokens [cu[s], cu[s+1])
//    of one packed row (offsets clamped into [0, T], so no offset array can
//    send an access outside the arrays); its NC_s chunks' cards start at
//    card chunk_off[s]*H + h*NC_s, chunk_off being the prefix sum of NC_s.
struct SeqSpan {
    int64_t tok0;     // first token (row index along the packed token axis)
    int64_t len;      // tokens
    int nc;           // chunks
    int64_t chunk0;   // packed batch: global index of the sequence's first chunk (0 for a uniform batch)
    int64_t card0;    // card index of chunk 0 of (sequence, head)
};
__device__ __forceinline__ void seq_bounds(const int32_t* cu, int64_t s, int64_t T, int64_t& st, int64_t& en) {
    const int64_t a = cu[s], b = cu[s + 1];
    st = a < 0 ? 0 : (a > T ? T : a);
    en = b < st ? st : (b > T ? T : b);
}
// nseq: sequences of a packed batch.  CLAMP: the chunk offsets were read
// back from a workspace an earlier call filled, so they are clamped to the
// chunks the workspace holds (ceil(T/C) + nseq) and to the sequence's own
// chunk count: whatever the workspace or cu_seqlens hold, no access leaves
// the workspace or the token arrays (offsets the plan kernel wrote for these
// cu_seqlens pass unchanged).  The prepare, which runs right after the plan
// kernel in the same call, takes them as they are.
template <bool CLAMP = true>
__device__ __forceinline__ SeqSpan seq_span(const int32_t* cu, const int64_t* chunk_off, int64_t T, int64_t rs,
                                            int NC, int64_t nseq, int64_t b, int h, int H) {
    SeqSpan r;
    if (cu) {
        int64_t st, en;
        seq_bounds(cu, b, T, st, en);
        r.tok0 = st;
        r.len = en - st;
        int64_t c0 = chunk_off[b], c1 = chunk_off[b + 1];
        if constexpr (CLAMP) {
            const int64_t maxc = (T + kChunk - 1) / kChunk + nseq;
            c0 = c0 < 0 ? 0 : (c0 > maxc ? maxc : c0);
            c1 = c1 < c0 ? c0 : (c1 > maxc ? maxc : c1);
            const int64_t need = (r.len + kChunk - 1) / kChunk;
            if (c1 - c0 > need) c1 = c0 + need;
        }
        r.nc = (int)(c1 - c0);
        r.chunk0 = c0;
        r.card0 = c0 * H + (int64_t)h * r.nc;
    } else {
        r.tok0 = b * (rs > 0 ? rs : T);
        r.len = T;
        r.nc = NC;
        r.chunk0 = 0;
        r.card0 = (b * H + h) * (int64_t)NC;
    }
    return r;
}

// Element index of (row, k) of an A operand with K columns in fragment order.
template <typename E>
__host__ __device__ constexpr int frag_index(int row, int k, int K) {
    return (((row >> 4) * (K / MM<E>::KS) + k / MM<E>::KS) * 64 +
            ((k % MM<E>::KS) / MM<E>::KF) * 16 + (row & 15)) * MM<E>::KF + (k % MM<E>::KF);
}

// Copy an R x K row-major LDS matrix (leading dimension ld) to global
// memory in MFMA A-fragment order (the Card layout above).
template <typename E, int R, int K>
__device__ __forceinline__ void store_frag_order(char* dst, const E* src, int ld, int t) {
    constexpr int KF = MM<E>::KF, KS = MM<E>::KS;
    if constexpr (KF == 8) {   // a lane fragment is one 16-byte run of a source row
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        for (int idx = t; idx < R * K / 8; idx += kThreads) {
            const int blk = idx >> 6, lane = idx & 63;
            const int row = 16 * (blk / (K / KS)) + (lane & 15);
            const int k = (blk % (K / KS)) * KS + (lane >> 4) * KF;
            *reinterpret_cast<u32x4*>(dst + (size_t)idx * 16) = *reinterpret_cast<const u32x4*>(src + row * ld + k);
        }
    } else {
        for (int idx = t; idx < R * K; idx += kThreads) {
            const int blk = idx >> 6, lane = idx & 63;
            const int row = 16 * (blk / (K / KS)) + (lane & 15);
            const int k = (blk % (K / KS)) * KS + (lane >> 4);
            reinterpret_cast<E*>(dst)[idx] = src[row * ld + k];
        }
    }
}

}  // namespace kda
