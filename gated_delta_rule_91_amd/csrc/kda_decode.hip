// kda_decode.hip -- one decode step for N independent sequences: the
// fixed-size memory is updated in place, no per-token cache grows
// [devpress.csdn.net K3 article §十六: KDA keeps a recursive state rather
// than per-token K/V; zuoshipin.com/article/18261 §二 for the step itself].
//
// Per (sequence, head), with S' = diag(e^lambda) S (retention with the floor):
//   p = S'^T kh,  r = S'^T qh     (one sweep over S)
//   u = beta (v - p)
//   S <- S' + kh u^T              (in place)
//   o = S^T qh = r + u (kh . qh); out = o * sigmoid(g)
//
// The step is bound by HBM: the fp32 state (64 KB per head at d = 128) is
// read once and written once, and everything else is < 2 KB.  One workgroup
// per (sequence, head), or two with half the value columns each at small
// batches (see the launch); thread (column group cg, row group rg) keeps a
// rows x 4-column block of S in registers between the read and the write.
// The state streams with non-temporal loads/stores (it is larger than the
// last-level cache), and the column partial sums of p and r are combined
// across row groups through LDS.  Residency is capped at two workgroups per
// CU (see the launch).
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

namespace {

template <typename E, int DK, int NSPLIT>
__global__ __launch_bounds__(kThreads) void kda_decode_kernel(DecodeArgs a) {
    constexpr int DV = DK;
    constexpr int DVS = DV / NSPLIT;    // this workgroup's value columns
    constexpr int CG = DVS / 4;         // 4-column groups
    constexpr int RG = kThreads / CG;   // row groups
    constexpr int RPT = DK / RG;        // rows per thread
    constexpr int EPL = DK / 64;        // elements per lane for the norm sweep
    static_assert(RPT >= 1 && RG * CG == kThreads, "whole rows per thread");

    __shared__ float red[2][RG][DVS];

    const int t = threadIdx.x, lane = t & 63, cg = t % CG, rg = t / CG;
    const size_t nh = blockIdx.x / NSPLIT;
    const int col0 = (int)(blockIdx.x % NSPLIT) * DVS;
    const E* q = reinterpret_cast<const E*>(a.q) + nh * DK;
    const E* k = reinterpret_cast<const E*>(a.k) + nh * DK;
    const E* v = reinterpret_cast<const E*>(a.v) + nh * DV;
    const E* gp = reinterpret_cast<const E*>(a.g) + nh * DV;
    const float* la = a.log_alpha + nh * DK;
    float* S = a.state + nh * DK * DV;

    // the state block first: RPT rows x 4 columns
    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (size_t)(rg * RPT + i) * DV + col0 + 4 * cg));

    // norms and k.q, each wave on its own (no LDS)
    float sk = 0.f, sq = 0.f, kq = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const float kk = to_f32(k[lane * EPL + e]), qq = to_f32(q[lane * EPL + e]);
        sk += kk * kk; sq += qq * qq; kq += kk * qq;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        sk += __shfl_xor(sk, off);
        sq += __shfl_xor(sq, off);
        kq += __shfl_xor(kq, off);
    }
    const float rk = 1.0f / fmaxf(sqrtf(sk), 1e-6f), rq = 1.0f / fmaxf(sqrtf(sq), 1e-6f);
    const float khqh = kq * rk * rq;
    const float bt = a.beta[nh];

    // retention and the two column sums over this thread's rows
    float kh[RPT];
    f32x4 pp = {0.f, 0.f, 0.f, 0.f}, rr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg * RPT + i;
        const float dec = __expf(fmaxf(la[r], a.floor_));
        kh[i] = to_f32(k[r]) * rk;
        const float qh = to_f32(q[r]) * rq;
        s[i] = s[i] * dec;
        pp += s[i] * kh[i];
        rr += s[i] * qh;
    }
    *reinterpret_cast<f32x4*>(&red[0][rg][4 * cg]) = pp;
    *reinterpret_cast<f32x4*>(&red[1][rg][4 * cg]) = rr;
    __syncthreads();
    f32x4 p = {0.f, 0.f, 0.f, 0.f}, r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < RG; ++j) {
        p += *reinterpret_cast<const f32x4*>(&red[0][j][4 * cg]);
        r += *reinterpret_cast<const f32x4*>(&red[1][j][4 * cg]);
    }
    const f32x4 vv = ld4(v + col0 + 4 * cg);
    const f32x4 u = bt * (vv - p);

    // corrective write, in place
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        __builtin_nontemporal_store(s[i] + kh[i] * u,
                                    reinterpret_cast<f32x4*>(S + (size_t)(rg * RPT + i) * DV + col0 + 4 * cg));

    if (rg == 0) {
        const f32x4 gg = ld4(gp + col0 + 4 * cg);
        const f32x4 o = r + u * khqh;
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = o[e] * sigmoidf_(gg[e]);
        st4(reinterpret_cast<E*>(a.out) + nh * DV + col0 + 4 * cg, y);
    }
}

// LDS reserved (and unused) per workgroup so that at most two workgroups
// share a CU: fewer state streams in flight at once run faster.  Measured at
// 256 sequences x 32 heads, d = 128: 177-179 us per step with two per CU,
// 189 us with three, 192 us with four (the register limit), 210 us with one.
constexpr unsigned kDecodeLdsReserve = 64 * 1024;

template <typename E, int DK, int NSPLIT>
hipError_t launch_decode_n(const DecodeArgs& a, hipStream_t s) {
    const int64_t blocks = a.N * (int64_t)a.H * NSPLIT;
    hipLaunchKernelGGL((kda_decode_kernel<E, DK, NSPLIT>), dim3((unsigned)blocks), dim3(kThreads), kDecodeLdsReserve,
                       s, a);
    return hipGetLastError();
}

// A head's value columns never interact once the norms are known, so with
// few (sequence, head) pairs each pair's state is split over two workgroups
// of d_v / 2 columns (each recomputes the norms): more state streams in
// flight.  Measured with H = 32, d = 128, steps replayed from a graph: 3.70
// against 4.10 us per step at 1 sequence, 4.22 against 4.64 at 4, 6.97
// against 7.57 at 8; from 16 sequences (512 pairs) on one workgroup per
// pair is faster (11.4 against 13.6 us), and four per pair was never better.
constexpr int64_t kDecodeSplitMaxPairs = 256;

template <typename E, int DK>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
    const int64_t pairs = a.N * (int64_t)a.H;
    if (pairs == 0) return hipSuccess;
    if (pairs <= kDecodeSplitMaxPairs) return launch_decode_n<E, DK, 2>(a, s);
    return launch_decode_n<E, DK, 1>(a, s);
}

}  // namespace

hipError_t launch_decode(bool bf16, int dk, const DecodeArgs& a, hipStream_t s) {
    if (bf16) return dk == 128 ? launch_decode_t<__bf16, 128>(a, s) : launch_decode_t<__bf16, 64>(a, s);
    return dk == 128 ? launch_decode_t<float, 128>(a, s) : launch_decode_t<float, 64>(a, s);
}

}  // namespace kda
