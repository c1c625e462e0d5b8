// kda_combine.hip -- in-order prefix merge of per-segment summaries
// [zuoshipin.com/article/18261 §三, "KDA 上下文并行" paragraph: the segments'
// fixed-size reports are merged in order to recover the exact state that
// enters every segment].
//
//   S(0) = state_init (or 0);  seg_state_in[n] = S(n);
//   S(n+1) = A_n S(n) + Bz_n;  state_final = S(n_seg)
//
// The columns of S evolve independently, so each (batch row, head, block of
// 16 columns) is one workgroup; the 16-column slice of S stays in LDS across
// the segments and each step is a d_k x d_k x 16 product in fp32 FMA, with
// each thread's whole row of A_n requested before the products.  The
// work is tiny (n_seg dependent steps per head); it is kept exact in fp32
// because every later segment starts from its result.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

namespace {

template <int DK>
__global__ __launch_bounds__(kThreads) void kda_combine_kernel(CombineArgs a) {
    constexpr int DV = DK;
    constexpr int NCB = DV / 16;             // column blocks per head
    constexpr int TPR = kThreads / DK;       // threads per row (2 or 4)
    constexpr int CPT = 16 / TPR;            // columns per thread (8 or 4)
    __shared__ __attribute__((aligned(16))) float sS[2][DK][16];

    const int t = threadIdx.x;
    const int64_t x = blockIdx.x;
    const int cb = (int)(x % NCB);
    const int64_t bh = x / NCB;
    const int64_t b = bh / a.H;
    const int h = (int)(bh % a.H);
    const int i = t / TPR, j0 = (t % TPR) * CPT;
    const int col0 = cb * 16;

    float cur[CPT];
#pragma unroll
    for (int e = 0; e < CPT; ++e)
        cur[e] = a.s0 ? a.s0[((size_t)bh * DK + i) * DV + col0 + j0 + e] : 0.f;
#pragma unroll
    for (int e = 0; e < CPT; ++e) sS[0][i][j0 + e] = cur[e];
    __syncthreads();

    int buf = 0;
    for (int sg = 0; sg < a.n_seg; ++sg) {
        const size_t sh = ((size_t)b * a.n_seg + sg) * a.H + h;
        float* dst = a.seg_in + (sh * DK + i) * DV + col0 + j0;
#pragma unroll
        for (int e = 0; e < CPT; ++e) dst[e] = cur[e];
        const float* Ar = a.A + (sh * DK + i) * DK;
        const float* Br = a.Bz + (sh * DK + i) * DV + col0 + j0;
        // the whole row of A_n is requested at once, so a step waits on one
        // memory latency rather than one per 16 bytes
        f32x4 av[DK / 4];
#pragma unroll
        for (int q = 0; q < DK / 4; ++q) av[q] = *reinterpret_cast<const f32x4*>(Ar + 4 * q);
        float acc[CPT];
#pragma unroll
        for (int e = 0; e < CPT; ++e) acc[e] = Br[e];
        __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of the products
#pragma unroll
        for (int q = 0; q < DK / 4; ++q)
#pragma unroll
            for (int cc = 0; cc < 4; ++cc)
#pragma unroll
                for (int e = 0; e < CPT; ++e) acc[e] = fmaf(av[q][cc], sS[buf][4 * q + cc][j0 + e], acc[e]);
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            cur[e] = acc[e];
            sS[buf ^ 1][i][j0 + e] = acc[e];
        }
        buf ^= 1;
        __syncthreads();
    }
    if (a.fin) {
#pragma unroll
        for (int e = 0; e < CPT; ++e) a.fin[((size_t)bh * DK + i) * DV + col0 + j0 + e] = cur[e];
    }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
    const int64_t blocks = a.B * (int64_t)a.H * (a.dv / 16);
    if (blocks == 0) return hipSuccess;
    if (a.dk == 128)
        hipLaunchKernelGGL(kda_combine_kernel<128>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(kda_combine_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace kda
