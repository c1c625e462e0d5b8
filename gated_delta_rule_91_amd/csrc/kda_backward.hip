// kda_backward.hip -- gradients of the KDA token mixer for training: with
// L = <d_out, out> + <d_state, S_T>, the gradients with respect to q, k, v,
// log_alpha, beta, g and the initial state (the pages say the fast kernels
// serve training throughput [zuoshipin.com/article/18261 §四, FlashKDA
// paragraph]; the recurrence is the one of the forward path, §二).
//
// This is the token-recurrent form of the adjoint, in fp32, one workgroup
// per (batch row, head):
//   phase 1  the forward recurrence over the whole sequence, storing the
//            state entering every chunk of 64 tokens (checkpoints);
//   phase 2  the chunks in reverse: the chunk's 64 entering states are
//            recomputed from its checkpoint into the workspace, then its
//            tokens are walked backwards.  Per token, with S_prev the entering
//            state, D = diag(e^lambda), S' = D S_prev, p = S'^T kh,
//            u = beta (v - p), S = S' + kh u^T, o = S^T qh, and dS the
//            gradient with respect to S:
//              do = d_out * sigmoid(g);  dg = d_out * o * sigmoid'(g)
//              dqh = S do;  dS += qh do^T
//              du = dS^T kh;  dbeta = du . (v - p);  dv = beta du;  dp = -beta du
//              dkh = dS u + S' dp;  dS' = dS + kh dp^T
//              dlambda_c = sum_j S'[c][j] dS'[c][j] (zero where the floor binds)
//              dS_prev = D dS';  dk, dq from dkh, dqh through the L2 normalisation
//
// Thread (column group cg, row group rg) keeps an RPT x 4 block of the state
// and of its gradient in registers.  Column sums over the rows go through
// LDS (one barrier each); row sums over the columns are lane shuffles inside
// the wave (a wave holds whole rows).
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

namespace {

template <typename E, int DK>
__global__ __launch_bounds__(kThreads) void kda_backward_kernel(BackwardArgs a) {
    constexpr int DV = DK;
    constexpr int C = kChunk;
    constexpr int CG = DV / 4;          // 4-column groups
    constexpr int RG = kThreads / CG;   // row groups
    constexpr int RPT = DK / RG;        // rows per thread
    constexpr int EPL = DK / 64;        // elements per lane for the norm sweep
    static_assert(64 % CG == 0, "a wave holds whole rows");
    static_assert(RPT <= CG, "lane cg == i writes row i of the thread's block");

    __shared__ float colred[3][RG][DV];   // partial column sums: p, o, du
    __shared__ float dotred[2][RG];       // partial kh . dkh, qh . dqh

    const int t = threadIdx.x, lane = t & 63, cg = t % CG, rg = t / CG;
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / a.H;
    const int h = (int)(bh % a.H);
    const int64_t T = a.T;
    const int NC = (int)((T + C - 1) / C);
    const size_t SZ = (size_t)DK * DV;
    // per (b, h): checkpoints [NC][DK][DV], then the chunk's entering states [C][DK][DV]
    // (no workspace, and no use of it, when T == 0)
    float* ckpt = a.ws + (T > 0 ? (size_t)bh * ((size_t)NC + C) * SZ : 0);
    float* hist = ckpt + (size_t)NC * SZ;                        // [C][DK][DV]
    const size_t blk = (size_t)(rg * RPT) * DV + 4 * cg;        // this thread's block origin

    auto row_of = [&](int64_t tok) { return ((size_t)b * T + tok) * a.H + h; };

    // column sum over all rows of this thread's partial x (4 columns)
    auto colsum = [&](int slot, f32x4 x) {
        *reinterpret_cast<f32x4*>(&colred[slot][rg][4 * cg]) = x;
        __syncthreads();
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < RG; ++j) s += *reinterpret_cast<const f32x4*>(&colred[slot][j][4 * cg]);
        return s;
    };
    // row sum over the CG column groups (lanes of one wave)
    auto rowsum = [&](float x) {
#pragma unroll
        for (int m = 1; m < CG; m <<= 1) x += __shfl_xor(x, m);
        return x;
    };
    // per-token row data: normalised k and q on this thread's rows, the
    // decays, and the norms (each wave sweeps the full vectors)
    struct Tok {
        float kh[RPT], qh[RPT], D[RPT], la[RPT];
        float nk, nq, beta;
        f32x4 v;
    };
    auto load_tok = [&](int64_t tok, Tok& x) {
        const size_t row = row_of(tok);
        const E* k = reinterpret_cast<const E*>(a.k) + row * DK;
        const E* q = reinterpret_cast<const E*>(a.q) + row * DK;
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const float kk = to_f32(k[lane * EPL + e]), qq = to_f32(q[lane * EPL + e]);
            sk += kk * kk; sq += qq * qq;
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            sk += __shfl_xor(sk, off);
            sq += __shfl_xor(sq, off);
        }
        x.nk = sqrtf(sk);
        x.nq = sqrtf(sq);
        const float rk = 1.0f / fmaxf(x.nk, 1e-6f), rq = 1.0f / fmaxf(x.nq, 1e-6f);
        const float* la = a.log_alpha + row * DK;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg * RPT + i;
            x.kh[i] = to_f32(k[r]) * rk;
            x.qh[i] = to_f32(q[r]) * rq;
            x.la[i] = la[r];
            x.D[i] = __expf(fmaxf(la[r], a.floor_));
        }
        x.beta = a.beta[row];
        x.v = ld4(reinterpret_cast<const E*>(a.v) + row * DV + 4 * cg);
    };

    f32x4 S[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        S[i] = a.state_in ? *reinterpret_cast<const f32x4*>(a.state_in + bh * SZ + blk + (size_t)i * DV)
                          : f32x4{0.f, 0.f, 0.f, 0.f};

    // one forward step on S (retention, prediction, corrective write)
    auto fwd = [&](const Tok& x) {
        f32x4 pp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            S[i] = S[i] * x.D[i];
            pp += S[i] * x.kh[i];
        }
        const f32x4 p = colsum(0, pp);
        const f32x4 u = x.beta * (x.v - p);
#pragma unroll
        for (int i = 0; i < RPT; ++i) S[i] += x.kh[i] * u;
        __syncthreads();   // colred[0] is reused by the next step
    };

    // ---- phase 1: checkpoints ----
    for (int64_t tok = 0; tok < T; ++tok) {
        if (tok % C == 0) {
#pragma unroll
            for (int i = 0; i < RPT; ++i)
                *reinterpret_cast<f32x4*>(ckpt + (size_t)(tok / C) * SZ + blk + (size_t)i * DV) = S[i];
        }
        Tok x;
        load_tok(tok, x);
        fwd(x);
    }

    // ---- phase 2: chunks in reverse ----
    f32x4 dS[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        dS[i] = a.d_state ? *reinterpret_cast<const f32x4*>(a.d_state + bh * SZ + blk + (size_t)i * DV)
                          : f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c = NC - 1; c >= 0; --c) {
        const int64_t t0 = (int64_t)c * C;
        const int n = (int)(T - t0 < C ? T - t0 : C);
        // recompute the entering states of the chunk's tokens
#pragma unroll
        for (int i = 0; i < RPT; ++i) S[i] = *reinterpret_cast<const f32x4*>(ckpt + (size_t)c * SZ + blk + (size_t)i * DV);
        for (int j = 0; j < n; ++j) {
#pragma unroll
            for (int i = 0; i < RPT; ++i) *reinterpret_cast<f32x4*>(hist + (size_t)j * SZ + blk + (size_t)i * DV) = S[i];
            if (j + 1 < n) {
                Tok x;
                load_tok(t0 + j, x);
                fwd(x);
            }
        }
        __syncthreads();
        // tokens in reverse
        for (int j = n - 1; j >= 0; --j) {
            const int64_t tok = t0 + j;
            const size_t row = row_of(tok);
            Tok x;
            load_tok(tok, x);
            f32x4 Sp[RPT];
            f32x4 pp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                Sp[i] = *reinterpret_cast<const f32x4*>(hist + (size_t)j * SZ + blk + (size_t)i * DV) * x.D[i];
                pp += Sp[i] * x.kh[i];
            }
            const f32x4 p = colsum(0, pp);
            const f32x4 u = x.beta * (x.v - p);
            f32x4 oo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < RPT; ++i) oo += (Sp[i] + x.kh[i] * u) * x.qh[i];
            const f32x4 o = colsum(1, oo);
            // output gate
            const f32x4 dy = a.d_out ? ld4(reinterpret_cast<const E*>(a.d_out) + row * DV + 4 * cg)
                                     : f32x4{0.f, 0.f, 0.f, 0.f};
            const f32x4 gg = ld4(reinterpret_cast<const E*>(a.g) + row * DV + 4 * cg);
            f32x4 dov, dgv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float sg = sigmoidf_(gg[e]);
                dov[e] = dy[e] * sg;
                dgv[e] = dy[e] * o[e] * sg * (1.f - sg);
            }
            if (rg == 0) st4(reinterpret_cast<E*>(a.dg) + row * DV + 4 * cg, dgv);
            // dqh = S do (S after the write), dS += qh do^T, du = dS^T kh
            float dqh[RPT];
            f32x4 dd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const f32x4 St = Sp[i] + x.kh[i] * u;
                dqh[i] = rowsum(St[0] * dov[0] + St[1] * dov[1] + St[2] * dov[2] + St[3] * dov[3]);
                dS[i] += x.qh[i] * dov;
                dd += dS[i] * x.kh[i];
            }
            const f32x4 du = colsum(2, dd);
            if (rg == 0) {
                st4(reinterpret_cast<E*>(a.dv) + row * DV + 4 * cg, x.beta * du);
                const f32x4 vp = x.v - p;
                const float db = rowsum(du[0] * vp[0] + du[1] * vp[1] + du[2] * vp[2] + du[3] * vp[3]);
                if (cg == 0) a.dbeta[row] = db;
            }
            const f32x4 dp = -x.beta * du;
            // dkh = dS u + S' dp; dS' = dS + kh dp^T; dlambda; dS_prev = D dS'
            float dkh[RPT];
            float kdot = 0.f, qdot = 0.f;
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const f32x4 m = dS[i] * u + Sp[i] * dp;
                dkh[i] = rowsum(m[0] + m[1] + m[2] + m[3]);
                dS[i] += x.kh[i] * dp;
                const f32x4 l = Sp[i] * dS[i];
                const float dl = rowsum(l[0] + l[1] + l[2] + l[3]);
                if (cg == i)   // one lane per row writes
                    a.dlog_alpha[row * DK + rg * RPT + i] = x.la[i] > a.floor_ ? dl : 0.f;
                dS[i] *= x.D[i];
                kdot += x.kh[i] * dkh[i];
                qdot += x.qh[i] * dqh[i];
            }
            // L2 normalisation: dx = (dxh - xh (xh . dxh)) / |x| (constant divisor below 1e-6)
            if (cg == 0) {
                dotred[0][rg] = kdot;
                dotred[1][rg] = qdot;
            }
            __syncthreads();
            float kd = 0.f, qd = 0.f;
#pragma unroll
            for (int r = 0; r < RG; ++r) { kd += dotred[0][r]; qd += dotred[1][r]; }
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                if (cg == i) {
                    const int r = rg * RPT + i;
                    reinterpret_cast<E*>(a.dk)[row * DK + r] =
                        from_f32<E>(x.nk < 1e-6f ? dkh[i] * 1e6f : (dkh[i] - x.kh[i] * kd) / x.nk);
                    reinterpret_cast<E*>(a.dq)[row * DK + r] =
                        from_f32<E>(x.nq < 1e-6f ? dqh[i] * 1e6f : (dqh[i] - x.qh[i] * qd) / x.nq);
                }
            }
            __syncthreads();   // colred and dotred are reused by the next token
        }
    }
    if (a.d_state_in) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) *reinterpret_cast<f32x4*>(a.d_state_in + bh * SZ + blk + (size_t)i * DV) = dS[i];
    }
}

template <typename E, int DK>
hipError_t launch_backward_t(const BackwardArgs& a, hipStream_t s) {
    const int64_t blocks = a.B * (int64_t)a.H;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((kda_backward_kernel<E, DK>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(int64_t B, int64_t T, int H, int dk) {
    const int64_t NC = (T + kChunk - 1) / kChunk;
    return T == 0 ? 0 : (size_t)B * H * (size_t)(NC + kChunk) * dk * dk * sizeof(float);
}

hipError_t launch_backward(bool bf16, int dk, const BackwardArgs& a, hipStream_t s) {
    if (bf16) return dk == 128 ? launch_backward_t<__bf16, 128>(a, s) : launch_backward_t<__bf16, 64>(a, s);
    return dk == 128 ? launch_backward_t<float, 128>(a, s) : launch_backward_t<float, 64>(a, s);
}

}  // namespace kda
