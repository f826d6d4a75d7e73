// Single-token TTT-Linear step (b = 1, primal form) on B x H independent
// states held in place: the fast-weight cache of the damodev.csdn.net TTT
// deep-dive (§5.2), with the update-then-apply rule of its §3.1:
//   z = xk W + b;  G = lnbwd(z, xv - xk)
//   W' = W - eta xk^T G;  b' = b - eta G
//   o  = xq + LN(xq W' + b')
// The state is read once and written once. The output uses the identity
//   xq W' + b' = (xq W + b) - eta (xq . xk + 1) G,
// so both dot products against W come out of the same single sweep over the
// state (no second read of W).
//
// One 256-thread workgroup per state. Thread (p, j) owns column j, rows
// p*RPT .. p*RPT+RPT-1 of W; for fixed rows a wave reads a contiguous row
// segment (coalesced). Column partials meet in LDS.
//
// Mini-batch decode (b > 1, mode != 0): the gradient is taken at the
// chunk-start state (Wc, bc) instead of (W, b); mode 1 starts a chunk (the
// current state is copied to Wc, bc first, and z uses it), mode 2 reads Wc,
// bc. The output identity still uses the current W: xq W' + b' =
// (xq W + b) - eta (xq . xk + 1) G.
//
// GATED: the step's rate comes from the learning-rate gate of the
// lryc.cn TTT article (§2.2), eta = eta_base * logistic(theta[h] . xk), x read
// as the key, instead of the eta array.
#include "common.hpp"
#include "launch.hpp"

namespace ttt {

template <int D, typename TIO, bool GATED, int MODE>
__global__ __launch_bounds__(256) void decode_step_kernel(
    int H, float eps, const TIO *__restrict__ xq, const TIO *__restrict__ xk,
    const TIO *__restrict__ xv, const float *__restrict__ eta, float *__restrict__ W,
    float *__restrict__ b, const float *__restrict__ gamma, const float *__restrict__ beta,
    TIO *__restrict__ o, float *__restrict__ Wc, float *__restrict__ bc,
    const float *__restrict__ theta, float eta_base) {
    constexpr int NT = 256, P = NT / D, RPT = D / P, E = D / 16;
    using io = io_traits<TIO>;
    __shared__ float sq[D], sk[D], sG[D];
    __shared__ float sPz[P * D], sPq[P * D];
    __shared__ float sCoef;

    const int tid = threadIdx.x;
    const long seq = blockIdx.x;
    const int h = static_cast<int>(seq % H);
    const int j = tid % D, p = tid / D;
    float *Ws = W + static_cast<size_t>(seq) * D * D;

    if (tid < D) {
        sq[tid] = io::load(xq, static_cast<size_t>(seq) * D + tid);
        sk[tid] = io::load(xk, static_cast<size_t>(seq) * D + tid);
    }
    float w[RPT], wz[RPT];  // current state; state the gradient is taken at
    float *Wcs = Wc ? Wc + static_cast<size_t>(seq) * D * D : nullptr;
#pragma unroll
    for (int r = 0; r < RPT; ++r) w[r] = Ws[static_cast<size_t>(p * RPT + r) * D + j];
#pragma unroll
    for (int r = 0; r < RPT; ++r)
        wz[r] = MODE == 2 ? Wcs[static_cast<size_t>(p * RPT + r) * D + j] : w[r];
    if constexpr (MODE == 1) {  // a chunk starts here: its start state is the current one
#pragma unroll
        for (int r = 0; r < RPT; ++r) Wcs[static_cast<size_t>(p * RPT + r) * D + j] = w[r];
    }
    __syncthreads();

    float pz = 0.f, pq = 0.f;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        pz += sk[p * RPT + r] * wz[r];
        pq += sq[p * RPT + r] * w[r];
    }
    sPz[p * D + j] = pz;
    sPq[p * D + j] = pq;
    __syncthreads();

    if (tid < 16) {
        float et;
        if constexpr (GATED) {  // the gate from the staged key
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) s += theta[static_cast<size_t>(h) * D + tid + 16 * e] * sk[tid + 16 * e];
            et = eta_base / (1.f + expf(-group_sum<16>(s)));
        } else {
            et = eta[seq];
        }
        float z[E], tau[E], g[E], zb[E], y[E], gm[E], bt[E], bb[E], q[E];
        float qk = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int jj = tid + 16 * e;
            float zs = 0.f, qs = 0.f;
#pragma unroll
            for (int pp = 0; pp < P; ++pp) {
                zs += sPz[pp * D + jj];
                qs += sPq[pp * D + jj];
            }
            bb[e] = b[static_cast<size_t>(seq) * D + jj];
            const size_t bi = static_cast<size_t>(seq) * D + jj;
            z[e] = zs + (MODE == 2 ? bc[bi] : bb[e]);
            if constexpr (MODE == 1) bc[bi] = bb[e];
            q[e] = qs;
            tau[e] = io::load(xv, static_cast<size_t>(seq) * D + jj) - sk[jj];
            gm[e] = gamma[static_cast<size_t>(h) * D + jj];
            bt[e] = beta[static_cast<size_t>(h) * D + jj];
            qk += sq[jj] * sk[jj];
        }
        qk = group_sum<16>(qk);
        ln_l2_grad<16, E>(z, tau, gm, bt, 1.0f / D, eps, g);
        const float c = et * (qk + 1.f);
#pragma unroll
        for (int e = 0; e < E; ++e) zb[e] = q[e] + bb[e] - c * g[e];
        ln_fwd<16, E>(zb, gm, bt, 1.0f / D, eps, y);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int jj = tid + 16 * e;
            io::store(o, static_cast<size_t>(seq) * D + jj, sq[jj] + y[e]);
            b[static_cast<size_t>(seq) * D + jj] = bb[e] - et * g[e];
            sG[jj] = g[e];
        }
        if (tid == 0) sCoef = et;
    }
    __syncthreads();

    const float et = sCoef, gj = sG[j];
#pragma unroll
    for (int r = 0; r < RPT; ++r)
        Ws[static_cast<size_t>(p * RPT + r) * D + j] = w[r] - et * sk[p * RPT + r] * gj;
}

template <int D, typename TIO, bool GATED, int MODE>
static hipError_t launch_decode_m(const DecodeArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL((decode_step_kernel<D, TIO, GATED, MODE>), dim3(a.B * a.H), dim3(256), 0, stream, a.H,
                       a.eps, static_cast<const TIO *>(a.xq), static_cast<const TIO *>(a.xk),
                       static_cast<const TIO *>(a.xv), a.eta, a.W, a.b, a.gamma, a.beta,
                       static_cast<TIO *>(a.o), a.Wc, a.bc, a.theta, a.eta_base);
    return hipGetLastError();
}

// mode (b > 1 decode): 0 plain b = 1 step, 1 starts a chunk, 2 continues one
template <int D, typename TIO, bool GATED>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t stream) {
    if (a.mode == 1) return launch_decode_m<D, TIO, GATED, 1>(a, stream);
    if (a.mode == 2) return launch_decode_m<D, TIO, GATED, 2>(a, stream);
    return launch_decode_m<D, TIO, GATED, 0>(a, stream);
}

template <bool GATED>
static hipError_t launch_decode_g(const DecodeArgs &a, hipStream_t stream) {
    if (a.d == 16) return a.io ? launch_decode_t<16, bf16_t, GATED>(a, stream) : launch_decode_t<16, float, GATED>(a, stream);
    if (a.d == 64) return a.io ? launch_decode_t<64, bf16_t, GATED>(a, stream) : launch_decode_t<64, float, GATED>(a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
    if (a.B * a.H == 0) return hipSuccess;
    return a.theta ? launch_decode_g<true>(a, stream) : launch_decode_g<false>(a, stream);
}

}  // namespace ttt
