// TTT-Linear prefill, fp32 VALU kernel: the path for fp32 storage, d = 16,
// and chunk sizes other than 16. One 256-thread workgroup per (n,h) sequence;
// the fp32 state W [d,d] and b [d] live in LDS for the whole sequence.
//
// Per chunk of up to 16 tokens (dual form of the damodev.csdn.net TTT
// deep-dive §4.2, with the LN-residual output of the lryc.cn article §2.1):
//   Z    = XK W + b                                  (chunk-start state)
//   G    = lnbwd(Z, XV - XK)                          (per row)
//   M    = tril((XQ XK^T + 1) * eta_col)              (token s <= t)
//   Zbar = XQ W + b - M G        ;  O = XQ + LN(Zbar)
//   W   -= (eta * XK)^T G        ;  b -= eta^T G
// Tokens past the end of a short last chunk carry eta = 0 and G = 0.
// With the learning-rate gate (theta set) eta_t = eta_base * logistic(theta_h .
// XK_t) is formed from the staged keys (the lryc.cn article §2.2 gate).
// Modular-TTT options: loss = 1 takes G from the inner-product loss
// -< XK + LN(Z), XV > (target XV, gh = -gamma * XV); weight decay lambda adds
// lambda * W_c to every token's W gradient (W_c = chunk-start state), so
//   Zbar_t = (1 - lambda * cum_t) XQ_t W_c + b - (M G)_t,  cum_t = sum_{s<=t} eta_s
//   W     <- (1 - lambda * cum_last) W_c - (eta * XK)^T G.
#include "common.hpp"
#include "launch.hpp"

namespace ttt {

template <int D, typename TIO>
__global__ __launch_bounds__(256) void linear_prefill_valu(
    int H, int L, int mb, float eps, const TIO *__restrict__ XQ, const TIO *__restrict__ XK,
    const TIO *__restrict__ XV, const float *__restrict__ eta, const float *__restrict__ theta,
    float eta_base, const float *W0, const float *b0, int w0_batched,
    const float *__restrict__ gamma,
    const float *__restrict__ beta, TIO *__restrict__ O, float *W_out, float *b_out, int loss,
    float wd) {
    constexpr int NT = 256, MB = 16, DP = D + 1;
    constexpr int R = MB * D / NT;  // outputs per thread in the row-by-column products
    constexpr int SS = NT / D;      // token stride between them
    constexpr int E = D / 16;       // features per lane in the 16-lane row groups
    using io = io_traits<TIO>;

    __shared__ float sW[D * D];
    __shared__ float sb[D];
    __shared__ float sQ[MB * DP], sK[MB * DP];
    __shared__ float sT[MB * D], sZ[MB * D], sG[MB * D];
    __shared__ float sEta[MB], sM[MB * MB];
    __shared__ float sTh[D];
    __shared__ float sDec[MB];  // 1 - lambda * cum_t (weight decay)
    __shared__ float sWbar[D], sBbar[1];  // row means of W0, mean of b0

    const int tid = threadIdx.x;
    const long seq = blockIdx.x;
    const int h = static_cast<int>(seq % H);
    const long n = seq / H;
    const size_t xbase = static_cast<size_t>(seq) * L * D;
    const size_t ebase = static_cast<size_t>(seq) * L;
    const size_t wofs = (w0_batched ? static_cast<size_t>(n) * H * D * D : 0) + static_cast<size_t>(h) * D * D;
    const size_t bofs = (w0_batched ? static_cast<size_t>(n) * H * D : 0) + static_cast<size_t>(h) * D;

    for (int e = tid; e < D * D; e += NT) sW[e] = W0[wofs + e];
    if (tid < D) sb[tid] = b0[bofs + tid];
    if (theta && tid < D) sTh[tid] = theta[static_cast<size_t>(h) * D + tid];

    const int rrow = tid / 16, rl = tid % 16;  // 16-lane row groups
    float gam[E], bet[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        gam[e] = gamma[static_cast<size_t>(h) * D + rl + 16 * e];
        bet[e] = beta[static_cast<size_t>(h) * D + rl + 16 * e];
    }
    const int cj = tid % D, cs0 = tid / D;  // column-product mapping
    __syncthreads();

    // Centred state: W - wbar 1^T and b - bbar (wbar the row means of W0,
    // bbar the mean of b0) shift every row of z by a per-token constant that
    // the layer norm and its backward do not see, and keep z small when the
    // caller's state carries a large offset (z is formed in fp32, so an
    // offset m would otherwise cost ulp(m) of the row's spread). The rows of
    // the gradient sum to zero, so the updates keep the centring; weight
    // decay scales wbar with W (rho). The state is restored on the way out.
    float rho = 1.f;
    if (L > 0) {
        if (tid < D) {
            float a = 0.f;
            for (int j = 0; j < D; ++j) a += sW[tid * D + j];
            sWbar[tid] = a * (1.0f / D);
        }
        if (tid == 0) {
            float a = 0.f;
            for (int j = 0; j < D; ++j) a += sb[j];
            sBbar[0] = a * (1.0f / D);
        }
        __syncthreads();
        for (int e = tid; e < D * D; e += NT) sW[e] -= sWbar[e / D];
        if (tid < D) sb[tid] -= sBbar[0];
        __syncthreads();
    }

    for (int t0 = 0; t0 < L; t0 += mb) {
        const int len = min(mb, L - t0);
        // 1. chunk -> LDS
        for (int e = tid; e < MB * D; e += NT) {
            const int s = e / D, j = e % D;
            float q = 0.f, k = 0.f, v = 0.f;
            if (s < len) {
                const size_t g = xbase + static_cast<size_t>(t0 + s) * D + j;
                q = io::load(XQ, g);
                k = io::load(XK, g);
                v = io::load(XV, g);
            }
            sQ[s * DP + j] = q;
            sK[s * DP + j] = k;
            sT[s * D + j] = loss ? v : v - k;  // the loss's target
        }
        if (!theta && tid < MB) sEta[tid] = tid < len ? eta[ebase + t0 + tid] : 0.f;
        __syncthreads();

        // 2. Z = XK W + b (and the gated eta, read after the next barrier)
        if (theta && tid < MB) {
            float s = 0.f;
            for (int i = 0; i < D; ++i) s = fmaf(sK[tid * DP + i], sTh[i], s);
            sEta[tid] = tid < len ? eta_base / (1.0f + __expf(-s)) : 0.f;
        }
        {
            float acc[R];
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = sb[cj];
            for (int i = 0; i < D; ++i) {
                const float w = sW[i * D + cj];
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r] += sK[(cs0 + r * SS) * DP + i] * w;
            }
#pragma unroll
            for (int r = 0; r < R; ++r) sZ[(cs0 + r * SS) * D + cj] = acc[r];
        }
        __syncthreads();

        // 3. G = lnbwd(Z, XV - XK) per row; M = causal (Gram + 1) * eta
        {
            float z[E], tau[E], g[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                z[e] = sZ[rrow * D + rl + 16 * e];
                tau[e] = sT[rrow * D + rl + 16 * e];
            }
            if (loss)
                ln_ip_grad<16, E>(z, tau, gam, 1.0f / D, eps, g);
            else
                ln_l2_grad<16, E>(z, tau, gam, bet, 1.0f / D, eps, g);
            if (tid < MB) {  // decay factor of token tid's W_c term
                float cum = 0.f;
                for (int s = 0; s <= tid; ++s) cum += sEta[s];
                sDec[tid] = 1.0f - wd * cum;
            }
#pragma unroll
            for (int e = 0; e < E; ++e) sG[rrow * D + rl + 16 * e] = rrow < len ? g[e] : 0.f;

            const int t = tid / MB, s = tid % MB;
            float a = 0.f;
            for (int i = 0; i < D; ++i) a += sQ[t * DP + i] * sK[s * DP + i];
            sM[t * MB + s] = (s <= t) ? sEta[s] * (a + 1.f) : 0.f;
        }
        __syncthreads();

        // 4. Zbar = (1 - lambda cum) XQ W + b - M G
        {
            float acc[R];
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = 0.f;
            for (int i = 0; i < D; ++i) {
                const float w = sW[i * D + cj];
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r] += sQ[(cs0 + r * SS) * DP + i] * w;
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
                acc[r] = (wd != 0.f ? acc[r] * sDec[cs0 + r * SS] : acc[r]) + sb[cj];
            for (int s = 0; s < MB; ++s) {
                const float gs = sG[s * D + cj];
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r] -= sM[(cs0 + r * SS) * MB + s] * gs;
            }
#pragma unroll
            for (int r = 0; r < R; ++r) sZ[(cs0 + r * SS) * D + cj] = acc[r];
        }
        __syncthreads();

        // 5. O = XQ + LN(Zbar); state update
        {
            float z[E], y[E];
#pragma unroll
            for (int e = 0; e < E; ++e) z[e] = sZ[rrow * D + rl + 16 * e];
            ln_fwd<16, E>(z, gam, bet, 1.0f / D, eps, y);
            if (rrow < len) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int j = rl + 16 * e;
                    io::store(O, xbase + static_cast<size_t>(t0 + rrow) * D + j, sQ[rrow * DP + j] + y[e]);
                }
            }
            const float dec = sDec[MB - 1];  // eta past the chunk's end is 0
            if (wd != 0.f) rho *= dec;
            for (int e = tid; e < D * D; e += NT) {
                const int i = e / D, j = e % D;
                float acc = 0.f;
#pragma unroll
                for (int s = 0; s < MB; ++s) acc += sEta[s] * sK[s * DP + i] * sG[s * D + j];
                sW[e] = (wd != 0.f ? sW[e] * dec : sW[e]) - acc;
            }
            if (tid < D) {
                float acc = 0.f;
#pragma unroll
                for (int s = 0; s < MB; ++s) acc += sEta[s] * sG[s * D + tid];
                sb[tid] -= acc;
            }
        }
        __syncthreads();
    }

    if (L > 0) {  // back to the caller's representation
        for (int e = tid; e < D * D; e += NT) sW[e] = fmaf(rho, sWbar[e / D], sW[e]);
        if (tid < D) sb[tid] += sBbar[0];
        __syncthreads();
    }
    if (W_out) {
        for (int e = tid; e < D * D; e += NT) W_out[static_cast<size_t>(seq) * D * D + e] = sW[e];
    }
    if (b_out && tid < D) b_out[static_cast<size_t>(seq) * D + tid] = sb[tid];
}

template <int D, typename TIO>
static hipError_t launch_valu_t(const LinearArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL((linear_prefill_valu<D, TIO>), dim3(a.B * a.H), dim3(256), 0, stream, a.H,
                       a.L, a.mb, a.eps, static_cast<const TIO *>(a.XQ),
                       static_cast<const TIO *>(a.XK), static_cast<const TIO *>(a.XV), a.eta,
                       a.theta, a.eta_base, a.W0, a.b0, a.w0_batched, a.gamma, a.beta, static_cast<TIO *>(a.O),
                       a.W_out, a.b_out, a.loss, a.wd);
    return hipGetLastError();
}

hipError_t launch_linear_valu(const LinearArgs &a, hipStream_t stream) {
    if (a.B * a.H == 0) return hipSuccess;
    if (a.d == 16) return a.io ? launch_valu_t<16, bf16_t>(a, stream) : launch_valu_t<16, float>(a, stream);
    if (a.d == 64) return a.io ? launch_valu_t<64, bf16_t>(a, stream) : launch_valu_t<64, float>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace ttt
