// TTT-MLP prefill (d = 64, hidden m = 4d = 256, exact GELU), mini-batch dual
// form. Hidden model from the lryc.cn TTT article §2.1 (d -> 4d GELU -> d
// inside the LN residual), inner loop from the damodev.csdn.net deep-dive
// §4.2. One 256-thread workgroup per (n,h) sequence:
//   thread k owns hidden unit k: column W1[:,k] (64 fp32 in registers), b1[k];
//   W2 [256,64] and b2 live in LDS for the whole sequence; per-chunk hidden
//   vectors (A, gelu'(Z1), G1, Ab) pass through LDS.
// Per chunk (state at chunk start; tokens s, t of the chunk, s <= t causal):
//   Z1 = XK W1 + b1, A = gelu(Z1), Z2 = A W2 + b2, G2 = lnbwd(Z2, XV - XK)
//   G1 = (G2 W2^T) * gelu'(Z1)
//   Zb1 = XQ W1 + b1 - M1 G1,     M1[t,s] = eta_s (XQ_t . XK_s + 1)
//   Ab  = gelu(Zb1)
//   Zb2 = Ab W2 + b2 - M2 G2,     M2[t,s] = eta_s (Ab_t . A_s + 1)
//   O = XQ + LN(Zb2)
//   W1 -= (eta XK)^T G1, b1 -= eta^T G1, W2 -= (eta A)^T G2, b2 -= eta^T G2
// Modular-TTT options (template): LOSS = 1 takes G2 from the inner-product
// loss -< XK + LN(Z2), XV > (target XV, no subtraction); DECAY adds
// lambda/2 (||W1||^2 + ||W2||^2) at the chunk-start state, so after token t
// the weights are d_t W + (loss updates), d_t = 1 - lambda sum_{s<=t} eta_s:
// the XQ W1 and Ab W2 products take a row factor d_t and the chunk ends with
// W scaled by d_last (the biases are not decayed). GATED forms each token's
// rate from its staged key, eta_t = eta_base * logistic(theta_lr[h] . XK_t)
// (the learning-rate gate of the lryc.cn article §2.2), instead of reading eta.
#include "common.hpp"
#include "launch.hpp"

namespace ttt {

template <typename TIO, int LOSS, bool DECAY, bool GATED>
__global__ __launch_bounds__(256) void mlp_prefill_valu(
    int H, int L, int mb, float eps, const TIO *__restrict__ XQ, const TIO *__restrict__ XK,
    const TIO *__restrict__ XV, const float *__restrict__ eta, const float *W1_0,
    const float *b1_0, const float *W2_0,
    const float *b2_0, int w0_batched, const float *__restrict__ gamma,
    const float *__restrict__ beta, TIO *__restrict__ O, float *W1_out, float *b1_out,
    float *W2_out, float *b2_out, float wd, const float *__restrict__ theta, float eta_base) {
    constexpr int D = 64, M = 256, MB = 16, NT = 256, DP = D + 1, MP = M + 1, E = D / 16;
    using io = io_traits<TIO>;

    __shared__ float sW2[M * DP];
    __shared__ float sb2[D];
    __shared__ float sA[MB * MP], sAb[MB * MP];
    __shared__ float sDA[MB * MP], sG1[MB * MP];  // gelu'(Z1), G1
    __shared__ float sQ[MB * DP], sK[MB * DP];
    __shared__ float sT[MB * D], sG2[MB * D], sZ2[MB * D];
    __shared__ float sEta[MB], sM[MB * MB], sDec[MB], sTh[D];
    __shared__ float sW2bar[M], sB2bar[1];  // row means of W2_0, mean of b2_0

    const int tid = threadIdx.x;
    const long seq = blockIdx.x;
    const int h = static_cast<int>(seq % H);
    const long n = seq / H;
    const size_t sb_ = w0_batched ? static_cast<size_t>(n) * H + h : static_cast<size_t>(h);
    const size_t xbase = static_cast<size_t>(seq) * L * D;
    const size_t ebase = static_cast<size_t>(seq) * L;

    // state
    const int k = tid;  // hidden unit owned by this thread
    float w1[D];
#pragma unroll
    for (int i = 0; i < D; ++i) w1[i] = W1_0[sb_ * D * M + static_cast<size_t>(i) * M + k];
    float b1 = b1_0[sb_ * M + k];
    for (int e = tid; e < M * D; e += NT) sW2[(e / D) * DP + (e % D)] = W2_0[sb_ * M * D + e];
    if (tid < D) sb2[tid] = b2_0[sb_ * D + tid];
    if (GATED && tid < D) sTh[tid] = theta[static_cast<size_t>(h) * D + tid];

    const int rrow = tid / 16, rl = tid % 16;
    float gam[E], bet[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        gam[e] = gamma[static_cast<size_t>(h) * D + rl + 16 * e];
        bet[e] = beta[static_cast<size_t>(h) * D + rl + 16 * e];
    }
    const int cj = tid % D, cs0 = tid / D;  // 4 outputs per thread: rows cs0 + 4r
    __syncthreads();

    // Centred output layer: W2 - w2bar 1^T and b2 - b2bar (row means of W2_0,
    // mean of b2_0) shift every row of Z2 and Zb2 by a per-token constant
    // that the layer norm and its backward do not see, and keep them small
    // when the caller's state carries a large offset (Z2 is formed in fp32).
    // G2 rows sum to zero, so G2 W2^T and the updates are unchanged and keep
    // the centring; weight decay scales w2bar with W2 (rho). The state is
    // restored on the way out.
    float rho = 1.f;
    if (L > 0) {
        {
            float a = 0.f;
            for (int j = 0; j < D; ++j) a += sW2[k * DP + j];
            sW2bar[k] = a * (1.0f / D);
        }
        if (tid == 0) {
            float a = 0.f;
            for (int j = 0; j < D; ++j) a += sb2[j];
            sB2bar[0] = a * (1.0f / D);
        }
        __syncthreads();
        for (int j = 0; j < D; ++j) sW2[k * DP + j] -= sW2bar[k];
        if (tid < D) sb2[tid] -= sB2bar[0];
        __syncthreads();
    }

    for (int t0 = 0; t0 < L; t0 += mb) {
        const int len = min(mb, L - t0);
        for (int e = tid; e < MB * D; e += NT) {
            const int s = e / D, j = e % D;
            float q = 0.f, kk = 0.f, v = 0.f;
            if (s < len) {
                const size_t g = xbase + static_cast<size_t>(t0 + s) * D + j;
                q = io::load(XQ, g);
                kk = io::load(XK, g);
                v = io::load(XV, g);
            }
            sQ[s * DP + j] = q;
            sK[s * DP + j] = kk;
            sT[s * D + j] = LOSS == 1 ? v : v - kk;
        }
        if (!GATED && tid < MB) sEta[tid] = tid < len ? eta[ebase + t0 + tid] : 0.f;
        __syncthreads();

        if (GATED && tid < MB) {  // the gate from the staged key
            float a = 0.f;
            for (int i = 0; i < D; ++i) a += sTh[i] * sK[tid * DP + i];
            sEta[tid] = tid < len ? eta_base / (1.f + expf(-a)) : 0.f;
        }
        // Z1 column k, A = gelu(Z1), gelu'(Z1)
#pragma unroll 1
        for (int s = 0; s < MB; ++s) {
            float acc = b1;
#pragma unroll
            for (int i = 0; i < D; ++i) acc += sK[s * DP + i] * w1[i];
            sA[s * MP + k] = gelu_f(acc);
            sDA[s * MP + k] = gelu_prime_f(acc);
        }
        __syncthreads();

        // decay factors d_t (eta is 0 past the end of the sequence)
        if (DECAY && tid < MB) {
            float a = 0.f;
            for (int s = 0; s <= tid; ++s) a += sEta[s];
            sDec[tid] = 1.f - wd * a;
        }
        // Z2 = A W2 + b2
        {
            float acc[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = sb2[cj];
            for (int q = 0; q < M; ++q) {
                const float w = sW2[q * DP + cj];
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] += sA[(cs0 + 4 * r) * MP + q] * w;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) sZ2[(cs0 + 4 * r) * D + cj] = acc[r];
        }
        __syncthreads();

        // G2 = lnbwd(Z2, XV - XK); M1 = causal (XQ XK^T + 1) * eta
        {
            float z[E], tau[E], g[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                z[e] = sZ2[rrow * D + rl + 16 * e];
                tau[e] = sT[rrow * D + rl + 16 * e];
            }
            if constexpr (LOSS == 1)
                ln_ip_grad<16, E>(z, tau, gam, 1.0f / D, eps, g);
            else
                ln_l2_grad<16, E>(z, tau, gam, bet, 1.0f / D, eps, g);
#pragma unroll
            for (int e = 0; e < E; ++e) sG2[rrow * D + rl + 16 * e] = rrow < len ? g[e] : 0.f;
            const int t = tid / MB, s = tid % MB;
            float a = 0.f;
            for (int i = 0; i < D; ++i) a += sQ[t * DP + i] * sK[s * DP + i];
            sM[t * MB + s] = (s <= t) ? sEta[s] * (a + 1.f) : 0.f;
        }
        __syncthreads();

        // G1 column k; Zb1 column k; Ab = gelu(Zb1)
#pragma unroll 1
        for (int s = 0; s < MB; ++s) {
            float acc = 0.f;
#pragma unroll 8
            for (int j = 0; j < D; ++j) acc += sG2[s * D + j] * sW2[k * DP + j];
            sG1[s * MP + k] = acc * sDA[s * MP + k];
        }
#pragma unroll 1
        for (int t = 0; t < MB; ++t) {
            float acc = DECAY ? 0.f : b1;
#pragma unroll
            for (int i = 0; i < D; ++i) acc += sQ[t * DP + i] * w1[i];
            if constexpr (DECAY) acc = fmaf(sDec[t], acc, b1);
#pragma unroll 4
            for (int s = 0; s < MB; ++s) acc -= sM[t * MB + s] * sG1[s * MP + k];
            sAb[t * MP + k] = gelu_f(acc);
        }
        __syncthreads();

        // M2 = causal (Ab A^T + 1) * eta
        {
            const int t = tid / MB, s = tid % MB;
            float a = 0.f;
            for (int q = 0; q < M; ++q) a += sAb[t * MP + q] * sA[s * MP + q];
            sM[t * MB + s] = (s <= t) ? sEta[s] * (a + 1.f) : 0.f;
        }
        __syncthreads();

        // Zb2 = Ab W2 + b2 - M2 G2
        {
            float acc[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = DECAY ? 0.f : sb2[cj];
            for (int q = 0; q < M; ++q) {
                const float w = sW2[q * DP + cj];
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] += sAb[(cs0 + 4 * r) * MP + q] * w;
            }
            if constexpr (DECAY) {
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = fmaf(sDec[cs0 + 4 * r], acc[r], sb2[cj]);
            }
            for (int s = 0; s < MB; ++s) {
                const float gs = sG2[s * D + cj];
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] -= sM[(cs0 + 4 * r) * MB + s] * gs;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) sZ2[(cs0 + 4 * r) * D + cj] = acc[r];
        }
        __syncthreads();

        // O = XQ + LN(Zb2); state updates
        {
            float z[E], y[E];
#pragma unroll
            for (int e = 0; e < E; ++e) z[e] = sZ2[rrow * D + rl + 16 * e];
            ln_fwd<16, E>(z, gam, bet, 1.0f / D, eps, y);
            if (rrow < len) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int j = rl + 16 * e;
                    io::store(O, xbase + static_cast<size_t>(t0 + rrow) * D + j, sQ[rrow * DP + j] + y[e]);
                }
            }
            const float alpha = DECAY ? sDec[MB - 1] : 1.f;
            rho *= alpha;
            if constexpr (DECAY) {
#pragma unroll
                for (int i = 0; i < D; ++i) w1[i] *= alpha;
            }
            float db1 = 0.f;
#pragma unroll 1
            for (int s = 0; s < MB; ++s) {
                const float eg = sEta[s] * sG1[s * MP + k];
                db1 += eg;
#pragma unroll
                for (int i = 0; i < D; ++i) w1[i] -= sK[s * DP + i] * eg;
            }
            b1 -= db1;
            for (int e = tid; e < M * D; e += NT) {
                const int q = e / D, j = e % D;
                float acc = 0.f;
#pragma unroll
                for (int s = 0; s < MB; ++s) acc += sEta[s] * sA[s * MP + q] * sG2[s * D + j];
                if constexpr (DECAY)
                    sW2[q * DP + j] = fmaf(alpha, sW2[q * DP + j], -acc);
                else
                    sW2[q * DP + j] -= acc;
            }
            if (tid < D) {
                float acc = 0.f;
#pragma unroll
                for (int s = 0; s < MB; ++s) acc += sEta[s] * sG2[s * D + tid];
                sb2[tid] -= acc;
            }
        }
        __syncthreads();
    }

    if (L > 0) {  // back to the caller's representation
        for (int j = 0; j < D; ++j) sW2[k * DP + j] = fmaf(rho, sW2bar[k], sW2[k * DP + j]);
        if (tid < D) sb2[tid] += sB2bar[0];
        __syncthreads();
    }
    if (W1_out) {
#pragma unroll
        for (int i = 0; i < D; ++i) W1_out[static_cast<size_t>(seq) * D * M + static_cast<size_t>(i) * M + k] = w1[i];
        b1_out[static_cast<size_t>(seq) * M + k] = b1;
        for (int e = tid; e < M * D; e += NT) W2_out[static_cast<size_t>(seq) * M * D + e] = sW2[(e / D) * DP + (e % D)];
        if (tid < D) b2_out[static_cast<size_t>(seq) * D + tid] = sb2[tid];
    }
}

template <typename TIO, int LOSS, bool DECAY, bool GATED = false>
static hipError_t launch_mlp_t(const MLPArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL((mlp_prefill_valu<TIO, LOSS, DECAY, GATED>), dim3(a.B * a.H), dim3(256), 0, stream, a.H, a.L,
                       a.mb, a.eps, static_cast<const TIO *>(a.XQ),
                       static_cast<const TIO *>(a.XK), static_cast<const TIO *>(a.XV), a.eta,
                       a.W1, a.b1, a.W2, a.b2, a.w0_batched, a.gamma, a.beta,
                       static_cast<TIO *>(a.O), a.W1_out, a.b1_out, a.W2_out, a.b2_out, a.wd,
                       a.theta, a.eta_base);
    return hipGetLastError();
}

template <typename TIO>
static hipError_t launch_mlp_io(const MLPArgs &a, hipStream_t stream) {
    if (a.theta) return launch_mlp_t<TIO, 0, false, true>(a, stream);  // the gate, default options
    const bool decay = a.wd != 0.f;
    if (a.loss == 1)
        return decay ? launch_mlp_t<TIO, 1, true>(a, stream) : launch_mlp_t<TIO, 1, false>(a, stream);
    return decay ? launch_mlp_t<TIO, 0, true>(a, stream) : launch_mlp_t<TIO, 0, false>(a, stream);
}

hipError_t launch_mlp(const MLPArgs &a, hipStream_t stream) {
    if (a.B * a.H == 0) return hipSuccess;
    if (a.d != 64 || (a.loss != 0 && a.loss != 1)) return hipErrorInvalidValue;
    return a.io ? launch_mlp_io<bf16_t>(a, stream) : launch_mlp_io<float>(a, stream);
}

}  // namespace ttt
