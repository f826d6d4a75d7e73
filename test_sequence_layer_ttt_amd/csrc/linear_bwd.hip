// Backward of the TTT-Linear inner loop: gradients of
//   loss = <dO, O> + <dW_out, W_L> + <db_out, b_L>
// with respect to XQ, XK, XV, eta, W0, b0, gamma and beta, the gradients a
// training step takes through the inner loop (the damodev.csdn.net TTT
// deep-dive, §6 and §7.1: the outer loop learns through the inner updates).
//
// Per chunk (state W, b at chunk start, m <= mb rows, row-vector convention)
// the forward is the dual form of the deep-dive's §4.2:
//   Z = XK W + b,  G = lnl2(Z, XV - XK),  E = -eta * G (rows),
//   T = tril(XQ XK^T + 1),  Zb = XQ W + b + T E,  O = XQ + LN(Zb),
//   W' = W + XK^T E,  b' = b + 1^T E.
// Its reverse, given dO and the adjoints dW', db' of the next chunk's state:
//   dZb = LN backward of dO;  dXQ = dO + dZb W^T + dA XK;
//   dA = (dZb E^T) masked to the causal triangle;  dXK = dA^T XQ + E dW'^T + ...
//   dE = T^T dZb + XK dW' + 1 db'^T;  deta_s = -G_s . dE_s;  dG = -eta * dE;
//   (dZ, dtau) = reverse of lnl2;  dXV = dtau;  dXK += dZ W^T - dtau;
//   dW = dW' + XQ^T dZb + XK^T dZ;  db = db' + 1^T dZb + 1^T dZ.
// lnl2(z, tau) = d/dz 1/2 ||gamma xhat + beta - tau||^2 with
// xhat = (z - mu) / sigma, sigma = sqrt(var + eps):
//   ghat = gamma (gamma xhat + beta - tau),  a = mean(ghat),  c = mean(ghat xhat),
//   G = (ghat - a - xhat c) / sigma,
// and its reverse for an incoming dG:
//   dghat = (dG - mean(dG) - xhat mean(dG xhat)) / sigma,
//   dxhat = gamma^2 dghat - (c dG + ghat mean(dG xhat)) / sigma,
//   dsigma = -sum(dG G) / sigma,  dtau = -gamma dghat,
//   dgamma += dghat (2 gamma xhat + beta - tau),  dbeta += gamma dghat,
//   dz = (dxhat - mean(dxhat) - xhat mean(dxhat xhat)) / sigma + dsigma xhat / d.
//
// One 256-thread workgroup per (n, h) sequence. A forward pass stores the
// state at every chunk start in the caller's workspace; the reverse pass
// reloads it, recomputes the chunk and applies the rules above, keeping the
// adjoint dW, db in LDS. Row work runs 16 threads per token row (thread
// (r, q) holds features q + 16u); products are fp32 FMAs over LDS tiles
// whose rows are padded to d + 1 floats so that the 16 row groups reading
// the same column hit different banks.
#include "common.hpp"
#include "launch.hpp"

namespace ttt {
namespace {

constexpr int NT = 256, RW = 16;  // threads; lanes per token row

template <int D>
struct BwdSmem {
    static constexpr int DP = D + 1;
    float W[D * DP], dW[D * DP];
    float b[D], db[D];
    float XQ[RW * DP], XK[RW * DP], E[RW * DP], dZb[RW * DP], dZ[RW * DP];
    float T[RW * (RW + 1)], dA[RW * (RW + 1)];
    float red[RW * D];  // final dgamma / dbeta reduction over rows
};

template <int D, typename TIO>
__global__ __launch_bounds__(NT) void linear_backward_kernel(
    int H, int L, int mb, float eps, const TIO *__restrict__ XQ, const TIO *__restrict__ XK,
    const TIO *__restrict__ XV, const float *__restrict__ eta, const float *__restrict__ W0,
    const float *__restrict__ b0, int w0_batched, const float *__restrict__ gamma,
    const float *__restrict__ beta, const float *__restrict__ dO, const float *__restrict__ dW_out,
    const float *__restrict__ db_out, float *__restrict__ dXQ, float *__restrict__ dXK,
    float *__restrict__ dXV, float *__restrict__ deta, float *__restrict__ dW0,
    float *__restrict__ db0, float *__restrict__ dgamma, float *__restrict__ dbeta,
    float *__restrict__ ws) {
    constexpr int NF = D / RW, DP = D + 1, TP = RW + 1;
    constexpr float inv_d = 1.0f / D;
    using io = io_traits<TIO>;
    __shared__ BwdSmem<D> sm;

    const int tid = threadIdx.x, r = tid / RW, q = tid % RW;
    const long seq = blockIdx.x;
    const int h = static_cast<int>(seq % H);
    const long n = seq / H;
    const int nch = (L + mb - 1) / mb;
    const size_t xbase = static_cast<size_t>(seq) * L * D;
    const size_t st = (w0_batched ? static_cast<size_t>(n) * H : 0) + static_cast<size_t>(h);
    float *wsq = ws + static_cast<size_t>(seq) * nch * (D * D + D);

    float gm[NF], bt[NF];
#pragma unroll
    for (int u = 0; u < NF; ++u) {
        gm[u] = gamma[h * D + q + RW * u];
        bt[u] = beta[h * D + q + RW * u];
    }
    for (int i = tid; i < D * D; i += NT) sm.W[(i / D) * DP + i % D] = W0[st * D * D + i];
    if (tid < D) sm.b[tid] = b0[st * D + tid];
    __syncthreads();

    // Z = XK W + b for this thread's row and features (XK row in LDS)
    auto xw = [&](const float *X, float (&out)[NF]) {
#pragma unroll
        for (int u = 0; u < NF; ++u) out[u] = sm.b[q + RW * u];
        for (int k = 0; k < D; ++k) {
            const float x = X[r * DP + k];
#pragma unroll
            for (int u = 0; u < NF; ++u) out[u] = fmaf(x, sm.W[k * DP + q + RW * u], out[u]);
        }
    };
    // layer-norm L2 gradient of one row (16 lanes) and what its reverse needs
    struct Lnl2 {
        float xh[NF], gh[NF], G[NF];
        float sigma, c;
    };
    auto lnl2 = [&](const float (&z)[NF], const float (&tau)[NF], Lnl2 &s) {
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int u = 0; u < NF; ++u) s1 += z[u];
        const float mu = group_sum<RW>(s1) * inv_d;
#pragma unroll
        for (int u = 0; u < NF; ++u) s2 += (z[u] - mu) * (z[u] - mu);
        s.sigma = sqrtf(group_sum<RW>(s2) * inv_d + eps);
        const float rs = 1.0f / s.sigma;
        float sa = 0.f, sc = 0.f;
#pragma unroll
        for (int u = 0; u < NF; ++u) {
            s.xh[u] = (z[u] - mu) * rs;
            s.gh[u] = gm[u] * fmaf(gm[u], s.xh[u], bt[u] - tau[u]);
            sa += s.gh[u];
            sc += s.gh[u] * s.xh[u];
        }
        const float a = group_sum<RW>(sa) * inv_d;
        s.c = group_sum<RW>(sc) * inv_d;
#pragma unroll
        for (int u = 0; u < NF; ++u) s.G[u] = (s.gh[u] - a - s.xh[u] * s.c) * rs;
    };
    auto load_rows = [&](int c, int m, float (&xk)[NF], float (&tau)[NF], float &et) {
        const bool ok = r < m;
        const size_t row = xbase + static_cast<size_t>(c * mb + (ok ? r : 0)) * D;
#pragma unroll
        for (int u = 0; u < NF; ++u) {
            const int f = q + RW * u;
            xk[u] = ok ? io::load(XK, row + f) : 0.f;
            tau[u] = ok ? io::load(XV, row + f) - xk[u] : 0.f;
            sm.XK[r * DP + f] = xk[u];
        }
        et = ok ? eta[static_cast<size_t>(seq) * L + c * mb + r] : 0.f;
    };

    // ===== forward: chunk-start states to the workspace ========================
    for (int c = 0; c < nch; ++c) {
        const int m = min(mb, L - c * mb);
        float *wc = wsq + static_cast<size_t>(c) * (D * D + D);
        for (int i = tid; i < D * D; i += NT) wc[i] = sm.W[(i / D) * DP + i % D];
        if (tid < D) wc[D * D + tid] = sm.b[tid];
        float xk[NF], tau[NF], et;
        load_rows(c, m, xk, tau, et);
        __syncthreads();
        float z[NF];
        xw(sm.XK, z);
        Lnl2 s;
        lnl2(z, tau, s);
#pragma unroll
        for (int u = 0; u < NF; ++u) sm.E[r * DP + q + RW * u] = -et * s.G[u];
        __syncthreads();
        // W += XK^T E, b += 1^T E
        for (int i = tid; i < D * D; i += NT) {
            const int a = i / D, bcol = i % D;
            float acc = sm.W[a * DP + bcol];
            for (int s2 = 0; s2 < m; ++s2) acc = fmaf(sm.XK[s2 * DP + a], sm.E[s2 * DP + bcol], acc);
            sm.W[a * DP + bcol] = acc;
        }
        if (tid < D) {
            float acc = sm.b[tid];
            for (int s2 = 0; s2 < m; ++s2) acc += sm.E[s2 * DP + tid];
            sm.b[tid] = acc;
        }
        __syncthreads();
    }

    // ===== reverse ================================================================
    const size_t sq = static_cast<size_t>(seq);
    for (int i = tid; i < D * D; i += NT)
        sm.dW[(i / D) * DP + i % D] = dW_out ? dW_out[sq * D * D + i] : 0.f;
    if (tid < D) sm.db[tid] = db_out ? db_out[sq * D + tid] : 0.f;
    float dg_acc[NF], db_acc[NF];
#pragma unroll
    for (int u = 0; u < NF; ++u) dg_acc[u] = db_acc[u] = 0.f;

    for (int c = nch - 1; c >= 0; --c) {
        const int m = min(mb, L - c * mb);
        const bool ok = r < m;
        const float *wc = wsq + static_cast<size_t>(c) * (D * D + D);
        __syncthreads();  // the previous chunk is done with every tile
        for (int i = tid; i < D * D; i += NT) sm.W[(i / D) * DP + i % D] = wc[i];
        if (tid < D) sm.b[tid] = wc[D * D + tid];
        float xk[NF], tau[NF], et, xq[NF], go[NF];
        load_rows(c, m, xk, tau, et);
        const size_t row = xbase + static_cast<size_t>(c * mb + (ok ? r : 0)) * D;
#pragma unroll
        for (int u = 0; u < NF; ++u) {
            const int f = q + RW * u;
            xq[u] = ok ? io::load(XQ, row + f) : 0.f;
            go[u] = ok ? dO[row + f] : 0.f;
            sm.XQ[r * DP + f] = xq[u];
        }
        __syncthreads();

        // recompute: Z, G, E; XQ W + b
        float z[NF], zq[NF];
        xw(sm.XK, z);
        xw(sm.XQ, zq);
        Lnl2 s;
        lnl2(z, tau, s);
#pragma unroll
        for (int u = 0; u < NF; ++u) sm.E[r * DP + q + RW * u] = -et * s.G[u];
        {  // T[t][s] = XQ_t . XK_s + 1 on the causal triangle of the chunk
            const int t = tid / RW, s2 = tid % RW;
            float acc = 0.f;
            for (int k = 0; k < D; ++k) acc = fmaf(sm.XQ[t * DP + k], sm.XK[s2 * DP + k], acc);
            sm.T[t * TP + s2] = (s2 <= t && t < m) ? acc + 1.f : 0.f;
        }
        __syncthreads();

        // Zb = XQ W + b + T E, its layer norm, and the reverse of O = XQ + LN(Zb)
        float zb[NF];
#pragma unroll
        for (int u = 0; u < NF; ++u) zb[u] = zq[u];
        for (int s2 = 0; s2 < RW; ++s2) {
            const float tv = sm.T[r * TP + s2];
#pragma unroll
            for (int u = 0; u < NF; ++u) zb[u] = fmaf(tv, sm.E[s2 * DP + q + RW * u], zb[u]);
        }
        {
            float s1 = 0.f, s2 = 0.f;
#pragma unroll
            for (int u = 0; u < NF; ++u) s1 += zb[u];
            const float mu = group_sum<RW>(s1) * inv_d;
#pragma unroll
            for (int u = 0; u < NF; ++u) s2 += (zb[u] - mu) * (zb[u] - mu);
            const float rs = 1.0f / sqrtf(group_sum<RW>(s2) * inv_d + eps);
            float xb[NF], dx[NF], m1 = 0.f, m2 = 0.f;
#pragma unroll
            for (int u = 0; u < NF; ++u) {
                xb[u] = (zb[u] - mu) * rs;
                dx[u] = gm[u] * go[u];
                dg_acc[u] = fmaf(go[u], xb[u], dg_acc[u]);
                db_acc[u] += go[u];
                m1 += dx[u];
                m2 += dx[u] * xb[u];
            }
            m1 = group_sum<RW>(m1) * inv_d;
            m2 = group_sum<RW>(m2) * inv_d;
#pragma unroll
            for (int u = 0; u < NF; ++u) sm.dZb[r * DP + q + RW * u] = (dx[u] - m1 - xb[u] * m2) * rs;
        }
        __syncthreads();

        // dXQ = dO + dZb W^T;  dE = T^T dZb + XK dW' + db';  dXK = E dW'^T;
        // dA = (dZb E^T) on the causal triangle (dW', db' not yet updated)
        float gq[NF], gk[NF], de[NF];
#pragma unroll
        for (int u = 0; u < NF; ++u) {
            gq[u] = go[u];
            gk[u] = 0.f;
            de[u] = sm.db[q + RW * u];
        }
        for (int j = 0; j < D; ++j) {
            const float dzb = sm.dZb[r * DP + j], e = sm.E[r * DP + j], x = sm.XK[r * DP + j];
#pragma unroll
            for (int u = 0; u < NF; ++u) {
                const int f = q + RW * u;
                gq[u] = fmaf(dzb, sm.W[f * DP + j], gq[u]);
                gk[u] = fmaf(e, sm.dW[f * DP + j], gk[u]);
                de[u] = fmaf(x, sm.dW[j * DP + f], de[u]);
            }
        }
        for (int t = 0; t < RW; ++t) {
            const float tv = sm.T[t * TP + r];
#pragma unroll
            for (int u = 0; u < NF; ++u) de[u] = fmaf(tv, sm.dZb[t * DP + q + RW * u], de[u]);
        }
        {
            const int t = tid / RW, s2 = tid % RW;
            float acc = 0.f;
            for (int k = 0; k < D; ++k) acc = fmaf(sm.dZb[t * DP + k], sm.E[s2 * DP + k], acc);
            sm.dA[t * TP + s2] = (s2 <= t && t < m) ? acc : 0.f;
        }
        __syncthreads();

        // dXQ += dA XK;  dXK += dA^T XQ
        for (int s2 = 0; s2 < RW; ++s2) {
            const float a1 = sm.dA[r * TP + s2], a2 = sm.dA[s2 * TP + r];
#pragma unroll
            for (int u = 0; u < NF; ++u) {
                gq[u] = fmaf(a1, sm.XK[s2 * DP + q + RW * u], gq[u]);
                gk[u] = fmaf(a2, sm.XQ[s2 * DP + q + RW * u], gk[u]);
            }
        }
        // E = -eta G:  deta = -G . dE,  dG = -eta dE;  then the reverse of lnl2
        float pe = 0.f;
#pragma unroll
        for (int u = 0; u < NF; ++u) pe = fmaf(s.G[u], de[u], pe);
        const float d_eta = -group_sum<RW>(pe);
        float dG[NF], mdg = 0.f, mdgx = 0.f, sgG = 0.f;
#pragma unroll
        for (int u = 0; u < NF; ++u) {
            dG[u] = -et * de[u];
            mdg += dG[u];
            mdgx += dG[u] * s.xh[u];
            sgG += dG[u] * s.G[u];
        }
        mdg = group_sum<RW>(mdg) * inv_d;
        mdgx = group_sum<RW>(mdgx) * inv_d;
        const float rs = 1.0f / s.sigma;
        const float dsig = -group_sum<RW>(sgG) * rs;
        float dxh[NF], mdx = 0.f, mdxx = 0.f, dtau[NF];
#pragma unroll
        for (int u = 0; u < NF; ++u) {
            const float dgh = (dG[u] - mdg - s.xh[u] * mdgx) * rs;
            dxh[u] = gm[u] * gm[u] * dgh - (s.c * dG[u] + s.gh[u] * mdgx) * rs;
            dtau[u] = -gm[u] * dgh;
            dg_acc[u] = fmaf(dgh, fmaf(2.f * gm[u], s.xh[u], bt[u] - tau[u]), dg_acc[u]);
            db_acc[u] = fmaf(gm[u], dgh, db_acc[u]);
            mdx += dxh[u];
            mdxx += dxh[u] * s.xh[u];
        }
        mdx = group_sum<RW>(mdx) * inv_d;
        mdxx = group_sum<RW>(mdxx) * inv_d;
#pragma unroll
        for (int u = 0; u < NF; ++u) {
            const float dz = fmaf(dsig * inv_d, s.xh[u], (dxh[u] - mdx - s.xh[u] * mdxx) * rs);
            sm.dZ[r * DP + q + RW * u] = ok ? dz : 0.f;
            gk[u] -= dtau[u];
        }
        __syncthreads();

        // dXK += dZ W^T; write the chunk's input gradients
        for (int j = 0; j < D; ++j) {
            const float dz = sm.dZ[r * DP + j];
#pragma unroll
            for (int u = 0; u < NF; ++u) gk[u] = fmaf(dz, sm.W[(q + RW * u) * DP + j], gk[u]);
        }
        if (ok) {
#pragma unroll
            for (int u = 0; u < NF; ++u) {
                const int f = q + RW * u;
                dXQ[row + f] = gq[u];
                dXK[row + f] = gk[u];
                dXV[row + f] = dtau[u];
            }
            if (q == 0) deta[static_cast<size_t>(seq) * L + c * mb + r] = d_eta;
        }
        // dW += XQ^T dZb + XK^T dZ;  db += 1^T (dZb + dZ)
        for (int i = tid; i < D * D; i += NT) {
            const int a = i / D, bcol = i % D;
            float acc = sm.dW[a * DP + bcol];
            for (int s2 = 0; s2 < m; ++s2)
                acc = fmaf(sm.XQ[s2 * DP + a], sm.dZb[s2 * DP + bcol],
                           fmaf(sm.XK[s2 * DP + a], sm.dZ[s2 * DP + bcol], acc));
            sm.dW[a * DP + bcol] = acc;
        }
        if (tid < D) {
            float acc = sm.db[tid];
            for (int s2 = 0; s2 < m; ++s2) acc += sm.dZb[s2 * DP + tid] + sm.dZ[s2 * DP + tid];
            sm.db[tid] = acc;
        }
    }
    __syncthreads();

    for (int i = tid; i < D * D; i += NT) dW0[sq * D * D + i] = sm.dW[(i / D) * DP + i % D];
    if (tid < D) db0[sq * D + tid] = sm.db[tid];
    // per-sequence dgamma, dbeta: sum the 16 row groups
#pragma unroll
    for (int u = 0; u < NF; ++u) sm.red[r * D + q + RW * u] = dg_acc[u];
    __syncthreads();
    if (tid < D) {
        float acc = 0.f;
        for (int rr = 0; rr < RW; ++rr) acc += sm.red[rr * D + tid];
        dgamma[sq * D + tid] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NF; ++u) sm.red[r * D + q + RW * u] = db_acc[u];
    __syncthreads();
    if (tid < D) {
        float acc = 0.f;
        for (int rr = 0; rr < RW; ++rr) acc += sm.red[rr * D + tid];
        dbeta[sq * D + tid] = acc;
    }
}

template <int D, typename TIO>
hipError_t launch_bwd_t(const LinearBwdArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL((linear_backward_kernel<D, TIO>), dim3(a.f.B * a.f.H), dim3(NT), 0, stream,
                       a.f.H, a.f.L, a.f.mb, a.f.eps, static_cast<const TIO *>(a.f.XQ),
                       static_cast<const TIO *>(a.f.XK), static_cast<const TIO *>(a.f.XV), a.f.eta,
                       a.f.W0, a.f.b0, a.f.w0_batched, a.f.gamma, a.f.beta, a.dO, a.dW_out, a.db_out,
                       a.dXQ, a.dXK, a.dXV, a.deta, a.dW0, a.db0, a.dgamma, a.dbeta, a.ws);
    return hipGetLastError();
}

}  // namespace

size_t linear_backward_workspace_floats(int B, int H, int L, int d, int mb) {
    const size_t nch = L > 0 ? static_cast<size_t>((L + mb - 1) / mb) : 0;
    return static_cast<size_t>(B) * H * nch * (static_cast<size_t>(d) * d + d);
}

hipError_t launch_linear_backward(const LinearBwdArgs &a, hipStream_t stream) {
    if (a.f.B * a.f.H == 0) return hipSuccess;
    if (a.f.d == 16) return a.f.io ? launch_bwd_t<16, bf16_t>(a, stream) : launch_bwd_t<16, float>(a, stream);
    if (a.f.d == 64) return a.f.io ? launch_bwd_t<64, bf16_t>(a, stream) : launch_bwd_t<64, float>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace ttt
