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
// adjoint dW, db in LDS. Row work (layer norms, their reverses) runs 16
// threads per token row, one DPP row (thread (r, q) holds features q + 16u;
// row sums are four v_add_f32_dpp steps). Every product
// runs on fp32 matrix cores (16x16x4 f32 MFMA: full fp32 products, fp32
// accumulation): wave u computes the 16-column tile u of each [16 x d]
// result, and tiles (rb, u) of each [d x d] state update, reading its
// operands from LDS tiles whose rows are padded to d + 1 floats.
#include "common.hpp"
#include <mutex>

#include "launch.hpp"
#include "ttt.h"
#include "tile.hpp"

namespace ttt {
namespace {

constexpr int NT = 256, RW = 16;  // threads; lanes per token row

using tile::f32x4;

template <int D>
struct BwdSmem {
    static constexpr int DP = D + 1, TP = RW + 1;
    float W[D * DP], dW[D * DP];
    float b[D], db[D];
    // [16 x d] row tiles (token rows, feature columns)
    float XQ[RW * DP], XK[RW * DP], Z[RW * DP], Zb[RW * DP], E[RW * DP], dZb[RW * DP];
    float dE[RW * DP], dZ[RW * DP], dT[RW * DP], dO[RW * DP];
    float T[RW * TP], dA[RW * TP];        // [t][s]
    float Tp[D / 16][RW * TP], Ap[D / 16][RW * TP];  // per-wave partials of T and dA over
                                                     // 16-feature slices (summed by the reader)
    float red[RW * D];              // final dgamma / dbeta reduction over rows
};

// One 16x16 output tile of C + A B over K (a multiple of 4) on fp32 MFMAs.
// Lane (g, c) supplies A[c][k] and B[k][c] for k = 4 kb + g and receives
// rows 4g .. 4g+3 of column c. A(m, k) and B(k, n) are accessors into LDS.
template <int K, typename FA, typename FB>
__device__ __forceinline__ f32x4 mma(FA A, FB B, int g, int c, f32x4 acc) {
#pragma unroll
    for (int kb = 0; kb < K / 4; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A(c, 4 * kb + g), B(4 * kb + g, c), acc, 0, 0, 0);
    return acc;
}

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
    constexpr int NF = D / RW, DP = D + 1, TP = RW + 1, NTL = D / 16;
    constexpr float inv_d = 1.0f / D;
    using io = io_traits<TIO>;
    __shared__ BwdSmem<D> sm;

    const int tid = threadIdx.x, r = tid / RW, q = tid % RW;
    const int w = tid / 64, lane = tid % 64, g = lane / 16, c = lane % 16;  // MFMA coordinates
    const bool mw = w < NTL;  // this wave owns column tile w
    const long seq = blockIdx.x;
    const int h = static_cast<int>(seq % H);
    const long n = seq / H;
    const int nch = (L + mb - 1) / mb;
    const size_t xbase = static_cast<size_t>(seq) * L * D;
    const size_t st = (w0_batched ? static_cast<size_t>(n) * H : 0) + static_cast<size_t>(h);
    float *wsq = ws + static_cast<size_t>(seq) * nch * (D * D + D);
    const f32x4 fz = {0.f, 0.f, 0.f, 0.f};

    // LDS accessors: row-major tiles and their transposes
    auto rowm = [](const float *M, int ld) { return [M, ld](int i, int j) { return M[i * ld + j]; }; };
    auto colm = [](const float *M, int ld) { return [M, ld](int i, int j) { return M[j * ld + i]; }; };
    // store a [16 x d] tile result (rows 4g+i, column 16 w + c)
    auto put = [&](float *M, f32x4 v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) M[(4 * g + i) * DP + 16 * w + c] = v[i];
    };
    auto get = [&](const float *M) {
        f32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = M[(4 * g + i) * DP + 16 * w + c];
        return v;
    };
    auto brow = [&](const float *bb) {  // b broadcast over the tile's rows
        const float x = bb[16 * w + c];
        return f32x4{x, x, x, x};
    };
    // M[d x d] += P^T Q over the m token rows, on tiles (rb, w); P, Q [16 x d]
    // (ck: also store the result to a checkpoint, row-major [d x d])
    auto state_update = [&](float *M, const float *P, const float *Q, const float *P2, const float *Q2,
                            float *ck) {
        if (!mw) return;
#pragma unroll
        for (int rb = 0; rb < NTL; ++rb) {
            f32x4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = M[(16 * rb + 4 * g + i) * DP + 16 * w + c];
            acc = mma<RW>(colm(P + 16 * rb, DP), rowm(Q + 16 * w, DP), g, c, acc);
            if (P2) acc = mma<RW>(colm(P2 + 16 * rb, DP), rowm(Q2 + 16 * w, DP), g, c, acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                M[(16 * rb + 4 * g + i) * DP + 16 * w + c] = acc[i];
                if (ck) ck[(16 * rb + 4 * g + i) * D + 16 * w + c] = acc[i];
            }
        }
    };
    // column sums of [16 x d] row tiles (padding rows are zero): all loads first
    auto colsum = [&](const float *P, const float *Q) {
        float v[RW];
#pragma unroll
        for (int s2 = 0; s2 < RW; ++s2) v[s2] = P[s2 * DP + tid] + (Q ? Q[s2 * DP + tid] : 0.f);
#pragma unroll
        for (int k = RW / 2; k >= 1; k >>= 1)
#pragma unroll
            for (int s2 = 0; s2 < k; ++s2) v[s2] += v[s2 + k];
        return v[0];
    };

    float gm[NF], bt[NF];
#pragma unroll
    for (int u = 0; u < NF; ++u) {
        gm[u] = gamma[h * D + q + RW * u];
        bt[u] = beta[h * D + q + RW * u];
    }
    for (int i = tid; i < D * D; i += NT) sm.W[(i / D) * DP + i % D] = W0[st * D * D + i];
    if (tid < D) sm.b[tid] = b0[st * D + tid];
    for (int i = tid; i < RW * DP; i += NT) sm.E[i] = 0.f;
    __syncthreads();

    // layer-norm L2 gradient of one row (16 lanes) and what its reverse needs
    struct Lnl2 {
        float xh[NF], gh[NF], G[NF];
        float sigma, c;
    };
    auto lnl2 = [&](const float (&z)[NF], const float (&tau)[NF], Lnl2 &s) {
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int u = 0; u < NF; ++u) s1 += z[u];
        const float mu = tile::row16_sum(s1) * inv_d;
#pragma unroll
        for (int u = 0; u < NF; ++u) s2 += (z[u] - mu) * (z[u] - mu);
        s.sigma = sqrtf(tile::row16_sum(s2) * inv_d + eps);
        const float rs = 1.0f / s.sigma;
        float sa = 0.f, sc = 0.f;
#pragma unroll
        for (int u = 0; u < NF; ++u) {
            s.xh[u] = (z[u] - mu) * rs;
            s.gh[u] = gm[u] * fmaf(gm[u], s.xh[u], bt[u] - tau[u]);
            sa += s.gh[u];
            sc += s.gh[u] * s.xh[u];
        }
        const float a = tile::row16_sum(sa) * inv_d;
        s.c = tile::row16_sum(sc) * inv_d;
#pragma unroll
        for (int u = 0; u < NF; ++u) s.G[u] = (s.gh[u] - a - s.xh[u] * s.c) * rs;
    };
    // Inputs of one chunk for this thread's row (zero past the end of the
    // sequence), and one chunk-start state: fetched into registers a chunk
    // ahead of their use so that the global-memory latency hides behind the
    // current chunk.
    constexpr int NWP = D * D / NT;
    // raw storage values (converted when staged), so that the loads stay in
    // flight until the next chunk instead of being waited on where they issue
    struct Rows {
        TIO xq[NF], xk[NF], xv[NF];
        float go[NF], et;
        bool ok;
    };
    struct State {
        float w[NWP], b;
    };
    // unconditional loads from a row clamped into the sequence; rows past its
    // end are zeroed when staged
    auto fetch_rows = [&](int ch, bool rev, Rows &R) {
        R.ok = r < min(mb, L - ch * mb);
        const int rr = R.ok ? r : 0;
        const size_t row = xbase + static_cast<size_t>(ch * mb + rr) * D;
#pragma unroll
        for (int u = 0; u < NF; ++u) {
            const int f = q + RW * u;
            R.xk[u] = XK[row + f];
            R.xv[u] = XV[row + f];
            if (rev) {
                R.xq[u] = XQ[row + f];
                R.go[u] = dO[row + f];
            }
        }
        R.et = eta[static_cast<size_t>(seq) * L + ch * mb + rr];
    };
    auto fetch_state = [&](int ch, State &S) {
        const float *wc = wsq + static_cast<size_t>(ch) * (D * D + D);
#pragma unroll
        for (int k = 0; k < NWP; ++k) S.w[k] = wc[tid + NT * k];
        S.b = tid < D ? wc[D * D + tid] : 0.f;
    };
    // stage a chunk's rows: XK (and XQ, dO) into LDS; tau and eta into registers
    auto stage_rows = [&](const Rows &R, bool rev, float (&tau)[NF], float &et, float (&go)[NF]) {
#pragma unroll
        for (int u = 0; u < NF; ++u) {
            const int f = q + RW * u;
            const float xk = R.ok ? io::load(R.xk, u) : 0.f;
            sm.XK[r * DP + f] = xk;
            tau[u] = R.ok ? io::load(R.xv, u) - xk : 0.f;
            if (rev) {
                sm.XQ[r * DP + f] = R.ok ? io::load(R.xq, u) : 0.f;
                go[u] = R.ok ? R.go[u] : 0.f;
                sm.dO[r * DP + f] = go[u];
            }
        }
        et = R.ok ? R.et : 0.f;
    };
    auto rowz = [&](const float *M, float (&z)[NF]) {
#pragma unroll
        for (int u = 0; u < NF; ++u) z[u] = M[r * DP + q + RW * u];
    };

    // ===== forward: chunk-start states to the workspace ========================
    Rows R;
    if (nch > 0) fetch_rows(0, false, R);
    if (nch > 0) {  // chunk 0's start state; the others are written by the updates
        for (int i = tid; i < D * D; i += NT) wsq[i] = W0[st * D * D + i];
        if (tid < D) wsq[D * D + tid] = b0[st * D + tid];
    }
    for (int ch = 0; ch < nch; ++ch) {
        float *wn = ch + 1 < nch ? wsq + static_cast<size_t>(ch + 1) * (D * D + D) : nullptr;
        float tau[NF], et, go_unused[NF];
        stage_rows(R, false, tau, et, go_unused);
        if (ch + 1 < nch) fetch_rows(ch + 1, false, R);
        __syncthreads();
        if (mw) put(sm.Z, mma<D>(rowm(sm.XK, DP), rowm(sm.W + 16 * w, DP), g, c, brow(sm.b)));
        __syncthreads();
        float z[NF];
        rowz(sm.Z, z);
        Lnl2 s;
        lnl2(z, tau, s);
#pragma unroll
        for (int u = 0; u < NF; ++u) sm.E[r * DP + q + RW * u] = -et * s.G[u];
        __syncthreads();
        state_update(sm.W, sm.XK, sm.E, nullptr, nullptr, wn);  // W += XK^T E
        if (tid < D) {
            const float bn = sm.b[tid] + colsum(sm.E, nullptr);
            sm.b[tid] = bn;
            if (wn) wn[D * D + tid] = bn;
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

    State S;
    if (nch > 0) {
        fetch_rows(nch - 1, true, R);
        fetch_state(nch - 1, S);
    }
    for (int ch = nch - 1; ch >= 0; --ch) {
        const int m = min(mb, L - ch * mb);
        const bool ok = r < m;
        __syncthreads();  // the previous chunk is done with every tile
#pragma unroll
        for (int k = 0; k < NWP; ++k) {
            const int i = tid + NT * k;
            sm.W[(i / D) * DP + i % D] = S.w[k];
        }
        if (tid < D) sm.b[tid] = S.b;
        float tau[NF], et, go[NF];
        stage_rows(R, true, tau, et, go);
        if (ch > 0) {
            fetch_rows(ch - 1, true, R);
            fetch_state(ch - 1, S);
        }
        __syncthreads();

        // Z = XK W + b, Zq = XQ W + b (tile w); T = XQ XK^T + 1 on the causal triangle
        if (mw) {
            put(sm.Z, mma<D>(rowm(sm.XK, DP), rowm(sm.W + 16 * w, DP), g, c, brow(sm.b)));
            put(sm.Zb, mma<D>(rowm(sm.XQ, DP), rowm(sm.W + 16 * w, DP), g, c, brow(sm.b)));
        }
        if (mw) {  // this wave's 16-feature slice of XQ XK^T
            const f32x4 t4 = mma<RW>(rowm(sm.XQ + 16 * w, DP), colm(sm.XK + 16 * w, DP), g, c, fz);
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.Tp[w][(4 * g + i) * TP + c] = t4[i];
        }
        __syncthreads();
        {  // T = tril(sum of the slices + 1) on the chunk's rows; one entry per thread
            const int t = tid / RW, s2 = tid % RW;
            float v = 0.f;
#pragma unroll
            for (int k = 0; k < NTL; ++k) v += sm.Tp[k][t * TP + s2];
            sm.T[t * TP + s2] = (s2 <= t && t < m) ? v + 1.f : 0.f;
        }
        float z[NF];
        rowz(sm.Z, z);
        Lnl2 s;
        lnl2(z, tau, s);
#pragma unroll
        for (int u = 0; u < NF; ++u) sm.E[r * DP + q + RW * u] = -et * s.G[u];
        __syncthreads();

        // Zb = XQ W + b + T E
        if (mw) put(sm.Zb, mma<RW>(rowm(sm.T, TP), rowm(sm.E + 16 * w, DP), g, c, get(sm.Zb)));
        __syncthreads();

        // the reverse of O = XQ + LN(Zb)
        {
            float zb[NF];
            rowz(sm.Zb, zb);
            float s1 = 0.f, s2 = 0.f;
#pragma unroll
            for (int u = 0; u < NF; ++u) s1 += zb[u];
            const float mu = tile::row16_sum(s1) * inv_d;
#pragma unroll
            for (int u = 0; u < NF; ++u) s2 += (zb[u] - mu) * (zb[u] - mu);
            const float rs = 1.0f / sqrtf(tile::row16_sum(s2) * inv_d + eps);
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
            m1 = tile::row16_sum(m1) * inv_d;
            m2 = tile::row16_sum(m2) * inv_d;
#pragma unroll
            for (int u = 0; u < NF; ++u) sm.dZb[r * DP + q + RW * u] = (dx[u] - m1 - xb[u] * m2) * rs;
        }
        __syncthreads();

        // dE = T^T dZb + XK dW' + db';  dXQ tile = dZb W^T;  dXK tile = E dW'^T;
        // dA = (dZb E^T) on the causal triangle  (dW', db' not yet updated)
        f32x4 gq = fz, gk = fz;
        if (mw) {
            f32x4 de = mma<D>(rowm(sm.XK, DP), rowm(sm.dW + 16 * w, DP), g, c, brow(sm.db));
            de = mma<RW>(colm(sm.T, TP), rowm(sm.dZb + 16 * w, DP), g, c, de);
            put(sm.dE, de);
            gq = mma<D>(rowm(sm.dZb, DP), colm(sm.W + 16 * w * DP, DP), g, c, fz);
            gk = mma<D>(rowm(sm.E, DP), colm(sm.dW + 16 * w * DP, DP), g, c, fz);
        }
        if (mw) {  // this wave's 16-feature slice of dZb E^T
            const f32x4 a4 = mma<RW>(rowm(sm.dZb + 16 * w, DP), colm(sm.E + 16 * w, DP), g, c, fz);
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.Ap[w][(4 * g + i) * TP + c] = a4[i];
        }
        __syncthreads();

        {  // dA = the slices summed on the causal triangle of the chunk's rows
            const int t = tid / RW, s2 = tid % RW;
            float v = 0.f;
#pragma unroll
            for (int k = 0; k < NTL; ++k) v += sm.Ap[k][t * TP + s2];
            sm.dA[t * TP + s2] = (s2 <= t && t < m) ? v : 0.f;
        }
        // row work: deta = -G . dE, dG = -eta dE, then the reverse of lnl2
        float de[NF];
        rowz(sm.dE, de);
        float pe = 0.f;
#pragma unroll
        for (int u = 0; u < NF; ++u) pe = fmaf(s.G[u], de[u], pe);
        const float d_eta = -tile::row16_sum(pe);
        float dG[NF], mdg = 0.f, mdgx = 0.f, sgG = 0.f;
#pragma unroll
        for (int u = 0; u < NF; ++u) {
            dG[u] = -et * de[u];
            mdg += dG[u];
            mdgx += dG[u] * s.xh[u];
            sgG += dG[u] * s.G[u];
        }
        mdg = tile::row16_sum(mdg) * inv_d;
        mdgx = tile::row16_sum(mdgx) * inv_d;
        const float rs = 1.0f / s.sigma;
        const float dsig = -tile::row16_sum(sgG) * rs;
        float dxh[NF], mdx = 0.f, mdxx = 0.f;
#pragma unroll
        for (int u = 0; u < NF; ++u) {
            const float dgh = (dG[u] - mdg - s.xh[u] * mdgx) * rs;
            dxh[u] = gm[u] * gm[u] * dgh - (s.c * dG[u] + s.gh[u] * mdgx) * rs;
            const float dtau = -gm[u] * dgh;
            sm.dT[r * DP + q + RW * u] = ok ? dtau : 0.f;
            dg_acc[u] = fmaf(dgh, fmaf(2.f * gm[u], s.xh[u], bt[u] - tau[u]), dg_acc[u]);
            db_acc[u] = fmaf(gm[u], dgh, db_acc[u]);
            mdx += dxh[u];
            mdxx += dxh[u] * s.xh[u];
        }
        mdx = tile::row16_sum(mdx) * inv_d;
        mdxx = tile::row16_sum(mdxx) * inv_d;
#pragma unroll
        for (int u = 0; u < NF; ++u) {
            const float dz = fmaf(dsig * inv_d, s.xh[u], (dxh[u] - mdx - s.xh[u] * mdxx) * rs);
            sm.dZ[r * DP + q + RW * u] = ok ? dz : 0.f;
        }
        if (ok) {
            if (q == 0) deta[static_cast<size_t>(seq) * L + ch * mb + r] = d_eta;
        }
        __syncthreads();

        // dXQ tile += dA XK + dO;  dXK tile += dA^T XQ + dZ W^T - dtau;  write the tiles
        if (mw) {
            gq = mma<RW>(rowm(sm.dA, TP), rowm(sm.XK + 16 * w, DP), g, c, gq);
            gk = mma<RW>(colm(sm.dA, TP), rowm(sm.XQ + 16 * w, DP), g, c, gk);
            gk = mma<D>(rowm(sm.dZ, DP), colm(sm.W + 16 * w * DP, DP), g, c, gk);
            const f32x4 dt4 = get(sm.dT), do4 = get(sm.dO);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 4 * g + i;
                if (t < m) {
                    const size_t at = xbase + static_cast<size_t>(ch * mb + t) * D + 16 * w + c;
                    dXQ[at] = gq[i] + do4[i];
                    dXK[at] = gk[i] - dt4[i];
                    dXV[at] = dt4[i];
                }
            }
        }
        // dW += XQ^T dZb + XK^T dZ;  db += 1^T (dZb + dZ)
        state_update(sm.dW, sm.XQ, sm.dZb, sm.XK, sm.dZ, nullptr);
        if (tid < D) sm.db[tid] += colsum(sm.dZb, sm.dZ);
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

// Fixed scratch of ttt_linear_backward_noalloc: the chunk-start checkpoints
// live here instead of in a caller workspace (64 MiB, held by every GPU the
// library runs on until the process ends). Host code must never pass the
// array's name to a kernel: on the host it is only a stand-in for the symbol;
// linear_backward_scratch below returns the device address.
constexpr size_t kScratchBytes = TTT_BACKWARD_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

size_t linear_backward_scratch_bytes() { return kScratchBytes; }

// Device address of `scratch` on the current device, looked up once per
// device (hipGetSymbolAddress with that device current) and kept.
hipError_t linear_backward_scratch(float **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static float *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = static_cast<float *>(p);
    }
    *ptr = addr[dev];
    return hipSuccess;
}

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
