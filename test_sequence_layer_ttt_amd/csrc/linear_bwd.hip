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
// Three launches of 256-thread workgroups. A forward sweep (one workgroup per
// (n, h) sequence) stores the state at every chunk start in the caller's
// workspace. A pre-pass (persistent workgroups taking the chunks in turn)
// recomputes each chunk from its stored state and applies every rule above
// that does not involve dW', db': Z, G, E, T, Zb, dZb, dA, dXQ in full, the
// dA^T XQ part of dXK and T^T dZb, storing what the rest needs in a per-chunk
// record. The reverse sweep (one workgroup per sequence, chunks from the last)
// applies the rest -- dE, deta, the reverse of lnl2, the E dW'^T and dZ W^T
// parts of dXK, dW and db -- keeping the adjoint dW, db in LDS. Row work (layer norms, their reverses) runs 16
// threads per token row, one DPP row (thread (r, q) holds features q + 16u;
// row sums are four v_add_f32_dpp steps). Every product
// runs on fp32 matrix cores (16x16x4 f32 MFMA: full fp32 products, fp32
// accumulation): wave u computes the 16-column tile u of each [16 x d]
// result, and tiles (rb, u) of each [d x d] state update, reading its
// operands from LDS tiles whose rows are padded to d + 1 floats.
#include "common.hpp"
#include <mutex>
#include <type_traits>

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

// The pre-pass's LDS (three workgroups per compute unit at d = 64): W, b, the
// chunk's rows, and tiles shared by values with disjoint lifetimes -- Z then
// dZb, Zb then the row-sum buffer, the T slices then the dA slices.
template <int D>
struct PreSmem {
    static constexpr int DP = D + 1, TP = RW + 1;
    float W[D * DP], b[D];
    float XQ[RW * DP], XK[RW * DP], Z[RW * DP], Zb[RW * DP], E[RW * DP], dO[RW * DP];
    float T[RW * TP], dA[RW * TP];
    float TA[D / 16][RW * TP];
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

// Record of one chunk, written by the pre-pass and read once by the reverse
// sweep: five [16 x d] row tensors (xhat, ghat and G of the layer-norm gradient,
// dZb, T^T dZb), sigma and c of the gradient rows, and the chunk's share of
// dgamma and dbeta from the output layer norm.
enum { RT_XH, RT_GH, RT_G, RT_DZB, RT_TDZ, NRT };
template <int D>
struct Rec {
    static constexpr int OS = NRT * RW * D, OGB = OS + 2 * RW, SIZE = OGB + 2 * D;
};

// The three launches: the forward sweep stores every chunk-start state (one
// workgroup per sequence); the pre-pass recomputes each chunk from its state
// and does all of the chunk's reverse that does not depend on the adjoint
// state (as many workgroups as run at once, each taking chunks in turn); the reverse sweep runs
// the adjoint-dependent rest, chunk by chunk from the last (one per sequence).
enum { FWD = 0, PRE = 1, REV = 2 };

template <int D, typename TIO, int MODE>
__global__ __launch_bounds__(NT) void linear_backward_kernel(
    int nseq, int H, int L, int mb, float eps, const TIO *__restrict__ XQ, const TIO *__restrict__ XK,
    const TIO *__restrict__ XV, const float *__restrict__ eta, const float *__restrict__ W0,
    const float *__restrict__ b0, int w0_batched, const float *__restrict__ gamma,
    const float *__restrict__ beta, const float *__restrict__ dO, const float *__restrict__ dW_out,
    const float *__restrict__ db_out, float *__restrict__ dXQ, float *__restrict__ dXK,
    float *__restrict__ dXV, float *__restrict__ deta, float *__restrict__ dW0,
    float *__restrict__ db0, float *__restrict__ dgamma, float *__restrict__ dbeta,
    float *__restrict__ ws) {
    constexpr int NF = D / RW, DP = D + 1, TP = RW + 1, NTL = D / 16, REC = Rec<D>::SIZE;
    constexpr int OS = Rec<D>::OS, OGB = Rec<D>::OGB;
    constexpr float inv_d = 1.0f / D;
    using io = io_traits<TIO>;
    __shared__ std::conditional_t<MODE == PRE, PreSmem<D>, BwdSmem<D>> sm;

    // (not const: the pre-pass's chunk loop makes them opaque per chunk)
    int tid = threadIdx.x, r = tid / RW, q = tid % RW;
    int w = tid / 64, lane = tid % 64, g = lane / 16, c = lane % 16;  // MFMA coordinates
    const bool mw = w < NTL;  // this wave owns column tile w
    const int nch = (L + mb - 1) / mb;
    // one sequence per workgroup in the sweeps; the pre-pass sets its sequence per chunk
    const long seq = MODE == PRE ? 0 : static_cast<long>(blockIdx.x);
    const int h = static_cast<int>(seq % H);
    const long n = seq / H;
    const size_t sq = static_cast<size_t>(seq);
    const size_t xbase = sq * L * D;
    const size_t st = (w0_batched ? static_cast<size_t>(n) * H : 0) + static_cast<size_t>(h);
    float *wsq = ws + sq * nch * (D * D + D);
    float *const recq = ws + static_cast<size_t>(nseq) * nch * (D * D + D) + sq * nch * REC;
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
    // sum over the 16 token rows of a per-thread row value (all threads, one
    // feature per thread for tid < D), through the [16 x d] LDS buffer red
    auto rowsum = [&](float *red, const float (&v)[NF]) {
#pragma unroll
        for (int u = 0; u < NF; ++u) red[r * D + q + RW * u] = v[u];
        __syncthreads();
        float acc = 0.f;
        if (tid < D)
            for (int rr = 0; rr < RW; ++rr) acc += red[rr * D + tid];
        __syncthreads();
        return acc;
    };

    float gm[NF], bt[NF];
#pragma unroll
    for (int u = 0; u < NF; ++u) {
        gm[u] = gamma[h * D + q + RW * u];
        bt[u] = beta[h * D + q + RW * u];
    }

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
    // (xb: the sequence's first element in the [.., L, d] arrays; sqi: its index)
    auto fetch_rows_at = [&](size_t xb, size_t sqi, int ch, bool xq, bool go, Rows &R) {
        R.ok = r < min(mb, L - ch * mb);
        const int rr = R.ok ? r : 0;
        const size_t row = xb + static_cast<size_t>(ch * mb + rr) * D;
#pragma unroll
        for (int u = 0; u < NF; ++u) {
            const int f = q + RW * u;
            R.xk[u] = XK[row + f];
            R.xv[u] = XV[row + f];
            if (xq) R.xq[u] = XQ[row + f];
            if (go) R.go[u] = dO[row + f];
        }
        R.et = eta[sqi * L + ch * mb + rr];
    };
    auto fetch_rows = [&](int ch, bool xq, bool go, Rows &R) { fetch_rows_at(xbase, sq, ch, xq, go, R); };
    auto fetch_state_at = [&](const float *wc, State &S) {
#pragma unroll
        for (int k = 0; k < NWP; ++k) S.w[k] = wc[tid + NT * k];
        S.b = tid < D ? wc[D * D + tid] : 0.f;
    };
    auto fetch_state = [&](int ch, State &S) { fetch_state_at(wsq + static_cast<size_t>(ch) * (D * D + D), S); };
    // stage a chunk's rows: XK (and XQ, dO) into LDS; tau and eta into registers
    auto stage_rows = [&](const Rows &R, bool xq, bool go, float (&tau)[NF], float &et, float (&gov)[NF]) {
#pragma unroll
        for (int u = 0; u < NF; ++u) {
            const int f = q + RW * u;
            const float xk = R.ok ? io::load(R.xk, u) : 0.f;
            sm.XK[r * DP + f] = xk;
            tau[u] = R.ok ? io::load(R.xv, u) - xk : 0.f;
            if (xq) sm.XQ[r * DP + f] = R.ok ? io::load(R.xq, u) : 0.f;
            if (go) {
                gov[u] = R.ok ? R.go[u] : 0.f;
                sm.dO[r * DP + f] = gov[u];
            }
        }
        et = R.ok ? R.et : 0.f;
    };
    auto rowz = [&](const float *M, float (&z)[NF]) {
#pragma unroll
        for (int u = 0; u < NF; ++u) z[u] = M[r * DP + q + RW * u];
    };

    if constexpr (MODE == FWD) {
        // ===== forward: chunk-start states to the workspace ========================
        // W stays in registers for the whole sweep: wave w holds the tiles (rb, w),
        // lane (g, c) rows 16 rb + 4g .. +3 of column 16 w + c (the output layout of
        // the update). Z = XK W + b takes them as its B operand directly, with the
        // contraction order k <-> 16 rb + 4g + i of the accumulator rows.
        f32x4 Wr[NTL];
        if (mw) {
#pragma unroll
            for (int rb = 0; rb < NTL; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) Wr[rb][i] = W0[st * D * D + (16 * rb + 4 * g + i) * D + 16 * w + c];
        }
        if (tid < D) sm.b[tid] = b0[st * D + tid];
        __syncthreads();
        Rows R;
        if (nch > 0) fetch_rows(0, false, false, R);
        if (nch > 0) {  // chunk 0's start state; the others are written by the updates
            for (int i = tid; i < D * D; i += NT) wsq[i] = W0[st * D * D + i];
            if (tid < D) wsq[D * D + tid] = b0[st * D + tid];
        }
        for (int ch = 0; ch + 1 < nch; ++ch) {
            float *wn = wsq + static_cast<size_t>(ch + 1) * (D * D + D);
            float tau[NF], et, go_unused[NF];
            stage_rows(R, false, false, tau, et, go_unused);
            if (ch + 2 < nch) fetch_rows(ch + 1, false, false, R);
            __syncthreads();
            if (mw) {
                f32x4 zt = brow(sm.b);
#pragma unroll
                for (int rb = 0; rb < NTL; ++rb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        zt = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.XK[c * DP + 16 * rb + 4 * g + i], Wr[rb][i], zt,
                                                                  0, 0, 0);
                put(sm.Z, zt);
            }
            __syncthreads();
            float z[NF];
            rowz(sm.Z, z);
            Lnl2 s;
            lnl2(z, tau, s);
#pragma unroll
            for (int u = 0; u < NF; ++u) sm.E[r * DP + q + RW * u] = -et * s.G[u];
            __syncthreads();
            if (mw) {  // W += XK^T E on the register tiles, and the checkpoint
#pragma unroll
                for (int rb = 0; rb < NTL; ++rb) {
                    Wr[rb] = mma<RW>(colm(sm.XK + 16 * rb, DP), rowm(sm.E + 16 * w, DP), g, c, Wr[rb]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) wn[(16 * rb + 4 * g + i) * D + 16 * w + c] = Wr[rb][i];
                }
            }
            if (tid < D) {
                const float bn = sm.b[tid] + colsum(sm.E, nullptr);
                sm.b[tid] = bn;
                wn[D * D + tid] = bn;
            }
            __syncthreads();
        }
    }

    if constexpr (MODE == PRE) {
        // ========== pre-pass: every chunk, everything independent of the adjoint ==========
        // Persistent workgroups: workgroup i takes the chunks i, i + grid, i + 2 grid, ...
        // of the sequence-major chunk list. Once a chunk is staged, the next one's
        // rows and checkpoint are fetched into the same registers, so the
        // global-memory latency hides behind a chunk's work.
        const long total = static_cast<long>(nseq) * nch;
        auto fetch = [&](long gi, Rows &R, State &S) {
            const long sqi = gi / nch;
            fetch_rows_at(static_cast<size_t>(sqi) * L * D, static_cast<size_t>(sqi), static_cast<int>(gi - sqi * nch),
                          true, true, R);
            fetch_state_at(ws + static_cast<size_t>(gi) * (D * D + D), S);
        };
        Rows R;
        State S;
        fetch(min(static_cast<long>(blockIdx.x), total - 1), R, S);
        for (long gi = blockIdx.x; gi < total; gi += gridDim.x) {
            // lane coordinates opaque per chunk: the per-lane LDS and record addresses are
            // formed where they are used instead of being hoisted out of the loop and held
            asm volatile("" : "+v"(tid), "+v"(r), "+v"(q), "+v"(g), "+v"(c));
            const long sqi = gi / nch;
            const int ch = static_cast<int>(gi - sqi * nch), hh = static_cast<int>(sqi % H);
            const size_t xb = static_cast<size_t>(sqi) * L * D;
            const int m = min(mb, L - ch * mb);
            float *rc = ws + static_cast<size_t>(total) * (D * D + D) + static_cast<size_t>(gi) * REC;
#pragma unroll
            for (int u = 0; u < NF; ++u) {
                gm[u] = gamma[hh * D + q + RW * u];
                bt[u] = beta[hh * D + q + RW * u];
            }
#pragma unroll
            for (int k = 0; k < NWP; ++k) {
                const int i = tid + NT * k;
                sm.W[(i / D) * DP + i % D] = S.w[k];
            }
            if (tid < D) sm.b[tid] = S.b;
            float tau[NF], et, go[NF];
            stage_rows(R, true, true, tau, et, go);
            fetch(min(gi + static_cast<long>(gridDim.x), total - 1), R, S);  // a valid chunk even past the end
            __syncthreads();

            // Z = XK W + b, Zq = XQ W + b (tile w); T = XQ XK^T + 1 on the causal triangle
            if (mw) {
                put(sm.Z, mma<D>(rowm(sm.XK, DP), rowm(sm.W + 16 * w, DP), g, c, brow(sm.b)));
                put(sm.Zb, mma<D>(rowm(sm.XQ, DP), rowm(sm.W + 16 * w, DP), g, c, brow(sm.b)));
                const f32x4 t4 = mma<RW>(rowm(sm.XQ + 16 * w, DP), colm(sm.XK + 16 * w, DP), g, c, fz);
#pragma unroll
                for (int i = 0; i < 4; ++i) sm.TA[w][(4 * g + i) * TP + c] = t4[i];
            }
            __syncthreads();
            {  // T = tril(sum of the slices + 1) on the chunk's rows; one entry per thread
                const int t = tid / RW, s2 = tid % RW;
                float v = 0.f;
#pragma unroll
                for (int k = 0; k < NTL; ++k) v += sm.TA[k][t * TP + s2];
                sm.T[t * TP + s2] = (s2 <= t && t < m) ? v + 1.f : 0.f;
            }
            {  // G = lnl2(Z, XV - XK), E = -eta G; the values the reverse of lnl2 needs to the record
                float z[NF];
                rowz(sm.Z, z);
                Lnl2 s;
                lnl2(z, tau, s);
#pragma unroll
                for (int u = 0; u < NF; ++u) {
                    const int f = q + RW * u;
                    sm.E[r * DP + f] = -et * s.G[u];
                    rc[RT_XH * RW * D + r * D + f] = s.xh[u];
                    rc[RT_GH * RW * D + r * D + f] = s.gh[u];
                    rc[RT_G * RW * D + r * D + f] = s.G[u];
                }
                if (q == 0) {
                    rc[OS + r] = s.sigma;
                    rc[OS + RW + r] = s.c;
                }
            }
            __syncthreads();

            // Zb = XQ W + b + T E
            if (mw) put(sm.Zb, mma<RW>(rowm(sm.T, TP), rowm(sm.E + 16 * w, DP), g, c, get(sm.Zb)));
            __syncthreads();

            // the reverse of O = XQ + LN(Zb): dZb, and the chunk's share of dgamma, dbeta
            float dgp[NF], dbp[NF];
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
                    dgp[u] = go[u] * xb[u];
                    dbp[u] = go[u];
                    m1 += dx[u];
                    m2 += dx[u] * xb[u];
                }
                m1 = tile::row16_sum(m1) * inv_d;
                m2 = tile::row16_sum(m2) * inv_d;
#pragma unroll
                for (int u = 0; u < NF; ++u) {
                    const float v = (dx[u] - m1 - xb[u] * m2) * rs;
                    sm.Z[r * DP + q + RW * u] = v;
                    rc[RT_DZB * RW * D + r * D + q + RW * u] = v;
                }
            }
            __syncthreads();  // every row of Zb read: its tile becomes the row-sum buffer
            {
                const float a = rowsum(sm.Zb, dgp), b = rowsum(sm.Zb, dbp);  // (two barriers each)
                if (tid < D) {
                    rc[OGB + tid] = a;
                    rc[OGB + D + tid] = b;
                }
            }

            // dXQ tile = dZb W^T; slices of dA = dZb E^T; T^T dZb, the adjoint-free part of dE
            f32x4 gq = fz;
            if (mw) {
                gq = mma<D>(rowm(sm.Z, DP), colm(sm.W + 16 * w * DP, DP), g, c, fz);
                const f32x4 a4 = mma<RW>(rowm(sm.Z + 16 * w, DP), colm(sm.E + 16 * w, DP), g, c, fz);
#pragma unroll
                for (int i = 0; i < 4; ++i) sm.TA[w][(4 * g + i) * TP + c] = a4[i];
                const f32x4 td = mma<RW>(colm(sm.T, TP), rowm(sm.Z + 16 * w, DP), g, c, fz);
#pragma unroll
                for (int i = 0; i < 4; ++i) rc[RT_TDZ * RW * D + (4 * g + i) * D + 16 * w + c] = td[i];
            }
            __syncthreads();
            {  // dA = the slices summed on the causal triangle of the chunk's rows
                const int t = tid / RW, s2 = tid % RW;
                float v = 0.f;
#pragma unroll
                for (int k = 0; k < NTL; ++k) v += sm.TA[k][t * TP + s2];
                sm.dA[t * TP + s2] = (s2 <= t && t < m) ? v : 0.f;
            }
            __syncthreads();

            // dXQ = dO + dZb W^T + dA XK;  dA^T XQ, the adjoint-free part of dXK
            if (mw) {
                gq = mma<RW>(rowm(sm.dA, TP), rowm(sm.XK + 16 * w, DP), g, c, gq);
                const f32x4 gk = mma<RW>(colm(sm.dA, TP), rowm(sm.XQ + 16 * w, DP), g, c, fz);
                const f32x4 do4 = get(sm.dO);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 4 * g + i;
                    if (t < m) {
                        const size_t at = xb + static_cast<size_t>(ch * mb + t) * D + 16 * w + c;
                        dXQ[at] = gq[i] + do4[i];
                        dXK[at] = gk[i];
                    }
                }
            }
            __syncthreads();  // the next chunk's staging overwrites every tile
        }
    }

    if constexpr (MODE == REV) {
        // ================ reverse sweep: the adjoint-dependent rest =====================
        for (int i = tid; i < D * D; i += NT)
            sm.dW[(i / D) * DP + i % D] = dW_out ? dW_out[sq * D * D + i] : 0.f;
        if (tid < D) sm.db[tid] = db_out ? db_out[sq * D + tid] : 0.f;
        float dg_acc[NF], db_acc[NF];
#pragma unroll
        for (int u = 0; u < NF; ++u) dg_acc[u] = db_acc[u] = 0.f;
        float accG = 0.f, accB = 0.f;  // the output layer norm's dgamma, dbeta from the records

        // what a chunk reads, loaded during the previous chunk: its rows, its start state,
        // the record's row values, T^T dZb and the pre-pass's part of dXK (tile layout)
        struct Ahead {
            Rows R;
            State S;
            float xh[NF], gh[NF], G[NF], dzb[NF], sig, cc, pg, pb;
            f32x4 tdz, xki;
        };
        auto load_ahead = [&](int ch, Ahead &N) {
            const float *rc = recq + static_cast<size_t>(ch) * REC;
            const int mc = min(mb, L - ch * mb);
            fetch_rows(ch, true, false, N.R);
            fetch_state(ch, N.S);
#pragma unroll
            for (int u = 0; u < NF; ++u) {
                const int o = r * D + q + RW * u;
                N.xh[u] = rc[RT_XH * RW * D + o];
                N.gh[u] = rc[RT_GH * RW * D + o];
                N.G[u] = rc[RT_G * RW * D + o];
                N.dzb[u] = rc[RT_DZB * RW * D + o];
            }
            N.sig = rc[OS + r];
            N.cc = rc[OS + RW + r];
            N.pg = tid < D ? rc[OGB + tid] : 0.f;
            N.pb = tid < D ? rc[OGB + D + tid] : 0.f;
            if (mw) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    N.tdz[i] = rc[RT_TDZ * RW * D + (4 * g + i) * D + 16 * w + c];
                    N.xki[i] = dXK[xbase + static_cast<size_t>(ch * mb + min(4 * g + i, mc - 1)) * D + 16 * w + c];
                }
            }
        };
        Ahead N;
        if (nch > 0) load_ahead(nch - 1, N);
        for (int ch = nch - 1; ch >= 0; --ch) {
            const int m = min(mb, L - ch * mb);
            const bool ok = r < m;
            __syncthreads();  // the previous chunk is done with every tile
#pragma unroll
            for (int k = 0; k < NWP; ++k) {
                const int i = tid + NT * k;
                sm.W[(i / D) * DP + i % D] = N.S.w[k];
            }
            if (tid < D) sm.b[tid] = N.S.b;
            float tau[NF], et, go_unused[NF];
            stage_rows(N.R, true, false, tau, et, go_unused);
            Lnl2 s;  // the forward values of this chunk's lnl2 rows, from the record
#pragma unroll
            for (int u = 0; u < NF; ++u) {
                s.xh[u] = N.xh[u];
                s.gh[u] = N.gh[u];
                s.G[u] = N.G[u];
                sm.E[r * DP + q + RW * u] = -et * N.G[u];
                sm.dZb[r * DP + q + RW * u] = N.dzb[u];
            }
            s.sigma = N.sig;
            s.c = N.cc;
            const f32x4 tdz = N.tdz, xki = N.xki;
            accG += N.pg;
            accB += N.pb;
            load_ahead(max(ch - 1, 0), N);  // unconditional: the last chunk reloads chunk 0
            __syncthreads();

            // dE = T^T dZb + XK dW' + db';  dXK tile = E dW'^T  (dW', db' not yet updated)
            f32x4 gk = fz;
            if (mw) {
                const f32x4 de = mma<D>(rowm(sm.XK, DP), rowm(sm.dW + 16 * w, DP), g, c, brow(sm.db));
                put(sm.dE, de + tdz);
                gk = mma<D>(rowm(sm.E, DP), colm(sm.dW + 16 * w * DP, DP), g, c, fz);
            }
            __syncthreads();

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
            if (ok && q == 0) deta[sq * L + ch * mb + r] = d_eta;
            __syncthreads();

            // dXK = dA^T XQ + E dW'^T + dZ W^T - dtau;  dXV = dtau;  write the tiles
            if (mw) {
                gk = mma<D>(rowm(sm.dZ, DP), colm(sm.W + 16 * w * DP, DP), g, c, gk);
                const f32x4 dt4 = get(sm.dT);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 4 * g + i;
                    if (t < m) {
                        const size_t at = xbase + static_cast<size_t>(ch * mb + t) * D + 16 * w + c;
                        dXK[at] = xki[i] + gk[i] - dt4[i];
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
        // per-sequence dgamma, dbeta: the 16 row groups of the lnl2 reverse plus the output norm's share
        const float a = rowsum(sm.red, dg_acc), b = rowsum(sm.red, db_acc);
        if (tid < D) {
            dgamma[sq * D + tid] = a + accG;
            dbeta[sq * D + tid] = b + accB;
        }
    }
}

template <int D, typename TIO, int MODE>
hipError_t launch_mode(const LinearBwdArgs &a, unsigned grid, hipStream_t stream) {
    hipLaunchKernelGGL((linear_backward_kernel<D, TIO, MODE>), dim3(grid), dim3(NT), 0, stream,
                       a.f.B * a.f.H, a.f.H, a.f.L, a.f.mb, a.f.eps, static_cast<const TIO *>(a.f.XQ),
                       static_cast<const TIO *>(a.f.XK), static_cast<const TIO *>(a.f.XV), a.f.eta,
                       a.f.W0, a.f.b0, a.f.w0_batched, a.f.gamma, a.f.beta, a.dO, a.dW_out, a.db_out,
                       a.dXQ, a.dXK, a.dXV, a.deta, a.dW0, a.db0, a.dgamma, a.dbeta, a.ws);
    return hipGetLastError();
}

template <int D, typename TIO>
hipError_t launch_bwd_t(const LinearBwdArgs &a, hipStream_t stream) {
    const size_t nseq = static_cast<size_t>(a.f.B) * a.f.H;
    const size_t nch = a.f.L > 0 ? static_cast<size_t>((a.f.L + a.f.mb - 1) / a.f.mb) : 0;
    if (nseq * nch > 0x7fffffffu) return hipErrorInvalidValue;
    hipError_t e;
    if (nch > 0) {
        if ((e = launch_mode<D, TIO, FWD>(a, static_cast<unsigned>(nseq), stream)) != hipSuccess) return e;
        // the pre-pass's persistent workgroups: as many as run at once, at most one per chunk
        int dev = 0, ncu = 0, per = 0;
        if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
        if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
        if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, linear_backward_kernel<D, TIO, PRE>, NT, 0)) !=
            hipSuccess)
            return e;
        const size_t pre = std::min(nseq * nch, static_cast<size_t>(std::max(1, ncu * per)));
        if ((e = launch_mode<D, TIO, PRE>(a, static_cast<unsigned>(pre), stream)) != hipSuccess) return e;
    }
    return launch_mode<D, TIO, REV>(a, static_cast<unsigned>(nseq), stream);
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

size_t linear_backward_chunk_floats(int d) {  // workspace floats per sequence and chunk
    if (d == 16) return 16 * 16 + 16 + Rec<16>::SIZE;
    if (d == 64) return 64 * 64 + 64 + Rec<64>::SIZE;
    return 0;
}

hipError_t launch_linear_backward(const LinearBwdArgs &a, hipStream_t stream) {
    if (a.f.B * a.f.H == 0) return hipSuccess;
    if (a.f.d == 16) return a.f.io ? launch_bwd_t<16, bf16_t>(a, stream) : launch_bwd_t<16, float>(a, stream);
    if (a.f.d == 64) return a.f.io ? launch_bwd_t<64, bf16_t>(a, stream) : launch_bwd_t<64, float>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace ttt
