// Backward of the TTT-MLP inner loop (d = 64, hidden m = 4d = 256, exact
// GELU; the lryc.cn TTT article §2.1 model, the mini-batch rule and dual form
// of the damodev.csdn.net deep-dive §4.1-4.2, trained through the inner loop as
// in its §6 and §7.1): gradients of
//   loss = <dO, O> + <dW1', W1_L> + <db1', b1_L> + <dW2', W2_L> + <db2', b2_L>
// with respect to XQ, XK, XV, eta, the initial state W1, b1, W2, b2, gamma and
// beta.
//
// Per chunk (state W1, b1, W2, b2 at the chunk start, rows = tokens, P = GELU'):
//   Z1 = XK W1 + b1,  A = gelu(Z1),  Z2 = A W2 + b2,  G2 = lnl2(Z2, XV - XK),
//   E2 = -eta * G2,  Q = E2 W2^T,  E1 = Q * P(Z1)         (the chunk-start gradients)
//   T1 = tril(XQ XK^T + 1),  Zb1 = XQ W1 + b1 + T1 E1,  Ab = gelu(Zb1),
//   T2 = tril(Ab A^T + 1),   Zb2 = Ab W2 + b2 + T2 E2,  O = XQ + LN(Zb2),
//   W1' = W1 + XK^T E1,  b1' = b1 + 1^T E1,  W2' = W2 + A^T E2,  b2' = b2 + 1^T E2.
// Reverse, given dO and the adjoints dW1', db1', dW2', db2' of the next state:
//   dZb2 = LN backward of dO;  dT2 = tril(dZb2 E2^T);
//   dAb = dZb2 W2^T + dT2 A;  dZb1 = dAb * P(Zb1);  dT1 = tril(dZb1 E1^T);
//   dE2 = T2^T dZb2 + A dW2' + 1 db2'^T + dQ W2,   with
//   dE1 = T1^T dZb1 + XK dW1' + 1 db1'^T,  dQ = dE1 * P(Z1);
//   deta = -rowsum(G2 * dE2);  (dZ2, dtau) = reverse of lnl2 for dG2 = -eta dE2;
//   dA = dT2^T Ab + E2 dW2'^T + dZ2 W2^T;
//   dZ1 = dA * P(Z1) + dE1 * Q * GELU''(Z1),  GELU''(x) = phi(x) (2 - x^2);
//   dXQ = dO + dZb1 W1^T + dT1 XK;  dXK = dT1^T XQ + E1 dW1'^T + dZ1 W1^T - dtau;
//   dXV = dtau;
//   dW1 = dW1' + XQ^T dZb1 + XK^T dZ1;       db1 = db1' + 1^T (dZb1 + dZ1);
//   dW2 = dW2' + Ab^T dZb2 + dQ^T E2 + A^T dZ2;  db2 = db2' + 1^T (dZb2 + dZ2).
// lnl2 and its reverse are the closed forms of the TTT-Linear backward.
//
// One 512-thread workgroup (8 waves) per sequence, fp32 throughout: every
// product on 16x16x4 fp32 MFMAs (lane (g, c) of a wave supplies row c of the
// left operand and column c of the right one at contraction index g of each
// step; the result tile's rows 4g..4g+3 of column c come back). Wave w owns
// the hidden units 32w..32w+31: it computes their [16 x 32] slices of every
// hidden-width tile and keeps them in registers, where a tile in the result
// layout is directly an operand of a product that contracts over the tokens
// (the contraction order permuted identically on both sides). Products that
// contract over the hidden units split them in two halves: wave w computes the
// half w / 4 of 16-feature tile w % 4 and the two partial tiles are summed by
// their reader. Hidden tiles read across waves or transposed go through LDS.
//
// Three launches. A forward sweep stores the state at every chunk start in the
// workspace. A pre-pass, one workgroup per chunk and all chunks at once,
// recomputes each chunk from its stored state and does every part of the
// chunk's reverse that does not involve the adjoint state of the chunk end
// (dZb2, dT2, dZb1, dT1, T2^T dZb2, dT2^T Ab, T1^T dZb1, dXQ in full, the dT1^T XQ
// part of dXK); it stores what the rest needs in a per-chunk record. The
// reverse sweep then runs the adjoint-dependent rest chunk by chunk from the
// last, keeping the running adjoint state in two workspace buffers used
// alternately (read the one, write the other), so no state matrix occupies LDS.
#include "common.hpp"

#include "launch.hpp"
#include "tile.hpp"

namespace ttt {
namespace {

constexpr int D = 64, M = 4 * D, NT = 512, RW = 16, NF = D / RW;
constexpr int DP = D + 1, MP = M + 1, TP = RW + 1;
// floats of one stored state: W1 transposed [M][D], b1 [M], W2 [M][D], b2 [D] (both weight
// matrices hidden-unit-major, as are the adjoint states, and stored as 16 x 16 tiles: see tix)
constexpr int CK = 2 * D * M + M + D;
constexpr int OB1 = D * M, OW2 = D * M + M, OB2 = 2 * D * M + M;

using tile::f32x4;

struct MlpBwdSmem {
    // [16 x D] token-row tiles
    float XQ[RW * DP], XK[RW * DP], dO[RW * DP], E2[RW * DP], dZb2[RW * DP], dZ2[RW * DP], dtau[RW * DP];
    float tau[RW * DP];
    // partials of the two hidden halves; partE holds dE2 and later the dXK partials
    float part[2][RW * DP], partE[2][RW * DP];
    // [16 x M] hidden tiles; HY holds Ab, later dQ, later dZ1
    float HA[RW * MP], HE[RW * MP], HX[RW * MP], HY[RW * MP];
    // row-work values: gamma, beta, eta of the chunk's rows, dgamma and dbeta per row
    float gam[D], bet[D], eta[RW], accg[RW * DP], accb[RW * DP];
    // [16 x 16] token-token tiles and per-wave partials
    float T1[RW * TP], T2[RW * TP], dT1[RW * TP];
    float gp[NT / 64][RW * TP];
    // what the reverse of lnl2 needs from the forward: xhat, ghat and G per row
    float lxh[RW * DP], lgh[RW * DP], lG[RW * DP], lsig[RW], lcc[RW];
};

// The forward sweep's tiles (the same LDS, reused): XK, A, the two Z2 halves,
// E2, and a copy of W2 (rows padded to 68 floats: the 16 rows one operand
// read touches start on distinct banks) for E2 W2^T and A W2.
constexpr int W2P = D + 4;
struct MlpFwdSmem {
    float XK[RW * DP], HA[RW * MP], part[2][RW * DP], E2[RW * DP];
    float W2[M * W2P], b2[D];
};
union MlpSmem {
    MlpBwdSmem r;
    MlpFwdSmem f;
};

// Offset of element (n, f) (hidden unit n, feature f) of a stored [M x D] state matrix: 16 x 16
// tiles, each 1 KB contiguous and row-major, tile (n / 16, f / 16) at (4 (n / 16) + f / 16) KB.
__device__ __forceinline__ int tix(int n, int f) {
    return ((n >> 4) * (D / 16) + (f >> 4)) * 256 + (n & 15) * 16 + (f & 15);
}

__device__ __forceinline__ f32x4 mf(float a, float b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

// Global access as a uniform base plus a 32-bit byte offset per lane, the
// form the scalar-base addressing of global loads and stores takes (one VGPR
// per address instead of a 64-bit pair).
__device__ __forceinline__ float gld(const float *base, unsigned idx) {
    return *reinterpret_cast<const float *>(reinterpret_cast<const char *>(base) + (idx << 2));
}
__device__ __forceinline__ void gst(float *base, unsigned idx, float v) {
    *reinterpret_cast<float *>(reinterpret_cast<char *>(base) + (idx << 2)) = v;
}
// 16-byte forms (base + idx 16-byte aligned)
__device__ __forceinline__ tile::f32x4 gld4(const float *base, unsigned idx) {
    return *reinterpret_cast<const tile::f32x4 *>(reinterpret_cast<const char *>(base) + (idx << 2));
}
__device__ __forceinline__ void gst4(float *base, unsigned idx, tile::f32x4 v) {
    *reinterpret_cast<tile::f32x4 *>(reinterpret_cast<char *>(base) + (idx << 2)) = v;
}

__device__ __forceinline__ tile::f32x2 gld2(const float *base, unsigned idx) {  // 8-byte form
    return *reinterpret_cast<const tile::f32x2 *>(reinterpret_cast<const char *>(base) + (idx << 2));
}
// two consecutive input elements in one load: raw bits and the two values as fp32
template <typename T> struct pair_io;
template <> struct pair_io<float> {
    typedef tile::f32x2 raw;
    static __device__ __forceinline__ raw ld(const float *base, unsigned idx) { return gld2(base, idx); }
    static __device__ __forceinline__ float lo(raw v) { return v[0]; }
    static __device__ __forceinline__ float hi(raw v) { return v[1]; }
};
template <> struct pair_io<bf16_t> {
    typedef uint32_t raw;
    static __device__ __forceinline__ raw ld(const bf16_t *base, unsigned idx) {
        return *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(base) + (idx << 1));
    }
    static __device__ __forceinline__ float lo(raw v) { return __uint_as_float(v << 16); }
    static __device__ __forceinline__ float hi(raw v) { return __uint_as_float(v & 0xffff0000u); }
};

// GELU(x) = x Phi(x), GELU'(x) = Phi(x) + x phi(x), GELU''(x) = phi(x) (2 - x^2), from one
// evaluation of Phi and phi (erf to |error| <= 1.5e-7, far below the fp32 products' bar)
__device__ __forceinline__ void gelu3(float x, float &g0, float &g1, float &g2) {
    float Phi, phi;
    normal_cdf_pdf(x, Phi, phi);
    g0 = x * Phi;
    g1 = fmaf(x, phi, Phi);
    g2 = phi * (2.0f - x * x);
}
__device__ __forceinline__ void gelu2(float x, float &g0, float &g1) {
    float Phi, phi;
    normal_cdf_pdf(x, Phi, phi);
    g0 = x * Phi;
    g1 = fmaf(x, phi, Phi);
}

// Record of one chunk, written by the pre-pass and read once by the reverse
// sweep: eight hidden tensors [16 x M] in the register layout of the waves that
// own them (tensor t, wave w, tile j, lane: four consecutive floats), five
// [16 x D] row tensors, sigma and c of the chunk's layer-norm gradient rows, and
// the chunk's share of dgamma and dbeta from the output layer norm.
constexpr int RH = RW * M;
enum { HT_A, HT_P, HT_RQ, HT_AB, HT_DZB1, HT_DAT, HT_TZ, HT_E1, NHT };
enum { RT_XH, RT_GH, RT_G, RT_DZB2, RT_T2Z, NRT };
constexpr int OR = NHT * RH, OS = OR + NRT * RW * D, OGB = OS + 2 * RW, REC = OGB + 2 * D;
static_assert(CK % 4 == 0 && REC % 4 == 0, "16-byte aligned records");

// The three launches: the forward sweep stores every chunk-start state (one
// workgroup per sequence); the pre-pass recomputes each chunk from its state
// and does all of the chunk's reverse that does not depend on the adjoint state
// (one workgroup per chunk, all chunks at once); the reverse sweep runs the
// adjoint-dependent rest, chunk by chunk from the last (one per sequence).
enum { FWD = 0, PRE = 1, REV = 2 };

template <typename TIO, int MODE>
__global__ __launch_bounds__(NT) void mlp_backward_kernel(
    int nseq, int H, int L, int mb, float eps, const TIO *__restrict__ XQ, const TIO *__restrict__ XK,
    const TIO *__restrict__ XV, const float *__restrict__ eta, const float *__restrict__ W1_0,
    const float *__restrict__ b1_0, const float *__restrict__ W2_0, const float *__restrict__ b2_0,
    int w0_batched, const float *__restrict__ gamma, const float *__restrict__ beta,
    const float *__restrict__ dO, const float *__restrict__ dW1_out, const float *__restrict__ db1_out,
    const float *__restrict__ dW2_out, const float *__restrict__ db2_out, float *__restrict__ dXQ,
    float *__restrict__ dXK, float *__restrict__ dXV, float *__restrict__ deta, float *__restrict__ dW1,
    float *__restrict__ db1, float *__restrict__ dW2, float *__restrict__ db2,
    float *__restrict__ dgamma, float *__restrict__ dbeta, float *__restrict__ ws) {
    constexpr float inv_d = 1.0f / D;
    using io = io_traits<TIO>;
    __shared__ MlpSmem smu;
    MlpBwdSmem &sm = smu.r;
    MlpFwdSmem &sf = smu.f;

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
    const int wu = __builtin_amdgcn_readfirstlane(w);  // the wave index as a uniform value
    const int u = wu & 3, hh = wu >> 2;        // feature tile and hidden half of split products
    const bool rowt = tid < RW * RW;           // row work: 16 lanes per token row
    const int r = (tid >> 4) & (RW - 1), q = tid & (RW - 1);
    const int nch = (L + mb - 1) / mb;
    // the pre-pass takes one chunk: workgroup index = sequence * chunks + chunk
    const long seq = MODE == PRE ? static_cast<long>(blockIdx.x) / nch : static_cast<long>(blockIdx.x);
    const int h = static_cast<int>(seq % H);
    const long n = seq / H;
    const size_t sq = static_cast<size_t>(seq);
    const size_t xbase = sq * L * D;
    const size_t st = (w0_batched ? static_cast<size_t>(n) * H : 0) + static_cast<size_t>(h);
    float *wsq = ws + sq * (static_cast<size_t>(nch) + 2) * CK;
    float *const adj0 = wsq + static_cast<size_t>(nch) * CK, *const adj1 = adj0 + CK;
    auto adj = [&](int k) { return (k & 1) ? adj1 : adj0; };
    float *const recq = ws + static_cast<size_t>(nseq) * (nch + 2) * CK + sq * nch * REC;
    const f32x4 fz = {0.f, 0.f, 0.f, 0.f};
    const int hc0 = 32 * wu + c;  // this lane's hidden column in own tile j: hc0 + 16 j
    // Global addresses are a uniform pointer plus one of a few per-lane offsets
    // (elements), so that the per-lane part stays one register per pattern.
    const unsigned lc = g * 16 + c, le = 4 * g * M + c, lf = 4 * g * D + c;
    // 16-byte per-lane runs: W2^T fragments and the transposed adjoint tiles
    const unsigned lbv = c * 16 + 4 * g, lg = c * 16 + 4 * g, lw = 64 * g + c;
    // record: a lane's four floats of a hidden tile; a row thread's features of a row tensor
    const unsigned lh = 4 * lane, lrq = r * D + q;

    // ---------------------------------------------------------------- products
    // the same with a token-token tile: [16 x 16] (LDS, transposed if tr) times X [16 x D]
    auto t_x = [&](const float *T, bool tr, const float *X, f32x4 acc) {
#pragma unroll
        for (int kb = 0; kb < RW / 4; ++kb) {
            const int k = 4 * kb + g;
            acc = mf(tr ? T[k * TP + c] : T[c * TP + k], X[k * DP + 16 * u + c], acc);
        }
        return acc;
    };
    // own hidden tile of T^T Hj: rows of T (LDS) contracted with the register tile Hj
    auto tt_h = [&](const float *T, f32x4 Hj, f32x4 acc) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = mf(T[(4 * g + i) * TP + c], Hj[i], acc);
        return acc;
    };
    // [D x M] update tile (rb, j) += X^T Hj over the tokens (X [16 x D] in LDS)
    auto xt_h = [&](const float *X, int rb, f32x4 Hj, f32x4 acc) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = mf(X[(4 * g + i) * DP + 16 * rb + c], Hj[i], acc);
        return acc;
    };
    // [M x D] update tile (j, uu) += Hj^T Y over the tokens (Y [16 x D] in LDS)
    auto ht_y = [&](f32x4 Hj, const float *Y, int uu, f32x4 acc) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = mf(Hj[i], Y[(4 * g + i) * DP + 16 * uu + c], acc);
        return acc;
    };
    auto put_h = [&](float *Hs, int j, f32x4 v) {
        int lo = 4 * g * MP + c;
        asm volatile("" : "+v"(lo));  // recomputed per use: no per-tile address held across the loop
        float *p = Hs + lo + 32 * wu + 16 * j;
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i * MP] = v[i];
    };
    auto put_d = [&](float *P, f32x4 v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) P[(4 * g + i) * DP + 16 * u + c] = v[i];
    };
    auto bcast = [](float x) { return f32x4{x, x, x, x}; };
    // Operand fragments: the right operands that one product reads from global
    // memory, loaded into registers as one block a phase ahead of the product,
    // so that their latency overlaps earlier work instead of stalling it.
    typedef float Frag[32];
    // V [M x D] transposed: own hidden tiles, contraction over D in the order
    // where load q of lane group g takes the features 16 q + 4 g .. + 3 (the four
    // groups of a row read 64 contiguous bytes per load)
    auto ld_vt = [&](const float *V, Frag &v) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const f32x4 t = gld4(V + (2 * wu + j) * 1024 + 256 * qq, lbv);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[16 * j + 4 * qq + e] = t[e];
            }
    };
    auto ld_v = [&](const float *V, Frag &v) {  // V [M x D]: feature tile u over hidden half hh
#pragma unroll
        for (int kb = 0; kb < M / 8; ++kb) v[kb] = gld(V + ((8 * hh + (kb >> 2)) * 4 + u) * 256 + 64 * (kb & 3), lc);
    };
    // feature tile u over hidden half hh of Y [16 x M] (LDS) times a fragment of ld_v
    auto mm_y = [&](const float *Y, const Frag &v, f32x4 acc) {
#pragma unroll
        for (int kb = 0; kb < M / 8; ++kb) acc = mf(Y[c * MP + M / 2 * hh + 4 * kb + g], v[kb], acc);
        return acc;
    };
    // own hidden tile j of X [16 x D] (LDS) times a fragment of ld_vt (step 4 q + e:
    // feature 16 q + 4 g + e)
    auto mm_xt = [&](const float *X, const Frag &v, int j, f32x4 acc) {
#pragma unroll
        for (int st = 0; st < D / 4; ++st)
            acc = mf(X[c * DP + 16 * (st >> 2) + 4 * g + (st & 3)], v[16 * j + st], acc);
        return acc;
    };
    auto issue = [] { __builtin_amdgcn_sched_barrier(0); };  // keeps the loads above where they are
    // token-token tile from per-wave partials: T[t][s] = sum + add on s <= t < m, else 0
    auto tri_sum = [&](float *T, int nparts, float add, int m) {
        if (tid < RW * RW) {
            const int t = tid >> 4, s = tid & 15;
            float v = 0.f;
            for (int k = 0; k < nparts; ++k) v += sm.gp[k][t * TP + s];
            T[t * TP + s] = (s <= t && t < m) ? v + add : 0.f;
        }
    };
    auto rowz2 = [&](const float *P0, const float *P1, float (&z)[NF]) {
#pragma unroll
        for (int k = 0; k < NF; ++k) z[k] = P0[r * DP + q + RW * k] + P1[r * DP + q + RW * k];
    };
    // a hidden tile of the record (tensor t, own tile j)
    auto put_rec = [&](float *rc, int t, int j, f32x4 v) { gst4(rc + t * RH + (2 * wu + j) * 256, lh, v); };
    auto get_rec = [&](const float *rc, int t, int j) { return gld4(rc + t * RH + (2 * wu + j) * 256, lh); };
    auto rrow = [&](int t) { return OR + t * RW * D; };  // offset of row tensor t in a record

    // layer-norm L2 gradient of one row (16 lanes) and what its reverse needs
    struct Lnl2 {
        float xh[NF], gh[NF], G[NF];
        float sigma, c;
    };
    auto lnl2 = [&](const float (&z)[NF], const float (&tau)[NF], const float (&gm)[NF], const float (&bt)[NF],
                    Lnl2 &s) {
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int k = 0; k < NF; ++k) s1 += z[k];
        const float mu = tile::row16_sum(s1) * inv_d;
#pragma unroll
        for (int k = 0; k < NF; ++k) s2 += (z[k] - mu) * (z[k] - mu);
        s.sigma = sqrtf(tile::row16_sum(s2) * inv_d + eps);
        const float rs = 1.0f / s.sigma;
        float sa = 0.f, sc = 0.f;
#pragma unroll
        for (int k = 0; k < NF; ++k) {
            s.xh[k] = (z[k] - mu) * rs;
            s.gh[k] = gm[k] * fmaf(gm[k], s.xh[k], bt[k] - tau[k]);
            sa += s.gh[k];
            sc += s.gh[k] * s.xh[k];
        }
        const float a = tile::row16_sum(sa) * inv_d;
        s.c = tile::row16_sum(sc) * inv_d;
#pragma unroll
        for (int k = 0; k < NF; ++k) s.G[k] = (s.gh[k] - a - s.xh[k] * s.c) * rs;
    };

    // Inputs of one chunk for this row thread; unconditional loads from a row
    // clamped into the sequence, rows past its end zeroed when staged.
    struct Rows {
        TIO xq[NF], xk[NF], xv[NF];
        float go[NF], et;
        bool ok;
    };
    auto fetch_rows = [&](int ch, bool xq, bool go, Rows &R) {
        R.ok = r < min(mb, L - ch * mb);
        const int rr = R.ok ? r : 0;
        const size_t row = xbase + static_cast<size_t>(ch * mb + rr) * D;
#pragma unroll
        for (int k = 0; k < NF; ++k) {
            const int f = q + RW * k;
            R.xk[k] = XK[row + f];
            R.xv[k] = XV[row + f];
            if (xq) R.xq[k] = XQ[row + f];
            if (go) R.go[k] = dO[row + f];
        }
        R.et = eta[sq * L + ch * mb + rr];
    };
    // one row of a [16 x D] tile (ld = 0: a [D] vector) for this row thread
    auto rowld = [&](const float *P, int ld, float (&z)[NF]) {
#pragma unroll
        for (int k = 0; k < NF; ++k) z[k] = P[r * ld + q + RW * k];
    };

    if constexpr (MODE == FWD) {
        // ======================= forward sweep: chunk-start states ===================
        // The state stays in registers in the result layout of its updates: wave w
        // holds W1[16 rb + 4 g + i][32 w + 16 j + c] and W2[32 w + 16 j + 4 g + i][16 uu + c],
        // which with the contraction order permuted identically is also the right
        // operand of XK W1. W2 is mirrored in LDS for A W2 and E2 W2^T. Every chunk
        // start is stored to the workspace (write-only).
        float gm[NF], bt[NF];
#pragma unroll
        for (int k = 0; k < NF; ++k) {
            gm[k] = gamma[h * D + q + RW * k];
            bt[k] = beta[h * D + q + RW * k];
        }
        f32x4 W1r[4][2], W2r[2][4];
        float b1r[2], b2r = 0.f;
        {
            const float *s1 = W1_0 + st * D * M, *s2 = b1_0 + st * M, *s3 = W2_0 + st * M * D, *s4 = b2_0 + st * D;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) W1r[rb][j][i] = gld(s1 + (16 * rb + i) * M + 32 * wu + 16 * j, le);
#pragma unroll
                for (int uu = 0; uu < 4; ++uu)
#pragma unroll
                    for (int i = 0; i < 4; ++i) W2r[j][uu][i] = gld(s3 + (32 * wu + 16 * j + i) * D + 16 * uu, lf);
                b1r[j] = gld(s2 + 32 * wu + 16 * j, c);
            }
            if (tid < D) b2r = s4[tid];
        }
        // the current state to the workspace checkpoint S and to the LDS mirror of W2
        auto put_state = [&](float *Sn) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) gst4(Sn + (2 * wu + j) * 1024 + 256 * rb, lg, W1r[rb][j]);
#pragma unroll
                for (int uu = 0; uu < 4; ++uu)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        gst(Sn + OW2 + ((2 * wu + j) * 4 + uu) * 256 + 16 * i, lw, W2r[j][uu][i]);
                        sf.W2[(32 * wu + 16 * j + 4 * g + i) * W2P + 16 * uu + c] = W2r[j][uu][i];
                    }
                if (g == 0) gst(Sn + OB1 + 32 * wu + 16 * j, c, b1r[j]);
            }
            if (tid < D) {
                gst(Sn + OB2, tid, b2r);
                sf.b2[tid] = b2r;
            }
        };
        Rows R;
        if (nch > 0) put_state(wsq);
        if (rowt && nch > 1) fetch_rows(0, false, false, R);
        for (int ch = 0; ch + 1 < nch; ++ch) {
            float tau[NF], et = 0.f;
            if (rowt) {
#pragma unroll
                for (int k = 0; k < NF; ++k) {
                    const float xk = R.ok ? io::load(R.xk, k) : 0.f;
                    sf.XK[r * DP + q + RW * k] = xk;
                    tau[k] = R.ok ? io::load(R.xv, k) - xk : 0.f;
                }
                et = R.ok ? R.et : 0.f;
                if (ch + 2 < nch) fetch_rows(ch + 1, false, false, R);
            }
            tile::lds_barrier();
            // Z1 = XK W1 + b1 on the own hidden tiles (W1 from registers); A = gelu(Z1), P = gelu'(Z1)
            f32x4 Ar[2], Pr[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                f32x4 z = bcast(b1r[j]);
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) z = mf(sf.XK[c * DP + 16 * rb + 4 * g + i], W1r[rb][j][i], z);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float g0, g1;
                    gelu2(z[i], g0, g1);
                    Ar[j][i] = g0;
                    Pr[j][i] = g1;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) sf.HA[(4 * g + i) * MP + hc0 + 16 * j] = Ar[j][i];
            }
            tile::lds_barrier();
            {  // Z2 = A W2 + b2, the two hidden halves (W2 from LDS)
                f32x4 acc = hh == 0 ? bcast(sf.b2[16 * u + c]) : fz;
#pragma unroll
                for (int kb = 0; kb < M / 8; ++kb) {
                    const int k = M / 2 * hh + 4 * kb + g;
                    acc = mf(sf.HA[c * MP + k], sf.W2[k * W2P + 16 * u + c], acc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) sf.part[hh][(4 * g + i) * DP + 16 * u + c] = acc[i];
            }
            tile::lds_barrier();
            if (rowt) {  // E2 = -eta lnl2(Z2, XV - XK)
                float z[NF];
                rowz2(sf.part[0], sf.part[1], z);
                Lnl2 s;
                lnl2(z, tau, gm, bt, s);
#pragma unroll
                for (int k = 0; k < NF; ++k) sf.E2[r * DP + q + RW * k] = -et * s.G[k];
            }
            tile::lds_barrier();
            // E1 = (E2 W2^T) * P;  W1 += XK^T E1, b1 += 1^T E1;  W2 += A^T E2, b2 += 1^T E2
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                f32x4 qv = fz;
#pragma unroll
                for (int kb = 0; kb < D / 4; ++kb)
                    qv = mf(sf.E2[c * DP + 4 * kb + g], sf.W2[(hc0 + 16 * j) * W2P + 4 * kb + g], qv);
                f32x4 e1;
#pragma unroll
                for (int i = 0; i < 4; ++i) e1[i] = qv[i] * Pr[j][i];
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) W1r[rb][j] = xt_h(sf.XK, rb, e1, W1r[rb][j]);
                b1r[j] += tile::rows4_sum((e1[0] + e1[1]) + (e1[2] + e1[3]));
#pragma unroll
                for (int uu = 0; uu < 4; ++uu) W2r[j][uu] = ht_y(Ar[j], sf.E2, uu, W2r[j][uu]);
            }
            if (tid < D) {
                float cs = 0.f;
                for (int t = 0; t < RW; ++t) cs += sf.E2[t * DP + tid];
                b2r += cs;
            }
            tile::lds_barrier();  // every read of the W2 mirror is done
            put_state(wsq + static_cast<size_t>(ch + 1) * CK);
        }
    }

    if constexpr (MODE == PRE) {
        // ============ pre-pass: one chunk, everything independent of the adjoint ============
        const int ch = static_cast<int>(blockIdx.x % nch);
        const int m = min(mb, L - ch * mb);
        const float *S = wsq + static_cast<size_t>(ch) * CK;
        float *rc = recq + static_cast<size_t>(ch) * REC;
        for (int i = tid; i < RW * DP; i += NT) sm.accg[i] = sm.accb[i] = 0.f;
        if (tid < D) {
            sm.gam[tid] = gamma[h * D + tid];
            sm.bet[tid] = beta[h * D + tid];
        }
        if (rowt) {  // the chunk's rows into LDS: XQ, XK, XV - XK, dO and eta (zero past the end)
            Rows R;
            fetch_rows(ch, true, true, R);
#pragma unroll
            for (int k = 0; k < NF; ++k) {
                const int f = q + RW * k;
                const float xk = R.ok ? io::load(R.xk, k) : 0.f;
                sm.XK[r * DP + f] = xk;
                sm.tau[r * DP + f] = R.ok ? io::load(R.xv, k) - xk : 0.f;
                sm.XQ[r * DP + f] = R.ok ? io::load(R.xq, k) : 0.f;
                sm.dO[r * DP + f] = R.ok ? R.go[k] : 0.f;
            }
            if (q == 0) sm.eta[r] = R.ok ? R.et : 0.f;
        }
        tile::lds_barrier();

        // Z1 = XK W1 + b1 and XQ W1 + b1 on the own hidden tiles; T1 slices
        Frag fA;
        ld_vt(S, fA);  // W1 (stored transposed)
        issue();
        f32x4 Ar[2], Pr[2], Rr[2], ZQ[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float b = gld(S + OB1 + 32 * wu + 16 * j, c);
            f32x4 z = bcast(b), zq = bcast(b);
#pragma unroll
            for (int st = 0; st < D / 4; ++st) {
                const int k = 16 * (st >> 2) + 4 * g + (st & 3);
                z = mf(sm.XK[c * DP + k], fA[16 * j + st], z);
                zq = mf(sm.XQ[c * DP + k], fA[16 * j + st], zq);
            }
            ZQ[j] = zq;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float g0, g1, g2;
                gelu3(z[i], g0, g1, g2);
                Ar[j][i] = g0;
                Pr[j][i] = g1;
                Rr[j][i] = g2;
            }
            put_h(sm.HA, j, Ar[j]);
            put_rec(rc, HT_A, j, Ar[j]);
            put_rec(rc, HT_P, j, Pr[j]);
        }
        if (w < 4) {  // T1 slice over features 16w..16w+15
            f32x4 t4 = fz;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                t4 = mf(sm.XQ[c * DP + 16 * w + 4 * kb + g], sm.XK[c * DP + 16 * w + 4 * kb + g], t4);
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.gp[w][(4 * g + i) * TP + c] = t4[i];
        }
        tile::lds_barrier();

        // Z2 = A W2 + b2 (two halves);  T1 = tril(XQ XK^T + 1)
        Frag fW;  // W2 rows of this wave's hidden half, held for A W2 and Ab W2
        ld_v(S + OW2, fW);
        issue();
        put_d(sm.part[hh], mm_y(sm.HA, fW, hh == 0 ? bcast(gld(S + OB2 + 16 * u, c)) : fz));
        tri_sum(sm.T1, 4, 1.f, m);
        tile::lds_barrier();

        if (rowt) {  // E2 = -eta lnl2(Z2, XV - XK); the lnl2 values its reverse needs go to the record
            float z[NF], tau[NF], gm[NF], bt[NF];
            rowz2(sm.part[0], sm.part[1], z);
            rowld(sm.tau, DP, tau);
            rowld(sm.gam, 0, gm);
            rowld(sm.bet, 0, bt);
            const float et = sm.eta[r];
            Lnl2 s;
            lnl2(z, tau, gm, bt, s);
#pragma unroll
            for (int k = 0; k < NF; ++k) {
                sm.E2[r * DP + q + RW * k] = -et * s.G[k];
                gst(rc + rrow(RT_XH) + RW * k, lrq, s.xh[k]);
                gst(rc + rrow(RT_GH) + RW * k, lrq, s.gh[k]);
                gst(rc + rrow(RT_G) + RW * k, lrq, s.G[k]);
            }
            if (q == 0) {
                gst(rc + OS, r, s.sigma);
                gst(rc + OS + RW, r, s.c);
            }
        }
        tile::lds_barrier();

        // Q = E2 W2^T, E1 = Q * P;  Zb1 = XQ W1 + b1 + T1 E1, Ab = gelu(Zb1), Pb = gelu'(Zb1)
        f32x4 E1r[2], Abr[2], Pbr[2];
        Frag fT;  // W2^T of this wave's hidden units, held for E2 W2^T and dZb2 W2^T
        ld_vt(S + OW2, fT);
        issue();
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const f32x4 qv = mm_xt(sm.E2, fT, j, fz);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                E1r[j][i] = qv[i] * Pr[j][i];
                Rr[j][i] *= qv[i];  // Q * GELU''(Z1), the factor of dE1 in dZ1
            }
            put_h(sm.HE, j, E1r[j]);
            put_rec(rc, HT_E1, j, E1r[j]);
            put_rec(rc, HT_RQ, j, Rr[j]);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            f32x4 zb = ZQ[j];
#pragma unroll
            for (int i = 0; i < 4; ++i) zb = mf(sm.T1[c * TP + 4 * g + i], E1r[j][i], zb);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float g0, g1;
                gelu2(zb[i], g0, g1);
                Abr[j][i] = g0;
                Pbr[j][i] = g1;
            }
            put_h(sm.HY, j, Abr[j]);
            put_rec(rc, HT_AB, j, Abr[j]);
        }
        tile::lds_barrier();

        // Ab W2 + b2 (two halves); slices of the Gram Ab A^T over the own hidden units
        put_d(sm.part[hh], mm_y(sm.HY, fW, hh == 0 ? bcast(gld(S + OB2 + 16 * u, c)) : fz));
        {
            f32x4 t4 = fz;
#pragma unroll
            for (int kb = 0; kb < 8; ++kb)
                t4 = mf(sm.HY[c * MP + 32 * w + 4 * kb + g], sm.HA[c * MP + 32 * w + 4 * kb + g], t4);
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.gp[w][(4 * g + i) * TP + c] = t4[i];
        }
        tile::lds_barrier();
        tri_sum(sm.T2, NT / 64, 1.f, m);  // T2 = tril(Ab A^T + 1)
        tile::lds_barrier();

        if (rowt) {  // Zb2 = Ab W2 + b2 + T2 E2;  dZb2 = LN backward of dO
            float zb[NF];
            rowz2(sm.part[0], sm.part[1], zb);
#pragma unroll
            for (int s2 = 0; s2 < RW; ++s2) {
                const float tv = sm.T2[r * TP + s2];
#pragma unroll
                for (int k = 0; k < NF; ++k) zb[k] = fmaf(tv, sm.E2[s2 * DP + q + RW * k], zb[k]);
            }
            float s1 = 0.f, s2 = 0.f;
#pragma unroll
            for (int k = 0; k < NF; ++k) s1 += zb[k];
            const float mu = tile::row16_sum(s1) * inv_d;
#pragma unroll
            for (int k = 0; k < NF; ++k) s2 += (zb[k] - mu) * (zb[k] - mu);
            const float rs = 1.0f / sqrtf(tile::row16_sum(s2) * inv_d + eps);
            float xb[NF], dx[NF], go[NF], gm[NF], m1 = 0.f, m2 = 0.f;
            rowld(sm.dO, DP, go);
            rowld(sm.gam, 0, gm);
#pragma unroll
            for (int k = 0; k < NF; ++k) {
                const int o = r * DP + q + RW * k;
                xb[k] = (zb[k] - mu) * rs;
                dx[k] = gm[k] * go[k];
                sm.accg[o] = go[k] * xb[k];
                sm.accb[o] = go[k];
                m1 += dx[k];
                m2 += dx[k] * xb[k];
            }
            m1 = tile::row16_sum(m1) * inv_d;
            m2 = tile::row16_sum(m2) * inv_d;
#pragma unroll
            for (int k = 0; k < NF; ++k) {
                const float v = (dx[k] - m1 - xb[k] * m2) * rs;
                sm.dZb2[r * DP + q + RW * k] = v;
                gst(rc + rrow(RT_DZB2) + RW * k, lrq, v);
            }
        }
        tile::lds_barrier();

        // the chunk's share of dgamma, dbeta: the output layer norm's sums over its rows
        if (tid < D) {
            float a = 0.f, b = 0.f;
            for (int rr = 0; rr < RW; ++rr) {
                a += sm.accg[rr * DP + tid];
                b += sm.accb[rr * DP + tid];
            }
            gst(rc + OGB, tid, a);
            gst(rc + OGB + D, tid, b);
        }
        // dT2 = tril(dZb2 E2^T) (every wave its own copy, result layout: row t = 4g+i, column s = c)
        f32x4 dt2 = fz;
#pragma unroll
        for (int kb = 0; kb < D / 4; ++kb) dt2 = mf(sm.dZb2[c * DP + 4 * kb + g], sm.E2[c * DP + 4 * kb + g], dt2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (c > 4 * g + i) dt2[i] = 0.f;
            sm.gp[w][(4 * g + i) * TP + c] = dt2[i];
        }
        if (hh == 0) {  // T2^T dZb2, the adjoint-free part of dE2
            const f32x4 e = t_x(sm.T2, true, sm.dZb2, fz);
#pragma unroll
            for (int i = 0; i < 4; ++i) gst(rc + rrow(RT_T2Z) + i * D + 16 * u, lf, e[i]);
        }
        // dAb = dZb2 W2^T + dT2 A, dZb1 = dAb * Pb;  dT2^T Ab, the adjoint-free part of dA
        f32x4 dZb1r[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            f32x4 v = mm_xt(sm.dZb2, fT, j, fz);
#pragma unroll
            for (int i = 0; i < 4; ++i) v = mf(sm.gp[w][c * TP + 4 * g + i], Ar[j][i], v);
#pragma unroll
            for (int i = 0; i < 4; ++i) dZb1r[j][i] = v[i] * Pbr[j][i];
            put_h(sm.HX, j, dZb1r[j]);
            put_rec(rc, HT_DZB1, j, dZb1r[j]);
            f32x4 a = fz;
#pragma unroll
            for (int i = 0; i < 4; ++i) a = mf(dt2[i], Abr[j][i], a);
            put_rec(rc, HT_DAT, j, a);
        }
        tile::lds_barrier();

        // slices of dT1 = dZb1 E1^T over the own hidden units;  T1^T dZb1, the adjoint-free part of dE1
        {
            f32x4 t4 = fz;
#pragma unroll
            for (int kb = 0; kb < 8; ++kb)
                t4 = mf(sm.HX[c * MP + 32 * w + 4 * kb + g], sm.HE[c * MP + 32 * w + 4 * kb + g], t4);
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.gp[w][(4 * g + i) * TP + c] = t4[i];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) put_rec(rc, HT_TZ, j, tt_h(sm.T1, dZb1r[j], fz));
        ld_v(S, fA);  // W1 (stored transposed), for dZb1 W1^T
        issue();
        tile::lds_barrier();
        tri_sum(sm.dT1, NT / 64, 0.f, m);
        tile::lds_barrier();

        // dXQ = dO + dZb1 W1^T + dT1 XK (halves);  dT1^T XQ, the adjoint-free part of dXK
        {
            f32x4 aq = hh == 0 ? t_x(sm.dT1, false, sm.XK, fz) : fz;
            aq = mm_y(sm.HX, fA, aq);
            put_d(sm.part[hh], aq);
            if (hh == 0) put_d(sm.partE[0], t_x(sm.dT1, true, sm.XQ, fz));
        }
        tile::lds_barrier();
        for (int e = tid; e < RW * D; e += NT) {
            const int t = e / D, f = e % D;
            if (t < m) {
                const size_t at = xbase + static_cast<size_t>(ch * mb + t) * D + f;
                dXQ[at] = sm.part[0][t * DP + f] + sm.part[1][t * DP + f] + sm.dO[t * DP + f];
                dXK[at] = sm.partE[0][t * DP + f];
            }
        }
    }

    if constexpr (MODE == REV) {
        // ================= reverse sweep: the adjoint-dependent rest ==================
        // the adjoint of the final state: the caller's dW1', db1', dW2', db2' (zero if absent)
        float *a0 = adj(nch - 1);
        if (nch > 0) {
            for (int i = tid; i < D * M; i += NT) {
                a0[tix(i % M, i / M)] = dW1_out ? dW1_out[sq * D * M + i] : 0.f;
                a0[OW2 + tix(i / D, i % D)] = dW2_out ? dW2_out[sq * M * D + i] : 0.f;
            }
            if (tid < M) a0[OB1 + tid] = db1_out ? db1_out[sq * M + tid] : 0.f;
            if (tid < D) a0[OB2 + tid] = db2_out ? db2_out[sq * D + tid] : 0.f;
        } else {  // no tokens: the state passes through unchanged
            for (int i = tid; i < D * M; i += NT) {
                dW1[sq * D * M + i] = dW1_out ? dW1_out[sq * D * M + i] : 0.f;
                dW2[sq * M * D + i] = dW2_out ? dW2_out[sq * M * D + i] : 0.f;
            }
            if (tid < M) db1[sq * M + tid] = db1_out ? db1_out[sq * M + tid] : 0.f;
            if (tid < D) db2[sq * D + tid] = db2_out ? db2_out[sq * D + tid] : 0.f;
        }
        for (int i = tid; i < RW * DP; i += NT) sm.accg[i] = sm.accb[i] = 0.f;
        if (tid < D) {
            sm.gam[tid] = gamma[h * D + tid];
            sm.bet[tid] = beta[h * D + tid];
        }
        float accG = 0.f, accB = 0.f;  // the output layer norm's dgamma, dbeta from the records
        // A chunk's staged values, loaded during the previous chunk: two consecutive
        // features (f, f + 1) of token row t of the inputs, of the record's row tensors
        // and of the pre-pass's part of dXK, the row's eta, and sigma, c of row tid % 16.
        using pio = pair_io<TIO>;
        const int at_t = tid >> 5, at_f = 2 * (tid & 31);
        struct Ahead {
            typename pio::raw xq, xk, xv;
            tile::f32x2 xh, gh, G, dzb2, dxk;
            float et, sig, cc, pg, pb;
            f32x4 t2z;
            bool ok;
        };
        auto load_ahead = [&](int ch, Ahead &N) {
            const int mc = min(mb, L - ch * mb);
            N.ok = at_t < mc;
            const unsigned o = (N.ok ? at_t : 0) * D + at_f, orec = at_t * D + at_f;
            const size_t r0 = xbase + static_cast<size_t>(ch) * mb * D;
            const float *rc = recq + static_cast<size_t>(ch) * REC;
            N.xq = pio::ld(XQ + r0, o);
            N.xk = pio::ld(XK + r0, o);
            N.xv = pio::ld(XV + r0, o);
            N.xh = gld2(rc + rrow(RT_XH), orec);
            N.gh = gld2(rc + rrow(RT_GH), orec);
            N.G = gld2(rc + rrow(RT_G), orec);
            N.dzb2 = gld2(rc + rrow(RT_DZB2), orec);
            N.dxk = gld2(dXK + r0, o);
            N.et = gld(eta + sq * L + static_cast<size_t>(ch) * mb, N.ok ? at_t : 0);
            N.sig = gld(rc + OS, tid & (RW - 1));
            N.cc = gld(rc + OS + RW, tid & (RW - 1));
            // T2^T dZb2 in the tile layout of the dE2 partial (hidden half 0), the chunk's dgamma, dbeta share
#pragma unroll
            for (int i = 0; i < 4; ++i) N.t2z[i] = gld(rc + rrow(RT_T2Z) + i * D + 16 * u, lf);
            N.pg = gld(rc + OGB, tid & (D - 1));
            N.pb = gld(rc + OGB + D, tid & (D - 1));
        };
        // into LDS: XQ, XK, XV - XK, E2 = -eta G2, dZb2, the lnl2 rows, eta, sigma, c, the dXK part
        // (inputs and eta zero on rows past the chunk)
        auto stage_ahead = [&](const Ahead &N) {
            const int o = at_t * DP + at_f;
            const float et = N.ok ? N.et : 0.f;
            const float q0 = N.ok ? pio::lo(N.xq) : 0.f, q1 = N.ok ? pio::hi(N.xq) : 0.f;
            const float k0 = N.ok ? pio::lo(N.xk) : 0.f, k1 = N.ok ? pio::hi(N.xk) : 0.f;
            const float v0 = N.ok ? pio::lo(N.xv) : 0.f, v1 = N.ok ? pio::hi(N.xv) : 0.f;
            sm.XQ[o] = q0;
            sm.XQ[o + 1] = q1;
            sm.XK[o] = k0;
            sm.XK[o + 1] = k1;
            sm.tau[o] = v0 - k0;
            sm.tau[o + 1] = v1 - k1;
            sm.lxh[o] = N.xh[0];
            sm.lxh[o + 1] = N.xh[1];
            sm.lgh[o] = N.gh[0];
            sm.lgh[o + 1] = N.gh[1];
            sm.lG[o] = N.G[0];
            sm.lG[o + 1] = N.G[1];
            sm.E2[o] = -et * N.G[0];
            sm.E2[o + 1] = -et * N.G[1];
            sm.dZb2[o] = N.dzb2[0];
            sm.dZb2[o + 1] = N.dzb2[1];
            sm.part[0][o] = N.dxk[0];
            sm.part[0][o + 1] = N.dxk[1];
            if ((tid & 31) == 0) sm.eta[at_t] = et;
            if (tid < RW) {
                sm.lsig[tid] = N.sig;
                sm.lcc[tid] = N.cc;
            }
        };
        Frag fA, fB, fW;
        Ahead N;
        if (nch > 0) load_ahead(nch - 1, N);
        for (int ch = nch - 1; ch >= 0; --ch) {
            const int m = min(mb, L - ch * mb);
            const bool ok = r < m;
            const float *S = wsq + static_cast<size_t>(ch) * CK;
            const float *rc = recq + static_cast<size_t>(ch) * REC;
            const float *Ad = adj(ch);  // adjoint of this chunk's end state
            float *dst1 = adj(ch + 1);  // adjoint of this chunk's start state
            float *dstb1 = dst1 + OB1, *dst2 = dst1 + OW2, *dstb2 = dst1 + OB2;
            __syncthreads();  // the previous chunk is done with every tile and its adjoint writes
            stage_ahead(N);
            // the record's hidden tiles of the first phases (own tiles of this wave)
            f32x4 Ar[2], Pr[2], Rr[2], TZr[2], E1r[2], Abr[2], dZb1r[2], dAr[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                TZr[j] = get_rec(rc, HT_TZ, j);
                Pr[j] = get_rec(rc, HT_P, j);
                Rr[j] = get_rec(rc, HT_RQ, j);
                Ar[j] = get_rec(rc, HT_A, j);
                E1r[j] = get_rec(rc, HT_E1, j);
            }
            const f32x4 t2z = N.t2z;
            if (tid < D) {
                accG += N.pg;
                accB += N.pb;
            }
            ld_vt(Ad, fA);  // dW1' (transposed)
            const float db1v[2] = {gld(Ad + OB1 + 32 * wu, c), gld(Ad + OB1 + 32 * wu + 16, c)};
            const float db2v = tid < D ? gld(Ad, OB2 + tid) : 0.f;
            const float db2u = gld(Ad + OB2 + 16 * u, c);  // db2' of this wave's feature tile
            issue();
            tile::lds_barrier();

            // dE1 = T1^T dZb1 + XK dW1' + db1' (zero on rows past the chunk), dQ = dE1 * P;
            // A and E1 into LDS for the products over the hidden units
            f32x4 dQr[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                f32x4 de = mm_xt(sm.XK, fA, j, bcast(db1v[j]));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = 4 * g + i < m ? de[i] + TZr[j][i] : 0.f;
                    dQr[j][i] = v * Pr[j][i];
                    Rr[j][i] *= v;  // dE1 * Q * GELU''(Z1)
                }
                put_h(sm.HY, j, dQr[j]);
                put_h(sm.HA, j, Ar[j]);
                put_h(sm.HE, j, E1r[j]);
            }
            ld_v(Ad + OW2, fB);  // dW2'
            ld_v(S + OW2, fW);   // W2
            issue();
            tile::lds_barrier();

            // dE2 = T2^T dZb2 + db2' + A dW2' + dQ W2 (two halves)
            {
                f32x4 e = hh == 0 ? t2z + bcast(db2u) : fz;
                e = mm_y(sm.HA, fB, e);
                e = mm_y(sm.HY, fW, e);
                put_d(sm.partE[hh], e);
            }
            ld_vt(Ad + OW2, fA);  // dW2' (transposed)
            ld_vt(S + OW2, fB);   // W2^T
#pragma unroll
            for (int j = 0; j < 2; ++j) {  // the record's tiles for dA and the adjoint-state update
                dAr[j] = get_rec(rc, HT_DAT, j);
                Abr[j] = get_rec(rc, HT_AB, j);
                dZb1r[j] = get_rec(rc, HT_DZB1, j);
            }
            issue();
            tile::lds_barrier();

            if (rowt) {  // deta = -G2 . dE2;  dG2 = -eta dE2;  reverse of lnl2 -> dZ2, dtau
                float de[NF], gm[NF], bt[NF], lxh[NF], lgh[NF], lG[NF], tau[NF];
                rowz2(sm.partE[0], sm.partE[1], de);
                rowld(sm.gam, 0, gm);
                rowld(sm.bet, 0, bt);
                rowld(sm.lxh, DP, lxh);
                rowld(sm.lgh, DP, lgh);
                rowld(sm.lG, DP, lG);
                rowld(sm.tau, DP, tau);
                const float et = sm.eta[r], l_sigma = sm.lsig[r], l_c = sm.lcc[r];
                float pe = 0.f;
#pragma unroll
                for (int k = 0; k < NF; ++k) pe = fmaf(lG[k], de[k], pe);
                const float d_eta = -tile::row16_sum(pe);
                float dG[NF], mdg = 0.f, mdgx = 0.f, sgG = 0.f;
#pragma unroll
                for (int k = 0; k < NF; ++k) {
                    dG[k] = -et * de[k];
                    mdg += dG[k];
                    mdgx += dG[k] * lxh[k];
                    sgG += dG[k] * lG[k];
                }
                mdg = tile::row16_sum(mdg) * inv_d;
                mdgx = tile::row16_sum(mdgx) * inv_d;
                const float rs = 1.0f / l_sigma;
                const float dsig = -tile::row16_sum(sgG) * rs;
                float dxh[NF], mdx = 0.f, mdxx = 0.f;
#pragma unroll
                for (int k = 0; k < NF; ++k) {
                    const int o = r * DP + q + RW * k;
                    const float dgh = (dG[k] - mdg - lxh[k] * mdgx) * rs;
                    dxh[k] = gm[k] * gm[k] * dgh - (l_c * dG[k] + lgh[k] * mdgx) * rs;
                    sm.dtau[o] = ok ? -gm[k] * dgh : 0.f;
                    sm.accg[o] = fmaf(dgh, fmaf(2.f * gm[k], lxh[k], bt[k] - tau[k]), sm.accg[o]);
                    sm.accb[o] = fmaf(gm[k], dgh, sm.accb[o]);
                    mdx += dxh[k];
                    mdxx += dxh[k] * lxh[k];
                }
                mdx = tile::row16_sum(mdx) * inv_d;
                mdxx = tile::row16_sum(mdxx) * inv_d;
#pragma unroll
                for (int k = 0; k < NF; ++k) {
                    const float dz = fmaf(dsig * inv_d, lxh[k], (dxh[k] - mdx - lxh[k] * mdxx) * rs);
                    sm.dZ2[r * DP + q + RW * k] = ok ? dz : 0.f;
                }
                if (ok && q == 0) gst(deta + sq * L + static_cast<size_t>(ch) * mb, r, d_eta);
            }
            tile::lds_barrier();

            // dA = dT2^T Ab + E2 dW2'^T + dZ2 W2^T;  dZ1 = dA * P + dE1 * Q * GELU'';
            // the adjoint state of the chunk start: dW2, dW1, db1, db2
            f32x4 dZ1r[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                f32x4 a = mm_xt(sm.E2, fA, j, dAr[j]);
                a = mm_xt(sm.dZ2, fB, j, a);
#pragma unroll
                for (int i = 0; i < 4; ++i) dZ1r[j][i] = fmaf(a[i], Pr[j][i], Rr[j][i]);
                put_h(sm.HY, j, dZ1r[j]);
            }
            // the dW1' tiles, read while the dW2 tiles are formed (layout of ld_vt)
            ld_vt(Ad, fB);
            issue();
            // dW2 = dW2' + Ab^T dZb2 + dQ^T E2 + A^T dZ2, accumulated transposed: a lane holds
            // four consecutive features of one hidden unit's row of dW2 -- the layout of the
            // dW2'^T fragment, which therefore starts each accumulator
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    f32x4 acc = {fA[16 * j + 4 * rb], fA[16 * j + 4 * rb + 1], fA[16 * j + 4 * rb + 2],
                                 fA[16 * j + 4 * rb + 3]};
                    acc = xt_h(sm.dZb2, rb, Abr[j], acc);
                    acc = xt_h(sm.E2, rb, dQr[j], acc);
                    acc = xt_h(sm.dZ2, rb, Ar[j], acc);
                    gst4(dst2 + (2 * wu + j) * 1024 + 256 * rb, lg, acc);
                }
            ld_v(S, fA);  // W1 (stored transposed), for dZ1 W1^T
            issue();
            // dW1 = dW1' + XQ^T dZb1 + XK^T dZ1: four consecutive features of one hidden unit's
            // row of the transposed dW1
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    f32x4 acc = {fB[16 * j + 4 * rb], fB[16 * j + 4 * rb + 1], fB[16 * j + 4 * rb + 2],
                                 fB[16 * j + 4 * rb + 3]};
                    acc = xt_h(sm.XQ, rb, dZb1r[j], acc);
                    acc = xt_h(sm.XK, rb, dZ1r[j], acc);
                    gst4(dst1 + (2 * wu + j) * 1024 + 256 * rb, lg, acc);
                }
                const float cs = tile::rows4_sum((dZb1r[j][0] + dZ1r[j][0]) + (dZb1r[j][1] + dZ1r[j][1]) +
                                                 ((dZb1r[j][2] + dZ1r[j][2]) + (dZb1r[j][3] + dZ1r[j][3])));
                if (g == 0) gst(dstb1 + 32 * wu + 16 * j, c, db1v[j] + cs);
            }
            if (tid < D) {
                float cs = 0.f;
                for (int t = 0; t < RW; ++t) cs += sm.dZb2[t * DP + tid] + sm.dZ2[t * DP + tid];
                gst(dstb2, tid, db2v + cs);
            }
            ld_v(Ad, fB);  // dW1' (transposed), for E1 dW1'^T
            load_ahead(max(ch - 1, 0), N);  // unconditional: the last chunk reloads chunk 0
            issue();
            tile::lds_barrier();

            // dXK = dT1^T XQ + E1 dW1'^T + dZ1 W1^T - dtau (halves);  dXV = dtau
            put_d(sm.partE[hh], mm_y(sm.HE, fB, mm_y(sm.HY, fA, fz)));
            tile::lds_barrier();
            {
                float *const oK = dXK + xbase + static_cast<size_t>(ch) * mb * D;
                float *const oV = dXV + xbase + static_cast<size_t>(ch) * mb * D;
                for (int e = tid; e < RW * D; e += NT) {
                    const int t = e / D, f = e % D;
                    if (t < m) {
                        const float dt = sm.dtau[t * DP + f];
                        gst(oK, e, sm.part[0][t * DP + f] + sm.partE[0][t * DP + f] + sm.partE[1][t * DP + f] - dt);
                        gst(oV, e, dt);
                    }
                }
            }
        }
        __syncthreads();
        if (nch > 0) {  // the adjoint of the initial state, from the workspace to the outputs
            const float *a = adj(1);
            for (int i = tid; i < D * M; i += NT) {
                dW1[sq * D * M + i] = a[tix(i % M, i / M)];
                dW2[sq * M * D + i] = a[OW2 + tix(i / D, i % D)];
            }
            if (tid < M) db1[sq * M + tid] = a[OB1 + tid];
            if (tid < D) db2[sq * D + tid] = a[OB2 + tid];
        }

        // per-sequence dgamma, dbeta: the 16 row groups of the lnl2 reverse plus the output norm's share
        if (tid < D) {
            float a = accG, b = accB;
            for (int rr = 0; rr < RW; ++rr) {
                a += sm.accg[rr * DP + tid];
                b += sm.accb[rr * DP + tid];
            }
            dgamma[sq * D + tid] = a;
            dbeta[sq * D + tid] = b;
        }
    }
}

template <typename TIO, int MODE>
hipError_t launch_mode(const MLPBwdArgs &a, unsigned grid, hipStream_t stream) {
    hipLaunchKernelGGL((mlp_backward_kernel<TIO, MODE>), dim3(grid), dim3(NT), 0, stream, a.f.B * a.f.H, a.f.H,
                       a.f.L, a.f.mb, a.f.eps, static_cast<const TIO *>(a.f.XQ), static_cast<const TIO *>(a.f.XK),
                       static_cast<const TIO *>(a.f.XV), a.f.eta, a.f.W1, a.f.b1, a.f.W2, a.f.b2,
                       a.f.w0_batched, a.f.gamma, a.f.beta, a.dO, a.dW1_out, a.db1_out, a.dW2_out,
                       a.db2_out, a.dXQ, a.dXK, a.dXV, a.deta, a.dW1, a.db1, a.dW2, a.db2, a.dgamma,
                       a.dbeta, a.ws);
    return hipGetLastError();
}

template <typename TIO>
hipError_t launch_t(const MLPBwdArgs &a, hipStream_t stream) {
    const size_t nseq = static_cast<size_t>(a.f.B) * a.f.H;
    const size_t nch = a.f.L > 0 ? static_cast<size_t>((a.f.L + a.f.mb - 1) / a.f.mb) : 0;
    if (nseq * nch > 0x7fffffffu) return hipErrorInvalidValue;
    hipError_t e;
    if (nch > 0) {
        if ((e = launch_mode<TIO, FWD>(a, static_cast<unsigned>(nseq), stream)) != hipSuccess) return e;
        if ((e = launch_mode<TIO, PRE>(a, static_cast<unsigned>(nseq * nch), stream)) != hipSuccess) return e;
    }
    return launch_mode<TIO, REV>(a, static_cast<unsigned>(nseq), stream);
}

}  // namespace

size_t mlp_backward_seq_floats(int L, int d, int mb) {
    if (d != D) return 0;
    const size_t nch = L > 0 ? static_cast<size_t>((L + mb - 1) / mb) : 0;
    return (nch + 2) * CK + nch * REC;
}

hipError_t launch_mlp_backward(const MLPBwdArgs &a, hipStream_t stream) {
    if (a.f.B * a.f.H == 0) return hipSuccess;
    if (a.f.d != D) return hipErrorInvalidValue;
    return a.f.io ? launch_t<bf16_t>(a, stream) : launch_t<float>(a, stream);
}

}  // namespace ttt
