// TTT-MLP prefill, MFMA path: bf16 storage, d = 64, hidden m = 4d = 256,
// mini-batch b = 16. The hidden model d -> 4d GELU -> d inside the LN
// residual is the one of the lryc.cn TTT article §2.1; the inner loop is the
// dual form of the damodev.csdn.net TTT deep-dive §4.2 applied to both layers.
//
// Per chunk (state W1, b1, W2, b2 at chunk start; E = -eta * G row-scaled):
//   Z1 = XK W1 + b1, A = gelu(Z1), Z2 = A W2 + b2, E2 = -eta lnbwd(Z2, XV - XK)
//   E1 = (E2 W2^T) * gelu'(Z1)
//   Zb1 = XQ W1 + b1 + T1 E1,   T1 = tril(XQ XK^T + 1),   Ab = gelu(Zb1)
//   Zb2 = Ab W2 + b2 + T2 E2,   T2 = tril(Ab A^T + 1),    O = XQ + LN(Zb2)
//   W1 += XK^T E1, b1 += 1^T E1, W2 += A^T E2, b2 += 1^T E2
// Modular-TTT options (template): LOSS = 1 takes E2 from the inner-product
// loss -< XK + LN(Z2), XV > (the staged row holds XV itself); DECAY adds
// lambda/2 (||W1||^2 + ||W2||^2) at the chunk-start state, which makes the
// weights after token t equal to d_t W + (loss updates) with
// d_t = 1 - lambda sum_{s<=t} eta_s: XQ W1 and Ab W2 take the factor d_t of
// their token and the chunk ends with W1, W2 scaled by d_15 (biases are not
// decayed).
// GATED (template): each token's rate is formed while its chunk is staged,
// eta_t = eta_base * logistic(theta_lr[h] . XK_t) (the learning-rate gate of
// the lryc.cn TTT article §2.2, x read as the key), and no eta array is read.
//
// Layout (gfx950, one 512-thread workgroup = 8 waves per (n,h) sequence, two
// per SIMD):
//  * wave w owns hidden units 32w .. 32w+31 (two hidden tiles t of 16). Its
//    share of the fp32 state lives in registers as MFMA accumulators, each in
//    the output layout of its own update (lane (g, c) holds rows 4g .. 4g+3 of
//    column c):
//      W1v[t][rb] = W1[in 16rb + 4g + i][hid 32w + 16t + c]    (XK^T E1)
//      b1v[t]     = b1[hid 32w + 16t + 4g + i]                 (E1^T 1)
//      W2v[u][rb] = W2[hid 32w + 16rb + 4g + i][out 16u + c]   (A^T E2)
//      b2w        = b2[out 16w + c]   (waves 0-3)               (1^T E2)
//    With the contraction index permuted identically on both operands these
//    are also the operand layouts of the forward products, so no product
//    reads the state through LDS. W2 is contracted over hidden units (A W2)
//    and over outputs (E2 W2^T); for the latter its fp16 tiles are transposed
//    each chunk by MFMAs with the identity.
//  * Z1 and Zb1 are computed transposed (hidden as the output row), so their
//    GELU outputs are directly the A operands of A W2 and Ab W2; A and E1 are
//    transposed by identity MFMAs for the token-contracting updates.
//  * contractions over all 256 hidden units (Z2 and Zb2) are summed across
//    the eight waves through LDS. T2 E2 needs no sum of its own: masking is
//    linear, so each wave adds tril(Ab_w A_w^T) E2 over its own hidden units
//    to its Zb2 partial (and wave 0 the tril(1) E2 term).
//  * row-layout work (16 lanes per token, DPP reductions): waves 0-3 run the
//    LN backward (Z2 -> E2) and load the input rows of their four tokens one
//    chunk ahead, staging a chunk into LDS a full iteration after its loads
//    were issued. Waves 4-7 emit O = XQ + LN(Zb2) of a chunk during the next
//    chunk's first phase, from Zb2 partials kept in a buffer of their own;
//    three LDS slots hold the previous chunk (its XQ rows for O), the current
//    one and the next. Three barriers per chunk.
//  * GELU: x Phi(x) with erf from Abramowitz & Stegun 7.1.26 (|error| <=
//    1.5e-7, far below the resolution of the MFMA operands); GELU and its
//    derivative share one exponential.
//  * precision: every MFMA takes fp16 operands (10-bit mantissa) and
//    accumulates in fp32. W1 and W2 grow along the sequence while a 16-bit
//    operand's rounding stays relative, so bf16 operands (7-bit mantissa)
//    would dominate the error. The bf16 inputs convert exactly above 2^-14;
//    the state, activations, E1, E2 and the Grams T1, T2 stay far below the
//    fp16 limit of 65504, and E values below 2^-14 keep an absolute
//    resolution of 2^-24. The transposes (identity MFMAs) add no rounding.
#include "launch.hpp"
#include "tile.hpp"

namespace ttt {
namespace {

using namespace tile;

constexpr int M = 4 * D;     // hidden units
constexpr int NW = 8, NT = 64 * NW;
constexpr int NRW = 4;       // waves running the row-layout work (16 tokens x 16 lanes)

struct alignas(16) MlpSmem {
    Slot slot[3];                          // chunks c - 1 (its XQ rows for O), c, c + 1
    alignas(16) float part[NW][MB * RS];   // per-wave partial sums of Z2
    alignas(16) float partb[NW][MB * RS];  // per-wave partial sums of Zb2 (read one chunk later)
    alignas(16) uint16_t e2[MB * RS];         // E2, fp16 rows [token][out]
    alignas(16) uint16_t e2t[D * KS];         // E2 transposed, fp16 [out][token]
};

// E = -eta * G for one row (row layout) under the selected loss. LOSS = 0 is
// the squared reconstruction error (tau = XV - XK); LOSS = 1 the inner product
// -< LN(z), v > with tau = v, whose gradient through the layer norm is
// G = rstd (ghat - mean(ghat) - xhat mean(ghat xhat)), ghat = -gamma v; with
// gamma = 1 this is a (z - mu) - rstd (v - mean v), a = rstd^3 mean(v (z - mu)).
template <bool IDENT, int LOSS>
__device__ __forceinline__ f32x4 row_grad(f32x4 z, f32x4 tau, float mutau, float eta_r,
                                          const float (&gam)[4], const float (&bet)[4],
                                          float eps) {
    if constexpr (LOSS == 0) {
        return ln_bwd_row<IDENT>(z, tau, mutau, eta_r, gam, bet, eps);
    } else {
        constexpr float inv_d = 1.0f / D;
        f32x4 ev;
        if constexpr (IDENT) {  // mean first, then centred sums (no E[z^2] - mu^2 cancellation)
            const float mu = row16_sum((z[0] + z[1]) + (z[2] + z[3])) * inv_d;
            f32x4 cz;
#pragma unroll
            for (int e = 0; e < 4; ++e) cz[e] = z[e] - mu;
            const float s2 = row16_sum(fmaf(cz[0], cz[0], cz[1] * cz[1]) + fmaf(cz[2], cz[2], cz[3] * cz[3]));
            const float s3 = row16_sum(fmaf(tau[0], cz[0], tau[1] * cz[1]) + fmaf(tau[2], cz[2], tau[3] * cz[3]));
            const float rstd = rsqrtf(s2 * inv_d + eps);
            const float a = rstd * rstd * rstd * (s3 * inv_d);
            const float ca = -eta_r * a, ct = eta_r * rstd;
#pragma unroll
            for (int e = 0; e < 4; ++e) ev[e] = fmaf(ca, cz[e], ct * (tau[e] - mutau));
        } else {
            const float mu = row16_sum((z[0] + z[1]) + (z[2] + z[3])) * inv_d;
            float cz[4], s2 = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                cz[e] = z[e] - mu;
                s2 += cz[e] * cz[e];
            }
            const float rstd = rsqrtf(row16_sum(s2) * inv_d + eps);
            float xh[4], gh[4], a1 = 0.f, a2 = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xh[e] = cz[e] * rstd;
                gh[e] = -gam[e] * tau[e];
                a1 += gh[e];
                a2 += gh[e] * xh[e];
            }
            const float m1 = row16_sum(a1) * inv_d, m2 = row16_sum(a2) * inv_d;
            const float ne = -eta_r * rstd;
#pragma unroll
            for (int e = 0; e < 4; ++e) ev[e] = ne * (gh[e] - m1 - xh[e] * m2);
        }
        return ev;
    }
}

static_assert(sizeof(MlpSmem) <= 160 * 1024, "MLP prefill LDS exceeds 160 KB");

}  // namespace

template <int LOSS, bool DECAY, bool GATED>
__global__ __launch_bounds__(NT) void mlp_prefill_mfma(
    int H, int L, float eps, const bf16_t *__restrict__ XQ, const bf16_t *__restrict__ XK,
    const bf16_t *__restrict__ XV, const float *__restrict__ eta,
    const float *W1_0, const float *b1_0, const float *W2_0, const float *b2_0,
    int w0_batched,
    const float *__restrict__ gamma, const float *__restrict__ beta, bf16_t *__restrict__ O,
    float *W1_out, float *b1_out, float *W2_out, float *b2_out, float wd,
    const float *__restrict__ theta, float eta_base) {
    __shared__ MlpSmem sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, g = lane >> 4, c = lane & 15;
    const long seq = blockIdx.x;
    const int h = static_cast<int>(seq % H);
    const long n = seq / H;
    const size_t st = w0_batched ? static_cast<size_t>(n) * H + h : static_cast<size_t>(h);
    const size_t xbase = static_cast<size_t>(seq) * L * D;
    const int nch = (L + MB - 1) / MB;
    const int hw = 32 * w;        // first hidden unit of this wave
    const bool roww = w < NRW;    // runs the row-layout work

    // ---- state (this wave's share) -------------------------------------------
    f32x4 W1v[2][4], W2v[4][2], b1v[2], b2w;
    {
        const float *W1s = W1_0 + st * D * M, *W2s = W2_0 + st * M * D;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) W1v[t][rb][i] = W1s[(16 * rb + 4 * g + i) * M + hw + 16 * t + c];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) W2v[u][rb][i] = W2s[(hw + 16 * rb + 4 * g + i) * D + 16 * u + c];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) b1v[t][i] = b1_0[st * M + hw + 16 * t + 4 * g + i];
        // b2 tile w (columns 16w .. 16w+15), held by waves 0-3 only
        const float bb = b2_0[st * D + 16 * (w & 3) + c];
        b2w = f32x4{bb, bb, bb, bb};
    }
    // row layout (waves 0-3): token r, features f0 .. f0+3
    const int r = 4 * (w & 3) + g, f0 = 4 * c;
    float gam[4], bet[4];
    bool ident = true;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        gam[e] = gamma[static_cast<size_t>(h) * D + f0 + e];
        bet[e] = beta[static_cast<size_t>(h) * D + f0 + e];
        ident = ident && gam[e] == 1.0f && bet[e] == 0.0f;
    }
    ident = __all(ident);  // every wave covers all 64 features: same vote everywhere

    const s16x4 ones = {0x3C00, 0x3C00, 0x3C00, 0x3C00};  // fp16 1.0
    s16x4 eye;  // identity as a B operand: B[k = 4g + i][n = c] (fp16)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        eye[i] = (4 * g + i == c) ? 0x3C00 : 0;
    }
    const f32x4 fzero = {0.f, 0.f, 0.f, 0.f};
    f32x4 tmask;
#pragma unroll
    for (int i = 0; i < 4; ++i) tmask[i] = (4 * g + i <= c) ? 1.f : 0.f;

    // ---- input rows of this lane's token, one chunk ahead (waves 0-3) --------
    const bf16_t *xq = XQ + xbase, *xk = XK + xbase, *xv = XV + xbase;
    const float *et = eta + static_cast<size_t>(seq) * L;
    PrepRegs R;
    auto load = [&](int ch) {
        const int tok = min(ch * MB + r, L - 1);
        const size_t off = static_cast<size_t>(tok) * D + f0;
        R.q = *reinterpret_cast<const uint2 *>(xq + off);
        R.k = *reinterpret_cast<const uint2 *>(xk + off);
        R.v = *reinterpret_cast<const uint2 *>(xv + off);
        if constexpr (!GATED) R.eta = et[tok];
    };
    // learning-rate gate: the dot product theta . XK_t split over the 16 lanes
    // of the token's row; exp2 and reciprocal are the hardware approximations
    f32x4 thv = {0.f, 0.f, 0.f, 0.f};  // -theta * log2(e) for features f0 .. f0+3
    if constexpr (GATED)
        thv = *reinterpret_cast<const f32x4 *>(theta + static_cast<size_t>(h) * D + f0) * -1.4426950408889634f;
    auto stage = [&](int ch) {
        Slot &S = sm.slot[ch % 3];
        const bool ok = ch * MB + r < L;
        const uint2 z2 = make_uint2(0u, 0u);
        const uint2 q = ok ? R.q : z2, k = ok ? R.k : z2, v = ok ? R.v : z2;
        const f32x4 qf = unpack4(q), kf = unpack4(k);
        const uint2 kh = make_uint2(pack2h(kf[0], kf[1]), pack2h(kf[2], kf[3]));
        *reinterpret_cast<uint2 *>(&S.xq[r * RS + f0]) = make_uint2(pack2h(qf[0], qf[1]), pack2h(qf[2], qf[3]));
        *reinterpret_cast<uint2 *>(&S.xk[r * RS + f0]) = kh;
        S.xkt[(f0 + 0) * KS + r] = static_cast<uint16_t>(kh.x & 0xffffu);
        S.xkt[(f0 + 1) * KS + r] = static_cast<uint16_t>(kh.x >> 16);
        S.xkt[(f0 + 2) * KS + r] = static_cast<uint16_t>(kh.y & 0xffffu);
        S.xkt[(f0 + 3) * KS + r] = static_cast<uint16_t>(kh.y >> 16);
        *reinterpret_cast<f32x4 *>(&S.xqf[r * RS + f0]) = qf;
        const f32x4 tau = LOSS == 1 ? unpack4(v) : unpack4(v) - kf;
        *reinterpret_cast<f32x4 *>(&S.tau[r * RS + f0]) = tau;
        const float mt = row16_sum((tau[0] + tau[1]) + (tau[2] + tau[3])) * (1.0f / D);
        float e;
        if constexpr (GATED) {
            const float ns = row16_sum(fmaf(thv[0], kf[0], thv[1] * kf[1]) + fmaf(thv[2], kf[2], thv[3] * kf[3]));
            e = eta_base * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(ns));
        } else {
            e = R.eta;
        }
        if (c == 0) {
            S.mutau[r] = mt;
            S.eta[r] = ok ? e : 0.f;
        }
    };
    if (roww && nch > 0) {
        load(0);
        stage(0);
        load(1);
    }
    lds_barrier();

    // O = XQ + LN(Zb2) of chunk ch from the Zb2 partials (row layout; waves 4-7)
    auto emit_out = [&](int ch) {
        const Slot &Sp = sm.slot[ch % 3];
        f32x4 zb2 = *reinterpret_cast<const f32x4 *>(&sm.partb[0][r * RS + f0]);
#pragma unroll
        for (int q = 1; q < NW; ++q) zb2 += *reinterpret_cast<const f32x4 *>(&sm.partb[q][r * RS + f0]);
        const f32x4 xqv = *reinterpret_cast<const f32x4 *>(&Sp.xqf[r * RS + f0]);
        const f32x4 o = ident ? ln_fwd_row<true>(zb2, xqv, gam, bet, eps)
                              : ln_fwd_row<false>(zb2, xqv, gam, bet, eps);
        if (ch * MB + r < L)
            *reinterpret_cast<uint2 *>(O + xbase + static_cast<size_t>(ch * MB + r) * D + f0) =
                make_uint2(pack2(o[0], o[1]), pack2(o[2], o[3]));
    };

    auto w1frag = [&](int t, int kb) { return pack8h(W1v[t][2 * kb], W1v[t][2 * kb + 1]); };
    auto rowh = [&](const uint16_t *tile, int kb) { return __builtin_bit_cast(f16x8, row_frag(tile, c, g, kb)); };

    for (int ch = 0; ch < nch; ++ch) {
        const Slot &S = sm.slot[ch % 3];
        float *P = sm.part[w] + (4 * g) * RS + c;

        // ===== A: Z1^T, A = gelu(Z1), Z2 partials, T1, A transposed ============
        // Row work beside it: waves 0-3 stage the next chunk (its slot last
        // served chunk ch - 2) and load the one after; waves 4-7 emit O of the
        // previous chunk from the Zb2 partials of phase C.
        if (roww) {
            if (ch + 1 < nch) {
                stage(ch + 1);
                load(ch + 2);
            }
        } else if (ch > 0) {
            emit_out(ch - 1);
        }
        // decay: dc = d_t of this lane's token column c, alpha = d_15
        float dc = 1.f, alpha = 1.f;
        if constexpr (DECAY) {
            float run = 0.f, cum = 0.f;
#pragma unroll
            for (int s = 0; s < MB; ++s) {
                run += S.eta[s];
                cum = s == c ? run : cum;
            }
            dc = fmaf(-wd, cum, 1.f);
            alpha = fmaf(-wd, run, 1.f);
        }
        f16x8 xkf[2], xqf[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            xkf[kb] = rowh(S.xk, kb);
            xqf[kb] = rowh(S.xq, kb);
        }
        f32x4 Aact[2], Ap[2], zq[2];  // [hid 16t + 4g + i][token c]
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const f16x8 wa = w1frag(t, 0), wb = w1frag(t, 1);
            f32x4 z = mfma32h(wa, xkf[0], b1v[t]);
            z = mfma32h(wb, xkf[1], z);
            if constexpr (DECAY) {  // (d_t XQ W1 + b1)^T
                const f32x4 p = mfma32h(wb, xqf[1], mfma32h(wa, xqf[0], fzero));
#pragma unroll
                for (int i = 0; i < 4; ++i) zq[t][i] = fmaf(dc, p[i], b1v[t][i]);
            } else {
                zq[t] = mfma32h(wb, xqf[1], mfma32h(wa, xqf[0], b1v[t]));  // (XQ W1 + b1)^T
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float Phi, phi;
                normal_cdf_pdf(z[i], Phi, phi);
                Aact[t][i] = z[i] * Phi;
                Ap[t][i] = fmaf(z[i], phi, Phi);
            }
        }
        const f16x8 Af = pack8h(Aact[0], Aact[1]);  // A operand [m = token c][k = this wave's hidden]
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            // chunk-start W2 as B operand [k = hidden][n = out]; b2 tile u added by wave u
            const f32x4 acc = mfma32h(Af, pack8h(W2v[u][0], W2v[u][1]), w == u ? b2w : fzero);
#pragma unroll
            for (int i = 0; i < 4; ++i) P[i * RS + 16 * u] = acc[i];
        }
        f32x4 gt = fzero;  // [s = 4g+i][t = c] = XQ_t . XK_s
        gt = mfma32h(xkf[0], xqf[0], gt);
        gt = mfma32h(xkf[1], xqf[1], gt);
        f32x4 tv;
#pragma unroll
        for (int i = 0; i < 4; ++i) tv[i] = fmaf(gt[i], tmask[i], tmask[i]);
        const s16x4 T1b = pack4h(tv);  // T1^T as a B operand: [k = s][n = t]
        s16x4 Atr[2];                 // A[token 4g+i][hid 16t + c]
#pragma unroll
        for (int t = 0; t < 2; ++t) Atr[t] = pack4h(mfma16h(pack4h(Aact[t]), eye, fzero));
        lds_barrier();

        // ===== B (row layout): Z2 -> E2 =====================================
        if (roww) {
            f32x4 z2 = *reinterpret_cast<const f32x4 *>(&sm.part[0][r * RS + f0]);
#pragma unroll
            for (int q = 1; q < NW; ++q) z2 += *reinterpret_cast<const f32x4 *>(&sm.part[q][r * RS + f0]);
            const f32x4 tau = *reinterpret_cast<const f32x4 *>(&S.tau[r * RS + f0]);
            const f32x4 ev = ident ? row_grad<true, LOSS>(z2, tau, S.mutau[r], S.eta[r], gam, bet, eps)
                                   : row_grad<false, LOSS>(z2, tau, S.mutau[r], S.eta[r], gam, bet, eps);
            const uint32_t p01 = pack2h(ev[0], ev[1]), p23 = pack2h(ev[2], ev[3]);
            *reinterpret_cast<uint2 *>(&sm.e2[r * RS + f0]) = make_uint2(p01, p23);
            sm.e2t[(f0 + 0) * KS + r] = static_cast<uint16_t>(p01 & 0xffffu);
            sm.e2t[(f0 + 1) * KS + r] = static_cast<uint16_t>(p01 >> 16);
            sm.e2t[(f0 + 2) * KS + r] = static_cast<uint16_t>(p23 & 0xffffu);
            sm.e2t[(f0 + 3) * KS + r] = static_cast<uint16_t>(p23 >> 16);
        }
        lds_barrier();

        // ===== C: E1, Zb1^T, Ab, Gram partials, Zb2 partials, state update ===
        // Repack W2 here rather than keep the packed copy of phase A alive
        // across the row-layout phase (the empty asm hides the equality).
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) asm volatile("" : "+v"(W2v[u][rb]));
        f16x8 W2f[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) W2f[u] = pack8h(W2v[u][0], W2v[u][1]);
        f16x8 e2f[2];  // E2 rows: B operand [k = out][n = token c]
        s16x4 e2b[4];   // E2 as B operand [k = token 4g+i][n = out 16u + c]
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) e2f[kb] = rowh(sm.e2, kb);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            e2b[u] = __builtin_bit_cast(s16x4, *reinterpret_cast<const uint2 *>(&sm.e2t[(16 * u + c) * KS + 4 * g]));
        s16x4 E1tr[2];  // E1[token 4g+i][hid 16t + c]
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            // W2 rows of hidden tile t, transposed: [out 16u + 4g + i][hid 16t + c]
            f32x4 w2t[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint4 pk = __builtin_bit_cast(uint4, W2f[u]);
                const s16x4 half = __builtin_bit_cast(s16x4, t ? make_uint2(pk.z, pk.w) : make_uint2(pk.x, pk.y));
                w2t[u] = mfma16h(half, eye, fzero);
            }
            f32x4 g1 = fzero;  // (E2 W2^T)^T: [hid 16t + 4g + i][token c]
            g1 = mfma32h(pack8h(w2t[0], w2t[1]), e2f[0], g1);
            g1 = mfma32h(pack8h(w2t[2], w2t[3]), e2f[1], g1);
            E1tr[t] = pack4h(mfma16h(pack4h(g1 * Ap[t]), eye, fzero));
        }
        f32x4 Ab[2];  // gelu(Zb1)^T: [hid 16t + 4g + i][token c]
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const f32x4 zb = mfma16h(E1tr[t], T1b, zq[t]);  // + (T1 E1)^T
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float Phi, phi;
                normal_cdf_pdf(zb[i], Phi, phi);
                Ab[t][i] = zb[i] * Phi;
            }
        }
        const f16x8 Abf = pack8h(Ab[0], Ab[1]);
        // A operand of Ab W2 (token c rows), with the decay factor of the token
        const f16x8 Abw = DECAY ? pack8h(Ab[0] * dc, Ab[1] * dc) : Abf;
        // This wave's share of T2 E2: the causal mask is linear, so
        // tril(Ab A^T + 1) E2 = sum over waves of tril(Ab_w A_w^T) E2, plus
        // tril(1) E2 added once (wave 0). The partial Gram
        // [s = 4g+i][t = c] = A_s . Ab_t over this wave's hidden units is in the
        // A-operand layout [m = t][k = s] as it stands.
        const f32x4 gw = mfma32h(Af, Abf, fzero);
        f32x4 t2;
#pragma unroll
        for (int i = 0; i < 4; ++i) t2[i] = (w == 0 ? gw[i] + 1.f : gw[i]) * tmask[i];
        const s16x4 t2h = pack4h(t2);
        // Zb2 partials: Ab_w W2_w + tril(Ab_w A_w^T (+1)) E2, plus the
        // chunk-start b2 tile u from wave u
        float *Pb = sm.partb[w] + (4 * g) * RS + c;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const f32x4 acc = mfma16h(t2h, e2b[u], mfma32h(Abw, W2f[u], w == u ? b2w : fzero));
#pragma unroll
            for (int i = 0; i < 4; ++i) Pb[i * RS + 16 * u] = acc[i];
        }
        // state update (the forward products above used the chunk-start state)
        {
            s16x4 xkt[4];  // XK^T as A operand [m = in 16rb + c][k = token 4g+i]
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
                xkt[rb] = __builtin_bit_cast(s16x4, *reinterpret_cast<const uint2 *>(&S.xkt[(16 * rb + c) * KS + 4 * g]));
            if constexpr (DECAY) {  // W <- d_15 W before the loss updates
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int rb = 0; rb < 4; ++rb) W1v[t][rb] = W1v[t][rb] * alpha;
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb) W2v[u][rb] = W2v[u][rb] * alpha;
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) W1v[t][rb] = mfma16h(xkt[rb], E1tr[t], W1v[t][rb]);
                b1v[t] = mfma16h(E1tr[t], ones, b1v[t]);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) W2v[u][rb] = mfma16h(Atr[rb], e2b[u], W2v[u][rb]);
            if (roww) {  // b2 tile w += 1^T E2
                const s16x4 e2w = __builtin_bit_cast(s16x4, *reinterpret_cast<const uint2 *>(&sm.e2t[(16 * w + c) * KS + 4 * g]));
                b2w = mfma16h(ones, e2w, b2w);
            }
        }
        lds_barrier();
    }
    if (!roww && nch > 0) emit_out(nch - 1);  // O of the last chunk

    if (W1_out) {
        // Recompute the lane coordinates here (opaque copy) instead of keeping
        // the store addresses alive through the chunk loop.
        int lane2 = lane;
        asm volatile("" : "+v"(lane2));
        const int g = lane2 >> 4, c = lane2 & 15;
        float *W1d = W1_out + static_cast<size_t>(seq) * D * M, *W2d = W2_out + static_cast<size_t>(seq) * M * D;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) W1d[(16 * rb + 4 * g + i) * M + hw + 16 * t + c] = W1v[t][rb][i];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) W2d[(hw + 16 * rb + 4 * g + i) * D + 16 * u + c] = W2v[u][rb][i];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) b1_out[static_cast<size_t>(seq) * M + hw + 16 * t + 4 * g + i] = b1v[t][i];
        if (roww && g == 0) b2_out[static_cast<size_t>(seq) * D + 16 * w + c] = b2w[0];
    }
}

bool mlp_mfma_supported(const MLPArgs &a) {
    return a.io == 1 && a.d == 64 && a.mb == 16 && (a.loss == 0 || a.loss == 1) &&
           (a.theta == nullptr || (a.loss == 0 && a.wd == 0.f));
}

template <int LOSS, bool DECAY, bool GATED>
static hipError_t launch_mlp_mfma_t(const MLPArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL((mlp_prefill_mfma<LOSS, DECAY, GATED>), dim3(a.B * a.H), dim3(NT), 0, stream, a.H, a.L, a.eps,
                       static_cast<const bf16_t *>(a.XQ), static_cast<const bf16_t *>(a.XK),
                       static_cast<const bf16_t *>(a.XV), a.eta, a.W1, a.b1, a.W2, a.b2,
                       a.w0_batched, a.gamma, a.beta, static_cast<bf16_t *>(a.O), a.W1_out,
                       a.b1_out, a.W2_out, a.b2_out, a.wd, a.theta, a.eta_base);
    return hipGetLastError();
}

hipError_t launch_mlp_mfma(const MLPArgs &a, hipStream_t stream) {
    if (a.B * a.H == 0) return hipSuccess;
    if (a.theta) return launch_mlp_mfma_t<0, false, true>(a, stream);  // the gate, default options
    const bool decay = a.wd != 0.f;
    if (a.loss == 1)
        return decay ? launch_mlp_mfma_t<1, true, false>(a, stream) : launch_mlp_mfma_t<1, false, false>(a, stream);
    return decay ? launch_mlp_mfma_t<0, true, false>(a, stream) : launch_mlp_mfma_t<0, false, false>(a, stream);
}

}  // namespace ttt
