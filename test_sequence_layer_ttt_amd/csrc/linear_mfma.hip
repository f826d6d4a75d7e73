// TTT-Linear prefill, MFMA path: bf16 storage, d = 64, mini-batch b = 16.
//
// What is computed (per sequence; chunk c of 16 tokens; W_c, b_c = state at
// the start of chunk c) -- the dual form of the damodev.csdn.net TTT
// deep-dive §4.2 with the LN-residual output of the lryc.cn TTT article §2.1:
//   Z_c    = XK_c W_c + b_c ;   E_c = -eta * lnbwd(Z_c, XV_c - XK_c)   (per row)
//   Zbar_c = XQ_c W_c + b_c + T_c E_c,   T_c = tril(XQ_c XK_c^T + 1)
//   O_c    = XQ_c + LN(Zbar_c)
//   W_{c+1} = W_c + XK_c^T E_c ;  b_{c+1} = b_c + 1^T E_c
//
// The serial chain runs Z_c -> E_c -> Z_{c+1}. Exact rewrites keep it short:
//  * two-step look-ahead: with K(j, i) = XK_j XK_i^T + 1 (the +1 is the bias
//    path),
//      Z_{c+1} = [XK_{c+1} W_{c-1} + b_{c-1} + K(c+1, c-1) E_{c-1}] + K(c+1, c) E_c,
//    so only the last product waits for E_c and the state update never sits
//    on the chain;
//  * the layer-norm backward needs one round of per-token row sums: with
//    gamma = 1, beta = 0 three (z, z^2, tau z) and
//      G = a (z - mu) - rstd (tau - mean tau),
//      a = rstd^2 (eps rstd^2 + rstd (mean(tau z) - mean(tau) mu));
//    otherwise seven (z, z^2, g^2 z, g^2 z^2, g b z, g tau z, g tau), from
//    which mean(ghat) and mean(ghat xhat) follow in closed form.
//
// Layout (gfx950, one 768-thread workgroup = 12 waves per (n,h) sequence):
//  * feature-major tiles: the products are formed transposed, [feature][token],
//    so lane (g = lane/16, c = lane%16) of a wave with feature tile u holds
//    features 16u + 4g .. +3 of token c. A token's row sum is four in-lane
//    values, a sum over the four lane rows (two lane swaps) and a sum over
//    the four waves of a role (a few floats per token through LDS).
//  * chain waves 0-3 (tile u = wave): Z^T = E^T K^T + bracket, the row sums,
//    E, and E transposed into the operand layout [feature][token] by an MFMA
//    with the identity (exact: the bf16 values pass through unchanged).
//  * state waves 4-7 (tile u = wave - 4) hold W[:, 16u .. 16u+15] and b as
//    fp32 MFMA accumulators for the whole sequence: lane (g, c) holds
//    W[16 rb + 4 g + i][16 u + c], the output layout of the XK^T E update
//    and, with the contraction index permuted identically on both operands,
//    the A-operand layout of W^T XK^T. They apply the updates, form the
//    brackets, K, XQ W + b and T, and emit O = XQ + LN(Zbar).
//  * prep waves 8-11 stream chunks three ahead into a 5-slot LDS ring and
//    form the token x token operands K(j, j-1), K(j, j-2) and T_j once per
//    chunk (they depend on the inputs only).
//  * LDS traffic is the scarce resource: operand fragments are 16 contiguous
//    bytes (the contraction order of the 16x16x32 products puts input
//    features 32 kb + 8 g .. +7 in lane row g; W's accumulator rows follow
//    that order), bf16 rows are padded to 72 elements and the row-sum
//    exchange to 36 floats per token so 16-byte accesses of eight
//    consecutive lanes hit distinct banks.
//  * two barriers per chunk. Phase 1: chain Z_c and its partial row sums;
//    state waves apply E_{c-1} and start O_{c-1}. Phase 2: chain E_c; state
//    waves finish O_{c-1} and prepare the operands of chunks c .. c+2.
//  * centred state: the state waves hold W - wbar 1^T and b - bbar (wbar the
//    row means of W_0, bbar the mean of b_0), which shifts every row of Z and
//    Zbar by a per-token constant that the layer norm and its backward do not
//    see; the rows of E sum to zero, so the updates keep the centring. The
//    one-pass row sums of z and z^2 therefore act on rows whose mean is near
//    zero, whatever offsets the caller's W_0 and b_0 carry.
//  Precision: W grows along the sequence and its bf16 rounding would dominate
//  the error of XK W and XQ W, so those products take W and the XQ / XK rows
//  in fp16 (the bf16 inputs convert exactly for |x| >= 2^-14, within 3e-8
//  below; W and the inputs lie far inside the fp16 range). The token x token
//  operands K and T, E and the transposed XK stay bf16, whose range cannot
//  overflow for any bf16 input. State, accumulation and row statistics are
//  fp32.
#include "launch.hpp"
#include "tile.hpp"

namespace ttt {
namespace {

using namespace tile;

constexpr int NCW = 4, NSW = 4, NPW = 4, NW = NCW + NSW + NPW, NT = 64 * NW;
constexpr int NSLOT = 5, AHEAD = 3;
constexpr int RB = 72;  // row stride (bf16) of the staged XQ / XK rows
constexpr int SB = 36;  // per-token stride (floats) of the row-sum exchange

// One staged chunk.
struct alignas(16) LSlot {
    alignas(16) uint16_t xq[MB * RB];       // fp16 rows
    alignas(16) uint16_t xk[MB * RB];       // fp16 rows
    alignas(16) uint16_t xkt[D * KS + 16];  // bf16, [permuted feature][token], see xkt_at
    alignas(16) float tau[MB * RS];    // the loss's target (XV - XK, or XV), fp32 rows
    alignas(16) float eta[MB];
};

struct alignas(16) Smem {
    LSlot slot[NSLOT];
    alignas(16) float stb[MB * SB];  // LN-backward partial row sums [token][value][chain wave]
    alignas(16) float stf[MB * SB];  // LN-forward partial row sums [token][value][state wave]
    alignas(16) uint2 ea[NCW][64];   // E of the newest chunk, bf16 operand layout, per tile
    alignas(16) f32x4 q[2][NCW][64];    // bracket of Z_j^T per tile, by chunk parity
    // token x token operands (B layout [k = s][n = t], bf16), by chunk parity:
    alignas(16) uint2 ka[2][64];        // K(j, j-1)
    alignas(16) uint2 k2[2][64];        // K(j, j-2)
    alignas(16) uint2 tb[2][64];        // T_j^T
    // weight decay, per slot: 1 - lambda * (sum of eta up to token t), and
    // alpha = 1 - lambda * (sum of the chunk's eta)
    alignas(16) float dec[NSLOT][MB];
    float alpha[NSLOT];
    // row means of W_0 and the mean of b_0 (the state is held centred)
    alignas(16) float wbar[D];
    float bbar;
};

struct Ctx {
    int L, nch, iters;
    float eps;
};

__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ s16x4 ld_s4(const void *p) {
    return __builtin_bit_cast(s16x4, *reinterpret_cast<const uint2 *>(p));
}
__device__ __forceinline__ void st_s4(void *p, s16x4 v) {
    *reinterpret_cast<uint2 *>(p) = __builtin_bit_cast(uint2, v);
}
__device__ __forceinline__ float sum4(f32x4 v) { return (v[0] + v[1]) + (v[2] + v[3]); }

// Input feature held in row m = 4 g + i of the state accumulator Wv[rb]:
// pack8h(Wv[2 kb], Wv[2 kb + 1]) then covers features 32 kb + 8 g .. +7.
__device__ __forceinline__ int win(int rb, int m) {
    return 32 * (rb >> 1) + 8 * (m >> 2) + 4 * (rb & 1) + (m & 3);
}
// Row of the transposed XK tile that holds feature f (so that row 16 rb + m
// holds feature win(rb, m), the order the update's A operand needs).
__device__ __forceinline__ int xkt_row(int f) {
    return 16 * (2 * (f >> 5) + ((f >> 2) & 1)) + 4 * ((f >> 3) & 3) + (f & 3);
}
// Element offset of (row, token) in the transposed XK tile. Each group of 16
// rows is shifted by two dwords so that the prep waves' stores (rows 16 apart
// in one instruction) fall into distinct banks; a reader's 16 rows share a
// group.
__device__ __forceinline__ int xkt_at(int row, int tok) { return row * KS + 4 * (row >> 4) + tok; }
// 16x16x32 operand fragment of an fp16 row tile: row c, features 32 kb + 8 g .. +7.
__device__ __forceinline__ f16x8 fragh(const uint16_t *rows, int c, int g, int kb) {
    return *reinterpret_cast<const f16x8 *>(&rows[c * RB + 32 * kb + 8 * g]);
}

// ---------------------------------------------------------------------------
// Prep waves: HBM -> registers -> LDS ring. Chunk j lives in slot j % NSLOT;
// chunk it + AHEAD is staged in phase 1 of iteration it (chunks 0 .. AHEAD-1
// before the prologue barriers). Loads run NSET chunks ahead of their
// staging and are unconditional (addresses clamped into the sequence, values
// past its end zeroed when staged); these waves never store to global
// memory, so their waits on the load counter stay precise. In phase 2 of
// iteration j they form K(j+2, j), K(j+2, j+1) and T_{j+1}; each is read in
// the next iteration (T_{j+1} in the one after) and rewritten two
// iterations later.
// ---------------------------------------------------------------------------
template <bool GATED, int LOSS, bool DECAY>
__device__ __forceinline__ void prep_waves(Smem &sm, int pw, int g, int c, int lane, const bf16_t *xq,
                                           const bf16_t *xk, const bf16_t *xv, const float *et,
                                           const float *th, float eta_base, float wd, int L,
                                           int iters) {
    constexpr int PRE = 2, BPI = 2;
    LSlot *slots = sm.slot;
    const int r = 4 * pw + g, f0 = 4 * c;  // token, first feature
    const int kr = xkt_row(f0);            // features f0 .. f0+3 -> rows kr .. kr+3
    if (L == 0) {  // same barrier count as the other waves
        for (int it = 0; it < PRE + iters * BPI; ++it) lds_barrier();
        return;
    }
    const char *bq = reinterpret_cast<const char *>(xq), *bk = reinterpret_cast<const char *>(xk),
               *bv = reinterpret_cast<const char *>(xv);
    const int last = (L - 1) / MB;  // the last chunk
    // Chunk ch's row r (both clamped into the sequence): a uniform 64-bit chunk base and a
    // 32-bit offset within the chunk, so the per-lane address arithmetic stays 32-bit.
    auto load = [&](PrepRegs &R, int ch) {
        const int cc = min(ch, last);
        const uint32_t rr = static_cast<uint32_t>(min(r, L - 1 - cc * MB));
        const size_t cb = static_cast<size_t>(cc) * (MB * D * 2);  // bytes
        const uint32_t off = (rr * D + f0) * 2u;
        R.q = *reinterpret_cast<const uint2 *>(bq + cb + off);
        R.k = *reinterpret_cast<const uint2 *>(bk + cb + off);
        R.v = *reinterpret_cast<const uint2 *>(bv + cb + off);
        if constexpr (!GATED) R.eta = (et + static_cast<size_t>(cc) * MB)[rr];
    };
    // learning-rate gate (GATED): eta = eta_base * logistic(theta . XK_t), the
    // dot product split over the 16 lanes of the token's DPP row; exp2 and
    // reciprocal are the hardware approximations (about 1 ulp each)
    f32x4 thv = {0.f, 0.f, 0.f, 0.f};
    if constexpr (GATED) thv = *reinterpret_cast<const f32x4 *>(th + f0) * -1.4426950408889634f;
    auto gate = [&](uint2 k) {  // thv holds -theta * log2(e)
        const f32x4 kf = unpack4(k);
        const float ns = row16_sum(fmaf(thv[0], kf[0], thv[1] * kf[1]) + fmaf(thv[2], kf[2], thv[3] * kf[3]));
        return eta_base * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(ns));
    };
    auto stage_rows = [&](LSlot &S, uint2 q, uint2 k, uint2 v, float e) {
        const f32x4 qf = unpack4(q), kf = unpack4(k);
        const uint2 qh = make_uint2(pack2h(qf[0], qf[1]), pack2h(qf[2], qf[3]));
        const uint2 kh = make_uint2(pack2h(kf[0], kf[1]), pack2h(kf[2], kf[3]));
        *reinterpret_cast<uint2 *>(&S.xq[r * RB + f0]) = qh;
        *reinterpret_cast<uint2 *>(&S.xk[r * RB + f0]) = kh;
        S.xkt[xkt_at(kr + 0, r)] = static_cast<uint16_t>(k.x & 0xffffu);
        S.xkt[xkt_at(kr + 1, r)] = static_cast<uint16_t>(k.x >> 16);
        S.xkt[xkt_at(kr + 2, r)] = static_cast<uint16_t>(k.y & 0xffffu);
        S.xkt[xkt_at(kr + 3, r)] = static_cast<uint16_t>(k.y >> 16);
        // target: XV - XK (squared error) or XV (inner-product loss)
        if constexpr (LOSS == 1)
            *reinterpret_cast<f32x4 *>(&S.tau[r * RS + f0]) = unpack4(v);
        else
            *reinterpret_cast<f32x4 *>(&S.tau[r * RS + f0]) = unpack4(v) - kf;
        if (c == 0) S.eta[r] = e;
    };
    auto stage = [&](const PrepRegs &R, int ch, int slot) {
        LSlot &S = slots[slot];
        float e;
        if constexpr (GATED)
            e = gate(R.k);  // all lanes (DPP sum)
        else
            e = R.eta;
        if (ch * MB + MB <= L) {  // whole chunk inside the sequence (uniform)
            stage_rows(S, R.q, R.k, R.v, e);
        } else {
            const bool ok = ch * MB + r < L;
            const uint2 z2 = make_uint2(0u, 0u);
            stage_rows(S, ok ? R.q : z2, ok ? R.k : z2, ok ? R.v : z2, ok ? e : 0.f);
        }
    };
    const f32x4 fzero = {0.f, 0.f, 0.f, 0.f}, fone = {1.f, 1.f, 1.f, 1.f};
    f32x4 tmask;  // causal mask of T^T[s = 4g + i][t = c]
#pragma unroll
    for (int i = 0; i < 4; ++i) tmask[i] = (4 * g + i <= c) ? 1.f : 0.f;
    // [s = 4g + i][t = c] = A_s . B_t + init for bf16 row tiles A, B, packed
    auto gram = [&](const uint16_t *A, const uint16_t *B, f32x4 init) {
        return mfma32h(fragh(A, c, g, 1), fragh(B, c, g, 1), mfma32h(fragh(A, c, g, 0), fragh(B, c, g, 0), init));
    };
    // weight decay factors of a staged chunk (one wave, lanes 0..15 = tokens)
    // (lane c of each DPP row holds token c: inclusive scan by row shifts)
    auto decay = [&](int si) {
        const float e = slots[si].eta[c];
        float cum = e;
        cum += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(cum), 0x111, 0xF, 0xF, true));
        cum += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(cum), 0x112, 0xF, 0xF, true));
        cum += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(cum), 0x114, 0xF, 0xF, true));
        cum += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(cum), 0x118, 0xF, 0xF, true));
        const float all = row16_sum(e);
        if (g == 0) sm.dec[si][c] = 1.0f - wd * cum;
        if (lane == 0) sm.alpha[si] = 1.0f - wd * all;
    };
    // K(j+2, j) with decay: alpha_{j+1} XK_{j+2} XK_j^T + 1 (the bias path is not decayed)
    auto gram_dec = [&](const uint16_t *A, const uint16_t *B, float alpha) {
        const f32x4 gt = gram(A, B, fzero);
        f32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = fmaf(alpha, gt[i], 1.f);
        return v;
    };
    auto tmat = [&](const LSlot &S) {  // T^T of a chunk as a B operand
        const f32x4 gt = gram(S.xk, S.xq, fzero);
        f32x4 tv;
#pragma unroll
        for (int i = 0; i < 4; ++i) tv[i] = fmaf(gt[i], tmask[i], tmask[i]);
        return pack4(tv);
    };

    PrepRegs R[NSET];
#pragma unroll
    for (int k = 0; k < NSET; ++k) load(R[k], k);
#pragma unroll
    for (int a = 0; a < AHEAD; ++a) {
        stage(R[a], a, a % NSLOT);
        load(R[a], a + NSET);
    }
    lds_barrier();
    // prologue operands K(1, 0) and T_0
    if (pw == 1) st_s4(&sm.ka[1][lane], pack4(gram(slots[0].xk, slots[1].xk, fone)));
    if (pw == 2) st_s4(&sm.tb[0][lane], tmat(slots[0]));
    if constexpr (DECAY) {
        if (pw == 3)
#pragma unroll
            for (int a = 0; a < AHEAD; ++a) decay(a);
    }
    lds_barrier();
    int slot = AHEAD % NSLOT;  // slot of chunk it + AHEAD
    for (int it = 0; it < iters; it += NSET) {
#pragma unroll
        for (int k = 0; k < NSET; ++k) {
            const int ks = (k + AHEAD) % NSET;
            // phase 1: stage chunk j+3 (j = it + k), load chunk j+3+NSET
            const int s2 = slot == 0 ? NSLOT - 1 : slot - 1;  // chunk j+2
            const int s1 = s2 == 0 ? NSLOT - 1 : s2 - 1;      // chunk j+1
            const int s0 = s1 == 0 ? NSLOT - 1 : s1 - 1;      // chunk j
            stage(R[ks], it + k + AHEAD, slot);
            load(R[ks], it + k + AHEAD + NSET);
            lds_barrier();
            // phase 2: K(j+2, j), K(j+2, j+1) and T_{j+1}
            const int par = (it + k) & 1;  // parity of j (= of j+2)
            if constexpr (DECAY) {
                if (pw == 0)
                    st_s4(&sm.k2[par][lane], pack4(gram_dec(slots[s0].xk, slots[s2].xk, sm.alpha[s1])));
                if (pw == 3) decay(slot);  // chunk j+3, staged in phase 1
            } else {
                if (pw == 0) st_s4(&sm.k2[par][lane], pack4(gram(slots[s0].xk, slots[s2].xk, fone)));
            }
            if (pw == 1) st_s4(&sm.ka[par][lane], pack4(gram(slots[s1].xk, slots[s2].xk, fone)));
            if (pw == 2) st_s4(&sm.tb[par ^ 1][lane], tmat(slots[s1]));
            slot = (slot + 1 == NSLOT) ? 0 : slot + 1;
            lds_barrier();
        }
    }
}

// ---------------------------------------------------------------------------
// Chain waves: Z_c^T (feature tile u) -> row sums -> E_c -> operand layout.
// ---------------------------------------------------------------------------
template <bool IDENT, int LOSS>
__device__ __forceinline__ void chain_waves(Smem &sm, const Ctx &cx, int u, int g, int c, int lane,
                                            const float *gam_h, const float *bet_h) {
    constexpr float inv_d = 1.0f / D;
    const int f0 = 16 * u + 4 * g;  // first feature of this lane
    s16x4 eye;                      // identity as a B operand: B[k = 4g + i][n = c] (bf16)
#pragma unroll
    for (int i = 0; i < 4; ++i) eye[i] = (4 * g + i == c) ? 0x3F80 : 0;
    const f32x4 fzero = {0.f, 0.f, 0.f, 0.f};

    // general layer norm: this lane's gamma and beta, and per-head sums
    f32x4 gm = {1.f, 1.f, 1.f, 1.f}, bt = fzero;
    float Sg2 = static_cast<float>(D), Sgb = 0.f;
    if constexpr (!IDENT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            gm[i] = gam_h[f0 + i];
            bt[i] = bet_h[f0 + i];
        }
        const float ga = gam_h[lane], ba = bet_h[lane];  // one feature per lane
        Sg2 = rows4_sum(row16_sum(ga * ga));
        Sgb = rows4_sum(row16_sum(ga * ba));
    }
    const f32x4 g2 = gm * gm, gb = gm * bt;

    lds_barrier();  // prologue chunks staged
    lds_barrier();  // first bracket and K written
    if (cx.nch == 0) {
        for (int it = 0; it < 2 * cx.iters; ++it) lds_barrier();
        return;
    }
    f32x4 Q = sm.q[0][u][lane];  // bracket of Z_0: XK_0 W_0 + b_0
    s16x4 EA = {0, 0, 0, 0};     // E_{c-1}, A operand [m = feature 16u + c][k = token 4g + i]
    s16x4 KB = {0, 0, 0, 0};     // K(c, c-1) as the B operand [k = s][n = t]
    int sc = 0;                  // slot of chunk it

    float *stw = &sm.stb[c * SB + u];  // this wave's column of token c

    for (int it = 0; it < cx.nch; ++it) {
        const LSlot &S = sm.slot[sc];
        // ===== phase 1: Z^T and partial row sums ==============================
        const f32x4 z = mfma16(EA, KB, Q);  // [feature f0 + i][token c]
        const f32x4 tau = ld4(&S.tau[c * RS + f0]);
        // lane row g receives this tile's partial sum number g of token c
        if constexpr (IDENT) {
            stw[4 * g] = rows4_reduce4(sum4(z), sum4(z * z), sum4(tau * z), sum4(tau));
        } else {
            const f32x4 g2z = g2 * z, gt = gm * tau;
            stw[4 * g] = rows4_reduce4(sum4(z), sum4(z * z), sum4(g2z), sum4(g2z * z));
            stw[16 + 4 * g] = rows4_reduce4(sum4(gb * z), sum4(gt * z), sum4(gt), 0.f);
        }
        lds_barrier();

        // ===== phase 2: E_c, transposed into the operand layout =============
        const f32x4 Qn = sm.q[(it + 1) & 1][u][lane];        // bracket of Z_{it+1}
        const s16x4 Kn = ld_s4(&sm.ka[(it + 1) & 1][lane]);  // K(it+1, it)
        const float et = S.eta[c];
        f32x4 ev;
        // lane row g adds value g over the four waves; the gather hands every
        // lane all four totals
        const f32x4 s = rows4_gather(sum4(ld4(&sm.stb[c * SB + 4 * g])));
        if constexpr (IDENT) {  // s = sums of z, z^2, tau z, tau
            // z comes from the centred state, so mu is small next to the row's
            // spread and s[1] / d - mu^2 does not cancel
            const float mut = s[3] * inv_d;
            const float mu = s[0] * inv_d;
            const float var = fmaxf(fmaf(s[1], inv_d, -mu * mu), 0.f);
            const float r = rsq(var + cx.eps);
            const float mtz = fmaf(s[2], inv_d, -mut * mu);
            const float r2 = r * r;
            // squared error: a = eps r^4 + r^3 mean((tau - mean tau)(z - mu));
            // inner product (ghat = -tau): the eps r^4 term from LN(z) drops out
            const float a = LOSS == 1 ? r2 * (r * mtz) : r2 * fmaf(r, mtz, cx.eps * r2);
            // E = -eta (a (z - mu) - r (tau - mean tau)) = cz z + ct tau + c0
            const float cz = -et * a, ct = et * r;
            const float c0 = et * fmaf(a, mu, -r * mut);
#pragma unroll
            for (int i = 0; i < 4; ++i) ev[i] = fmaf(cz, z[i], fmaf(ct, tau[i], c0));
        } else {
            const f32x4 s2 = rows4_gather(sum4(ld4(&sm.stb[c * SB + 16 + 4 * g])));
            const float mu = s[0] * inv_d;
            const float var = fmaxf(fmaf(s[1], inv_d, -mu * mu), 0.f);
            const float r = rsq(var + cx.eps);
            if constexpr (LOSS == 1) {
                // ghat = -gamma tau: mean(ghat) = -sum(g tau)/d,
                // mean(ghat xhat) = -r (sum(g tau z) - mu sum(g tau))/d;
                // E = -eta r (ghat - m1 - xhat m2)
                const float m1 = -s2[2] * inv_d;
                const float m2 = -r * fmaf(-mu, s2[2], s2[1]) * inv_d;
                const float k1 = et * r, k2 = et * r * r * m2, k3 = et * r * m1;
#pragma unroll
                for (int i = 0; i < 4; ++i) ev[i] = fmaf(k1 * gm[i], tau[i], fmaf(k2, z[i] - mu, k3));
            } else {
            // mean(ghat) and mean(ghat xhat), ghat = gamma (gamma xhat + beta - tau)
            const float m1 = (fmaf(r, fmaf(-mu, Sg2, s[2]), Sgb) - s2[2]) * inv_d;
            const float q2 = fmaf(mu, fmaf(mu, Sg2, -2.f * s[2]), s[3]);       // sum g^2 (z - mu)^2
            const float q1 = fmaf(-mu, Sgb, s2[0]) - fmaf(-mu, s2[2], s2[1]);  // sum g (b - tau)(z - mu)
            const float m2 = fmaf(r * r, q2, r * q1) * inv_d;
            // E = -eta r [r (g^2 - m2)(z - mu) + g (b - tau) - m1]
            const float k1 = -et * r * r, k2 = -et * r, k3 = et * r * m1;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ev[i] = fmaf(k1 * (g2[i] - m2), z[i] - mu, fmaf(k2 * gm[i], bt[i] - tau[i], k3));
            }
        }
        // [token c][feature f0 + i] as the A operand times the identity gives
        // [token 4g + i][feature 16u + c]: E^T in the operand layout.
        EA = pack4(mfma16(pack4(ev), eye, fzero));
        st_s4(&sm.ea[u][lane], EA);
        Q = Qn;
        KB = Kn;
        sc = (sc + 1 == NSLOT) ? 0 : sc + 1;
        lds_barrier();
    }
    for (int it = cx.nch; it < cx.iters; ++it) {
        lds_barrier();
        lds_barrier();
    }
}

// ---------------------------------------------------------------------------
// State waves: W, b of feature tile u; brackets and K; outputs.
// ---------------------------------------------------------------------------
template <bool IDENT, bool DECAY>
__device__ __forceinline__ void state_waves(Smem &sm, const Ctx &cx, int u, int g, int c, int lane,
                                            const float *W0s, const float *b0s, const float *gam_h,
                                            const float *bet_h, bf16_t *Oseq, float *W_out,
                                            float *b_out, float wd) {
    constexpr float inv_d = 1.0f / D;
    const int f0 = 16 * u + 4 * g;
    const s16x4 ones = {0x3F80, 0x3F80, 0x3F80, 0x3F80};  // bf16 1.0
    const f32x4 fzero = {0.f, 0.f, 0.f, 0.f}, fone = {1.f, 1.f, 1.f, 1.f};

    f32x4 Wv[4];  // W[16 rb + 4g + i][16u + c]
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) Wv[rb][i] = W0s[win(rb, 4 * g + i) * D + 16 * u + c];
    f32x4 bv = ld4(b0s + f0);  // b[f0 + i]
    // Centred state: the waves hold W' = W - wbar 1^T and b' = b - bbar, with
    // wbar the row means of W_0 and bbar the mean of b_0. Every row of Z and
    // Zbar is then shifted by the per-token constant XK_t wbar + bbar (or
    // XQ_t wbar + bbar), which the layer norm and its backward do not see, so
    // the one-pass sums of z and z^2 below work on rows whose mean is near
    // zero however large the caller's offsets are. The updates keep the
    // centring: the rows of E sum to zero (the layer-norm gradient of a row
    // sums to zero), so XK^T E and 1^T E have zero row means; weight decay
    // scales wbar by the same factors as W (rho below). The caller's
    // representation is restored when the state is written out.
    const bool centre = cx.nch > 0;  // uniform; L = 0 passes the state through bit for bit
    if (centre) {
        const int t = 64 * u + lane, row = t >> 2, q = t & 3;  // 256 threads: a quarter row each
        const f32x4 *wr = reinterpret_cast<const f32x4 *>(W0s + row * D + 16 * q);
        float s = sum4(wr[0]) + sum4(wr[1]) + (sum4(wr[2]) + sum4(wr[3]));
        s = dpp_add<0xB1>(s);  // quad_perm [1,0,3,2]
        s = dpp_add<0x4E>(s);  // quad_perm [2,3,0,1]
        if (q == 0) sm.wbar[row] = s * (1.0f / D);
        if (u == 0) {
            const float bs = rows4_sum(row16_sum(b0s[lane]));
            if (lane == 0) sm.bbar = bs * (1.0f / D);
        }
    }
    float rho = 1.f;  // product of the decay factors applied so far
    f32x4 gm = fone, bt = fzero;
    if constexpr (!IDENT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            gm[i] = gam_h[f0 + i];
            bt[i] = bet_h[f0 + i];
        }
    }
    // W as the A operand [m = out][k = in] (fp16)
    auto wfrag = [&](int kb) { return pack8h(Wv[2 * kb], Wv[2 * kb + 1]); };
    auto xfrag = [&](const uint16_t *rows, int kb) { return fragh(rows, c, g, kb); };
    // [feature f0 + i][token c] = (X W + b)^T for an fp16 row tile X
    auto xw = [&](const f16x8 (&wf)[2], const uint16_t *rows) {
        return mfma32h(wf[1], xfrag(rows, 1), mfma32h(wf[0], xfrag(rows, 0), bv));
    };

    lds_barrier();  // prologue chunks 0 .. 2 staged (and the means above written)
    f32x4 Pp = fzero;  // XK_{j+2} W_j + b_j, waiting for E_j (with decay: XK_{j+2} W_j alone)
    float pk = 1.f, zk = 1.f;  // weight decay: the factors Pp and Zq still need (then + b)
    if (cx.nch > 0) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) Wv[rb][i] -= sm.wbar[win(rb, 4 * g + i)];
        bv = bv - sm.bbar;
        const f16x8 wf[2] = {wfrag(0), wfrag(1)};
        sm.q[0][u][lane] = xw(wf, sm.slot[0].xk);  // bracket of Z_0 = XK_0 W_0 + b_0
        if constexpr (DECAY) {  // alpha_0 XK_1 W_0 + b_0, alpha_0 from chunk 0's eta
            const float *e = sm.slot[0].eta;
            float all = 0.f;
#pragma unroll
            for (int s = 0; s < MB; ++s) all += e[s];
            Pp = mfma32h(wf[1], xfrag(sm.slot[1].xk, 1), mfma32h(wf[0], xfrag(sm.slot[1].xk, 0), fzero));
            pk = 1.0f - wd * all;
        } else {
            Pp = xw(wf, sm.slot[1].xk);  // XK_1 W_0 + b_0 (E_{-1} = 0)
        }
    }
    lds_barrier();

    f32x4 Zq = fzero;  // (XQ_j W_j + b_j)^T of the chunk awaiting its E
    int sm1 = NSLOT - 1, s0 = 0, s1 = 1, s2 = 2;  // slots of chunks it-1 .. it+2

    // One iteration: apply E_{it-1} and emit O_{it-1} (upd); write the bracket
    // of Z_{it+1} and prepare the operands of chunks it .. it+2 (fwd). Each
    // phase issues all of its LDS reads first, so one round trip covers them.
    auto iteration = [&](int it, bool upd, bool fwd) {
        // ===== phase 1 ==========================================================
        s16x4 EAp = {0, 0, 0, 0}, xkt[4], K2 = {0, 0, 0, 0}, TB;
        if (upd) {
            const LSlot &P = sm.slot[sm1];
            EAp = ld_s4(&sm.ea[u][lane]);  // E_{it-1}, A operand [feature][token]
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) xkt[rb] = ld_s4(&P.xkt[xkt_at(16 * rb + c, 4 * g)]);
            K2 = ld_s4(&sm.k2[(it + 1) & 1][lane]);  // K(it+1, it-1)
            TB = ld_s4(&sm.tb[(it - 1) & 1][lane]);  // T_{it-1}^T
        }
        __builtin_amdgcn_sched_barrier(0);  // all reads of the phase in flight together
        if constexpr (DECAY) {  // the deferred factors; bv is still b of the chunk they were formed at
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Pp[i] = fmaf(pk, Pp[i], bv[i]);
                Zq[i] = fmaf(zk, Zq[i], bv[i]);
            }
        }
        if (fwd) sm.q[(it + 1) & 1][u][lane] = upd ? mfma16(EAp, K2, Pp) : Pp;
        f32x4 zb = fzero;
        if (upd) {
            zb = mfma16(EAp, TB, Zq);  // Zbar_{it-1}^T
            // rows 0, 1 receive the tile's sum of zb, rows 2, 3 that of zb^2
            sm.stf[c * SB + 4 * g + u] = rows4_reduce2(sum4(zb), sum4(zb * zb));
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) Wv[rb] = mfma16(xkt[rb], EAp, Wv[rb]);  // (W already decayed)
            bv = mfma16(EAp, ones, bv);
        }
        lds_barrier();

        // ===== phase 2 ==========================================================
        f32x4 st;
        uint2 xqb;
        f16x8 q0[2], k2[2];
        if constexpr (DECAY) {  // token c's XQ factor; alpha_it alpha_{it+1} (applied next phase)
            if (fwd) {
                zk = sm.dec[s0][c];
                pk = sm.alpha[s0] * sm.alpha[s1];
            }
        }
        if (upd) {
            st = ld4(&sm.stf[c * SB + 4 * (g & 2)]);  // rows 0, 1: sums of zb; rows 2, 3: of zb^2
            xqb = *reinterpret_cast<const uint2 *>(&sm.slot[sm1].xq[c * RB + f0]);
        }
        if (fwd) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                k2[kb] = xfrag(sm.slot[s2].xk, kb);
                q0[kb] = xfrag(sm.slot[s0].xq, kb);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (fwd) {
            const f16x8 wf[2] = {wfrag(0), wfrag(1)};
            if constexpr (DECAY) {
                // XK_{it+2} W_it and XQ_it W_it; their factors and b_it follow
                // in the next phase, off this phase's MFMA latency
                Pp = mfma32h(wf[1], k2[1], mfma32h(wf[0], k2[0], fzero));
                Zq = mfma32h(wf[1], q0[1], mfma32h(wf[0], q0[0], fzero));
                // W_{it+1} = alpha_it W_it + XK_it^T E_it: the decay now (the
                // products above took W_it as fp16 copies), the update next phase
                const float a_it = sm.alpha[s0];
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) Wv[rb] = Wv[rb] * a_it;
                rho *= a_it;
            } else {
                Pp = mfma32h(wf[1], k2[1], mfma32h(wf[0], k2[0], bv));  // XK_{it+2} W_it + b_it
                Zq = mfma32h(wf[1], q0[1], mfma32h(wf[0], q0[0], bv));  // XQ_it W_it + b_it
            }
        }
        if (upd) {
            const uint32_t sb = __float_as_uint(sum4(st));
            const auto tt = __builtin_amdgcn_permlane32_swap(sb, sb, false, false);
            const float t1 = __uint_as_float(tt[0]), t2 = __uint_as_float(tt[1]);
            const float mu = t1 * inv_d;
            const f32x4 xq = unpack4h(xqb);
            const float r = rsq(fmaxf(fmaf(t2, inv_d, -mu * mu), 0.f) + cx.eps);
            f32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (IDENT)
                    o[i] = fmaf(zb[i] - mu, r, xq[i]);
                else
                    o[i] = xq[i] + fmaf(gm[i], (zb[i] - mu) * r, bt[i]);
            }
            uint2 ov = make_uint2(pack2(o[0], o[1]), pack2(o[2], o[3]));
            asm volatile("" : "+v"(ov));  // keep the math out of the store's branch
            const int tok = (it - 1) * MB + c;
            if (tok < cx.L)
                *reinterpret_cast<uint2 *>(Oseq + static_cast<size_t>(it - 1) * (MB * D) + (c * D + f0)) = ov;
        }
        sm1 = s0;
        s0 = s1;
        s1 = s2;
        s2 = (s2 + 1 == NSLOT) ? 0 : s2 + 1;
        lds_barrier();
    };

    const int nch = cx.nch;
    int it = 0;
    if (nch > 0) {
        iteration(0, false, true);
        for (it = 1; it < nch; ++it) iteration(it, true, true);
        iteration(nch, true, false);
        it = nch + 1;
    }
    for (; it < cx.iters; ++it) {
        lds_barrier();
        lds_barrier();
    }

    if (centre) {  // back to the caller's representation: W = W' + rho wbar 1^T, b = b' + bbar
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) Wv[rb][i] = fmaf(rho, sm.wbar[win(rb, 4 * g + i)], Wv[rb][i]);
        bv = bv + sm.bbar;
    }
    if (W_out) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) W_out[win(rb, 4 * g + i) * D + 16 * u + c] = Wv[rb][i];
    }
    if (b_out && c == 0) *reinterpret_cast<f32x4 *>(b_out + f0) = bv;
}

}  // namespace

// LOSS: 0 squared error, 1 inner product; DECAY: weight decay wd on W.
template <int LOSS, bool DECAY>
__global__ __launch_bounds__(NT) void linear_prefill_mfma(
    int H, int L, float eps, const bf16_t *__restrict__ XQ, const bf16_t *__restrict__ XK,
    const bf16_t *__restrict__ XV, const float *__restrict__ eta, const float *__restrict__ theta,
    float eta_base, const float *W0, const float *b0, int w0_batched,
    const float *__restrict__ gamma, const float *__restrict__ beta, bf16_t *__restrict__ O,
    float *W_out, float *b_out, float wd) {
    __shared__ Smem sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, g = lane >> 4, c = lane & 15;
    const long seq = blockIdx.x;
    const int h = static_cast<int>(seq % H);
    const long n = seq / H;
    Ctx cx;
    cx.L = L;
    cx.nch = (L + MB - 1) / MB;
    cx.iters = (cx.nch + 1 + NSET - 1) / NSET * NSET;  // whole turns of the prep ring
    cx.eps = eps;
    const size_t xbase = static_cast<size_t>(seq) * L * D;
    const float *gam_h = gamma + static_cast<size_t>(h) * D, *bet_h = beta + static_cast<size_t>(h) * D;

    if (w >= NCW + NSW) {
        if (theta)
            prep_waves<true, LOSS, DECAY>(sm, w - NCW - NSW, g, c, lane, XQ + xbase, XK + xbase,
                                          XV + xbase, nullptr, theta + static_cast<size_t>(h) * D,
                                          eta_base, wd, L, cx.iters);
        else
            prep_waves<false, LOSS, DECAY>(sm, w - NCW - NSW, g, c, lane, XQ + xbase, XK + xbase,
                                           XV + xbase, eta + static_cast<size_t>(seq) * L, nullptr,
                                           0.f, wd, L, cx.iters);
        return;
    }
    // gamma = 1 and beta = 0 over the head (one feature per lane; same vote in every wave)
    const bool ident = __all(gam_h[lane] == 1.0f && bet_h[lane] == 0.0f);

    if (w < NCW) {
        if (ident)
            chain_waves<true, LOSS>(sm, cx, w, g, c, lane, gam_h, bet_h);
        else
            chain_waves<false, LOSS>(sm, cx, w, g, c, lane, gam_h, bet_h);
        return;
    }
    const size_t st = (w0_batched ? static_cast<size_t>(n) * H : 0) + static_cast<size_t>(h);
    float *Wd = W_out ? W_out + static_cast<size_t>(seq) * D * D : nullptr;
    float *bd = b_out ? b_out + static_cast<size_t>(seq) * D : nullptr;
    if (ident)
        state_waves<true, DECAY>(sm, cx, w - NCW, g, c, lane, W0 + st * D * D, b0 + st * D, gam_h,
                                 bet_h, O + xbase, Wd, bd, wd);
    else
        state_waves<false, DECAY>(sm, cx, w - NCW, g, c, lane, W0 + st * D * D, b0 + st * D, gam_h,
                                  bet_h, O + xbase, Wd, bd, wd);
}

bool linear_mfma_supported(const LinearArgs &a) { return a.io == 1 && a.d == 64 && a.mb == 16; }

template <int LOSS, bool DECAY>
static hipError_t launch_mfma_t(const LinearArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL((linear_prefill_mfma<LOSS, DECAY>), dim3(a.B * a.H), dim3(NT), 0, stream, a.H,
                       a.L, a.eps, static_cast<const bf16_t *>(a.XQ),
                       static_cast<const bf16_t *>(a.XK), static_cast<const bf16_t *>(a.XV), a.eta,
                       a.theta, a.eta_base, a.W0, a.b0, a.w0_batched, a.gamma, a.beta,
                       static_cast<bf16_t *>(a.O), a.W_out, a.b_out, a.wd);
    return hipGetLastError();
}

hipError_t launch_linear_mfma(const LinearArgs &a, hipStream_t stream) {
    if (a.B * a.H == 0) return hipSuccess;
    const bool decay = a.wd != 0.f;
    if (a.loss == 1) return decay ? launch_mfma_t<1, true>(a, stream) : launch_mfma_t<1, false>(a, stream);
    return decay ? launch_mfma_t<0, true>(a, stream) : launch_mfma_t<0, false>(a, stream);
}

}  // namespace ttt
