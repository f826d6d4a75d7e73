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
// The serial chain runs through Z -> E -> state. Two exact rewrites shorten it:
//  * look-ahead: Z_{c+1} = P_{c+1} + K_c E_c with P_{c+1} = XK_{c+1} W_c + b_c
//    and K_c = XK_{c+1} XK_c^T + 1 (both known one chunk early), so between
//    two layer-norm backwards sits a single 16x16x16 MFMA;
//  * with gamma = 1, beta = 0 the gradient has the closed form
//      G = a (z - mu) - rstd (tau - mean tau),
//      a = rstd^2 (eps rstd^2 + rstd (mean(tau z) - mean(tau) mu)),
//    which needs one round of row sums (z, z^2, tau z) instead of two.
//
// Layout (gfx950, one 512-thread workgroup per (n,h) sequence):
//  * waves 0-3 compute. Wave w owns columns 16w..16w+15 of the fp32 state:
//    lane (g = lane/16, c = lane%16) holds W[16 rb + 4 g + i][16 w + c] --
//    the output layout of the 16x16x16 MFMA that applies the update and, with
//    the contraction index permuted identically on both operands, the
//    B-operand layout of the 16x16x32 MFMAs that form XK W and XQ W. The bias
//    lives alongside and is updated by an MFMA with an all-ones A operand.
//    MFMA operands are bf16; state and accumulation are fp32.
//  * row-wise layer-norm work uses a row layout: 16 lanes per token, four
//    consecutive features each, DPP row reductions; tiles cross between the
//    MFMA layout and the row layout through LDS.
//  * waves 4-7 prepare inputs: 8-byte loads issued four chunks ahead into a
//    register ring (these waves never store, so their load waits stay
//    precise), then bf16 rows, the transposed XK, fp32 XQ, the target
//    XV - XK with its row mean, and eta are staged in a 5-chunk LDS ring.
//  * per chunk two barriers: phase X (MFMA layout: Z_c, Zbar_{c-1}; row
//    layout: O_{c-2}) and phase Y (row layout: E_c; MFMA layout: state update
//    with E_{c-1}, P_{c+1}, XQ_c W_c, Gram, K_c).
#include <type_traits>

#include "launch.hpp"
#include "tile.hpp"

namespace ttt {
namespace {

using namespace tile;

constexpr int NCW = 4, NPW = 4, NT = 64 * (NCW + NPW);
constexpr int NSLOT = 5;  // LDS ring: chunks c-2 .. c+2

struct alignas(16) Smem {
    Slot slot[NSLOT];
    alignas(16) float z[MB * RS];          // Z_c
    alignas(16) float zbar[2][MB * RS];    // Zbar, two chunks in flight
    alignas(16) uint16_t e[MB * RS];       // E_c, bf16 rows
};

struct Ctx {
    int L, nch, iters;
    float eps;
    bf16_t *Oseq;  // output rows of this sequence
};

// Compute waves: the chain and the output, two barriers per iteration.
// The state is kept as MFMA accumulators: Wv[rb] holds rows 16 rb + 4 g .. +3
// of column 16 w + c, bv holds b[16 w + c] in all four slots.
template <bool IDENT>
__device__ __forceinline__ void compute_loop(Smem &sm, const Ctx &cx, int w, int g, int c,
                                             f32x4 (&Wv)[4], f32x4 &bv, const float (&gam)[4],
                                             const float (&bet)[4]) {
    const int col = 16 * w + c;           // MFMA layout column
    const int r = 4 * w + g, f0 = 4 * c;  // row layout token / first feature
    const int nch = cx.nch;
    const s16x4 ones = {0x3F80, 0x3F80, 0x3F80, 0x3F80};  // bf16 1.0
    const s16x4 zero4 = {0, 0, 0, 0};
    const f32x4 fzero = {0.f, 0.f, 0.f, 0.f};
    // causal mask of T[t = c][s = 4g + i] as 0/1 factors: T = (Gram + 1) * m
    f32x4 tmask;
#pragma unroll
    for (int i = 0; i < 4; ++i) tmask[i] = (4 * g + i <= c) ? 1.f : 0.f;

    auto cvt_state = [&](bf16x8 (&wb)[2]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            wb[kb] = __builtin_bit_cast(
                bf16x8, make_uint4(pack2(Wv[2 * kb][0], Wv[2 * kb][1]), pack2(Wv[2 * kb][2], Wv[2 * kb][3]),
                                   pack2(Wv[2 * kb + 1][0], Wv[2 * kb + 1][1]),
                                   pack2(Wv[2 * kb + 1][2], Wv[2 * kb + 1][3])));
    };

    // P_0 = XK_0 W_0 + b_0
    f32x4 P = bv, Zq = fzero;
    s16x4 Ka = zero4, Ta = zero4;
    if (nch > 0) {
        bf16x8 wb[2];
        cvt_state(wb);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) P = mfma32(row_frag(sm.slot[0].xk, c, g, kb), wb[kb], P);
    }

    const uint16_t *Ecol = sm.e + (4 * g) * RS + col;  // E[4g + i][col] at Ecol[i * RS]
    float *Zw = sm.z + (4 * g) * RS + col;             // MFMA-layout writes
    const float *Zr = sm.z + r * RS + f0;              // row-layout reads
    int sc = 0, sp = NSLOT - 1, sp2 = NSLOT - 2, sn = 1;  // slots of chunks it, it-1, it-2, it+1

    // One iteration. chain: Z_it and E_it; upd: apply E_{it-1}; out: O_{it-2}.
    // In the steady state all three hold and the body is one straight block,
    // so the scheduler can interleave its independent LDS, MFMA and VALU work.
    auto iteration = [&](int it, auto chain_t, auto upd_t, auto out_t, bool chain_r, bool upd_r,
                         bool out_r) {
        constexpr bool CT = decltype(chain_t)::value, UT = decltype(upd_t)::value,
                       OT = decltype(out_t)::value;
        const bool chain = CT || chain_r, upd = UT || upd_r, out = OT || out_r;

        // ===== phase X ========================================================
        // Every LDS read of the phase is issued before any LDS write (the
        // compiler cannot reorder them past writes it cannot disambiguate).
        s16x4 eb = zero4;  // E_{it-1} as the B operand: E[4g + i][col]
        if (upd) {
            const uint32_t e01 = static_cast<uint32_t>(Ecol[0]) | (static_cast<uint32_t>(Ecol[RS]) << 16);
            const uint32_t e23 = static_cast<uint32_t>(Ecol[2 * RS]) | (static_cast<uint32_t>(Ecol[3 * RS]) << 16);
            eb = __builtin_bit_cast(s16x4, make_uint2(e01, e23));
        }
        f32x4 zbr = fzero, xqr = fzero;
        if (out) {
            zbr = *reinterpret_cast<const f32x4 *>(&sm.zbar[it & 1][r * RS + f0]);  // Zbar_{it-2}
            xqr = *reinterpret_cast<const f32x4 *>(&sm.slot[sp2].xqf[r * RS + f0]);
        }
        f32x4 z = P, zb = fzero;
        if (chain && (UT || it > 0)) z = mfma16(Ka, eb, P);
        if (upd) zb = mfma16(Ta, eb, Zq);
        f32x4 o = fzero;
        if (out) o = ln_fwd_row<IDENT>(zbr, xqr, gam, bet, cx.eps);
        if (chain) {
#pragma unroll
            for (int i = 0; i < 4; ++i) Zw[i * RS] = z[i];
        }
        if (upd) {
            float *Zb = sm.zbar[(it - 1) & 1] + (4 * g) * RS + col;
#pragma unroll
            for (int i = 0; i < 4; ++i) Zb[i * RS] = zb[i];
        }
        if (out) {
            const int oc = it - 2;
            if (oc * MB + r < cx.L)
                *reinterpret_cast<uint2 *>(cx.Oseq + static_cast<uint32_t>((oc * MB + r) * D + f0)) =
                    make_uint2(pack2(o[0], o[1]), pack2(o[2], o[3]));
        }
        lds_barrier();

        // ===== phase Y ========================================================
        const Slot &S = sm.slot[sc], &N = sm.slot[sn];
        f32x4 zz = fzero, tau = fzero;
        float mutau = 0.f, eta_r = 0.f;
        bf16x8 akc[2], aqc[2], akn[2];
        s16x4 ka[4];
        if (chain) {
            zz = *reinterpret_cast<const f32x4 *>(Zr);
            tau = *reinterpret_cast<const f32x4 *>(&S.tau[r * RS + f0]);
            mutau = S.mutau[r];
            eta_r = S.eta[r];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                akc[kb] = row_frag(S.xk, c, g, kb);
                aqc[kb] = row_frag(S.xq, c, g, kb);
                akn[kb] = row_frag(N.xk, c, g, kb);
            }
        }
        if (upd) {
            const uint16_t *XKT = sm.slot[sp].xkt + c * KS + 4 * g;
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
                ka[rb] = __builtin_bit_cast(s16x4, *reinterpret_cast<const uint2 *>(XKT + 16 * rb * KS));
        }
        // state update with E_{it-1}
        if (upd) {
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) Wv[rb] = mfma16(ka[rb], eb, Wv[rb]);
            bv = mfma16(ones, eb, bv);
        }
        // chain: E_it (the critical path of the loop) goes out first
        if (chain) {
            const f32x4 ev = ln_bwd_row<IDENT>(zz, tau, mutau, eta_r, gam, bet, cx.eps);
            *reinterpret_cast<uint2 *>(&sm.e[r * RS + f0]) = make_uint2(pack2(ev[0], ev[1]), pack2(ev[2], ev[3]));
        }
        if (chain) {
            bf16x8 wb[2];
            cvt_state(wb);
            f32x4 p = bv, zq = bv, gt = fzero, kt = fzero;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                p = mfma32(akn[kb], wb[kb], p);
                zq = mfma32(aqc[kb], wb[kb], zq);
                gt = mfma32(akc[kb], aqc[kb], gt);  // [s = 4g+i][t = c] = XQ_t . XK_s
                kt = mfma32(akc[kb], akn[kb], kt);  // [s = 4g+i][t = c] = XK_{it+1, t} . XK_{it, s}
            }
            P = p;
            Zq = zq;
            // A operands (row t = c, contraction s = 4g + i)
            Ta = __builtin_bit_cast(s16x4, make_uint2(pack2(fmaf(gt[0], tmask[0], tmask[0]), fmaf(gt[1], tmask[1], tmask[1])),
                                                      pack2(fmaf(gt[2], tmask[2], tmask[2]), fmaf(gt[3], tmask[3], tmask[3]))));
            Ka = __builtin_bit_cast(s16x4, make_uint2(pack2(kt[0] + 1.f, kt[1] + 1.f), pack2(kt[2] + 1.f, kt[3] + 1.f)));
        }
        lds_barrier();
        // rotate the ring
        sp2 = sp;
        sp = sc;
        sc = sn;
        sn = (sn + 1 == NSLOT) ? 0 : sn + 1;
    };

    using F = std::false_type;
    using T = std::true_type;
    const int steady_end = max(nch, 2);
    int it = 0;
    for (; it < min(2, cx.iters); ++it)  // warm-up: no update / no output yet
        iteration(it, F{}, F{}, F{}, it < nch, it >= 1 && it <= nch, false);
    for (; it < steady_end; ++it)        // steady state: branch-free body
        iteration(it, T{}, T{}, T{}, true, true, true);
    for (; it < cx.iters; ++it)          // drain (and padding to the prep ring)
        iteration(it, F{}, F{}, F{}, it < nch, it >= 1 && it <= nch, it >= 2 && it <= nch + 1);
}

}  // namespace

__global__ __launch_bounds__(NT) void linear_prefill_mfma(
    int H, int L, float eps, const bf16_t *__restrict__ XQ, const bf16_t *__restrict__ XK,
    const bf16_t *__restrict__ XV, const float *__restrict__ eta,
    const float *__restrict__ W0, const float *__restrict__ b0, int w0_batched,
    const float *__restrict__ gamma, const float *__restrict__ beta, bf16_t *__restrict__ O,
    float *W_out, float *b_out) {
    __shared__ Smem sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, g = lane >> 4, c = lane & 15;
    const long seq = blockIdx.x;
    const int h = static_cast<int>(seq % H);
    const long n = seq / H;
    Ctx cx;
    cx.L = L;
    cx.nch = (L + MB - 1) / MB;
    cx.iters = (cx.nch + 2 + NSET - 1) / NSET * NSET;  // whole turns of the prep ring
    cx.eps = eps;
    const size_t xbase = static_cast<size_t>(seq) * L * D;
    cx.Oseq = O + xbase;

    if (w >= NCW) {
        // prep waves: chunk it + 2 is staged during iteration it; two barriers
        // per iteration
        prep_waves<NSLOT, 2, 2>(sm.slot, w - NCW, g, c, XQ + xbase, XK + xbase, XV + xbase,
                                eta + static_cast<size_t>(seq) * L, L, cx.iters);
        return;
    }

    // =========== compute waves ==============================================
    const size_t wofs = (w0_batched ? static_cast<size_t>(n) * H * D * D : 0) + static_cast<size_t>(h) * D * D;
    const size_t bofs = (w0_batched ? static_cast<size_t>(n) * H * D : 0) + static_cast<size_t>(h) * D;
    const int col = 16 * w + c;
    f32x4 Wv[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) Wv[rb][i] = W0[wofs + static_cast<size_t>(16 * rb + 4 * g + i) * D + col];
    const float b_init = b0[bofs + col];
    f32x4 bv = {b_init, b_init, b_init, b_init};
    float gam[4], bet[4];
    bool ident = true;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        gam[e] = gamma[static_cast<size_t>(h) * D + 4 * c + e];
        bet[e] = beta[static_cast<size_t>(h) * D + 4 * c + e];
        ident = ident && gam[e] == 1.0f && bet[e] == 0.0f;
    }
    // every compute wave covers all 64 features in its row layout, so the
    // wave-wide vote is the same in all four waves
    ident = __all(ident);

    lds_barrier();
    if (ident)
        compute_loop<true>(sm, cx, w, g, c, Wv, bv, gam, bet);
    else
        compute_loop<false>(sm, cx, w, g, c, Wv, bv, gam, bet);

    if (W_out) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                W_out[static_cast<size_t>(seq) * D * D + static_cast<size_t>(16 * rb + 4 * g + i) * D + col] = Wv[rb][i];
    }
    if (b_out && g == 0) b_out[static_cast<size_t>(seq) * D + col] = bv[0];
}

bool linear_mfma_supported(const LinearArgs &a) { return a.io == 1 && a.d == 64 && a.mb == 16; }

hipError_t launch_linear_mfma(const LinearArgs &a, hipStream_t stream) {
    if (a.B * a.H == 0) return hipSuccess;
    hipLaunchKernelGGL(linear_prefill_mfma, dim3(a.B * a.H), dim3(NT), 0, stream, a.H, a.L, a.eps,
                       static_cast<const bf16_t *>(a.XQ), static_cast<const bf16_t *>(a.XK),
                       static_cast<const bf16_t *>(a.XV), a.eta, a.W0, a.b0, a.w0_batched, a.gamma,
                       a.beta, static_cast<bf16_t *>(a.O), a.W_out, a.b_out);
    return hipGetLastError();
}

}  // namespace ttt
