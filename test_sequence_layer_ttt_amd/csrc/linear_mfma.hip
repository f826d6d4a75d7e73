// TTT-Linear prefill, MFMA path: bf16 storage, d = 64, mini-batch b = 16.
//
// What is computed (per sequence, chunk of 16 tokens, state W, b at chunk
// start) -- the dual form of the damodev.csdn.net TTT deep-dive §4.2 with the
// LN-residual output of the lryc.cn TTT article §2.1:
//   Z    = XK W + b ;  G = lnbwd(Z, XV - XK) ;  E = -eta * G      (per row)
//   T    = tril(XQ XK^T + 1)                      (token s <= t)
//   Zbar = XQ W + b + T E ;  O = XQ + LN(Zbar)
//   W   += XK^T E ;  b += 1^T E
//
// Design (gfx950, one 256-thread workgroup = 4 waves per (n,h) sequence):
//   * The fp32 state never leaves registers. Wave w owns columns
//     16w..16w+15 of W; lane (g = lane/16, c = lane%16) holds
//     W[16 rb + 4 g + i][16 w + c] for rb, i in 0..3 -- exactly the output
//     layout of the 16x16x16 MFMA that applies the update, and (with the
//     contraction index permuted consistently on both operands) the B-operand
//     layout of the 16x16x32 MFMAs that form XK W and XQ W.
//   * The bias is kept the same way (b[16 w + c] on every lane) and updated by
//     an MFMA with an all-ones A operand, which sums E over tokens.
//   * MFMA operands are bf16 (state and gradients rounded once per chunk),
//     accumulation and state are fp32.
//   * The row-wise layer-norm work runs in a "row layout": 16 lanes share a
//     token, 4 consecutive features each, reduced with DPP row operations;
//     tiles move between the MFMA layout and the row layout through LDS.
//   * Q/K/V chunks stream from HBM with 8-byte loads issued three chunks
//     ahead into a ring of register sets; each thread's loads are exactly the
//     values its row-layout work needs (XV never goes to LDS), and XQ/XK are
//     staged into LDS (XK also transposed, for the update's A operand).
#include "common.hpp"
#include "launch.hpp"

namespace ttt {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int D = 64, MB = 16;
constexpr int NCW = 4;              // compute waves
constexpr int NT = 64 * (NCW + 1);  // + one loader wave
constexpr int QK_STRIDE = 72;       // bf16 per staged XQ / XK / XV row (64 + pad)
constexpr int KT_STRIDE = 20;       // bf16 per transposed-XK row (16 tokens + pad)
constexpr int Z_STRIDE = 68;        // fp32 per Z / Zbar row (64 + pad)
constexpr int ET_STRIDE = 20;       // bf16 per transposed-E row
constexpr int NSET = 4;             // register sets in the loader's ring

// One chunk as held by the loader wave: lane l covers token 8p + l/8,
// features 8 (l%8) .. +7 of XQ, XK, XV (p = 0, 1), and eta of token l (l < 16).
struct ChunkRegs {
    uint4 q[2], k[2], v[2];
    float eta;
};

__device__ __forceinline__ float lo_bf(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ void unpack4(uint2 p, float (&f)[4]) {
    f[0] = lo_bf(p.x);
    f[1] = hi_bf(p.x);
    f[2] = lo_bf(p.y);
    f[3] = hi_bf(p.y);
}
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    const __bf16 x = static_cast<__bf16>(a), y = static_cast<__bf16>(b);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, x)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, y)) << 16);
}

// Sum over the 16 lanes of a DPP row; every lane receives the total.
__device__ __forceinline__ float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));  // quad [1,0,3,2]
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));  // quad [2,3,0,1]
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)); // half-row mirror
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)); // row mirror
    return v;
}

struct alignas(16) Smem {
    alignas(16) uint16_t xq[2][MB * QK_STRIDE];
    alignas(16) uint16_t xk[2][MB * QK_STRIDE];
    alignas(16) uint16_t xv[2][MB * QK_STRIDE];
    alignas(16) uint16_t xkt[2][D * KT_STRIDE];
    alignas(16) float eta[2][MB];
    alignas(16) float z[MB * Z_STRIDE];
    alignas(16) uint16_t et[D * ET_STRIDE];
};

// Barrier for LDS hand-offs only: waits for this wave's LDS operations, not
// for its outstanding global loads / stores.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
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
    const size_t xbase = static_cast<size_t>(seq) * L * D;
    const size_t ebase = static_cast<size_t>(seq) * L;
    const int nch = (L + MB - 1) / MB;

    const int nch_pad = (nch + NSET - 1) / NSET * NSET;  // loader ring runs in whole turns

    if (w == NCW) {
        // ================= loader wave: HBM -> registers -> LDS =============
        // Loads run NSET chunks ahead of their staging and are issued
        // unconditionally (addresses clamped into the sequence, values past
        // its end zeroed when staged); this wave issues no stores, so its
        // waits on the load counter stay precise.
        if (nch == 0) return;
        auto load = [&](ChunkRegs &R, int ch) {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int tok = min(ch * MB + 8 * p + (lane >> 3), L - 1);
                const size_t off = xbase + static_cast<size_t>(tok) * D + 8 * (lane & 7);
                R.q[p] = *reinterpret_cast<const uint4 *>(XQ + off);
                R.k[p] = *reinterpret_cast<const uint4 *>(XK + off);
                R.v[p] = *reinterpret_cast<const uint4 *>(XV + off);
            }
            R.eta = eta[ebase + min(ch * MB + (lane & 15), L - 1)];
        };
        auto stage = [&](const ChunkRegs &R, int ch) {
            const int s = ch & 1;
            const uint4 zero = make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int tok = 8 * p + (lane >> 3), f = 8 * (lane & 7);
                const bool ok = ch * MB + tok < L;
                const uint4 q = ok ? R.q[p] : zero, k = ok ? R.k[p] : zero, v = ok ? R.v[p] : zero;
                *reinterpret_cast<uint4 *>(&sm.xq[s][tok * QK_STRIDE + f]) = q;
                *reinterpret_cast<uint4 *>(&sm.xk[s][tok * QK_STRIDE + f]) = k;
                *reinterpret_cast<uint4 *>(&sm.xv[s][tok * QK_STRIDE + f]) = v;
                const uint32_t kw[4] = {k.x, k.y, k.z, k.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sm.xkt[s][(f + 2 * e) * KT_STRIDE + tok] = static_cast<uint16_t>(kw[e] & 0xffffu);
                    sm.xkt[s][(f + 2 * e + 1) * KT_STRIDE + tok] = static_cast<uint16_t>(kw[e] >> 16);
                }
            }
            if (lane < MB) sm.eta[s][lane] = (ch * MB + lane < L) ? R.eta : 0.f;
        };

        ChunkRegs R[NSET];
#pragma unroll
        for (int k = 0; k < NSET; ++k) load(R[k], k);
        stage(R[0], 0);
        load(R[0], NSET);
        lds_barrier();
        for (int ch = 0; ch < nch_pad; ch += NSET) {
#pragma unroll
            for (int k = 0; k < NSET; ++k) {
                // during chunk ch + k: stage chunk ch + k + 1, refill its set
                const int kn = (k + 1) % NSET;
                stage(R[kn], ch + k + 1);
                load(R[kn], ch + k + 1 + NSET);
                lds_barrier();
                lds_barrier();
                lds_barrier();
                lds_barrier();
            }
        }
        return;
    }

    // ===================== compute waves ====================================
    const size_t wofs = (w0_batched ? static_cast<size_t>(n) * H * D * D : 0) + static_cast<size_t>(h) * D * D;
    const size_t bofs = (w0_batched ? static_cast<size_t>(n) * H * D : 0) + static_cast<size_t>(h) * D;

    // state in the MFMA layout
    const int col = 16 * w + c;
    float Wr[4][4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) Wr[rb][i] = W0[wofs + static_cast<size_t>(16 * rb + 4 * g + i) * D + col];
    float bv = b0[bofs + col];

    // row layout: token r = tid / 16, features f0 .. f0 + 3
    const int r = tid >> 4, f0 = 4 * c;
    float gam[4], bet[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        gam[e] = gamma[static_cast<size_t>(h) * D + f0 + e];
        bet[e] = beta[static_cast<size_t>(h) * D + f0 + e];
    }
    const float inv_d = 1.0f / D;
    const s16x4 ones = {0x3F80, 0x3F80, 0x3F80, 0x3F80};  // bf16 1.0

    lds_barrier();
    for (int ch = 0; ch < nch; ++ch) {
        const int s = ch & 1;
        const int len = min(MB, L - ch * MB);

        // ---- phase A: Z = XK W + b, Zq = XQ W + b, Gram^T = XK XQ^T ------
        bf16x8 wb[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                wb[kb][j] = static_cast<__bf16>(Wr[2 * kb][j]);
                wb[kb][4 + j] = static_cast<__bf16>(Wr[2 * kb + 1][j]);
            }
        bf16x8 ak[2], aq[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const uint2 k0 = *reinterpret_cast<const uint2 *>(&sm.xk[s][c * QK_STRIDE + 32 * kb + 4 * g]);
            const uint2 k1 = *reinterpret_cast<const uint2 *>(&sm.xk[s][c * QK_STRIDE + 32 * kb + 16 + 4 * g]);
            const uint2 q0 = *reinterpret_cast<const uint2 *>(&sm.xq[s][c * QK_STRIDE + 32 * kb + 4 * g]);
            const uint2 q1 = *reinterpret_cast<const uint2 *>(&sm.xq[s][c * QK_STRIDE + 32 * kb + 16 + 4 * g]);
            ak[kb] = __builtin_bit_cast(bf16x8, make_uint4(k0.x, k0.y, k1.x, k1.y));
            aq[kb] = __builtin_bit_cast(bf16x8, make_uint4(q0.x, q0.y, q1.x, q1.y));
        }
        f32x4 z = {bv, bv, bv, bv}, zq = {bv, bv, bv, bv}, gt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak[kb], wb[kb], z, 0, 0, 0);
            zq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[kb], wb[kb], zq, 0, 0, 0);
            gt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak[kb], aq[kb], gt, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.z[(4 * g + i) * Z_STRIDE + col] = z[i];
        lds_barrier();

        // ---- phase B (row layout): E = -eta * lnbwd(Z, XV - XK) ----------
        {
            const f32x4 zz = *reinterpret_cast<const f32x4 *>(&sm.z[r * Z_STRIDE + f0]);
            float xv[4], xk[4];
            unpack4(*reinterpret_cast<const uint2 *>(&sm.xv[s][r * QK_STRIDE + f0]), xv);
            unpack4(*reinterpret_cast<const uint2 *>(&sm.xk[s][r * QK_STRIDE + f0]), xk);
            const float et_r = sm.eta[s][r];
            const float mu = row16_sum((zz[0] + zz[1]) + (zz[2] + zz[3])) * inv_d;
            float cz[4], s2 = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                cz[e] = zz[e] - mu;
                s2 += cz[e] * cz[e];
            }
            const float rstd = rsqrtf(row16_sum(s2) * inv_d + eps);
            float xh[4], gh[4], a1 = 0.f, a2 = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xh[e] = cz[e] * rstd;
                gh[e] = gam[e] * (gam[e] * xh[e] + bet[e] - (xv[e] - xk[e]));
                a1 += gh[e];
                a2 += gh[e] * xh[e];
            }
            const float m1 = row16_sum(a1) * inv_d, m2 = row16_sum(a2) * inv_d;
            const float ne = -et_r * rstd;
            float ev[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) ev[e] = ne * (gh[e] - m1 - xh[e] * m2);
            const uint32_t p01 = pack2(ev[0], ev[1]), p23 = pack2(ev[2], ev[3]);
            sm.et[(f0 + 0) * ET_STRIDE + r] = static_cast<uint16_t>(p01 & 0xffffu);
            sm.et[(f0 + 1) * ET_STRIDE + r] = static_cast<uint16_t>(p01 >> 16);
            sm.et[(f0 + 2) * ET_STRIDE + r] = static_cast<uint16_t>(p23 & 0xffffu);
            sm.et[(f0 + 3) * ET_STRIDE + r] = static_cast<uint16_t>(p23 >> 16);
        }
        lds_barrier();

        // ---- phase C: state update, bias update, Zbar = Zq + T E ---------
        {
            const s16x4 eb = __builtin_bit_cast(s16x4, *reinterpret_cast<const uint2 *>(&sm.et[col * ET_STRIDE + 4 * g]));
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const s16x4 ka = __builtin_bit_cast(
                    s16x4, *reinterpret_cast<const uint2 *>(&sm.xkt[s][(16 * rb + c) * KT_STRIDE + 4 * g]));
                f32x4 acc = {Wr[rb][0], Wr[rb][1], Wr[rb][2], Wr[rb][3]};
                acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ka, eb, acc, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) Wr[rb][i] = acc[i];
            }
            f32x4 bacc = {bv, bv, bv, bv};
            bacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones, eb, bacc, 0, 0, 0);
            bv = bacc[0];
            // T[t = c][s = 4g + i] = Gram + 1 on and below the diagonal
            const uint32_t t01 = pack2((4 * g + 0 <= c) ? gt[0] + 1.f : 0.f, (4 * g + 1 <= c) ? gt[1] + 1.f : 0.f);
            const uint32_t t23 = pack2((4 * g + 2 <= c) ? gt[2] + 1.f : 0.f, (4 * g + 3 <= c) ? gt[3] + 1.f : 0.f);
            const s16x4 ta = __builtin_bit_cast(s16x4, make_uint2(t01, t23));
            zq = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ta, eb, zq, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.z[(4 * g + i) * Z_STRIDE + col] = zq[i];
        }
        lds_barrier();

        // ---- phase D (row layout): O = XQ + LN(Zbar) -----------------------
        {
            const f32x4 zz = *reinterpret_cast<const f32x4 *>(&sm.z[r * Z_STRIDE + f0]);
            float xq[4], o[4];
            unpack4(*reinterpret_cast<const uint2 *>(&sm.xq[s][r * QK_STRIDE + f0]), xq);
            const float mu = row16_sum((zz[0] + zz[1]) + (zz[2] + zz[3])) * inv_d;
            float cz[4], s2 = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                cz[e] = zz[e] - mu;
                s2 += cz[e] * cz[e];
            }
            const float rstd = rsqrtf(row16_sum(s2) * inv_d + eps);
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = xq[e] + gam[e] * (cz[e] * rstd) + bet[e];
            if (r < len) {
                const size_t t = static_cast<size_t>(ch) * MB + r;
                *reinterpret_cast<uint2 *>(O + xbase + t * D + f0) = make_uint2(pack2(o[0], o[1]), pack2(o[2], o[3]));
            }
        }
        lds_barrier();
    }
    for (int ch = nch; ch < nch_pad; ++ch) {  // keep step with the loader's ring
        lds_barrier();
        lds_barrier();
        lds_barrier();
        lds_barrier();
    }

    if (W_out) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                W_out[static_cast<size_t>(seq) * D * D + static_cast<size_t>(16 * rb + 4 * g + i) * D + col] = Wr[rb][i];
    }
    if (b_out && g == 0) b_out[static_cast<size_t>(seq) * D + col] = bv;
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
