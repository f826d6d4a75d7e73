// Shared pieces of the MFMA prefill kernels (gfx950): operand types, bf16
// packing, DPP row reductions, LDS-only barriers, row-layout layer norms, and
// the prep waves that stream Q/K/V chunks from HBM into an LDS ring.
//
// Layout conventions (d = 64, chunks of MB = 16 tokens):
//  * MFMA layout: lane (g = lane/16, c = lane%16) of a 16x16 tile holds rows
//    4g .. 4g+3 of column c (the MFMA output layout).
//  * row layout: 16 lanes per token, each with four consecutive features.
#pragma once

#include "common.hpp"

namespace ttt {
namespace tile {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr int D = 64, MB = 16;
constexpr int RS = 68;   // row stride (elements) of a [16][64] tile in LDS
constexpr int KS = 20;   // row stride (bf16) of a transposed [64][16] tile
constexpr int NSET = 4;  // prep register ring depth (chunks)

__device__ __forceinline__ float lo_bf(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ f32x4 unpack4(uint2 p) {
    return f32x4{lo_bf(p.x), hi_bf(p.x), lo_bf(p.y), hi_bf(p.y)};
}
// Two floats -> packed bf16 pair (round to nearest even), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ s16x4 pack4(f32x4 v) {
    return __builtin_bit_cast(s16x4, make_uint2(pack2(v[0], v[1]), pack2(v[2], v[3])));
}
// Two MFMA-layout quads (rows 4g..4g+3 of two 16-row blocks) -> one 16x16x32
// operand fragment in the permuted contraction order used throughout.
__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi) {
    return __builtin_bit_cast(bf16x8, make_uint4(pack2(lo[0], lo[1]), pack2(lo[2], lo[3]),
                                                 pack2(hi[0], hi[1]), pack2(hi[2], hi[3])));
}

// Sum over the 16 lanes of a DPP row; every lane receives the total. Each
// step is one v_add_f32_dpp (identity 0 for lanes outside the pattern).
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_sum(float v) {
    v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]
    v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]
    v = dpp_add<0x141>(v);  // row_half_mirror
    v = dpp_add<0x140>(v);  // row_mirror
    return v;
}

// Barrier for LDS hand-offs only: waits for this wave's LDS operations, not
// for its outstanding global loads or stores.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Operand fragment of a bf16 [16][64] row tile for 16x16x32 MFMAs over
// k-block kb. Lane (g, c) takes row c, features 32kb + 4g .. +3 and
// 32kb + 16 + 4g .. +3: the same contraction order as pack8 of two MFMA
// quads. Serves as an A operand (rows = M) or a B operand (rows = N).
__device__ __forceinline__ bf16x8 row_frag(const uint16_t *tile, int c, int g, int kb) {
    const uint2 a = *reinterpret_cast<const uint2 *>(&tile[c * RS + 32 * kb + 4 * g]);
    const uint2 b = *reinterpret_cast<const uint2 *>(&tile[c * RS + 32 * kb + 16 + 4 * g]);
    return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}

// Layer-norm + L2 backward of one row (row layout), returning E = -eta * G
// where G = d/dz 1/2 ||LN(z) - tau||^2 (the fused step of the damodev.csdn.net
// TTT deep-dive §4.2). With gamma = 1, beta = 0 it uses the closed form
//   G = a (z - mu) - rstd (tau - mean tau),
//   a = rstd^2 (eps rstd^2 + rstd (mean(tau z) - mean(tau) mu)),
// which needs one round of row sums; otherwise the general two-round form.
template <bool IDENT>
__device__ __forceinline__ f32x4 ln_bwd_row(f32x4 z, f32x4 tau, float mutau, float eta_r,
                                            const float (&gam)[4], const float (&bet)[4],
                                            float eps) {
    constexpr float inv_d = 1.0f / D;
    f32x4 ev;
    if constexpr (IDENT) {
        const float s1 = row16_sum((z[0] + z[1]) + (z[2] + z[3]));
        const float s2 = row16_sum(z[0] * z[0] + z[1] * z[1] + z[2] * z[2] + z[3] * z[3]);
        const float s3 = row16_sum(tau[0] * z[0] + tau[1] * z[1] + tau[2] * z[2] + tau[3] * z[3]);
        const float mu = s1 * inv_d;
        const float var = fmaxf(s2 * inv_d - mu * mu, 0.f);
        const float rstd = rsqrtf(var + eps);
        const float mtz = s3 * inv_d - mutau * mu;
        const float a = rstd * rstd * (eps * rstd * rstd + rstd * mtz);
        // E = -eta (a (z - mu) - rstd (tau - mutau)) = cz z + ct tau + c0
        const float cz = -eta_r * a, ct = eta_r * rstd;
        const float c0 = eta_r * (a * mu - rstd * mutau);
#pragma unroll
        for (int e = 0; e < 4; ++e) ev[e] = fmaf(cz, z[e], fmaf(ct, tau[e], c0));
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
            gh[e] = gam[e] * (gam[e] * xh[e] + bet[e] - tau[e]);
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

// O row = XQ row + LN(Zbar row) (row layout; LN-residual output of the
// lryc.cn TTT article §2.1).
template <bool IDENT>
__device__ __forceinline__ f32x4 ln_fwd_row(f32x4 z, f32x4 xq, const float (&gam)[4],
                                            const float (&bet)[4], float eps) {
    constexpr float inv_d = 1.0f / D;
    const float mu = row16_sum((z[0] + z[1]) + (z[2] + z[3])) * inv_d;
    float cz[4], s2 = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        cz[e] = z[e] - mu;
        s2 += cz[e] * cz[e];
    }
    const float rstd = rsqrtf(row16_sum(s2) * inv_d + eps);
    f32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (IDENT)
            o[e] = fmaf(cz[e], rstd, xq[e]);
        else
            o[e] = xq[e] + fmaf(gam[e], cz[e] * rstd, bet[e]);
    }
    return o;
}

// One staged chunk in LDS.
struct alignas(16) Slot {
    alignas(16) uint16_t xq[MB * RS];   // bf16 rows
    alignas(16) uint16_t xk[MB * RS];   // bf16 rows
    alignas(16) uint16_t xkt[D * KS];   // bf16, [feature][token]
    alignas(16) float xqf[MB * RS];     // fp32 rows
    alignas(16) float tau[MB * RS];     // XV - XK, fp32 rows
    alignas(16) float eta[MB];
    alignas(16) float mutau[MB];        // mean over features of tau
};

struct PrepRegs {
    uint2 q, k, v;  // 4 bf16 features of one token
    float eta;
};

// Prep waves: stream chunks HBM -> registers -> LDS ring. Chunk j lives in
// slots[j % NSLOT]; chunk it + AHEAD is staged during compute iteration it
// (chunks 0 .. AHEAD-1 before the first barrier), each iteration ends with
// BPI barriers, and `iters` is a multiple of NSET. Loads are issued NSET
// chunks before their staging and unconditionally (addresses clamped into
// the sequence, values past its end zeroed when staged); these waves never
// store to global memory, so their waits on the load counter stay precise.
template <int NSLOT, int AHEAD, int BPI>
__device__ __forceinline__ void prep_waves(Slot *slots, int pw, int g, int c, const bf16_t *xq,
                                           const bf16_t *xk, const bf16_t *xv, const float *et,
                                           int L, int iters) {
    const int r = 4 * pw + g, f0 = 4 * c;  // token, first feature
    if (L == 0) {  // same barrier count as the compute waves
        lds_barrier();
        for (int it = 0; it < iters * BPI; ++it) lds_barrier();
        return;
    }
    auto load = [&](PrepRegs &R, int ch) {
        const uint32_t tok = static_cast<uint32_t>(min(ch * MB + r, L - 1));
        const uint32_t off = tok * D + f0;
        R.q = *reinterpret_cast<const uint2 *>(xq + off);
        R.k = *reinterpret_cast<const uint2 *>(xk + off);
        R.v = *reinterpret_cast<const uint2 *>(xv + off);
        R.eta = et[tok];
    };
    auto stage_rows = [&](Slot &S, uint2 q, uint2 k, uint2 v, float e) {
        *reinterpret_cast<uint2 *>(&S.xq[r * RS + f0]) = q;
        *reinterpret_cast<uint2 *>(&S.xk[r * RS + f0]) = k;
        S.xkt[(f0 + 0) * KS + r] = static_cast<uint16_t>(k.x & 0xffffu);
        S.xkt[(f0 + 1) * KS + r] = static_cast<uint16_t>(k.x >> 16);
        S.xkt[(f0 + 2) * KS + r] = static_cast<uint16_t>(k.y & 0xffffu);
        S.xkt[(f0 + 3) * KS + r] = static_cast<uint16_t>(k.y >> 16);
        *reinterpret_cast<f32x4 *>(&S.xqf[r * RS + f0]) = unpack4(q);
        const f32x4 tau = unpack4(v) - unpack4(k);
        *reinterpret_cast<f32x4 *>(&S.tau[r * RS + f0]) = tau;
        const float mt = row16_sum((tau[0] + tau[1]) + (tau[2] + tau[3])) * (1.0f / D);
        if (c == 0) {
            S.mutau[r] = mt;
            S.eta[r] = e;
        }
    };
    auto stage = [&](const PrepRegs &R, int ch, int slot) {
        Slot &S = slots[slot];
        if (ch * MB + MB <= L) {  // whole chunk inside the sequence (uniform)
            stage_rows(S, R.q, R.k, R.v, R.eta);
        } else {
            const bool ok = ch * MB + r < L;
            const uint2 z2 = make_uint2(0u, 0u);
            stage_rows(S, ok ? R.q : z2, ok ? R.k : z2, ok ? R.v : z2, ok ? R.eta : 0.f);
        }
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
    int slot = AHEAD % NSLOT;  // slot of chunk it + AHEAD
    for (int it = 0; it < iters; it += NSET) {
#pragma unroll
        for (int k = 0; k < NSET; ++k) {
            const int ks = (k + AHEAD) % NSET;
            stage(R[ks], it + k + AHEAD, slot);
            load(R[ks], it + k + AHEAD + NSET);
            slot = (slot + 1 == NSLOT) ? 0 : slot + 1;
#pragma unroll
            for (int b = 0; b < BPI; ++b) lds_barrier();
        }
    }
}

}  // namespace tile
}  // namespace ttt
