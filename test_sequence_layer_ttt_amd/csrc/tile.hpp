// Shared pieces of the MFMA prefill kernels (gfx950): operand types, bf16
// packing, DPP and lane-swap row reductions, LDS-only barriers, row-layout
// layer norms and the staged-chunk layout.
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
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

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

// Sum over the four DPP rows (lanes c, c+16, c+32, c+48); every lane receives
// the total, bitwise identical across the four rows. Each step swaps halves
// (v_permlane32_swap), then odd and even rows (v_permlane16_swap), and adds.
__device__ __forceinline__ float rows4_sum(float v) {
    const uint32_t b = __float_as_uint(v);
    const auto h = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    v = __uint_as_float(h[0]) + __uint_as_float(h[1]);
    const uint32_t b2 = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane16_swap(b2, b2, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Four row sums at once (butterfly over the four DPP rows): the lane in row
// k (= lane / 16) receives the sum of v_k over lanes c, c+16, c+32, c+48.
// The half swap pairs (v0, v2) and (v1, v3), the row swap pairs the results.
__device__ __forceinline__ float rows4_reduce4(float v0, float v1, float v2, float v3) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v0), __float_as_uint(v2), false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v1), __float_as_uint(v3), false, false);
    const float A = __uint_as_float(a[0]) + __uint_as_float(a[1]);  // rows 0,1: v0; rows 2,3: v2
    const float B = __uint_as_float(b[0]) + __uint_as_float(b[1]);  // rows 0,1: v1; rows 2,3: v3
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(A), __float_as_uint(B), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two row sums at once: rows 0 and 1 receive the sum of v0, rows 2 and 3 that of v1.
__device__ __forceinline__ float rows4_reduce2(float v0, float v1) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v0), __float_as_uint(v1), false, false);
    const float A = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t b = __float_as_uint(A);
    const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Inverse of the row reductions: the lane in row k holds S_k; every lane
// receives (S_0, S_1, S_2, S_3). Element 0 of a swap result is the first
// operand's new value, element 1 the second's.
__device__ __forceinline__ f32x4 rows4_gather(float x) {
    const uint32_t b = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane32_swap(b, b, false, false);  // rows (S0,S1,S0,S1), (S2,S3,S2,S3)
    const auto lo = __builtin_amdgcn_permlane16_swap(a[0], a[0], false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap(a[1], a[1], false, false);
    return f32x4{__uint_as_float(lo[0]), __uint_as_float(lo[1]), __uint_as_float(hi[0]),
                 __uint_as_float(hi[1])};
}

// 1/sqrt(x) for a normal (non-denormal) x: one v_rsq_f32, no rescaling.
__device__ __forceinline__ float rsq(float x) { return __builtin_amdgcn_rsqf(x); }

// Barrier for LDS hand-offs only: waits for this wave's LDS operations, not
// for its outstanding global loads or stores.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Two floats -> packed fp16 pair (round to nearest even).
__device__ __forceinline__ uint32_t pack2h(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}
__device__ __forceinline__ f16x8 pack8h(f32x4 lo, f32x4 hi) {
    return __builtin_bit_cast(f16x8, make_uint4(pack2h(lo[0], lo[1]), pack2h(lo[2], lo[3]),
                                                pack2h(hi[0], hi[1]), pack2h(hi[2], hi[3])));
}
__device__ __forceinline__ s16x4 pack4h(f32x4 v) {
    return __builtin_bit_cast(s16x4, make_uint2(pack2h(v[0], v[1]), pack2h(v[2], v[3])));
}
__device__ __forceinline__ f32x4 unpack4h(uint2 p) {
    typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
    return __builtin_convertvector(__builtin_bit_cast(f16x4, p), f32x4);
}
__device__ __forceinline__ f32x4 mfma32h(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// 16x16x16 fp16 product on operands held as 4 x 16-bit containers.
__device__ __forceinline__ f32x4 mfma16h(s16x4 a, s16x4 b, f32x4 c) {
    typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c,
                                                 0, 0, 0);
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
// which needs the mean and then two centred row sums (the variance and
// mean(tau (z - mu)) are sums of centred products, so a large common offset
// of the row cancels exactly instead of in E[z^2] - mu^2); otherwise the
// general two-round form.
template <bool IDENT>
__device__ __forceinline__ f32x4 ln_bwd_row(f32x4 z, f32x4 tau, float mutau, float eta_r,
                                            const float (&gam)[4], const float (&bet)[4],
                                            float eps) {
    constexpr float inv_d = 1.0f / D;
    f32x4 ev;
    if constexpr (IDENT) {
        const float mu = row16_sum((z[0] + z[1]) + (z[2] + z[3])) * inv_d;
        f32x4 cz;
#pragma unroll
        for (int e = 0; e < 4; ++e) cz[e] = z[e] - mu;
        const float s2 = row16_sum(fmaf(cz[0], cz[0], cz[1] * cz[1]) + fmaf(cz[2], cz[2], cz[3] * cz[3]));
        const float s3 = row16_sum(fmaf(tau[0], cz[0], tau[1] * cz[1]) + fmaf(tau[2], cz[2], tau[3] * cz[3]));
        const float rstd = rsqrtf(s2 * inv_d + eps);
        const float mtz = s3 * inv_d;  // mean((tau - mean tau)(z - mu)): the centred z sums to 0
        const float a = rstd * rstd * (eps * rstd * rstd + rstd * mtz);
        // E = -eta (a (z - mu) - rstd (tau - mutau))
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
    alignas(16) uint16_t xq[MB * RS];   // 16-bit rows (fp16 in the MLP kernel)
    alignas(16) uint16_t xk[MB * RS];   // 16-bit rows (fp16 in the MLP kernel)
    alignas(16) uint16_t xkt[D * KS];   // 16-bit, [feature][token] (fp16 in the MLP kernel)
    alignas(16) float xqf[MB * RS];     // fp32 rows
    alignas(16) float tau[MB * RS];     // XV - XK, fp32 rows
    alignas(16) float eta[MB];
    alignas(16) float mutau[MB];        // mean over features of tau
};

struct PrepRegs {
    uint2 q, k, v;  // 4 bf16 features of one token
    float eta;
};

}  // namespace tile
}  // namespace ttt
