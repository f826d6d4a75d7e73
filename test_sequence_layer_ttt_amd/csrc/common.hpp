// Device helpers shared by the gfx950 kernels of libttt.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

typedef uint16_t bf16_t;  // bfloat16 storage (raw bits)

// ---------------------------------------------------------------------------
// bfloat16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Round to nearest, ties to even (finite inputs; NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
}

template <typename T> struct io_traits;
template <> struct io_traits<float> {
    static __device__ __forceinline__ float load(const float *p, size_t i) { return p[i]; }
    static __device__ __forceinline__ void store(float *p, size_t i, float v) { p[i] = v; }
};
template <> struct io_traits<bf16_t> {
    static __device__ __forceinline__ float load(const bf16_t *p, size_t i) {
        return bf16_to_f32(p[i]);
    }
    static __device__ __forceinline__ void store(bf16_t *p, size_t i, float v) {
        p[i] = f32_to_bf16(v);
    }
};

// ---------------------------------------------------------------------------
// Reductions over aligned groups of W lanes (W in {4, 8, 16, 32, 64}).
// ---------------------------------------------------------------------------
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = W / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, W);
    return v;
}

// Phi(x) and phi(x) (standard normal cdf / pdf) with erf from Abramowitz &
// Stegun 7.1.26: erf(y) = 1 - (a1 t + ... + a5 t^5) exp(-y^2), t = 1/(1 + p y).
__device__ __forceinline__ void normal_cdf_pdf(float x, float &Phi, float &phi) {
    const float y = fabsf(x) * 0.70710678118654752f;  // |x| / sqrt(2)
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, y, 1.0f));
    const float p = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f),
                                     -0.284496736f), 0.254829592f);
    const float e = __expf(-y * y);                   // exp(-x^2 / 2)
    const float half_erfc = 0.5f * p * e;             // erfc(|x| / sqrt(2)) / 2
    Phi = x >= 0.f ? 1.0f - half_erfc : half_erfc;
    phi = 0.39894228040143268f * e;
}

// Exact GELU x * Phi(x) and its derivative.
__device__ __forceinline__ float gelu_f(float x) {
    return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}
__device__ __forceinline__ float gelu_prime_f(float x) {
    const float Phi = 0.5f * (1.0f + erff(x * 0.70710678118654752f));
    const float phi = 0.39894228040143268f * __expf(-0.5f * x * x);
    return Phi + x * phi;
}

// ---------------------------------------------------------------------------
// Layer-norm helpers over one row of D features spread over a group of
// GL lanes, each lane holding E = D / GL values (element j = lane + GL * e).
// ---------------------------------------------------------------------------
// Centred row cz = z - mean(z) and rstd = 1 / sqrt(var + eps), in three
// rounds: the mean m1, then the mean of z - m1 (the rounding error of m1,
// which a large common offset of the row makes comparable to the row's
// spread), then the variance as the mean of the squared centred values.
// Nothing subtracts two large sums, so the result keeps its accuracy
// whatever the row's offset.
template <int GL, int E>
__device__ __forceinline__ void row_centre(const float (&z)[E], float inv_d, float eps,
                                           float (&cz)[E], float &rstd) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) s += z[e];
    const float m1 = group_sum<GL>(s) * inv_d;
    float s1 = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        cz[e] = z[e] - m1;
        s1 += cz[e];
    }
    const float dm = group_sum<GL>(s1) * inv_d;
    float v = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        cz[e] -= dm;
        v += cz[e] * cz[e];
    }
    rstd = rsqrtf(group_sum<GL>(v) * inv_d + eps);
}

// G = d/dz 1/2 ||gamma * xhat + beta - tau||^2
//   = rstd * (gh - mean(gh) - xhat * mean(gh * xhat)),  gh = gamma * (y - tau)
template <int GL, int E>
__device__ __forceinline__ void ln_l2_grad(const float (&z)[E], const float (&tau)[E],
                                           const float (&gamma)[E], const float (&beta)[E],
                                           float inv_d, float eps, float (&G)[E]) {
    float cz[E], rstd;
    row_centre<GL, E>(z, inv_d, eps, cz, rstd);
    float xh[E], gh[E];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        xh[e] = cz[e] * rstd;
        gh[e] = gamma[e] * (gamma[e] * xh[e] + beta[e] - tau[e]);
        s1 += gh[e];
        s2 += gh[e] * xh[e];
    }
    s1 = group_sum<GL>(s1) * inv_d;
    s2 = group_sum<GL>(s2) * inv_d;
#pragma unroll
    for (int e = 0; e < E; ++e) G[e] = rstd * (gh[e] - s1 - xh[e] * s2);
}

// Gradient of the inner-product loss -< x + LN(z), v > with respect to z:
// the upstream gradient is -v, so gh = -gamma * v (beta drops out).
template <int GL, int E>
__device__ __forceinline__ void ln_ip_grad(const float (&z)[E], const float (&v)[E],
                                           const float (&gamma)[E], float inv_d, float eps,
                                           float (&G)[E]) {
    float cz[E], rstd;
    row_centre<GL, E>(z, inv_d, eps, cz, rstd);
    float xh[E], gh[E];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        xh[e] = cz[e] * rstd;
        gh[e] = -gamma[e] * v[e];
        s1 += gh[e];
        s2 += gh[e] * xh[e];
    }
    s1 = group_sum<GL>(s1) * inv_d;
    s2 = group_sum<GL>(s2) * inv_d;
#pragma unroll
    for (int e = 0; e < E; ++e) G[e] = rstd * (gh[e] - s1 - xh[e] * s2);
}

template <int GL, int E>
__device__ __forceinline__ void ln_fwd(const float (&z)[E], const float (&gamma)[E],
                                       const float (&beta)[E], float inv_d, float eps,
                                       float (&y)[E]) {
    float cz[E], rstd;
    row_centre<GL, E>(z, inv_d, eps, cz, rstd);
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = gamma[e] * (cz[e] * rstd) + beta[e];
}

}  // namespace ttt
