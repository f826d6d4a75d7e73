// Learning-rate gate of the lryc.cn TTT article (§2.2): each token's inner-loop
// rate is eta_t = eta_base * logistic(theta_h . x_t), with the gate input x_t
// taken as the head's key XK_t. The prefill kernels evaluate it in their load
// stage; the two kernels here serve the other callers:
//
//   eta_gate_fwd  eta [B,H,L] from XK [B,H,L,d] and theta [H,d]. Streams XK
//                 once (HBM-bound: d*esize + 4 bytes per token).
//   eta_gate_bwd_dx      given deta = dLoss/deta (the inner-loop backward's
//                        output): dXK += deta * eta_base * logistic'(s) * theta_h
//                        in place, over the whole chip (HBM-bound).
//   eta_gate_bwd_dtheta  dtheta[n,h] = sum_t deta * eta_base * logistic'(s) * XK_t,
//                        one workgroup per sequence; the sum over tokens runs
//                        in a fixed order (repeatable bit for bit).
//
// Both split a token over LPT lanes that each hold 16 bytes of its key, so a
// wave reads 1 KiB of contiguous keys per load; the dot product theta . x is a
// shuffle sum over those lanes.
#include "common.hpp"
#include "launch.hpp"

namespace ttt {
namespace {

constexpr int NT = 256;

template <typename TIO> struct Vec16;
template <> struct Vec16<float> {  // 4 fp32 values
    static constexpr int N = 4;
    typedef float4 Raw;
    static __device__ __forceinline__ Raw raw(const float *p) { return *reinterpret_cast<const float4 *>(p); }
    static __device__ __forceinline__ void unpack(const Raw &v, float (&x)[N]) {
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    }
    static __device__ __forceinline__ void load(const float *p, float (&x)[N]) { unpack(raw(p), x); }
};
template <> struct Vec16<bf16_t> {  // 8 bf16 values
    static constexpr int N = 8;
    typedef uint4 Raw;
    static __device__ __forceinline__ Raw raw(const bf16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
    static __device__ __forceinline__ void unpack(const Raw &v, float (&x)[N]) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void load(const bf16_t *p, float (&x)[N]) { unpack(raw(p), x); }
};

// logistic(s) and its derivative without overflow: with E = exp(-|s|) <= 1,
// logistic(|s|) = 1 / (1 + E) and logistic'(s) = E / (1 + E)^2 (even in s).
__device__ __forceinline__ void logistic(float s, float &sig, float &dsig) {
    const float E = __expf(-fabsf(s));
    const float r = 1.0f / (1.0f + E);
    sig = s >= 0.f ? r : E * r;
    dsig = E * r * r;
}

template <int D, typename TIO>
__global__ __launch_bounds__(NT) void eta_gate_fwd(long ntok, int H, int L, const TIO *__restrict__ XK,
                                                   const float *__restrict__ theta, float eta_base,
                                                   float *__restrict__ eta) {
    constexpr int V = Vec16<TIO>::N, LPT = D / V, TPB = NT / LPT;
    const int j = threadIdx.x % LPT, tl = threadIdx.x / LPT;
    for (long base = static_cast<long>(blockIdx.x) * TPB; base < ntok;
         base += static_cast<long>(gridDim.x) * TPB) {
        const long t = base + tl;
        const bool ok = t < ntok;  // the shuffle below runs on every lane
        const long tc = ok ? t : ntok - 1;
        const int h = static_cast<int>((tc / L) % H);
        float x[V];
        Vec16<TIO>::load(XK + tc * D + j * V, x);
        const float *th = theta + static_cast<size_t>(h) * D + j * V;
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < V; ++i) p = fmaf(th[i], x[i], p);
        const float s = group_sum<LPT>(p);
        if (ok && j == 0) eta[t] = eta_base / (1.0f + __expf(-s));
    }
}

// deta * eta_base * logistic'(s), s = theta . x for the token of this lane's
// group (x already unpacked: this lane's V features)
template <int D, typename TIO>
__device__ __forceinline__ float gate_weight(const float (&x)[Vec16<TIO>::N],
                                             const float (&th)[Vec16<TIO>::N], float de,
                                             float eta_base) {
    constexpr int V = Vec16<TIO>::N, LPT = D / V;
    float p = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i) p = fmaf(th[i], x[i], p);
    float sig, dsig;
    logistic(group_sum<LPT>(p), sig, dsig);
    return de * eta_base * dsig;
}

// dXK += w_t * theta_h over every token (grid-stride over all sequences)
template <int D, typename TIO>
__global__ __launch_bounds__(NT) void eta_gate_bwd_dx(long ntok, int H, int L, const TIO *__restrict__ XK,
                                                      const float *__restrict__ theta, float eta_base,
                                                      const float *__restrict__ deta,
                                                      float *__restrict__ dXK) {
    constexpr int V = Vec16<TIO>::N, LPT = D / V, TPB = NT / LPT;
    const int j = threadIdx.x % LPT, tl = threadIdx.x / LPT;
    for (long base = static_cast<long>(blockIdx.x) * TPB; base < ntok;
         base += static_cast<long>(gridDim.x) * TPB) {
        const long t = base + tl;
        const bool ok = t < ntok;  // the shuffle in gate_weight runs on every lane
        const long tc = ok ? t : ntok - 1;
        const int h = static_cast<int>((tc / L) % H);
        float th[V], x[V];
#pragma unroll
        for (int i = 0; i < V; ++i) th[i] = theta[static_cast<size_t>(h) * D + j * V + i];
        Vec16<TIO>::load(XK + tc * D + j * V, x);
        const float w = gate_weight<D, TIO>(x, th, deta[tc], eta_base);
        if (ok) {
            float4 *q = reinterpret_cast<float4 *>(dXK + t * D + j * V);
#pragma unroll
            for (int k = 0; k < V / 4; ++k) {
                float4 v = q[k];
                v.x = fmaf(w, th[4 * k + 0], v.x);
                v.y = fmaf(w, th[4 * k + 1], v.y);
                v.z = fmaf(w, th[4 * k + 2], v.z);
                v.w = fmaf(w, th[4 * k + 3], v.w);
                q[k] = v;
            }
        }
    }
}

// dtheta[n,h] = sum_t w_t XK_t: one 1024-thread workgroup per sequence, the
// sum over tokens in a fixed order (per-thread, then over rows in LDS)
constexpr int NTR = 1024;
template <int D, typename TIO>
__global__ __launch_bounds__(NTR) void eta_gate_bwd_dtheta(int H, int L, const TIO *__restrict__ XK,
                                                           const float *__restrict__ theta,
                                                           float eta_base,
                                                           const float *__restrict__ deta,
                                                           float *__restrict__ dtheta) {
    constexpr int V = Vec16<TIO>::N, LPT = D / V, TPB = NTR / LPT;
    __shared__ float red[TPB][D + 1];
    const int j = threadIdx.x % LPT, tl = threadIdx.x / LPT;
    const long seq = blockIdx.x;
    const int h = static_cast<int>(seq % H);
    const TIO *xk = XK + static_cast<size_t>(seq) * L * D;
    const float *de = deta + static_cast<size_t>(seq) * L;
    float th[V], acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        th[i] = theta[static_cast<size_t>(h) * D + j * V + i];
        acc[i] = 0.f;
    }
    // U tokens per lane group in flight: all loads of a batch are issued first
    constexpr int U = 8;
    for (int base = 0; base < L; base += U * TPB) {
        typename Vec16<TIO>::Raw raw[U];
        float dv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tc = min(base + u * TPB + tl, L - 1);
            raw[u] = Vec16<TIO>::raw(xk + static_cast<size_t>(tc) * D + j * V);
            dv[u] = de[tc];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float x[V];
            Vec16<TIO>::unpack(raw[u], x);
            float w = gate_weight<D, TIO>(x, th, dv[u], eta_base);
            if (base + u * TPB + tl >= L) w = 0.f;  // clamped duplicate of the last token
#pragma unroll
            for (int i = 0; i < V; ++i) acc[i] = fmaf(w, x[i], acc[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < V; ++i) red[tl][j * V + i] = acc[i];
    __syncthreads();
    if (threadIdx.x < D) {
        float s = 0.f;
        for (int r = 0; r < TPB; ++r) s += red[r][threadIdx.x];
        dtheta[static_cast<size_t>(seq) * D + threadIdx.x] = s;
    }
}

template <int D, typename TIO>
hipError_t gate_fwd_t(int B, int H, int L, const void *XK, const float *theta, float eta_base,
                      float *eta, hipStream_t stream) {
    constexpr int TPB = NT / (D / Vec16<TIO>::N);
    const long ntok = static_cast<long>(B) * H * L;
    const long blocks = (ntok + TPB - 1) / TPB;
    const int grid = static_cast<int>(blocks < 4096 ? blocks : 4096);
    hipLaunchKernelGGL((eta_gate_fwd<D, TIO>), dim3(grid), dim3(NT), 0, stream, ntok, H, L,
                       static_cast<const TIO *>(XK), theta, eta_base, eta);
    return hipGetLastError();
}

template <int D, typename TIO>
hipError_t gate_bwd_t(int B, int H, int L, const void *XK, const float *theta, float eta_base,
                      const float *deta, float *dXK, float *dtheta, hipStream_t stream) {
    constexpr int TPB = NT / (D / Vec16<TIO>::N);
    const long ntok = static_cast<long>(B) * H * L;
    if (ntok > 0) {
        const long blocks = (ntok + TPB - 1) / TPB;
        const int grid = static_cast<int>(blocks < 4096 ? blocks : 4096);
        hipLaunchKernelGGL((eta_gate_bwd_dx<D, TIO>), dim3(grid), dim3(NT), 0, stream, ntok, H, L,
                           static_cast<const TIO *>(XK), theta, eta_base, deta, dXK);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((eta_gate_bwd_dtheta<D, TIO>), dim3(B * H), dim3(NTR), 0, stream, H, L,
                       static_cast<const TIO *>(XK), theta, eta_base, deta, dtheta);
    return hipGetLastError();
}

template <typename TIO>
hipError_t gate_fwd_io(int B, int H, int L, int d, const void *XK, const float *theta,
                       float eta_base, float *eta, hipStream_t s) {
    if (d == 16) return gate_fwd_t<16, TIO>(B, H, L, XK, theta, eta_base, eta, s);
    if (d == 32) return gate_fwd_t<32, TIO>(B, H, L, XK, theta, eta_base, eta, s);
    return gate_fwd_t<64, TIO>(B, H, L, XK, theta, eta_base, eta, s);
}

template <typename TIO>
hipError_t gate_bwd_io(int B, int H, int L, int d, const void *XK, const float *theta,
                       float eta_base, const float *deta, float *dXK, float *dtheta, hipStream_t s) {
    if (d == 16) return gate_bwd_t<16, TIO>(B, H, L, XK, theta, eta_base, deta, dXK, dtheta, s);
    if (d == 32) return gate_bwd_t<32, TIO>(B, H, L, XK, theta, eta_base, deta, dXK, dtheta, s);
    return gate_bwd_t<64, TIO>(B, H, L, XK, theta, eta_base, deta, dXK, dtheta, s);
}

}  // namespace

hipError_t launch_eta_gate(int B, int H, int L, int d, int io, const void *XK, const float *theta,
                           float eta_base, float *eta, hipStream_t stream) {
    if (static_cast<long>(B) * H * L == 0) return hipSuccess;
    return io == 1 ? gate_fwd_io<bf16_t>(B, H, L, d, XK, theta, eta_base, eta, stream)
                   : gate_fwd_io<float>(B, H, L, d, XK, theta, eta_base, eta, stream);
}

hipError_t launch_eta_gate_backward(int B, int H, int L, int d, int io, const void *XK,
                                    const float *theta, float eta_base, const float *deta,
                                    float *dXK, float *dtheta, hipStream_t stream) {
    if (B * H == 0) return hipSuccess;
    return io == 1 ? gate_bwd_io<bf16_t>(B, H, L, d, XK, theta, eta_base, deta, dXK, dtheta, stream)
                   : gate_bwd_io<float>(B, H, L, d, XK, theta, eta_base, deta, dXK, dtheta, stream);
}

}  // namespace ttt
