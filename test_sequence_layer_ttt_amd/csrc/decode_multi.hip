// T consecutive single-token TTT-Linear steps (b = 1, primal form) on B x H
// independent d = 64 states, with every state held in registers for the
// whole launch: the fast-weight cache of the damodev.csdn.net TTT deep-dive
// (§5.2) carried through a run of decode steps, each step following the
// update-then-apply rule of its §3.1:
//   z = xk W + b;  E = -eta lnbwd(z, xv - xk)
//   W' = W + xk^T E;  b' = b + E
//   o  = xq + LN(xq W' + b')
// The output uses the identity xq W' + b' = (xq W + b) + (xq . xk + 1) E, so
// both dot products against W are taken before the update.
//
// One wave per state. Lane j owns column j of W (64 fp32 registers), so
// z_j and (xq W)_j are sums over the lane's own registers; element i of xk
// and xq reaches every lane as a DPP row broadcast folded into the FMA. The
// layer-norm sums over the 64 features are wave reductions (DPP row sums,
// then row swaps). HBM carries only the per-step inputs and outputs; W and b
// are read once at the start and written once at the end.
//
// Mini-batch decode (CH, b = mb > 1): the tokens of a chunk take their
// gradient at the chunk-start state, held as a second register copy (wc, bc)
// that is refreshed from (W, b) when a chunk starts; z uses the copy, the
// output and the update use the current state, so the identity above still
// holds with W the current state.
//
// GATED: each step's rate comes from the learning-rate gate of the lryc.cn TTT
// article (§2.2), eta = eta_base * logistic(theta[h] . xk), x read as the key;
// theta . xk is a wave sum taken together with xq . xk, then one exp2 and one
// reciprocal (hardware approximations); no eta array is read.
#include "common.hpp"
#include "launch.hpp"
#include "tile.hpp"

#include <utility>

namespace ttt {
namespace {

using namespace tile;
constexpr int DM = 64;

__device__ __forceinline__ float wave_sum(float v) { return rows4_sum(row16_sum(v)); }
// Four wave sums at once; every lane receives all four totals.
__device__ __forceinline__ f32x4 wave_sum4(float a, float b, float c, float d) {
    return rows4_gather(rows4_reduce4(row16_sum(a), row16_sum(b), row16_sum(c), row16_sum(d)));
}
// Two wave sums at once.
__device__ __forceinline__ f32x4 wave_sum2(float a, float b) {
    return rows4_gather(rows4_reduce2(row16_sum(a), row16_sum(b)));
}

// acc + x[lane n of this lane's DPP row] * w: the broadcast is the DPP
// source modifier of the FMA itself (row_newbcast), so it costs nothing.
// A DPP source must be written at least two wait states before it is read;
// the compiler does not see DPP inside asm, so dpp_guard (an s_nop 1 that
// takes the sources as operands, hence follows their last write) precedes
// each run of these FMAs, and both are volatile so they keep that order.
template <int N>
__device__ __forceinline__ float fmac_bcast(float acc, float x, float w) {
    asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
        : "+v"(acc)
        : "v"(x), "v"(w), "n"(N));
    return acc;
}

// Broadcast layout of a 64-element input vector: lane l holds elements
// 4 (l mod 16) + m in x[m], so every DPP row (16 lanes) holds the whole
// vector and element 4 n + m is x[m] of lane n of the row. Raw<TIO> is what
// one lane loads for that (four elements) plus its own element j; it stays
// packed until the step that uses it, so the load is in flight meanwhile.
template <typename TIO> struct Raw;
template <> struct Raw<bf16_t> {
    uint2 v4;
    bf16_t v1;
    __device__ __forceinline__ void load(const bf16_t *v, int j) {
        v4 = *reinterpret_cast<const uint2 *>(v + 4 * (j & 15));
        v1 = v[j];
    }
    __device__ __forceinline__ void bcast(float (&x)[4]) const {
        x[0] = lo_bf(v4.x);
        x[1] = hi_bf(v4.x);
        x[2] = lo_bf(v4.y);
        x[3] = hi_bf(v4.y);
    }
    __device__ __forceinline__ float own() const { return bf16_to_f32(v1); }
};
template <> struct Raw<float> {
    float4 v4;
    float v1;
    __device__ __forceinline__ void load(const float *v, int j) {
        v4 = *reinterpret_cast<const float4 *>(v + 4 * (j & 15));
        v1 = v[j];
    }
    __device__ __forceinline__ void bcast(float (&x)[4]) const {
        x[0] = v4.x;
        x[1] = v4.y;
        x[2] = v4.z;
        x[3] = v4.w;
    }
    __device__ __forceinline__ float own() const { return v1; }
};

__device__ __forceinline__ void dpp_guard(const float (&x)[4]) {
    asm volatile("s_nop 1" ::"v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]));
}

// a0 + a1 = sum over i of x_i w[i] (two accumulators).
template <int... N>
__device__ __forceinline__ void dot_bcast(const float (&x)[4], const float (&w)[DM], float &a0,
                                          float &a1, std::integer_sequence<int, N...>) {
    dpp_guard(x);
    ((a0 = fmac_bcast<N>(a0, x[0], w[4 * N]), a1 = fmac_bcast<N>(a1, x[1], w[4 * N + 1]),
      a0 = fmac_bcast<N>(a0, x[2], w[4 * N + 2]), a1 = fmac_bcast<N>(a1, x[3], w[4 * N + 3])),
     ...);
}
// w[i] += x_i e.
template <int... N>
__device__ __forceinline__ void axpy_bcast(const float (&x)[4], float e, float (&w)[DM],
                                           std::integer_sequence<int, N...>) {
    dpp_guard(x);
    ((w[4 * N] = fmac_bcast<N>(w[4 * N], x[0], e), w[4 * N + 1] = fmac_bcast<N>(w[4 * N + 1], x[1], e),
      w[4 * N + 2] = fmac_bcast<N>(w[4 * N + 2], x[2], e),
      w[4 * N + 3] = fmac_bcast<N>(w[4 * N + 3], x[3], e)),
     ...);
}
using Rows16 = std::make_integer_sequence<int, 16>;

template <typename TIO, bool IDENT, bool CH, bool GATED>
__device__ __forceinline__ void run_steps(int T, int BH, float eps, int seq, int j,
                                          const TIO *__restrict__ xq, const TIO *__restrict__ xk,
                                          const TIO *__restrict__ xv, const float *__restrict__ eta,
                                          float *__restrict__ Ws, float *__restrict__ bs, float gm,
                                          float bt, TIO *__restrict__ o, int mb, int pos,
                                          float *__restrict__ Wcs, float *__restrict__ bcs,
                                          float thj, float eta_base) {
    using io = io_traits<TIO>;
    constexpr float inv_d = 1.0f / DM;
    float w[DM];  // W[i][j], i = 0 .. 63
#pragma unroll
    for (int i = 0; i < DM; ++i) w[i] = Ws[i * DM + j];
    float bj = bs[j];
    float wc[DM];  // CH: chunk-start W[i][j] (read when the first step continues a chunk)
    float bcj = 0.f;
    if constexpr (CH) {
        if (pos > 0) {
#pragma unroll
            for (int i = 0; i < DM; ++i) wc[i] = Wcs[i * DM + j];
            bcj = bcs[j];
        }
    }
    int k = pos;  // CH: position of step t within its chunk
    // per-head constants of the general layer-norm backward
    float Sg2 = static_cast<float>(DM), Sgb = 0.f;
    if constexpr (!IDENT) {
        Sg2 = wave_sum(gm * gm);
        Sgb = wave_sum(gm * bt);
    }
    const float g2 = gm * gm;

    size_t base = static_cast<size_t>(seq) * DM;  // step 0
    Raw<TIO> rq, rk;
    rq.load(xq + base, j);
    rk.load(xk + base, j);
    TIO rv = xv[base + j];
    float et = GATED ? 0.f : eta[seq];

    for (int t = 0; t < T; ++t) {
        const bool more = t + 1 < T;  // uniform
        const size_t nbase = base + static_cast<size_t>(BH) * DM;
        float qb[4], kb[4];
        rq.bcast(qb);
        rk.bcast(kb);
        const float xqj = rq.own(), xkj = rk.own(), xvj = io::load(&rv, 0);
        float etc = et;
        // the next step's inputs, in flight during this one
        if (more) {
            rq.load(xq + nbase, j);
            rk.load(xk + nbase, j);
            rv = xv[nbase + j];
            if constexpr (!GATED) et = eta[static_cast<size_t>(t + 1) * BH + seq];
        }
        const float tau = xvj - xkj;
        float qk;
        if constexpr (GATED) {  // xq . xk and theta . xk in one pair of wave sums
            const f32x4 s = wave_sum2(xqj * xkj, thj * xkj);
            qk = s[0];
            etc = eta_base * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * s[2]));
        } else {
            qk = wave_sum(xqj * xkj);
        }

        // (xq W)_j and z_j = (xk W + b)_j, W, b at the chunk start for z
        float p0 = 0.f, p1 = 0.f, z0, z1 = 0.f;
        dot_bcast(qb, w, p0, p1, Rows16{});
        if constexpr (CH) {
            if (k == 0) {  // a chunk starts: its start state is the current one
#pragma unroll
                for (int i = 0; i < DM; ++i) wc[i] = w[i];
                bcj = bj;
            }
            z0 = bcj;
            dot_bcast(kb, wc, z0, z1, Rows16{});
            k = (k + 1 == mb) ? 0 : k + 1;
        } else {
            z0 = bj;
            dot_bcast(kb, w, z0, z1, Rows16{});
        }
        const float z = z0 + z1, p = p0 + p1;

        // E_j = -eta * d/dz_j [ 1/2 || LN(z) - tau ||^2 ]
        float e;
        if constexpr (IDENT) {
            const f32x4 s = wave_sum4(z, z * z, tau * z, tau);
            const float mu = s[0] * inv_d, mut = s[3] * inv_d;
            const float var = fmaxf(fmaf(s[1], inv_d, -mu * mu), 0.f);
            const float r = rsq(var + eps);
            const float r2 = r * r;
            const float a = r2 * fmaf(r, fmaf(s[2], inv_d, -mut * mu), eps * r2);
            e = -etc * fmaf(a, z - mu, -r * (tau - mut));
        } else {
            const f32x4 s = wave_sum4(z, z * z, g2 * z, g2 * z * z);
            const f32x4 s2 = wave_sum4(gm * bt * z, gm * tau * z, gm * tau, 0.f);
            const float mu = s[0] * inv_d;
            const float var = fmaxf(fmaf(s[1], inv_d, -mu * mu), 0.f);
            const float r = rsq(var + eps);
            // mean(ghat) and mean(ghat xhat), ghat = gamma (gamma xhat + beta - tau)
            const float m1 = (fmaf(r, fmaf(-mu, Sg2, s[2]), Sgb) - s2[2]) * inv_d;
            const float q2 = fmaf(mu, fmaf(mu, Sg2, -2.f * s[2]), s[3]);
            const float q1 = fmaf(-mu, Sgb, s2[0]) - fmaf(-mu, s2[2], s2[1]);
            const float m2 = fmaf(r * r, q2, r * q1) * inv_d;
            e = -etc * r * (fmaf(r * (g2 - m2), z - mu, gm * (bt - tau)) - m1);
        }

        // W += xk^T E (column j)
        axpy_bcast(kb, e, w, Rows16{});

        // o = xq + LN(xq W' + b'),  xq W' + b' = xq W + b + (xq . xk + 1) E
        const float zb = fmaf(qk + 1.f, e, p + bj);
        bj += e;
        const f32x4 f = wave_sum2(zb, zb * zb);
        const float mu = f[0] * inv_d;
        const float r = rsq(fmaxf(fmaf(f[2], inv_d, -mu * mu), 0.f) + eps);
        io::store(o, base + j, IDENT ? fmaf(zb - mu, r, xqj) : xqj + fmaf(gm, (zb - mu) * r, bt));

        base = nbase;
    }
#pragma unroll
    for (int i = 0; i < DM; ++i) Ws[i * DM + j] = w[i];
    bs[j] = bj;
    if constexpr (CH) {  // the start state of the chunk the last step belongs to
#pragma unroll
        for (int i = 0; i < DM; ++i) Wcs[i * DM + j] = wc[i];
        bcs[j] = bcj;
    }
}

template <typename TIO, bool CH, bool GATED>
__global__ __launch_bounds__(64) void decode_steps_kernel(
    int T, int BH, int H, float eps, const TIO *__restrict__ xq, const TIO *__restrict__ xk,
    const TIO *__restrict__ xv, const float *__restrict__ eta, float *__restrict__ W,
    float *__restrict__ b, const float *__restrict__ gamma, const float *__restrict__ beta,
    TIO *__restrict__ o, int mb, int pos, float *__restrict__ Wc, float *__restrict__ bc,
    const float *__restrict__ theta, float eta_base) {
    const int j = threadIdx.x;
    const int seq = blockIdx.x;
    const int h = seq % H;
    float *Ws = W + static_cast<size_t>(seq) * DM * DM;
    float *bs = b + static_cast<size_t>(seq) * DM;
    float *Wcs = CH ? Wc + static_cast<size_t>(seq) * DM * DM : nullptr;
    float *bcs = CH ? bc + static_cast<size_t>(seq) * DM : nullptr;
    const float gm = gamma[h * DM + j], bt = beta[h * DM + j];
    const float thj = GATED ? theta[h * DM + j] : 0.f;
    if (__all(gm == 1.0f && bt == 0.0f))
        run_steps<TIO, true, CH, GATED>(T, BH, eps, seq, j, xq, xk, xv, eta, Ws, bs, gm, bt, o, mb,
                                        pos, Wcs, bcs, thj, eta_base);
    else
        run_steps<TIO, false, CH, GATED>(T, BH, eps, seq, j, xq, xk, xv, eta, Ws, bs, gm, bt, o, mb,
                                         pos, Wcs, bcs, thj, eta_base);
}

template <typename TIO, bool CH, bool GATED>
hipError_t launch_steps_t(const DecodeArgs &a, int T, hipStream_t stream) {
    hipLaunchKernelGGL((decode_steps_kernel<TIO, CH, GATED>), dim3(a.B * a.H), dim3(64), 0, stream, T,
                       a.B * a.H, a.H, a.eps, static_cast<const TIO *>(a.xq),
                       static_cast<const TIO *>(a.xk), static_cast<const TIO *>(a.xv), a.eta, a.W,
                       a.b, a.gamma, a.beta, static_cast<TIO *>(a.o), a.mb, a.pos, a.Wc, a.bc,
                       a.theta, a.eta_base);
    return hipGetLastError();
}

}  // namespace

bool decode_steps_resident(int d) { return d == DM; }

hipError_t launch_decode_steps(const DecodeArgs &a, int T, hipStream_t stream) {
    if (a.B * a.H == 0 || T == 0) return hipSuccess;
    const bool ch = a.Wc != nullptr;  // mini-batch decode
    if (a.theta) {
        if (a.io) return ch ? launch_steps_t<bf16_t, true, true>(a, T, stream) : launch_steps_t<bf16_t, false, true>(a, T, stream);
        return ch ? launch_steps_t<float, true, true>(a, T, stream) : launch_steps_t<float, false, true>(a, T, stream);
    }
    if (a.io) return ch ? launch_steps_t<bf16_t, true, false>(a, T, stream) : launch_steps_t<bf16_t, false, false>(a, T, stream);
    return ch ? launch_steps_t<float, true, false>(a, T, stream) : launch_steps_t<float, false, false>(a, T, stream);
}

}  // namespace ttt
