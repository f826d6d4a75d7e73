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

// DPP row-broadcast FMAs. Element i = 4 n + m of a broadcast-layout vector
// x (see Raw below) is x[m] of lane n of each 16-lane DPP row, so
// row_newbcast:n as the FMA's own source modifier hands it to every lane at
// no cost. The compiler does not fold a DPP move into an FMA, so these are
// written in assembly, sixteen FMAs (rows 4 NB .. 4 NB + 3) to a block. A DPP
// instruction must not read a VGPR within two wait states of a VALU write to
// it (five after an EXEC write); each block therefore opens with s_nop 4 and
// takes every register it reads as an operand, so nothing the compiler
// schedules can fall between the guard and the FMAs. Inside a block no FMA
// reads a register written by either of the two instructions before it: the
// dot product rotates four accumulators (one per m) and the update writes
// sixteen distinct elements.

// a[m] += sum over n in 4 NB .. 4 NB + 3 of x_{4n+m} w[4n+m]
template <int NB>
__device__ __forceinline__ void dot_block(const float (&x)[4], const float (&w)[DM], float (&a)[4]) {
    asm("s_nop 4\n\t"
        "v_fmac_f32_dpp %0, %4, %8 row_newbcast:%24 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %9 row_newbcast:%24 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %10 row_newbcast:%24 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %11 row_newbcast:%24 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %12 row_newbcast:%25 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %13 row_newbcast:%25 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %14 row_newbcast:%25 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %15 row_newbcast:%25 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %16 row_newbcast:%26 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %17 row_newbcast:%26 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %18 row_newbcast:%26 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %19 row_newbcast:%26 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %20 row_newbcast:%27 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %21 row_newbcast:%27 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %22 row_newbcast:%27 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %23 row_newbcast:%27 row_mask:0xf bank_mask:0xf\n\t"
        : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3])
        : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(w[16 * NB + 0]), "v"(w[16 * NB + 1]),
          "v"(w[16 * NB + 2]), "v"(w[16 * NB + 3]), "v"(w[16 * NB + 4]), "v"(w[16 * NB + 5]),
          "v"(w[16 * NB + 6]), "v"(w[16 * NB + 7]), "v"(w[16 * NB + 8]), "v"(w[16 * NB + 9]),
          "v"(w[16 * NB + 10]), "v"(w[16 * NB + 11]), "v"(w[16 * NB + 12]), "v"(w[16 * NB + 13]),
          "v"(w[16 * NB + 14]), "v"(w[16 * NB + 15]), "n"(4 * NB), "n"(4 * NB + 1), "n"(4 * NB + 2),
          "n"(4 * NB + 3));
}
// w[4n+m] += x_{4n+m} e for n in 4 NB .. 4 NB + 3
template <int NB>
__device__ __forceinline__ void axpy_block(const float (&x)[4], float e, float (&w)[DM]) {
    asm("s_nop 4\n\t"
        "v_fmac_f32_dpp %0, %16, %20 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %17, %20 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %18, %20 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %19, %20 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %16, %20 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %17, %20 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %18, %20 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %19, %20 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %8, %16, %20 row_newbcast:%23 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %9, %17, %20 row_newbcast:%23 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %10, %18, %20 row_newbcast:%23 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %11, %19, %20 row_newbcast:%23 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %12, %16, %20 row_newbcast:%24 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %13, %17, %20 row_newbcast:%24 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %14, %18, %20 row_newbcast:%24 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %15, %19, %20 row_newbcast:%24 row_mask:0xf bank_mask:0xf\n\t"
        : "+v"(w[16 * NB + 0]), "+v"(w[16 * NB + 1]), "+v"(w[16 * NB + 2]), "+v"(w[16 * NB + 3]),
          "+v"(w[16 * NB + 4]), "+v"(w[16 * NB + 5]), "+v"(w[16 * NB + 6]), "+v"(w[16 * NB + 7]),
          "+v"(w[16 * NB + 8]), "+v"(w[16 * NB + 9]), "+v"(w[16 * NB + 10]), "+v"(w[16 * NB + 11]),
          "+v"(w[16 * NB + 12]), "+v"(w[16 * NB + 13]), "+v"(w[16 * NB + 14]), "+v"(w[16 * NB + 15])
        : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(e), "n"(4 * NB), "n"(4 * NB + 1),
          "n"(4 * NB + 2), "n"(4 * NB + 3));
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

// sum over i of x_i w[i], as four partial sums
__device__ __forceinline__ float dot64(const float (&x)[4], const float (&w)[DM], float init) {
    float a[4] = {init, 0.f, 0.f, 0.f};
    dot_block<0>(x, w, a);
    dot_block<1>(x, w, a);
    dot_block<2>(x, w, a);
    dot_block<3>(x, w, a);
    return (a[0] + a[1]) + (a[2] + a[3]);
}
// w[i] += x_i e
__device__ __forceinline__ void axpy64(const float (&x)[4], float e, float (&w)[DM]) {
    axpy_block<0>(x, e, w);
    axpy_block<1>(x, e, w);
    axpy_block<2>(x, e, w);
    axpy_block<3>(x, e, w);
}

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
    // Centred state for the whole call: W - wbar 1^T and b - bbar (wbar the
    // row means of W, bbar the mean of b, each wave sum bitwise identical in
    // every lane). Every z and zbar then moves by a per-token constant that
    // the layer norm and its backward do not see, and the per-step updates
    // (rows of E sum to zero, so they keep the centring) accumulate into
    // small numbers instead of into a large offset, whose fp32 spacing would
    // swallow them. The chunk-start copy takes the same shift. The caller's
    // representation is restored before the state is stored.
    float wb_own = 0.f;  // lane j keeps wbar_j for the way out
#pragma unroll
    for (int i = 0; i < DM; ++i) {
        const float m = wave_sum(w[i]) * inv_d;
        wb_own = (i == j) ? m : wb_own;
        w[i] -= m;
        if constexpr (CH) {
            if (pos > 0) wc[i] -= m;  // (pos == 0: set when the first step starts its chunk)
        }
        __builtin_amdgcn_sched_barrier(0);  // one reduction at a time: no register peak here
    }
    asm volatile("" : "+v"(wb_own));  // formed here, not sunk to its use after the loop
    const float bbar = wave_sum(bj) * inv_d;
    bj -= bbar;
    if constexpr (CH) bcj -= bbar;
    int k = pos;  // CH: position of step t within its chunk
    // per-head constants of the general layer-norm backward
    float Sgb = 0.f;
    if constexpr (!IDENT) Sgb = wave_sum(gm * bt);
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

        // (xq W)_j and z_j = (xk W + b)_j, W, b at the chunk start for z
        const float p = dot64(qb, w, 0.f);
        float z;
        if constexpr (CH) {
            if (k == 0) {  // a chunk starts: its start state is the current one
#pragma unroll
                for (int i = 0; i < DM; ++i) wc[i] = w[i];
                bcj = bj;
            }
            z = dot64(kb, wc, bcj);
            k = (k + 1 == mb) ? 0 : k + 1;
        } else {
            z = dot64(kb, w, bj);
        }

        // E_j = -eta * d/dz_j [ 1/2 || LN(z) - tau ||^2 ]. Layer-norm sums in
        // two rounds: the means first (with xq . xk and the gate's theta . xk),
        // then sums of centred products, so a large common offset of z cancels
        // exactly instead of in E[z^2] - mu^2.
        const float qkp = xqj * xkj, thp = GATED ? thj * xkj : 0.f;
        float e, qk;
        if constexpr (IDENT) {
            const f32x4 s = wave_sum4(z, tau, qkp, thp);
            qk = s[2];
            if constexpr (GATED)
                etc = eta_base * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * s[3]));
            const float cz = z - s[0] * inv_d, ct = tau - s[1] * inv_d;
            const f32x4 q = wave_sum2(cz * cz, ct * cz);
            const float r = rsq(fmaf(q[0], inv_d, eps));
            const float r2 = r * r;
            // a = r^2 (eps r^2 + r mean((tau - mean tau)(z - mu)))
            const float a = r2 * fmaf(r, q[2] * inv_d, eps * r2);
            e = -etc * fmaf(a, cz, -r * ct);
        } else {
            const f32x4 s = wave_sum4(z, gm * tau, qkp, thp);
            qk = s[2];
            if constexpr (GATED)
                etc = eta_base * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * s[3]));
            const float cz = z - s[0] * inv_d;
            const float gbt = gm * (bt - tau);
            const f32x4 q = wave_sum4(cz * cz, g2 * cz, g2 * cz * cz, gbt * cz);
            const float r = rsq(fmaf(q[0], inv_d, eps));
            // mean(ghat) and mean(ghat xhat), ghat = gamma (gamma xhat + beta - tau), xhat = r cz
            const float m1 = (fmaf(r, q[1], Sgb) - s[1]) * inv_d;
            const float m2 = r * fmaf(r, q[2], q[3]) * inv_d;
            e = -etc * r * (fmaf(r * (g2 - m2), cz, gbt) - m1);
        }

        // W += xk^T E (column j)
        axpy64(kb, e, w);

        // o = xq + LN(xq W' + b'),  xq W' + b' = xq W + b + (xq . xk + 1) E
        const float zb = fmaf(qk + 1.f, e, p + bj);
        bj += e;
        const float cb = zb - wave_sum(zb) * inv_d;
        const float r = rsq(fmaf(wave_sum(cb * cb), inv_d, eps));
        io::store(o, base + j, IDENT ? fmaf(cb, r, xqj) : xqj + fmaf(gm, cb * r, bt));

        base = nbase;
    }
    // wbar in the broadcast layout (lane l: elements 4 (l mod 16) + m), then
    // w[i] += 1 * wbar_i with the broadcast FMAs (exact product, one rounding)
    float wbb[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
        wbb[m] = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (4 * (j & 15) + m), __float_as_int(wb_own)));
    axpy64(wbb, 1.0f, w);
    if constexpr (CH) axpy64(wbb, 1.0f, wc);  // the start state of the last step's chunk
#pragma unroll
    for (int i = 0; i < DM; ++i) Ws[i * DM + j] = w[i];
    bs[j] = bj + bbar;
    if constexpr (CH) {
#pragma unroll
        for (int i = 0; i < DM; ++i) Wcs[i * DM + j] = wc[i];
        bcs[j] = bcj + bbar;
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
