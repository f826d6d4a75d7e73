// Input projections of the layer: the query, key and value views XQ, XK, XV
// of the layer input X, made by the outer-loop weights theta_Q, theta_K,
// theta_V (lryc.cn TTT article §2.2; the damodev.csdn.net deep-dive §4.2
// feeds the three views to the inner loop):
//     out_v[b,h,t,j] = sum_k X[b,t,k] theta[v][h d + j][k],   v = Q, K, V.
//
// One bf16 GEMM with fp32 accumulation, computed transposed, C^T = Theta X^T:
// rows = the 3 H d output features, columns = the B L tokens, contraction
// over d_model. With Theta as the A operand of the 16x16x32 MFMA, a lane's
// four accumulator values are four consecutive features of one token, which
// go straight to the [B,H,L,d] layout the prefill kernels read as one 8-byte
// store.
//  * block tile 256 features x 256 tokens, contraction steps of 64; 8 waves
//    (2 along the features x 4 along the tokens), 128 x 64 per wave = 8 x 4
//    MFMA tiles, 32 fp32 accumulator quads;
//  * operands staged in LDS, two stages, by direct global-to-LDS loads: each
//    step's loads into the other stage are issued before its MFMAs and land
//    while they run (no register staging, no LDS store instructions), one
//    barrier per step after a wait for this wave's loads. A load instruction
//    puts lane i at 16 i bytes, so rows are unpadded 128 bytes with their
//    16-byte chunks XOR-swizzled by row & 7: the 8 rows that one fragment
//    read's lanes c = 0 .. 7 touch then use distinct chunk positions. Within
//    a step each A fragment is read three groups ahead of its four products;
//  * XCD-aware order: workgroups go to the 8 XCDs round robin and workgroup
//    i takes feature block i % nfb of token block i / nfb. When the number of
//    feature blocks nfb is a multiple of 8, XCD x is given the feature blocks
//    x, x + 8, ... (its slice of Theta stays in its L2) over every token
//    block; otherwise the blocks still spread evenly over the XCDs.
#include "launch.hpp"
#include "tile.hpp"

namespace ttt {
namespace {

using namespace tile;

constexpr int PT = 256;  // tokens per block
constexpr int PK = 64;   // contraction step
constexpr int PNT = 512; // threads (8 waves)
constexpr int WT = 64;   // tokens per wave tile

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;  // 16 bytes

// PF output features per block (256, or 128 when the 256-feature tiles would
// leave most compute units idle in a last round); a wave tile is PF / 2 x 64
template <int PF>
struct ProjSmem {
    uint16_t a[2][PF * PK];  // Theta rows [feature][k], 16-byte chunks XOR-swizzled by row & 7
    uint16_t b[2][PT * PK];  // X rows [token][k], same swizzle
};
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void glb_void;

template <int PF>
__global__ __launch_bounds__(PNT) void qkv_project_kernel(int NF, int M, int K, int HD, int H, int L,
                                                          const bf16_t *X, const bf16_t *theta,
                                                          bf16_t *XQ, bf16_t *XK, bf16_t *XV) {
    constexpr int WF = PF / 2, NTA = WF / 16;  // features per wave tile, its MFMA row tiles
    __shared__ ProjSmem<PF> sm;
    const int nfb = (NF + PF - 1) / PF;
    const int blk_id = blockIdx.x, fb = blk_id % nfb, tb = blk_id / nfb;
    const int f0 = fb * PF, t0 = tb * PT;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c = lane & 15;
    const int wf0 = (w & 1) * WF, wt0 = (w >> 1) * WT;

    // global -> LDS directly: wave w, instruction q fills rows 8 (4w + q) .. +7
    // (1 KB) of X, and for q < PF / 64 rows 8 ((PF / 64) w + q) .. +7 of Theta; lane i lands
    // at 16 i bytes, i.e. row 8 blk + i / 8, physical
    // chunk i % 8, which holds logical chunk (i % 8) ^ (i / 8) of that row.
    // Rows past the end read row 0: a feature row only reaches the outputs of
    // that feature and a token row those of that token, which are not stored,
    // so the values need no masking.
    auto dma = [&](int kt, int stg) {
        const int k0 = kt * PK;
        const int rl = lane >> 3, lc = (lane & 7) ^ rl;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int blk = 4 * w + q, tr = t0 + 8 * blk + rl;
            const bf16_t *sb = X + static_cast<size_t>(tr < M ? tr : 0) * K + k0 + lc * 8;
            if (q < PF / 64) {  // compile-time after unrolling; Theta rows 8 ((PF / 64) w + q) .. +7
                const int blka = (PF / 64) * w + q, fr = f0 + 8 * blka + rl;
                const bf16_t *sa = theta + static_cast<size_t>(fr < NF ? fr : 0) * K + k0 + lc * 8;
                __builtin_amdgcn_global_load_lds((glb_void *)sa, (lds_void *)&sm.a[stg][8 * blka * PK], 16, 0, 0);
            }
            __builtin_amdgcn_global_load_lds((glb_void *)sb, (lds_void *)&sm.b[stg][8 * blk * PK], 16, 0, 0);
        }
    };

    f32x4 acc[NTA][4];
#pragma unroll
    for (int t = 0; t < NTA; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[t][s] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = K / PK;
    dma(0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        if (kt + 1 < nk) dma(kt + 1, st ^ 1);
        __builtin_amdgcn_sched_barrier(0);
        auto rd_a = [&](int idx) {
            const int kk = idx / NTA, t = idx % NTA;
            const int j = (4 * kk + g) ^ (c & 7);
            return __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4 *>(&sm.a[st][(wf0 + 16 * t + c) * PK + 8 * j]));
        };
        auto rd_x = [&](int kk, int s) {
            const int j = (4 * kk + g) ^ (c & 7);
            return __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4 *>(&sm.b[st][(wt0 + 16 * s + c) * PK + 8 * j]));
        };
        constexpr int PD = 3, NG = 2 * NTA;  // read-ahead depth; groups of four products per step
        bf16x8 fa[NG], fx[2][4];
#pragma unroll
        for (int s = 0; s < 4; ++s) fx[0][s] = rd_x(0, s);
#pragma unroll
        for (int i = 0; i < PD; ++i) fa[i] = rd_a(i);
#pragma unroll
        for (int idx = 0; idx < NG; ++idx) {
            if (idx + PD < NG) fa[idx + PD] = rd_a(idx + PD);
            if (idx == 2) {
#pragma unroll
                for (int s = 0; s < 4; ++s) fx[1][s] = rd_x(1, s);
            }
            __builtin_amdgcn_sched_barrier(0);
            const int kk = idx / NTA, t = idx % NTA;
#pragma unroll
            for (int s = 0; s < 4; ++s) acc[t][s] = mfma32(fa[idx], fx[kk][s], acc[t][s]);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads into the other stage have landed
        __syncthreads();
    }

    // lane (g, c) of tile (t, s): features f0 + wf0 + 16 t + 4 g .. +3 of token t0 + wt0 + 16 s + c
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int m = t0 + wt0 + 16 * s + c;
        if (m >= M) continue;
        const int bi = m / L, tp = m - bi * L;
#pragma unroll
        for (int t = 0; t < NTA; ++t) {
            const int n = f0 + wf0 + 16 * t + 4 * g;
            if (n >= NF) continue;
            const int v = n / HD, hj = n - v * HD, h = hj / D, j = hj - h * D;
            bf16_t *out = v == 0 ? XQ : (v == 1 ? XK : XV);
            bf16_t *dst = out + ((static_cast<size_t>(bi) * H + h) * L + tp) * D + j;
            *reinterpret_cast<uint2 *>(dst) = make_uint2(pack2(acc[t][s][0], acc[t][s][1]),
                                                        pack2(acc[t][s][2], acc[t][s][3]));
        }
    }
}

}  // namespace

template <int PF>
hipError_t launch_pf(int NF, int M, int dm, int HD, int H, int L, const void *X, const void *theta, void *XQ,
                     void *XK, void *XV, hipStream_t stream) {
    const long blocks = static_cast<long>((NF + PF - 1) / PF) * ((M + PT - 1) / PT);
    hipLaunchKernelGGL(qkv_project_kernel<PF>, dim3(static_cast<unsigned>(blocks)), dim3(PNT), 0, stream, NF, M,
                       dm, HD, H, L, static_cast<const bf16_t *>(X), static_cast<const bf16_t *>(theta),
                       static_cast<bf16_t *>(XQ), static_cast<bf16_t *>(XK), static_cast<bf16_t *>(XV));
    return hipGetLastError();
}

hipError_t launch_qkv_project(int B, int L, int dm, int H, const void *X, const void *theta, void *XQ,
                              void *XK, void *XV, hipStream_t stream) {
    const int HD = H * D, NF = 3 * HD;
    const long Ml = static_cast<long>(B) * L;
    const int M = static_cast<int>(Ml);
    const long ntb = (M + PT - 1) / PT, t256 = ntb * ((NF + 255) / 256), t128 = ntb * ((NF + 127) / 128);
    if (t256 <= 0) return hipSuccess;
    // One 256 x 256 tile per compute unit at a time (128 KB of LDS). Rounds of the grid over the
    // chip, a 128-feature tile costing about 0.6 of a 256-feature one: take the 128-feature tiles
    // when they finish in fewer tile-times.
    int dev = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    ncu = ncu > 0 ? ncu : 1;
    const long r256 = (t256 + ncu - 1) / ncu, r128 = (t128 + ncu - 1) / ncu;
    if (3 * r128 < 5 * r256)
        return launch_pf<128>(NF, M, dm, HD, H, L, X, theta, XQ, XK, XV, stream);
    return launch_pf<256>(NF, M, dm, HD, H, L, X, theta, XQ, XK, XV, stream);
}

}  // namespace ttt
