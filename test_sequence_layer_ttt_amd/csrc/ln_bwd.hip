// Fused layer-norm + L2 backward, row-wise (the "ln_fused_l2_bwd" step of the
// damodev.csdn.net TTT deep-dive, §4.2): for each row,
//   G = d/dz 1/2 ||LN_{gamma,beta}(z) - target||^2.
// Sixteen lanes share a row (D/16 features each); the four row reductions are
// 16-lane butterflies. 16 rows per 256-thread block.
#include "common.hpp"
#include "launch.hpp"

namespace ttt {

template <int D>
__global__ __launch_bounds__(256) void ln_l2_bwd_kernel(int rows, const float *__restrict__ Z,
                                                        const float *__restrict__ T,
                                                        const float *__restrict__ gamma,
                                                        const float *__restrict__ beta,
                                                        float eps, float *__restrict__ G) {
    constexpr int GL = 16, E = D / GL;
    const int lane = threadIdx.x % GL;
    const long row = static_cast<long>(blockIdx.x) * 16 + threadIdx.x / GL;
    const bool valid = row < rows;
    const long r = valid ? row : 0;  // every lane of a group takes part in the shuffles
    float z[E], t[E], g[E], b[E], out[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int j = lane + GL * e;
        z[e] = valid ? Z[r * D + j] : 0.f;
        t[e] = valid ? T[r * D + j] : 0.f;
        g[e] = gamma[j];
        b[e] = beta[j];
    }
    ln_l2_grad<GL, E>(z, t, g, b, 1.0f / D, eps, out);
    if (valid) {
#pragma unroll
        for (int e = 0; e < E; ++e) G[r * D + lane + GL * e] = out[e];
    }
}

hipError_t launch_ln_l2_bwd(int rows, int d, const float *Z, const float *T, const float *gamma,
                            const float *beta, float eps, float *G, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    const dim3 grid((rows + 15) / 16), block(256);
    switch (d) {
    case 16: hipLaunchKernelGGL(ln_l2_bwd_kernel<16>, grid, block, 0, stream, rows, Z, T, gamma, beta, eps, G); break;
    case 32: hipLaunchKernelGGL(ln_l2_bwd_kernel<32>, grid, block, 0, stream, rows, Z, T, gamma, beta, eps, G); break;
    case 64: hipLaunchKernelGGL(ln_l2_bwd_kernel<64>, grid, block, 0, stream, rows, Z, T, gamma, beta, eps, G); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ttt
