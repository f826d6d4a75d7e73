// Internal launchers (host side) of libttt.so. Arguments are validated by the
// C ABI before these are called; each enqueues on `stream` and returns the
// launch status.
#pragma once

#include <hip/hip_runtime.h>

namespace ttt {

struct LinearArgs {
    int B, H, L, d, mb, io;
    float eps;
    const void *XQ, *XK, *XV;
    const float *eta, *W0, *b0;
    int w0_batched;
    const float *gamma, *beta;
    void *O;
    float *W_out, *b_out;
    // learning-rate gate: when theta is set, eta is ignored and each token's
    // rate is eta_base * logistic(theta[h] . XK_t), evaluated in the kernel
    const float *theta = nullptr;
    float eta_base = 0.f;
    // inner loss (0: squared reconstruction error, 1: inner product) and
    // weight decay lambda on W; the MFMA kernel takes only the defaults
    int loss = 0;
    float wd = 0.f;
};

struct LinearBwdArgs {
    LinearArgs f;  // forward arguments (O, W_out, b_out unused)
    const float *dO, *dW_out, *db_out;
    float *dXQ, *dXK, *dXV, *deta, *dW0, *db0, *dgamma, *dbeta;
    float *ws;  // chunk-start states and chunk records: B*H*ceil(L/mb)*linear_backward_chunk_floats
};

struct MLPArgs {
    int B, H, L, d, mb, io;
    float eps;
    const void *XQ, *XK, *XV;
    const float *eta, *W1, *b1, *W2, *b2;
    int w0_batched;
    const float *gamma, *beta;
    void *O;
    float *W1_out, *b1_out, *W2_out, *b2_out;
    int loss = 0;    // 0 squared error, 1 inner product
    float wd = 0.f;  // weight decay on W1 and W2
    const float *theta = nullptr;  // learning-rate gate [H,d] (eta unused when set)
    float eta_base = 0.f;
};

struct MLPBwdArgs {
    MLPArgs f;  // forward arguments (O and the state outputs unused)
    const float *dO, *dW1_out, *db1_out, *dW2_out, *db2_out;
    float *dXQ, *dXK, *dXV, *deta, *dW1, *db1, *dW2, *db2, *dgamma, *dbeta;
    float *ws;  // chunk-start states, two adjoint states and chunk records: B*H*mlp_backward_seq_floats
};

struct DecodeArgs {
    int B, H, d, io;
    float eps;
    const void *xq, *xk, *xv;
    const float *eta;
    float *W, *b;
    const float *gamma, *beta;
    void *o;
    // mini-batch decode (b = mb > 1): every token of a chunk takes its
    // gradient at the chunk-start state (Wc, bc). Single-step kernel: mode
    // 1 starts a chunk (Wc, bc <- W, b first), mode 2 continues one; multi-
    // step kernel: pos = position of the first step within its chunk.
    float *Wc = nullptr, *bc = nullptr;
    int mode = 0, mb = 1, pos = 0;
    // learning-rate gate: eta_t = eta_base * logistic(theta[h] . xk_t) in the
    // kernel (eta unused when theta is set)
    const float *theta = nullptr;
    float eta_base = 0.f;
};

hipError_t launch_ln_l2_bwd(int rows, int d, const float *Z, const float *T, const float *gamma,
                            const float *beta, float eps, float *G, hipStream_t stream);
hipError_t launch_linear_valu(const LinearArgs &a, hipStream_t stream);
bool linear_mfma_supported(const LinearArgs &a);
hipError_t launch_linear_mfma(const LinearArgs &a, hipStream_t stream);
hipError_t launch_qkv_project(int B, int L, int dm, int H, const void *X, const void *theta, void *XQ,
                              void *XK, void *XV, hipStream_t stream);
hipError_t launch_eta_gate(int B, int H, int L, int d, int io, const void *XK, const float *theta,
                           float eta_base, float *eta, hipStream_t stream);
hipError_t launch_eta_gate_backward(int B, int H, int L, int d, int io, const void *XK,
                                    const float *theta, float eta_base, const float *deta,
                                    float *dXK, float *dtheta, hipStream_t stream);

size_t linear_backward_chunk_floats(int d);  // workspace floats per sequence and chunk
// the fixed device scratch of ttt_linear_backward_noalloc: its size, and its
// address on the current device
size_t linear_backward_scratch_bytes();
hipError_t linear_backward_scratch(float **ptr);
hipError_t launch_linear_backward(const LinearBwdArgs &a, hipStream_t stream);
size_t mlp_backward_seq_floats(int L, int d, int mb);  // workspace floats per sequence
hipError_t launch_mlp_backward(const MLPBwdArgs &a, hipStream_t stream);
hipError_t launch_mlp(const MLPArgs &a, hipStream_t stream);
bool mlp_mfma_supported(const MLPArgs &a);
hipError_t launch_mlp_mfma(const MLPArgs &a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
bool decode_steps_resident(int d);
hipError_t launch_decode_steps(const DecodeArgs &a, int T, hipStream_t stream);

}  // namespace ttt
