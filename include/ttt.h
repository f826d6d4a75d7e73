/*
 * ttt.h -- C ABI of libttt.so: the TTT layer inner loop on AMD Instinct MI355X
 * (gfx950).
 *
 * Source pages (citation key):
 *   [D] damodev.csdn.net TTT deep-dive: §3.1 update/apply equation, §4.1
 *       mini-batch TTT, §4.2 inner-loop excerpt (reconstruction target
 *       XV - XK, forward XK W + b, fused LN + L2 backward, dual-form state
 *       update), §4.3 fast-weight shapes [heads, d, d] and [heads, 1, d],
 *       §5.2 the fast-weight cache used for decode.
 *   [Y] lryc.cn "测试时学习（TTT）" article: §2.1 LN-residual output
 *       f(x) = x + LN(f_res(x)) and the d -> 4d GELU -> d MLP, §2.2 the
 *       per-token learning-rate gate, §2.4 mini-batch b = 16 and the dual form.
 *   [X] xiaohu.ai TTT summary: mini-batch TTT and the dual form.
 *   [M] ai-feeds.com "Modular TTT" summary: inner loss (MSE or inner
 *       product) and weight decay as design axes of the fast-weight learner.
 *
 * Computation (per independent sequence (n,h), tokens t = 0..L-1, chunks of
 * `mb` tokens aligned at t = 0, the last chunk possibly shorter):
 *   for each chunk, at the chunk-start state (W, b):
 *     G_s = d/dz [ 1/2 || LN_{gamma,beta}(z) - (xv_s - xk_s) ||^2 ] at
 *           z = xk_s W + b                                   ([D] §4.2)
 *   then for each token t of the chunk, in order:
 *     W <- W - eta_t xk_t^T G_t ;  b <- b - eta_t G_t        ([D] §3.1, §4.2)
 *     o_t = xq_t + LN_{gamma,beta}(xq_t W + b)               ([Y] §2.1)
 *   W_out, b_out = the state after the last token.
 * LN uses the biased variance over the d features with ln_eps inside the
 * square root; the same gamma/beta serve the loss and the output. Row-vector
 * convention: W[i][j] maps input feature i to output feature j.
 * The MLP variant replaces x W + b by GELU(x W1 + b1) W2 + b2 (exact GELU,
 * hidden width 4d) and updates W1, b1, W2, b2 with their gradients.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers to row-major contiguous arrays owned
 *     by the caller. The library never allocates, frees or synchronises; each
 *     call enqueues its kernel(s) on `stream` and returns.
 *   - Validation runs on the host before any HIP call. A pointer may be NULL
 *     only when the array it addresses has zero elements (or is documented as
 *     optional). Every pointer must be aligned to its element size; the
 *     prefill entry points also need 16-byte alignment of XQ, XK, XV, O and
 *     the state arrays (their kernels use 16-byte vector accesses).
 *   - Return value: TTT_OK (0) or a negative TTT_E_* code; ttt_last_error()
 *     then returns a message (thread-local, valid until the next call on the
 *     same thread). Faults inside a kernel surface at the caller's next
 *     synchronisation of `stream`.
 *   - Calls on one stream are ordered; calls that write the same buffers on
 *     different streams race.
 */
#ifndef TTT_H
#define TTT_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TTT_OK 0
#define TTT_E_NULL (-1)  /* a required pointer is NULL                          */
#define TTT_E_SHAPE (-2) /* negative size, unsupported d / mb, bad ln_eps or  */
                         /* another scalar argument out of its range         */
#define TTT_E_DTYPE (-3) /* io is not TTT_F32 / TTT_BF16                       */
#define TTT_E_ALIGN (-4) /* a pointer is not aligned as required               */
#define TTT_E_ALIAS (-5) /* an output overlaps an input or another output      */
#define TTT_E_HIP (-6)   /* the kernel launch failed                           */

/* Longest sequence any prefill entry point accepts (tokens per (n,h));
 * longer L is TTT_E_SHAPE. Token and chunk indices inside the kernels are
 * 32-bit ints; byte offsets are 64-bit. */
#define TTT_MAX_L (1 << 30)

/* Inner loss of ttt_linear_forward_opts and ttt_mlp_forward_opts. */
#define TTT_LOSS_MSE 0           /* 1/2 ||LN(f_res(XK)) - (XV - XK)||^2 per token */
#define TTT_LOSS_INNER_PRODUCT 1 /* -< XK + LN(f_res(XK)), XV > per token        */

/* Storage type of XQ/XK/XV and O. State, eta and LN parameters are fp32. */
typedef enum { TTT_F32 = 0, TTT_BF16 = 1 } ttt_dtype;

/*
 * TTT-Linear prefill over [B,H,L,d] inputs, mini-batch form, computed in the
 * dual form ([D] §4.2 dual branch; [X]; [Y] §2.4).
 *   B, H >= 0, L >= 0; d in {16, 64}; 1 <= mb <= 16. L need not be a multiple
 *   of mb: the last chunk is then shorter.
 *   io       : storage type of XQ, XK, XV, O.
 *   XQ,XK,XV : [B,H,L,d] io.         eta : [B,H,L] fp32 per-token rate
 *              (already gated, e.g. eta_base * sigmoid(theta_lr . x), [Y] §2.2).
 *   W0, b0   : fp32, [H,d,d] and [H,d] shared by every n when w0_batched == 0
 *              (the per-head parameter of [D] §4.3), else [B,H,d,d], [B,H,d].
 *   ln_gamma, ln_beta : [H,d] fp32.
 *   O        : [B,H,L,d] io, written.  Must not overlap any other argument.
 *   W_out, b_out : [B,H,d,d], [B,H,d] fp32, the final state; optional (NULL
 *              skips the store). With w0_batched == 1 they may be exactly
 *              W0 / b0 (in-place resume); any other overlap is TTT_E_ALIAS.
 *   ln_eps   : a positive normal float (>= FLT_MIN, finite), else TTT_E_SHAPE
 *              (the same for every entry point below). L > TTT_MAX_L is
 *              TTT_E_SHAPE (also for every prefill and backward entry point).
 *   W0 and b0 may carry any offset: the layer-norm statistics are sums of
 *   centred values (the bf16 d = 64 kernel holds the state with its row means
 *   removed, which shifts z by a per-token constant the layer norm does not
 *   see; the other kernels centre each row before squaring), so rows whose
 *   mean is large against their spread keep their accuracy.
 * Numerics: state, accumulation and layer-norm statistics in fp32. On the
 * bf16 path with d = 64 and mb = 16 the products XK W and XQ W take W and
 * the XQ / XK rows as fp16 MFMA operands (the bf16 inputs convert exactly;
 * |XQ|, |XK| and |W| must stay below 65504, the fp16 range); the products
 * with E and with the token x token matrices XK XK^T + 1 and XQ XK^T + 1
 * take bf16 operands.
 */
int ttt_linear_forward(int B, int H, int L, int d, int mb, int io, float ln_eps,
                       const void *XQ, const void *XK, const void *XV, const float *eta,
                       const float *W0, const float *b0, int w0_batched,
                       const float *ln_gamma, const float *ln_beta, void *O,
                       float *W_out, float *b_out, hipStream_t stream);

/*
 * ttt_linear_forward with each token's rate taken from the learning-rate gate
 * of [Y] §2.2 inside the kernel (no eta array is read):
 *   eta_t = eta_base * logistic(theta_lr[h] . XK_t),  logistic(s) = 1/(1+e^-s).
 * The gate input x is read as the head's key XK_t ([Y] leaves x open).
 *   theta_lr : [H,d] fp32, 16-byte aligned.  eta_base : finite, else TTT_E_SHAPE.
 * Every other argument, and the numerics, as ttt_linear_forward; the gate
 * itself is evaluated in fp32 (dot product, exp, divide).
 */
int ttt_linear_forward_gated(int B, int H, int L, int d, int mb, int io, float ln_eps,
                             const void *XQ, const void *XK, const void *XV,
                             const float *theta_lr, float eta_base, const float *W0,
                             const float *b0, int w0_batched, const float *ln_gamma,
                             const float *ln_beta, void *O, float *W_out, float *b_out,
                             hipStream_t stream);

/*
 * ttt_linear_forward with two design choices of the Modular-TTT page ([M]:
 * inner loss and weight decay on the fast weights), which names them without
 * an update rule; the readings taken:
 *   inner_loss   : TTT_LOSS_MSE (the layer above) or TTT_LOSS_INNER_PRODUCT,
 *                  each token's loss -< XK_t + LN(XK_t W + b), XV_t >; any other
 *                  value is TTT_E_SHAPE.
 *   weight_decay : lambda >= 0 (finite, else TTT_E_SHAPE); every token's loss
 *                  gains lambda/2 ||W||^2 (W only, not b), its gradient taken at
 *                  the chunk-start state W_c like the rest, so a chunk maps
 *                  W_c -> (1 - lambda * sum_t eta_t) W_c - (eta * XK)^T G.
 * Every other argument, and the numerics, as ttt_linear_forward: the bf16
 * path with d = 64 and mb = 16 runs the MFMA prefill for every option value
 * (the defaults, TTT_LOSS_MSE and 0, are exactly ttt_linear_forward), other
 * shapes the fp32 VALU prefill.
 */
int ttt_linear_forward_opts(int B, int H, int L, int d, int mb, int io, float ln_eps,
                            const void *XQ, const void *XK, const void *XV, const float *eta,
                            const float *W0, const float *b0, int w0_batched,
                            const float *ln_gamma, const float *ln_beta, int inner_loss,
                            float weight_decay, void *O, float *W_out, float *b_out,
                            hipStream_t stream);

/*
 * The learning-rate gate of [Y] §2.2 on its own, for the paths that take eta
 * as an array (the backward, the single-step decode, the prefills with the
 * loss options):
 *   eta[n,h,t] = eta_base * logistic(theta_lr[h] . XK[n,h,t]).
 *   B, H, L >= 0; d in {16, 32, 64}; io as above.
 *   XK [B,H,L,d] io, 16-byte aligned; theta_lr [H,d] fp32; eta [B,H,L] fp32,
 *   written, must not overlap XK or theta_lr. eta_base finite. fp32 throughout.
 */
int ttt_eta_gate(int B, int H, int L, int d, int io, const void *XK, const float *theta_lr,
                 float eta_base, float *eta, hipStream_t stream);

/*
 * Backward of ttt_eta_gate: with deta = dLoss/deta (e.g. ttt_linear_backward's
 * deta) and logistic'(s) = logistic(s) (1 - logistic(s)), s = theta_lr[h] . XK_t:
 *   dXK[n,h,t,:] += deta * eta_base * logistic'(s) * theta_lr[h]   (in place)
 *   dtheta[n,h,:] = sum_t deta * eta_base * logistic'(s) * XK[n,h,t,:]
 * dXK [B,H,L,d] fp32 (16-byte aligned) is read and updated, so passing the
 * inner-loop backward's dXK yields the key's total gradient. dtheta
 * [B,H,d] fp32 is written per sequence (the parameter's gradient is its sum
 * over n); its sum over t runs in a fixed order, so repeated calls give the
 * same bits. Other arguments as ttt_eta_gate; no output may overlap an input.
 */
int ttt_eta_gate_backward(int B, int H, int L, int d, int io, const void *XK,
                          const float *theta_lr, float eta_base, const float *deta, float *dXK,
                          float *dtheta, hipStream_t stream);

/*
 * Input projections of the layer: the query, key and value views of the
 * layer input ([Y] §2.2: the outer loop learns theta_Q, theta_K, theta_V;
 * [D] §4.2 feeds the views XQ, XK, XV to the inner loop). With the weights
 * stored output-major, like a linear layer's,
 *   XQ[b,h,t,j] = sum_k X[b,t,k] theta[0][h*d + j][k]   (XK: theta[1], XV: theta[2]),
 * written in the [B,H,L,d] layout every prefill entry point reads.
 *   B, L, H >= 0; d = 64; d_model a positive multiple of 64; B*L and 3*H*d
 *   at most INT_MAX, else TTT_E_SHAPE.
 *   X [B,L,d_model] bf16 and theta [3,H*d,d_model] bf16, 16-byte aligned,
 *   read only. XQ, XK, XV [B,H,L,d] bf16, 16-byte aligned, written; none may
 *   overlap another argument (TTT_E_ALIAS).
 *   Arithmetic: bf16 products, fp32 accumulation, outputs rounded to bf16
 *   (nearest even). Empty outputs (B, L or H = 0): nothing is read or launched.
 * The per-token rates then come from ttt_eta_gate on XK.
 */
int ttt_qkv_project(int B, int L, int d_model, int H, int d, const void *X, const void *theta, void *XQ,
                    void *XK, void *XV, hipStream_t stream);

/*
 * TTT-MLP prefill ([Y] §2.1: f_res(x) = GELU(x W1 + b1) W2 + b2, hidden m = 4d,
 * exact GELU x * Phi(x)), mini-batch form as above.
 *   d = 64 (m = 256); 1 <= mb <= 16.
 *   W1_0 [.,H,d,m], b1_0 [.,H,m], W2_0 [.,H,m,d], b2_0 [.,H,d] fp32, where
 *   "." is absent (shared over B) when w0_batched == 0, else B.
 *   Outputs W1_out [B,H,d,m], b1_out [B,H,m], W2_out [B,H,m,d], b2_out [B,H,d]
 *   are optional as a group (all NULL or all non-NULL) and may equal the
 *   corresponding inputs when w0_batched == 1.
 * Numerics: state, accumulation and layer-norm statistics in fp32; on the
 *   bf16 path (mb = 16) every product takes fp16 MFMA operands (inputs,
 *   state, activations, E1, E2 and the Grams rounded to fp16, accumulated in
 *   fp32), so |W1|, |W2|, the activations and the Gram entries must stay
 *   below 65504.
 */
int ttt_mlp_forward(int B, int H, int L, int d, int mb, int io, float ln_eps,
                    const void *XQ, const void *XK, const void *XV, const float *eta,
                    const float *W1_0, const float *b1_0, const float *W2_0,
                    const float *b2_0, int w0_batched, const float *ln_gamma,
                    const float *ln_beta, void *O, float *W1_out, float *b1_out,
                    float *W2_out, float *b2_out, hipStream_t stream);

/*
 * ttt_mlp_forward with each token's rate taken from the learning-rate gate of
 * [Y] §2.2 while the kernel stages the token (no eta array is read):
 *   eta_t = eta_base * logistic(theta_lr[h] . XK_t),  logistic(s) = 1/(1+e^-s),
 * the gate input x read as the head's key XK_t, as in ttt_linear_forward_gated.
 *   theta_lr : [H,d] fp32, 16-byte aligned.  eta_base : finite, else TTT_E_SHAPE.
 * Every other argument, and the numerics, as ttt_mlp_forward; the gate itself
 * is evaluated in fp32 (on the bf16 mb = 16 path with the hardware exp2 and
 * reciprocal, about 1 ulp each).
 */
int ttt_mlp_forward_gated(int B, int H, int L, int d, int mb, int io, float ln_eps,
                          const void *XQ, const void *XK, const void *XV,
                          const float *theta_lr, float eta_base, const float *W1_0,
                          const float *b1_0, const float *W2_0, const float *b2_0,
                          int w0_batched, const float *ln_gamma, const float *ln_beta, void *O,
                          float *W1_out, float *b1_out, float *W2_out, float *b2_out,
                          hipStream_t stream);

/*
 * ttt_mlp_forward with the two Modular-TTT options of ttt_linear_forward_opts
 * ([M]: inner loss and weight decay on the fast weights), read for the MLP:
 *   inner_loss   : TTT_LOSS_MSE (as ttt_mlp_forward) or TTT_LOSS_INNER_PRODUCT,
 *                  each token's loss -< XK_t + LN(f_res(XK_t)), XV_t >; any
 *                  other value is TTT_E_SHAPE.
 *   weight_decay : lambda >= 0 (finite, else TTT_E_SHAPE); every token's loss
 *                  gains lambda/2 (||W1||^2 + ||W2||^2) (the weight matrices,
 *                  not b1, b2), its gradient taken at the chunk-start state, so
 *                  a chunk scales W1 and W2 by 1 - lambda * sum_t eta_t before
 *                  the loss updates, and token t inside the chunk sees them
 *                  scaled by 1 - lambda * sum_{s<=t} eta_s.
 * Every other argument, and the numerics, as ttt_mlp_forward; the bf16 path
 * with mb = 16 runs the MFMA kernel for every option value, other shapes the
 * fp32 VALU kernel.
 */
int ttt_mlp_forward_opts(int B, int H, int L, int d, int mb, int io, float ln_eps,
                         const void *XQ, const void *XK, const void *XV, const float *eta,
                         const float *W1_0, const float *b1_0, const float *W2_0,
                         const float *b2_0, int w0_batched, const float *ln_gamma,
                         const float *ln_beta, int inner_loss, float weight_decay, void *O,
                         float *W1_out, float *b1_out, float *W2_out, float *b2_out,
                         hipStream_t stream);

/*
 * Backward of ttt_linear_forward: the gradients of
 *   loss = <dO, O> + <dW_out, W_L> + <db_out, b_L>
 * with respect to XQ, XK, XV, eta, W0, b0, gamma and beta, the gradients a
 * training step takes through the inner loop ([D] §6, §7.1). Arguments as
 * ttt_linear_forward for the forward inputs (same B, H, L, d, mb, io,
 * ln_eps, w0_batched), plus:
 *   dO [B,H,L,d] fp32; dW_out [B,H,d,d], db_out [B,H,d] fp32 or NULL (zero).
 *   Outputs, fp32 and per sequence: dXQ, dXK, dXV [B,H,L,d]; deta [B,H,L];
 *   dW0 [B,H,d,d]; db0, dgamma, dbeta [B,H,d]. Parameters shared over the
 *   batch (W0 and b0 when w0_batched == 0, gamma, beta) need the caller's
 *   sum over B.
 *   workspace: device memory of at least the size ttt_linear_backward_workspace
 *   reports (the state at every chunk start and, per chunk, the reverse's
 *   values that do not depend on dW', db'), caller-owned, overwritten. The
 *   call is three launches on `stream`: the forward sweep, a pre-pass over all
 *   chunks at once, the reverse sweep.
 * No output may overlap an input, another output or the workspace.
 * Numerics: fp32 throughout (bf16 inputs widened); the forward is recomputed
 * chunk by chunk from the stored states in the dual form ([D] §4.2).
 * Errors as ttt_linear_forward; TTT_E_SHAPE also for a short workspace.
 */
int ttt_linear_backward(int B, int H, int L, int d, int mb, int io, float ln_eps,
                        const void *XQ, const void *XK, const void *XV, const float *eta,
                        const float *W0, const float *b0, int w0_batched,
                        const float *ln_gamma, const float *ln_beta, const float *dO,
                        const float *dW_out, const float *db_out, float *dXQ, float *dXK,
                        float *dXV, float *deta, float *dW0, float *db0, float *dgamma,
                        float *dbeta, void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

/* Workspace bytes ttt_linear_backward needs:
 * B*H*ceil(L/mb)*(d*d + d + 80d + 2d + 32)*4 (a chunk-start state and a
 * chunk record per chunk; d = 64: 37,760 bytes per chunk and sequence).
 * Validates B, H, L, d, mb as ttt_linear_backward does; TTT_E_SHAPE also
 * when B*H*ceil(L/mb) exceeds 2^31 - 1. */
int ttt_linear_backward_workspace(int B, int H, int L, int d, int mb, size_t *bytes);

/*
 * ttt_linear_backward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving or training loops, harnesses that
 * forbid hipMalloc. Same arguments, results and kernel as
 * ttt_linear_backward, minus the workspace: the chunk-start checkpoints and
 * chunk records go to a fixed device array inside the library,
 * TTT_BACKWARD_SCRATCH_BYTES (64 MiB) on every GPU the library runs on, held
 * until the process ends.
 *   - ttt_linear_backward_workspace's size must not exceed
 *     TTT_BACKWARD_SCRATCH_BYTES, else TTT_E_SHAPE before any HIP call
 *     (d = 64: at most 1777 chunks B*H*ceil(L/mb), e.g. B*H = 3 at L = 9472
 *     with mb = 16).
 *   - Calls no hipMalloc, hipFree or allocating library routine. The first
 *     call on a device looks up the array's device address once
 *     (hipGetSymbolAddress with that device current).
 *   - `stream` must belong to the current device (else TTT_E_HIP).
 *   - Every call on one GPU shares that GPU's array and it keeps the last
 *     call's contents; a call reads only values it wrote itself, so nothing
 *     needs clearing. Calls that overlap in time on one GPU (other
 *     streams, other host threads) race on the array and give wrong
 *     gradients: order them, e.g. on one stream.
 */
#define TTT_BACKWARD_SCRATCH_BYTES ((size_t)64 << 20)
int ttt_linear_backward_noalloc(int B, int H, int L, int d, int mb, int io, float ln_eps,
                                const void *XQ, const void *XK, const void *XV,
                                const float *eta, const float *W0, const float *b0,
                                int w0_batched, const float *ln_gamma, const float *ln_beta,
                                const float *dO, const float *dW_out, const float *db_out,
                                float *dXQ, float *dXK, float *dXV, float *deta, float *dW0,
                                float *db0, float *dgamma, float *dbeta, hipStream_t stream);

/*
 * Backward of ttt_mlp_forward: the gradients of
 *   loss = <dO, O> + <dW1_out, W1_L> + <db1_out, b1_L> + <dW2_out, W2_L> + <db2_out, b2_L>
 * with respect to XQ, XK, XV, eta, the initial state W1, b1, W2, b2, gamma
 * and beta -- the TTT-MLP of [Y] §2.1 (d -> 4d exact-GELU -> d, LN residual)
 * under the mini-batch rule of [D] §4.1-4.2, trained through the inner loop
 * as in [D] §6, §7.1. Arguments as ttt_mlp_forward for the forward inputs
 * (d = 64 only, any 1 <= mb <= 16, any L >= 0, io, ln_eps, w0_batched), plus:
 *   dO [B,H,L,d] fp32; dW1_out [B,H,d,4d], db1_out [B,H,4d], dW2_out [B,H,4d,d],
 *   db2_out [B,H,d] fp32, each NULL for zero.
 *   Outputs, fp32 and per sequence: dXQ, dXK, dXV [B,H,L,d]; deta [B,H,L];
 *   dW1 [B,H,d,4d]; db1 [B,H,4d]; dW2 [B,H,4d,d]; db2, dgamma, dbeta [B,H,d].
 *   Parameters shared over the batch (the initial state when w0_batched == 0,
 *   gamma, beta) need the caller's sum over B.
 *   workspace: device memory of at least ttt_mlp_backward_workspace bytes
 *   (the state at every chunk start, two adjoint states and, per chunk, the
 *   reverse's values that do not depend on the adjoint state), caller-owned,
 *   overwritten. The call is three launches on `stream`: the forward sweep,
 *   a pre-pass over all chunks at once, the reverse sweep.
 * No output may overlap an input, another output or the workspace.
 * Numerics: fp32 throughout (bf16 inputs widened); the forward is recomputed
 * chunk by chunk from the stored states in the dual form ([D] §4.2).
 * Errors as ttt_mlp_forward; TTT_E_SHAPE also for a short workspace.
 */
int ttt_mlp_backward(int B, int H, int L, int d, int mb, int io, float ln_eps, const void *XQ,
                     const void *XK, const void *XV, const float *eta, const float *W1_0,
                     const float *b1_0, const float *W2_0, const float *b2_0, int w0_batched,
                     const float *ln_gamma, const float *ln_beta, const float *dO,
                     const float *dW1_out, const float *db1_out, const float *dW2_out,
                     const float *db2_out, float *dXQ, float *dXK, float *dXV, float *deta,
                     float *dW1, float *db1, float *dW2, float *db2, float *dgamma, float *dbeta,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes ttt_mlp_backward needs, with n = ceil(L/mb):
 * B*H*((n+2)*(8d*d+5d) + n*(594d+32))*4 (d = 64: 284,544 bytes per chunk and
 * sequence plus 264,704 per sequence). Validates B, H, L, d, mb as
 * ttt_mlp_backward does; TTT_E_SHAPE also when B*H*n exceeds 2^31 - 1. */
int ttt_mlp_backward_workspace(int B, int H, int L, int d, int mb, size_t *bytes);

/*
 * One single-token TTT-Linear step (b = 1, primal form) for B x H independent
 * states held in place -- the fast-weight cache of [D] §5.2:
 *   G = lnbwd(xk W + b, xv - xk);  W <- W - eta xk^T G;  b <- b - eta G;
 *   o = xq + LN(xq W + b)   (with the updated W, b).
 *   d in {16, 64}.  xq, xk, xv : [B,H,d] io;  eta : [B,H] fp32;
 *   W [B,H,d,d], b [B,H,d] fp32, read and overwritten;  o [B,H,d] io.
 */
int ttt_decode_step(int B, int H, int d, int io, float ln_eps, const void *xq,
                    const void *xk, const void *xv, const float *eta, float *W, float *b,
                    const float *ln_gamma, const float *ln_beta, void *o,
                    hipStream_t stream);

/*
 * T consecutive single-token steps, each exactly as ttt_decode_step, on the
 * same B x H states: step t reads xq[t], xk[t], xv[t], eta[t] and writes
 * o[t]; W and b hold the state after the last step. This is the cache of
 * [D] §5.2 carried through a run of decode steps whose inputs are known in
 * advance (teacher-forced decoding, b = 1 prefill).
 *   T >= 0 (T = 0 leaves W and b unchanged); d in {16, 64}.
 *   xq, xk, xv, o : [T,B,H,d] io, step-major;  eta : [T,B,H] fp32;
 *   W [B,H,d,d], b [B,H,d] fp32, read and overwritten.
 * For d = 64 one launch keeps every state in registers for all T steps, so
 * only the per-step inputs and outputs cross HBM; for d = 16 it issues one
 * single-step launch per step. Numerics: fp32 throughout (as
 * ttt_decode_step; the two differ only in summation order).
 * Errors as ttt_decode_step, plus TTT_E_SHAPE for T < 0.
 */
int ttt_decode_steps(int T, int B, int H, int d, int io, float ln_eps, const void *xq,
                     const void *xk, const void *xv, const float *eta, float *W, float *b,
                     const float *ln_gamma, const float *ln_beta, void *o,
                     hipStream_t stream);

/*
 * Mini-batch decode: T consecutive tokens under the mini-batch rule of [D]
 * §4.1 with b = mb, so that a prefill followed by any sequence of these calls
 * gives the same outputs and state as one prefill over the whole sequence
 * (chunks aligned at its first token). The cache of [D] §5.2 then holds two
 * states: the current one (W, b) and the start state of the current chunk
 * (W_chunk, b_chunk), at which every token of the chunk takes its gradient:
 *   at a chunk's first token   W_chunk, b_chunk <- W, b
 *   z = xk W_chunk + b_chunk;  G = lnbwd(z, xv - xk)
 *   W <- W - eta xk^T G;  b <- b - eta G;  o = xq + LN(xq W + b)
 *   mb  : 1 <= mb <= 16 (mb = 1 is ttt_decode_steps).
 *   pos : 0 <= pos < mb, the position of the first step within its chunk
 *         (the number of the chunk's tokens already processed); the next
 *         call continues at (pos + T) mod mb.
 *   W_chunk, b_chunk : [B,H,d,d], [B,H,d] fp32, read when pos > 0, written
 *         with the start state of the chunk of the last step (so a call
 *         ending inside a chunk can be continued). Required when mb > 1,
 *         ignored when mb = 1; must not overlap any other argument.
 * Every other argument, the layouts and the errors as ttt_decode_steps, plus
 * TTT_E_SHAPE for mb or pos out of range. d = 64 keeps both states in
 * registers for all T steps; d = 16 runs one launch per step.
 */
int ttt_decode_steps_mb(int T, int B, int H, int d, int io, float ln_eps, int mb, int pos,
                        const void *xq, const void *xk, const void *xv, const float *eta,
                        float *W_chunk, float *b_chunk, float *W, float *b,
                        const float *ln_gamma, const float *ln_beta, void *o,
                        hipStream_t stream);

/*
 * ttt_decode_steps_mb with each step's rate taken from the learning-rate gate
 * of [Y] §2.2 (no eta array is read):
 *   eta_t = eta_base * logistic(theta_lr[h] . xk_t),  logistic(s) = 1/(1+e^-s),
 * the gate input x read as the head's key, as in the gated prefills, so a
 * gated prefill followed by these calls equals one gated prefill over the
 * whole sequence. mb = 1 is plain b = 1 decode (W_chunk, b_chunk ignored).
 *   theta_lr : [H,d] fp32.  eta_base : finite, else TTT_E_SHAPE.
 * Every other argument, the layouts and the errors as ttt_decode_steps_mb.
 * The gate is evaluated in fp32 (d = 64: a wave sum, then the hardware exp2
 * and reciprocal, about 1 ulp each; d = 16: expf and a divide).
 */
int ttt_decode_steps_gated(int T, int B, int H, int d, int io, float ln_eps, int mb, int pos,
                           const void *xq, const void *xk, const void *xv,
                           const float *theta_lr, float eta_base, float *W_chunk,
                           float *b_chunk, float *W, float *b, const float *ln_gamma,
                           const float *ln_beta, void *o, hipStream_t stream);

/*
 * The fused layer-norm + L2 backward step on its own ([D] §4.2), row-wise:
 *   G[r] = d/dz [ 1/2 || LN_{gamma,beta}(z) - target[r] ||^2 ] at z = Z[r].
 *   rows >= 0; d in {16, 32, 64}. Z, target, G : [rows,d] fp32;
 *   gamma, beta : [d] fp32. G must not overlap Z or target.
 */
int ttt_ln_l2_bwd(int rows, int d, const float *Z, const float *target,
                  const float *ln_gamma, const float *ln_beta, float ln_eps, float *G,
                  hipStream_t stream);

/* Message for the last non-zero return on this thread ("" if none). */
const char *ttt_last_error(void);

/* ABI version (incremented on incompatible changes). */
int ttt_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TTT_H */
