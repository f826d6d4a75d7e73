// extern "C" entry points of libttt.so (declared and documented in ttt.h).
// Every argument is validated on the host before any HIP call; the kernels
// are then enqueued on the caller's stream. Nothing here allocates or
// synchronises.
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <cfloat>
#include <climits>
#include <cmath>

#include "launch.hpp"
#include "ttt.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return TTT_OK;
}

struct Buf {
    const void *p;
    size_t bytes;
    const char *name;
    bool optional;
    unsigned align;  // required alignment in bytes
};

bool mul_ok(size_t a, size_t b, size_t *out) { return !__builtin_mul_overflow(a, b, out); }

// product of non-negative ints as bytes; false on overflow
bool nbytes(size_t *out, std::initializer_list<size_t> dims) {
    size_t r = 1;
    for (size_t v : dims)
        if (!mul_ok(r, v, &r)) return false;
    *out = r;
    return true;
}

int check_bufs(const Buf *b, int n) {
    for (int i = 0; i < n; ++i) {
        if (!b[i].p) {
            if (b[i].bytes && !b[i].optional)
                return fail(TTT_E_NULL, "%s is NULL (%zu bytes expected)", b[i].name, b[i].bytes);
            continue;
        }
        if (reinterpret_cast<uintptr_t>(b[i].p) & (b[i].align - 1))
            return fail(TTT_E_ALIGN, "%s (%p) is not %u-byte aligned", b[i].name, b[i].p, b[i].align);
    }
    return TTT_OK;
}

bool overlaps(const Buf &a, const Buf &b) {
    if (!a.p || !b.p || !a.bytes || !b.bytes) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Outputs must not overlap any other buffer, except that an output may be
// exactly the same buffer as its paired input (`same_ok[out] == in`).
int check_alias(const Buf *outs, int nout, const Buf *ins, int nin, const int *pair) {
    for (int o = 0; o < nout; ++o) {
        for (int i = 0; i < nin; ++i) {
            if (!overlaps(outs[o], ins[i])) continue;
            if (pair && pair[o] == i && outs[o].p == ins[i].p && outs[o].bytes == ins[i].bytes) continue;
            return fail(TTT_E_ALIAS, "%s overlaps %s", outs[o].name, ins[i].name);
        }
        for (int o2 = o + 1; o2 < nout; ++o2)
            if (overlaps(outs[o], outs[o2]))
                return fail(TTT_E_ALIAS, "%s overlaps %s", outs[o].name, outs[o2].name);
    }
    return TTT_OK;
}

int check_common(int B, int H, int L, int mb, int io) {
    if (B < 0 || H < 0 || L < 0) return fail(TTT_E_SHAPE, "negative size (B=%d H=%d L=%d)", B, H, L);
    if (io != TTT_F32 && io != TTT_BF16) return fail(TTT_E_DTYPE, "io dtype %d is not TTT_F32/TTT_BF16", io);
    if (mb < 1 || mb > 16) return fail(TTT_E_SHAPE, "mini-batch size %d not in [1, 16]", mb);
    // token and chunk indices inside the kernels are 32-bit ints
    if (L > TTT_MAX_L) return fail(TTT_E_SHAPE, "L = %d exceeds TTT_MAX_L = %d", L, TTT_MAX_L);
    if (static_cast<long long>(B) * H > INT_MAX) return fail(TTT_E_SHAPE, "B*H = %lld too large", static_cast<long long>(B) * H);
    return TTT_OK;
}

// The layer norms evaluate 1/sqrt(var + eps) with var >= 0, which needs a
// positive normal eps.
int check_eps(float eps) {
    if (!(eps >= FLT_MIN) || !std::isfinite(eps))
        return fail(TTT_E_SHAPE, "ln_eps = %g is not a positive normal float", static_cast<double>(eps));
    return TTT_OK;
}

int launched(hipError_t e) {
    if (e != hipSuccess) return fail(TTT_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

// ttt_linear_backward with a caller workspace, or (fixed_scratch) with the
// library's fixed device scratch: the same validation and the same kernel.
int linear_backward(int B, int H, int L, int d, int mb, int io, float ln_eps, const void *XQ,
                    const void *XK, const void *XV, const float *eta, const float *W0,
                    const float *b0, int w0_batched, const float *ln_gamma, const float *ln_beta,
                    const float *dO, const float *dW_out, const float *db_out, float *dXQ,
                    float *dXK, float *dXV, float *deta, float *dW0, float *db0, float *dgamma,
                    float *dbeta, void *workspace, size_t workspace_bytes, bool fixed_scratch,
                    hipStream_t stream) {
    int st;
    if ((st = check_common(B, H, L, mb, io)) || (st = check_eps(ln_eps))) return st;
    if (d != 16 && d != 64) return fail(TTT_E_SHAPE, "d = %d not in {16, 64}", d);
    const size_t es = io == TTT_BF16 ? 2 : 4;
    const size_t nb = w0_batched ? static_cast<size_t>(B) : 1;
    size_t xb, fb, eb, wb, bb, ob_w, ob_b, pb, need;
    if (!nbytes(&xb, {size_t(B), size_t(H), size_t(L), size_t(d), es}) ||
        !nbytes(&fb, {size_t(B), size_t(H), size_t(L), size_t(d), sizeof(float)}) ||
        !nbytes(&eb, {size_t(B), size_t(H), size_t(L), sizeof(float)}) ||
        !nbytes(&wb, {nb, size_t(H), size_t(d), size_t(d), sizeof(float)}) ||
        !nbytes(&bb, {nb, size_t(H), size_t(d), sizeof(float)}) ||
        !nbytes(&ob_w, {size_t(B), size_t(H), size_t(d), size_t(d), sizeof(float)}) ||
        !nbytes(&ob_b, {size_t(B), size_t(H), size_t(d), sizeof(float)}) ||
        !nbytes(&pb, {size_t(H), size_t(d), sizeof(float)}))
        return fail(TTT_E_SHAPE, "sizes overflow");
    if ((st = ttt_linear_backward_workspace(B, H, L, d, mb, &need))) return st;
    const Buf in[] = {{XQ, xb, "XQ", false, 16},        {XK, xb, "XK", false, 16},
                      {XV, xb, "XV", false, 16},        {eta, eb, "eta", false, 4},
                      {W0, wb, "W0", false, 16},        {b0, bb, "b0", false, 16},
                      {ln_gamma, pb, "ln_gamma", false, 4}, {ln_beta, pb, "ln_beta", false, 4},
                      {dO, fb, "dO", false, 4},         {dW_out, ob_w, "dW_out", true, 4},
                      {db_out, ob_b, "db_out", true, 4}};
    const Buf out[] = {{dXQ, fb, "dXQ", false, 4},   {dXK, fb, "dXK", false, 4},
                       {dXV, fb, "dXV", false, 4},   {deta, eb, "deta", false, 4},
                       {dW0, ob_w, "dW0", false, 4}, {db0, ob_b, "db0", false, 4},
                       {dgamma, ob_b, "dgamma", false, 4}, {dbeta, ob_b, "dbeta", false, 4},
                       {workspace, need, "workspace", false, 4}};
    const int nout = fixed_scratch ? 8 : 9;  // the workspace is the last output
    if ((st = check_bufs(in, 11)) || (st = check_bufs(out, nout))) return st;
    if (fixed_scratch) {
        if (need > ttt::linear_backward_scratch_bytes())
            return fail(TTT_E_SHAPE,
                        "the checkpoints and chunk records need %zu bytes; the no-allocation entry "
                        "point's scratch holds %zu (ttt_linear_backward_workspace must not exceed it)",
                        need, ttt::linear_backward_scratch_bytes());
    } else if (workspace_bytes < need) {
        return fail(TTT_E_SHAPE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    }
    if ((st = check_alias(out, nout, in, 11, nullptr))) return st;
    if (B * H == 0) return ok();
    if (fixed_scratch) {  // the scratch of the device the stream runs on
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return fail(TTT_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
        if (stream) {
            hipDevice_t sd = 0;
            if ((e = hipStreamGetDevice(stream, &sd)) != hipSuccess)
                return fail(TTT_E_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
            if (sd != cur)
                return fail(TTT_E_HIP, "stream belongs to device %d, the current device is %d",
                            static_cast<int>(sd), cur);
        }
        float *p = nullptr;
        if ((e = ttt::linear_backward_scratch(&p)) != hipSuccess)
            return fail(TTT_E_HIP, "scratch address: %s", hipGetErrorString(e));
        workspace = p;
    }
    ttt::LinearBwdArgs a{{B, H, L, d, mb, io, ln_eps, XQ, XK, XV, eta, W0, b0, w0_batched ? 1 : 0,
                          ln_gamma, ln_beta, nullptr, nullptr, nullptr},
                         dO, dW_out, db_out, dXQ, dXK, dXV, deta, dW0, db0, dgamma, dbeta,
                         static_cast<float *>(workspace)};
    return launched(ttt::launch_linear_backward(a, stream));
}

}  // namespace

extern "C" {

int ttt_version(void) { return 1; }

const char *ttt_last_error(void) { return g_err; }

int ttt_ln_l2_bwd(int rows, int d, const float *Z, const float *target, const float *ln_gamma,
                  const float *ln_beta, float ln_eps, float *G, hipStream_t stream) {
    if (rows < 0) return fail(TTT_E_SHAPE, "rows = %d < 0", rows);
    if (check_eps(ln_eps)) return TTT_E_SHAPE;
    if (d != 16 && d != 32 && d != 64) return fail(TTT_E_SHAPE, "d = %d not in {16, 32, 64}", d);
    size_t rb;
    if (!nbytes(&rb, {static_cast<size_t>(rows), static_cast<size_t>(d), sizeof(float)}))
        return fail(TTT_E_SHAPE, "rows*d overflows");
    const Buf in[] = {{Z, rb, "Z", false, 4}, {target, rb, "target", false, 4},
                      {ln_gamma, d * sizeof(float), "ln_gamma", false, 4},
                      {ln_beta, d * sizeof(float), "ln_beta", false, 4}};
    const Buf out[] = {{G, rb, "G", false, 4}};
    int st;
    if ((st = check_bufs(in, 4)) || (st = check_bufs(out, 1))) return st;
    if ((st = check_alias(out, 1, in, 4, nullptr))) return st;
    return launched(ttt::launch_ln_l2_bwd(rows, d, Z, target, ln_gamma, ln_beta, ln_eps, G, stream));
}

}  // extern "C"

namespace {

// TTT-Linear prefill with eta given (theta == nullptr) or from the gate.
int linear_forward(int B, int H, int L, int d, int mb, int io, float ln_eps, const void *XQ,
                   const void *XK, const void *XV, const float *eta, const float *theta,
                   float eta_base, const float *W0, const float *b0, int w0_batched,
                   const float *ln_gamma, const float *ln_beta, void *O, float *W_out,
                   float *b_out, hipStream_t stream, bool gated, int loss = TTT_LOSS_MSE,
                   float weight_decay = 0.f) {
    int st;
    if ((st = check_common(B, H, L, mb, io)) || (st = check_eps(ln_eps))) return st;
    if (d != 16 && d != 64) return fail(TTT_E_SHAPE, "d = %d not in {16, 64}", d);
    if (loss != TTT_LOSS_MSE && loss != TTT_LOSS_INNER_PRODUCT)
        return fail(TTT_E_SHAPE, "inner_loss = %d is not TTT_LOSS_MSE / TTT_LOSS_INNER_PRODUCT", loss);
    if (!(weight_decay >= 0.f) || !std::isfinite(weight_decay))
        return fail(TTT_E_SHAPE, "weight_decay = %g is not a finite value >= 0",
                    static_cast<double>(weight_decay));
    if (gated && !std::isfinite(eta_base))
        return fail(TTT_E_SHAPE, "eta_base = %g is not finite", static_cast<double>(eta_base));
    const size_t es = io == TTT_BF16 ? 2 : 4;
    const size_t nb = w0_batched ? static_cast<size_t>(B) : 1;
    size_t xb, eb, wb, bb, ob_w, ob_b;
    if (!nbytes(&xb, {size_t(B), size_t(H), size_t(L), size_t(d), es}) ||
        !nbytes(&eb, {size_t(B), size_t(H), size_t(L), sizeof(float)}) ||
        !nbytes(&wb, {nb, size_t(H), size_t(d), size_t(d), sizeof(float)}) ||
        !nbytes(&bb, {nb, size_t(H), size_t(d), sizeof(float)}) ||
        !nbytes(&ob_w, {size_t(B), size_t(H), size_t(d), size_t(d), sizeof(float)}) ||
        !nbytes(&ob_b, {size_t(B), size_t(H), size_t(d), sizeof(float)}))
        return fail(TTT_E_SHAPE, "sizes overflow");
    const size_t pb = static_cast<size_t>(H) * d * sizeof(float);
    const Buf in[] = {{XQ, xb, "XQ", false, 16}, {XK, xb, "XK", false, 16},
                      {XV, xb, "XV", false, 16},
                      gated ? Buf{theta, pb, "theta_lr", false, 16} : Buf{eta, eb, "eta", false, 4},
                      {W0, wb, "W0", false, 16}, {b0, bb, "b0", false, 16},
                      {ln_gamma, pb, "ln_gamma", false, 4}, {ln_beta, pb, "ln_beta", false, 4}};
    const Buf out[] = {{O, xb, "O", false, 16}, {W_out, ob_w, "W_out", true, 16},
                       {b_out, ob_b, "b_out", true, 16}};
    if ((st = check_bufs(in, 8)) || (st = check_bufs(out, 3))) return st;
    // W_out may be exactly W0 (and b_out exactly b0) when the state is per batch.
    const int pair[] = {-1, w0_batched ? 4 : -1, w0_batched ? 5 : -1};
    if ((st = check_alias(out, 3, in, 8, pair))) return st;
    if (B * H == 0) return ok();

    ttt::LinearArgs a{B, H, L, d, mb, io, ln_eps, XQ, XK, XV, gated ? nullptr : eta, W0, b0,
                      w0_batched ? 1 : 0, ln_gamma, ln_beta, O, W_out, b_out};
    if (gated) {
        a.theta = theta;
        a.eta_base = eta_base;
    }
    a.loss = loss;
    a.wd = weight_decay;
    if (ttt::linear_mfma_supported(a)) return launched(ttt::launch_linear_mfma(a, stream));
    return launched(ttt::launch_linear_valu(a, stream));
}

// XK, theta and eta/deta checks shared by the two gate entry points.
int gate_common(int B, int H, int L, int d, int io, float eta_base, size_t *xb, size_t *eb,
                size_t *pb) {
    int st;
    if ((st = check_common(B, H, L, 1, io))) return st;
    if (d != 16 && d != 32 && d != 64) return fail(TTT_E_SHAPE, "d = %d not in {16, 32, 64}", d);
    if (!std::isfinite(eta_base))
        return fail(TTT_E_SHAPE, "eta_base = %g is not finite", static_cast<double>(eta_base));
    const size_t es = io == TTT_BF16 ? 2 : 4;
    if (!nbytes(xb, {size_t(B), size_t(H), size_t(L), size_t(d), es}) ||
        !nbytes(eb, {size_t(B), size_t(H), size_t(L), sizeof(float)}))
        return fail(TTT_E_SHAPE, "sizes overflow");
    *pb = static_cast<size_t>(H) * d * sizeof(float);
    return TTT_OK;
}

// TTT-MLP prefill with the loss / weight-decay options (shared by the plain
// and the options entry points).
int mlp_forward(int B, int H, int L, int d, int mb, int io, float ln_eps, const void *XQ,
                const void *XK, const void *XV, const float *eta, const float *theta,
                float eta_base, const float *W1_0, const float *b1_0, const float *W2_0,
                const float *b2_0, int w0_batched, const float *ln_gamma,
                const float *ln_beta, void *O, float *W1_out, float *b1_out, float *W2_out,
                float *b2_out, hipStream_t stream, bool gated, int loss, float weight_decay) {
    int st;
    if ((st = check_common(B, H, L, mb, io)) || (st = check_eps(ln_eps))) return st;
    if (d != 64) return fail(TTT_E_SHAPE, "d = %d: the MLP supports d = 64 only", d);
    if (loss != TTT_LOSS_MSE && loss != TTT_LOSS_INNER_PRODUCT)
        return fail(TTT_E_SHAPE, "inner_loss = %d is not TTT_LOSS_MSE / TTT_LOSS_INNER_PRODUCT", loss);
    if (!(weight_decay >= 0.f) || !std::isfinite(weight_decay))
        return fail(TTT_E_SHAPE, "weight_decay = %g is not a finite value >= 0",
                    static_cast<double>(weight_decay));
    if (gated && !std::isfinite(eta_base))
        return fail(TTT_E_SHAPE, "eta_base = %g is not finite", static_cast<double>(eta_base));
    const int nout = (W1_out != nullptr) + (b1_out != nullptr) + (W2_out != nullptr) + (b2_out != nullptr);
    if (nout != 0 && nout != 4) return fail(TTT_E_NULL, "state outputs must be all NULL or all non-NULL");
    const size_t es = io == TTT_BF16 ? 2 : 4, m = 4 * static_cast<size_t>(d);
    const size_t nb = w0_batched ? static_cast<size_t>(B) : 1;
    size_t xb, eb, w1b, b1b, w2b, b2b, o1, o2, o3, o4;
    if (!nbytes(&xb, {size_t(B), size_t(H), size_t(L), size_t(d), es}) ||
        !nbytes(&eb, {size_t(B), size_t(H), size_t(L), sizeof(float)}) ||
        !nbytes(&w1b, {nb, size_t(H), size_t(d), m, sizeof(float)}) ||
        !nbytes(&b1b, {nb, size_t(H), m, sizeof(float)}) ||
        !nbytes(&w2b, {nb, size_t(H), m, size_t(d), sizeof(float)}) ||
        !nbytes(&b2b, {nb, size_t(H), size_t(d), sizeof(float)}) ||
        !nbytes(&o1, {size_t(B), size_t(H), size_t(d), m, sizeof(float)}) ||
        !nbytes(&o2, {size_t(B), size_t(H), m, sizeof(float)}) ||
        !nbytes(&o3, {size_t(B), size_t(H), m, size_t(d), sizeof(float)}) ||
        !nbytes(&o4, {size_t(B), size_t(H), size_t(d), sizeof(float)}))
        return fail(TTT_E_SHAPE, "sizes overflow");
    const size_t pb = static_cast<size_t>(H) * d * sizeof(float);
    const Buf in[] = {{XQ, xb, "XQ", false, 16}, {XK, xb, "XK", false, 16},
                      {XV, xb, "XV", false, 16},
                      gated ? Buf{theta, pb, "theta_lr", false, 16} : Buf{eta, eb, "eta", false, 4},
                      {W1_0, w1b, "W1_0", false, 16}, {b1_0, b1b, "b1_0", false, 16},
                      {W2_0, w2b, "W2_0", false, 16}, {b2_0, b2b, "b2_0", false, 16},
                      {ln_gamma, pb, "ln_gamma", false, 4}, {ln_beta, pb, "ln_beta", false, 4}};
    const Buf out[] = {{O, xb, "O", false, 16}, {W1_out, o1, "W1_out", true, 16},
                       {b1_out, o2, "b1_out", true, 16}, {W2_out, o3, "W2_out", true, 16},
                       {b2_out, o4, "b2_out", true, 16}};
    if ((st = check_bufs(in, 10)) || (st = check_bufs(out, 5))) return st;
    const int pair[] = {-1, w0_batched ? 4 : -1, w0_batched ? 5 : -1, w0_batched ? 6 : -1,
                        w0_batched ? 7 : -1};
    if ((st = check_alias(out, 5, in, 10, pair))) return st;
    if (B * H == 0) return ok();
    ttt::MLPArgs a{B, H, L, d, mb, io, ln_eps, XQ, XK, XV, gated ? nullptr : eta, W1_0, b1_0,
                   W2_0, b2_0, w0_batched ? 1 : 0, ln_gamma, ln_beta, O, W1_out, b1_out,
                   W2_out, b2_out};
    a.loss = loss;
    a.wd = weight_decay;
    if (gated) {
        a.theta = theta;
        a.eta_base = eta_base;
    }
    if (ttt::mlp_mfma_supported(a)) return launched(ttt::launch_mlp_mfma(a, stream));
    return launched(ttt::launch_mlp(a, stream));
}

int mlp_backward(int B, int H, int L, int d, int mb, int io, float ln_eps, const void *XQ,
                 const void *XK, const void *XV, const float *eta, const float *W1_0,
                 const float *b1_0, const float *W2_0, const float *b2_0, int w0_batched,
                 const float *ln_gamma, const float *ln_beta, const float *dO,
                 const float *dW1_out, const float *db1_out, const float *dW2_out,
                 const float *db2_out, float *dXQ, float *dXK, float *dXV, float *deta,
                 float *dW1, float *db1, float *dW2, float *db2, float *dgamma, float *dbeta,
                 void *workspace, size_t workspace_bytes, hipStream_t stream) {
    int st;
    if ((st = check_common(B, H, L, mb, io)) || (st = check_eps(ln_eps))) return st;
    if (d != 64) return fail(TTT_E_SHAPE, "d = %d: the MLP supports d = 64 only", d);
    const size_t es = io == TTT_BF16 ? 2 : 4, m = 4 * static_cast<size_t>(d);
    const size_t nb = w0_batched ? static_cast<size_t>(B) : 1;
    size_t xb, fb, eb, w1b, b1b, w2b, b2b, o1, o2, o3, o4, need;
    if (!nbytes(&xb, {size_t(B), size_t(H), size_t(L), size_t(d), es}) ||
        !nbytes(&fb, {size_t(B), size_t(H), size_t(L), size_t(d), sizeof(float)}) ||
        !nbytes(&eb, {size_t(B), size_t(H), size_t(L), sizeof(float)}) ||
        !nbytes(&w1b, {nb, size_t(H), size_t(d), m, sizeof(float)}) ||
        !nbytes(&b1b, {nb, size_t(H), m, sizeof(float)}) ||
        !nbytes(&w2b, {nb, size_t(H), m, size_t(d), sizeof(float)}) ||
        !nbytes(&b2b, {nb, size_t(H), size_t(d), sizeof(float)}) ||
        !nbytes(&o1, {size_t(B), size_t(H), size_t(d), m, sizeof(float)}) ||
        !nbytes(&o2, {size_t(B), size_t(H), m, sizeof(float)}) ||
        !nbytes(&o3, {size_t(B), size_t(H), m, size_t(d), sizeof(float)}) ||
        !nbytes(&o4, {size_t(B), size_t(H), size_t(d), sizeof(float)}))
        return fail(TTT_E_SHAPE, "sizes overflow");
    if ((st = ttt_mlp_backward_workspace(B, H, L, d, mb, &need))) return st;
    const size_t pb = static_cast<size_t>(H) * d * sizeof(float);
    const Buf in[] = {{XQ, xb, "XQ", false, 16},       {XK, xb, "XK", false, 16},
                      {XV, xb, "XV", false, 16},       {eta, eb, "eta", false, 4},
                      {W1_0, w1b, "W1_0", false, 4},   {b1_0, b1b, "b1_0", false, 4},
                      {W2_0, w2b, "W2_0", false, 4},   {b2_0, b2b, "b2_0", false, 4},
                      {ln_gamma, pb, "ln_gamma", false, 4}, {ln_beta, pb, "ln_beta", false, 4},
                      {dO, fb, "dO", false, 4},        {dW1_out, o1, "dW1_out", true, 4},
                      {db1_out, o2, "db1_out", true, 4}, {dW2_out, o3, "dW2_out", true, 4},
                      {db2_out, o4, "db2_out", true, 4}};
    const Buf out[] = {{dXQ, fb, "dXQ", false, 4},  {dXK, fb, "dXK", false, 4},
                       {dXV, fb, "dXV", false, 4},  {deta, eb, "deta", false, 4},
                       {dW1, o1, "dW1", false, 4},  {db1, o2, "db1", false, 4},
                       {dW2, o3, "dW2", false, 4},  {db2, o4, "db2", false, 4},
                       {dgamma, o4, "dgamma", false, 4}, {dbeta, o4, "dbeta", false, 4},
                       {workspace, need, "workspace", false, 4}};
    if ((st = check_bufs(in, 15)) || (st = check_bufs(out, 11))) return st;
    if (workspace_bytes < need)
        return fail(TTT_E_SHAPE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    if ((st = check_alias(out, 11, in, 15, nullptr))) return st;
    if (B * H == 0) return ok();
    ttt::MLPBwdArgs a{{B, H, L, d, mb, io, ln_eps, XQ, XK, XV, eta, W1_0, b1_0, W2_0, b2_0,
                       w0_batched ? 1 : 0, ln_gamma, ln_beta, nullptr, nullptr, nullptr, nullptr,
                       nullptr},
                      dO, dW1_out, db1_out, dW2_out, db2_out, dXQ, dXK, dXV, deta, dW1, db1, dW2,
                      db2, dgamma, dbeta, static_cast<float *>(workspace)};
    return launched(ttt::launch_mlp_backward(a, stream));
}

}  // namespace

extern "C" {

int ttt_linear_forward(int B, int H, int L, int d, int mb, int io, float ln_eps,
                       const void *XQ, const void *XK, const void *XV, const float *eta,
                       const float *W0, const float *b0, int w0_batched,
                       const float *ln_gamma, const float *ln_beta, void *O,
                       float *W_out, float *b_out, hipStream_t stream) {
    return linear_forward(B, H, L, d, mb, io, ln_eps, XQ, XK, XV, eta, nullptr, 0.f, W0, b0,
                          w0_batched, ln_gamma, ln_beta, O, W_out, b_out, stream, false);
}

int ttt_linear_forward_gated(int B, int H, int L, int d, int mb, int io, float ln_eps,
                             const void *XQ, const void *XK, const void *XV,
                             const float *theta_lr, float eta_base, const float *W0,
                             const float *b0, int w0_batched, const float *ln_gamma,
                             const float *ln_beta, void *O, float *W_out, float *b_out,
                             hipStream_t stream) {
    return linear_forward(B, H, L, d, mb, io, ln_eps, XQ, XK, XV, nullptr, theta_lr, eta_base,
                          W0, b0, w0_batched, ln_gamma, ln_beta, O, W_out, b_out, stream, true);
}

int ttt_linear_forward_opts(int B, int H, int L, int d, int mb, int io, float ln_eps,
                            const void *XQ, const void *XK, const void *XV, const float *eta,
                            const float *W0, const float *b0, int w0_batched,
                            const float *ln_gamma, const float *ln_beta, int inner_loss,
                            float weight_decay, void *O, float *W_out, float *b_out,
                            hipStream_t stream) {
    return linear_forward(B, H, L, d, mb, io, ln_eps, XQ, XK, XV, eta, nullptr, 0.f, W0, b0,
                          w0_batched, ln_gamma, ln_beta, O, W_out, b_out, stream, false,
                          inner_loss, weight_decay);
}

int ttt_eta_gate(int B, int H, int L, int d, int io, const void *XK, const float *theta_lr,
                 float eta_base, float *eta, hipStream_t stream) {
    size_t xb, eb, pb;
    int st;
    if ((st = gate_common(B, H, L, d, io, eta_base, &xb, &eb, &pb))) return st;
    const Buf in[] = {{XK, xb, "XK", false, 16}, {theta_lr, pb, "theta_lr", false, 4}};
    const Buf out[] = {{eta, eb, "eta", false, 4}};
    if ((st = check_bufs(in, 2)) || (st = check_bufs(out, 1))) return st;
    if ((st = check_alias(out, 1, in, 2, nullptr))) return st;
    return launched(ttt::launch_eta_gate(B, H, L, d, io, XK, theta_lr, eta_base, eta, stream));
}

int ttt_eta_gate_backward(int B, int H, int L, int d, int io, const void *XK,
                          const float *theta_lr, float eta_base, const float *deta, float *dXK,
                          float *dtheta, hipStream_t stream) {
    size_t xb, eb, pb, gb, tb;
    int st;
    if ((st = gate_common(B, H, L, d, io, eta_base, &xb, &eb, &pb))) return st;
    if (!nbytes(&gb, {size_t(B), size_t(H), size_t(L), size_t(d), sizeof(float)}) ||
        !nbytes(&tb, {size_t(B), size_t(H), size_t(d), sizeof(float)}))
        return fail(TTT_E_SHAPE, "sizes overflow");
    const Buf in[] = {{XK, xb, "XK", false, 16}, {theta_lr, pb, "theta_lr", false, 4},
                      {deta, eb, "deta", false, 4}};
    const Buf out[] = {{dXK, gb, "dXK", false, 16}, {dtheta, tb, "dtheta", false, 4}};
    if ((st = check_bufs(in, 3)) || (st = check_bufs(out, 2))) return st;
    if ((st = check_alias(out, 2, in, 3, nullptr))) return st;
    return launched(ttt::launch_eta_gate_backward(B, H, L, d, io, XK, theta_lr, eta_base, deta,
                                                  dXK, dtheta, stream));
}

int ttt_qkv_project(int B, int L, int d_model, int H, int d, const void *X, const void *theta, void *XQ,
                    void *XK, void *XV, hipStream_t stream) {
    if (B < 0 || L < 0 || H < 0) return fail(TTT_E_SHAPE, "negative size (B=%d L=%d H=%d)", B, L, H);
    if (d != 64) return fail(TTT_E_SHAPE, "d = %d: the projection kernel serves d = 64", d);
    if (d_model <= 0 || d_model % 64)
        return fail(TTT_E_SHAPE, "d_model = %d is not a positive multiple of 64", d_model);
    if (L > TTT_MAX_L) return fail(TTT_E_SHAPE, "L = %d exceeds TTT_MAX_L", L);
    if (static_cast<long long>(B) * L > INT_MAX || 3LL * H * d > INT_MAX)
        return fail(TTT_E_SHAPE, "B*L or 3*H*d exceeds INT_MAX");
    size_t xb, tb, ob;
    if (!nbytes(&xb, {size_t(B), size_t(L), size_t(d_model), 2}) ||
        !nbytes(&tb, {3, size_t(H), size_t(d), size_t(d_model), 2}) ||
        !nbytes(&ob, {size_t(B), size_t(H), size_t(L), size_t(d), 2}))
        return fail(TTT_E_SHAPE, "sizes overflow");
    const bool work = ob > 0;  // nothing to write: no input is read
    const Buf in[] = {{X, work ? xb : 0, "X", false, 16}, {theta, work ? tb : 0, "theta", false, 16}};
    const Buf out[] = {{XQ, ob, "XQ", false, 16}, {XK, ob, "XK", false, 16}, {XV, ob, "XV", false, 16}};
    int st;
    if ((st = check_bufs(in, 2)) || (st = check_bufs(out, 3))) return st;
    if ((st = check_alias(out, 3, in, 2, nullptr)) || (st = check_alias(out, 1, out + 1, 2, nullptr)) ||
        (st = check_alias(out + 1, 1, out + 2, 1, nullptr)))
        return st;
    if (!work) return TTT_OK;
    return launched(ttt::launch_qkv_project(B, L, d_model, H, X, theta, XQ, XK, XV, stream));
}

int ttt_linear_backward_workspace(int B, int H, int L, int d, int mb, size_t *bytes) {
    int st;
    if ((st = check_common(B, H, L, mb, TTT_F32))) return st;
    if (d != 16 && d != 64) return fail(TTT_E_SHAPE, "d = %d not in {16, 64}", d);
    if (!bytes) return fail(TTT_E_NULL, "bytes is NULL");
    const size_t nch = L > 0 ? static_cast<size_t>((L + mb - 1) / mb) : 0;
    if (static_cast<size_t>(B) * H * nch > 0x7fffffffu)
        return fail(TTT_E_SHAPE, "B*H*ceil(L/mb) = %zu chunks exceeds 2^31 - 1", static_cast<size_t>(B) * H * nch);
    if (!nbytes(bytes, {size_t(B), size_t(H), nch, ttt::linear_backward_chunk_floats(d), sizeof(float)}))
        return fail(TTT_E_SHAPE, "sizes overflow");
    return ok();
}

int ttt_linear_backward(int B, int H, int L, int d, int mb, int io, float ln_eps,
                        const void *XQ, const void *XK, const void *XV, const float *eta,
                        const float *W0, const float *b0, int w0_batched,
                        const float *ln_gamma, const float *ln_beta, const float *dO,
                        const float *dW_out, const float *db_out, float *dXQ, float *dXK,
                        float *dXV, float *deta, float *dW0, float *db0, float *dgamma,
                        float *dbeta, void *workspace, size_t workspace_bytes,
                        hipStream_t stream) {
    return linear_backward(B, H, L, d, mb, io, ln_eps, XQ, XK, XV, eta, W0, b0, w0_batched,
                           ln_gamma, ln_beta, dO, dW_out, db_out, dXQ, dXK, dXV, deta, dW0, db0,
                           dgamma, dbeta, workspace, workspace_bytes, false, stream);
}

int ttt_linear_backward_noalloc(int B, int H, int L, int d, int mb, int io, float ln_eps,
                                const void *XQ, const void *XK, const void *XV,
                                const float *eta, const float *W0, const float *b0,
                                int w0_batched, const float *ln_gamma, const float *ln_beta,
                                const float *dO, const float *dW_out, const float *db_out,
                                float *dXQ, float *dXK, float *dXV, float *deta, float *dW0,
                                float *db0, float *dgamma, float *dbeta, hipStream_t stream) {
    return linear_backward(B, H, L, d, mb, io, ln_eps, XQ, XK, XV, eta, W0, b0, w0_batched,
                           ln_gamma, ln_beta, dO, dW_out, db_out, dXQ, dXK, dXV, deta, dW0, db0,
                           dgamma, dbeta, nullptr, 0, true, stream);
}

int ttt_mlp_backward_workspace(int B, int H, int L, int d, int mb, size_t *bytes) {
    int st;
    if ((st = check_common(B, H, L, mb, TTT_F32))) return st;
    if (d != 64) return fail(TTT_E_SHAPE, "d = %d: the MLP supports d = 64 only", d);
    if (!bytes) return fail(TTT_E_NULL, "bytes is NULL");
    const size_t nch = L > 0 ? static_cast<size_t>((L + mb - 1) / mb) : 0;
    if (static_cast<size_t>(B) * H * nch > 0x7fffffffu)
        return fail(TTT_E_SHAPE, "B*H*ceil(L/mb) = %zu chunks exceeds 2^31 - 1", static_cast<size_t>(B) * H * nch);
    if (!nbytes(bytes, {size_t(B), size_t(H), ttt::mlp_backward_seq_floats(L, d, mb), sizeof(float)}))
        return fail(TTT_E_SHAPE, "sizes overflow");
    return ok();
}

int ttt_mlp_backward(int B, int H, int L, int d, int mb, int io, float ln_eps, const void *XQ,
                     const void *XK, const void *XV, const float *eta, const float *W1_0,
                     const float *b1_0, const float *W2_0, const float *b2_0, int w0_batched,
                     const float *ln_gamma, const float *ln_beta, const float *dO,
                     const float *dW1_out, const float *db1_out, const float *dW2_out,
                     const float *db2_out, float *dXQ, float *dXK, float *dXV, float *deta,
                     float *dW1, float *db1, float *dW2, float *db2, float *dgamma, float *dbeta,
                     void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return mlp_backward(B, H, L, d, mb, io, ln_eps, XQ, XK, XV, eta, W1_0, b1_0, W2_0, b2_0,
                        w0_batched, ln_gamma, ln_beta, dO, dW1_out, db1_out, dW2_out, db2_out, dXQ,
                        dXK, dXV, deta, dW1, db1, dW2, db2, dgamma, dbeta, workspace,
                        workspace_bytes, stream);
}

int ttt_mlp_forward(int B, int H, int L, int d, int mb, int io, float ln_eps,
                    const void *XQ, const void *XK, const void *XV, const float *eta,
                    const float *W1_0, const float *b1_0, const float *W2_0,
                    const float *b2_0, int w0_batched, const float *ln_gamma,
                    const float *ln_beta, void *O, float *W1_out, float *b1_out,
                    float *W2_out, float *b2_out, hipStream_t stream) {
    return mlp_forward(B, H, L, d, mb, io, ln_eps, XQ, XK, XV, eta, nullptr, 0.f, W1_0, b1_0,
                       W2_0, b2_0, w0_batched, ln_gamma, ln_beta, O, W1_out, b1_out, W2_out,
                       b2_out, stream, false, TTT_LOSS_MSE, 0.f);
}

int ttt_mlp_forward_gated(int B, int H, int L, int d, int mb, int io, float ln_eps,
                          const void *XQ, const void *XK, const void *XV,
                          const float *theta_lr, float eta_base, const float *W1_0,
                          const float *b1_0, const float *W2_0, const float *b2_0,
                          int w0_batched, const float *ln_gamma, const float *ln_beta, void *O,
                          float *W1_out, float *b1_out, float *W2_out, float *b2_out,
                          hipStream_t stream) {
    return mlp_forward(B, H, L, d, mb, io, ln_eps, XQ, XK, XV, nullptr, theta_lr, eta_base,
                       W1_0, b1_0, W2_0, b2_0, w0_batched, ln_gamma, ln_beta, O, W1_out, b1_out,
                       W2_out, b2_out, stream, true, TTT_LOSS_MSE, 0.f);
}

int ttt_mlp_forward_opts(int B, int H, int L, int d, int mb, int io, float ln_eps,
                         const void *XQ, const void *XK, const void *XV, const float *eta,
                         const float *W1_0, const float *b1_0, const float *W2_0,
                         const float *b2_0, int w0_batched, const float *ln_gamma,
                         const float *ln_beta, int inner_loss, float weight_decay, void *O,
                         float *W1_out, float *b1_out, float *W2_out, float *b2_out,
                         hipStream_t stream) {
    return mlp_forward(B, H, L, d, mb, io, ln_eps, XQ, XK, XV, eta, nullptr, 0.f, W1_0, b1_0,
                       W2_0, b2_0, w0_batched, ln_gamma, ln_beta, O, W1_out, b1_out, W2_out,
                       b2_out, stream, false, inner_loss, weight_decay);
}

int ttt_decode_step(int B, int H, int d, int io, float ln_eps, const void *xq,
                    const void *xk, const void *xv, const float *eta, float *W, float *b,
                    const float *ln_gamma, const float *ln_beta, void *o,
                    hipStream_t stream) {
    int st;
    if ((st = check_common(B, H, 1, 1, io)) || (st = check_eps(ln_eps))) return st;
    if (d != 16 && d != 64) return fail(TTT_E_SHAPE, "d = %d not in {16, 64}", d);
    const size_t es = io == TTT_BF16 ? 2 : 4;
    size_t xb, eb, wb, bb;
    if (!nbytes(&xb, {size_t(B), size_t(H), size_t(d), es}) ||
        !nbytes(&eb, {size_t(B), size_t(H), sizeof(float)}) ||
        !nbytes(&wb, {size_t(B), size_t(H), size_t(d), size_t(d), sizeof(float)}) ||
        !nbytes(&bb, {size_t(B), size_t(H), size_t(d), sizeof(float)}))
        return fail(TTT_E_SHAPE, "sizes overflow");
    const size_t pb = static_cast<size_t>(H) * d * sizeof(float);
    const unsigned ea = static_cast<unsigned>(es);
    const Buf in[] = {{xq, xb, "xq", false, ea}, {xk, xb, "xk", false, ea},
                      {xv, xb, "xv", false, ea}, {eta, eb, "eta", false, 4},
                      {ln_gamma, pb, "ln_gamma", false, 4}, {ln_beta, pb, "ln_beta", false, 4}};
    const Buf out[] = {{W, wb, "W", false, 4}, {b, bb, "b", false, 4}, {o, xb, "o", false, ea}};
    if ((st = check_bufs(in, 6)) || (st = check_bufs(out, 3))) return st;
    if ((st = check_alias(out, 3, in, 6, nullptr))) return st;
    if (B * H == 0) return ok();
    ttt::DecodeArgs a{B, H, d, io, ln_eps, xq, xk, xv, eta, W, b, ln_gamma, ln_beta, o};
    return launched(ttt::launch_decode(a, stream));
}

}  // extern "C"

namespace {

// T decode steps; mb = 1 is b = 1 TTT (Wc, bc unused), mb > 1 the mini-batch
// rule with the chunk-start state in (Wc, bc) and the first step at position
// pos of its chunk.
int decode_steps(int T, int B, int H, int d, int io, float ln_eps, int mb, int pos,
                 const void *xq, const void *xk, const void *xv, const float *eta, float *Wc,
                 float *bc, float *W, float *b, const float *ln_gamma, const float *ln_beta,
                 void *o, hipStream_t stream, const float *theta = nullptr, float eta_base = 0.f,
                 bool gated = false) {
    int st;
    if (T < 0) return fail(TTT_E_SHAPE, "T = %d is negative", T);
    if (gated && !std::isfinite(eta_base))
        return fail(TTT_E_SHAPE, "eta_base = %g is not finite", static_cast<double>(eta_base));
    if ((st = check_common(B, H, 1, mb, io)) || (st = check_eps(ln_eps))) return st;
    if (pos < 0 || pos >= mb) return fail(TTT_E_SHAPE, "pos = %d not in [0, mb = %d)", pos, mb);
    if (d != 16 && d != 64) return fail(TTT_E_SHAPE, "d = %d not in {16, 64}", d);
    const bool ch = mb > 1;
    const size_t es = io == TTT_BF16 ? 2 : 4;
    size_t xb, eb, wb, bb;
    if (!nbytes(&xb, {size_t(T), size_t(B), size_t(H), size_t(d), es}) ||
        !nbytes(&eb, {size_t(T), size_t(B), size_t(H), sizeof(float)}) ||
        !nbytes(&wb, {size_t(B), size_t(H), size_t(d), size_t(d), sizeof(float)}) ||
        !nbytes(&bb, {size_t(B), size_t(H), size_t(d), sizeof(float)}))
        return fail(TTT_E_SHAPE, "sizes overflow");
    const size_t pb = static_cast<size_t>(H) * d * sizeof(float);
    const unsigned ea = static_cast<unsigned>(es);
    const Buf in[] = {{xq, xb, "xq", false, ea}, {xk, xb, "xk", false, ea},
                      {xv, xb, "xv", false, ea},
                      gated ? Buf{theta, pb, "theta_lr", false, 4} : Buf{eta, eb, "eta", false, 4},
                      {ln_gamma, pb, "ln_gamma", false, 4}, {ln_beta, pb, "ln_beta", false, 4}};
    const Buf out[] = {{W, wb, "W", false, 4}, {b, bb, "b", false, 4}, {o, xb, "o", false, ea},
                       {ch ? Wc : nullptr, ch ? wb : 0, "W_chunk", false, 4},
                       {ch ? bc : nullptr, ch ? bb : 0, "b_chunk", false, 4}};
    const int nout = ch ? 5 : 3;
    if ((st = check_bufs(in, 6)) || (st = check_bufs(out, nout))) return st;
    if ((st = check_alias(out, nout, in, 6, nullptr))) return st;
    if (B * H == 0 || T == 0) return ok();
    if (ttt::decode_steps_resident(d)) {
        ttt::DecodeArgs a{B, H, d, io, ln_eps, xq, xk, xv, gated ? nullptr : eta, W, b, ln_gamma,
                          ln_beta, o};
        if (gated) {
            a.theta = theta;
            a.eta_base = eta_base;
        }
        if (ch) {
            a.Wc = Wc;
            a.bc = bc;
            a.mb = mb;
            a.pos = pos;
        }
        return launched(ttt::launch_decode_steps(a, T, stream));
    }
    // other d: one launch of the single-step kernel per step
    const size_t step = static_cast<size_t>(B) * H * d * es;
    const size_t estep = static_cast<size_t>(B) * H;
    for (int t = 0; t < T; ++t) {
        ttt::DecodeArgs a{B, H, d, io, ln_eps,
                          static_cast<const char *>(xq) + t * step, static_cast<const char *>(xk) + t * step,
                          static_cast<const char *>(xv) + t * step, gated ? nullptr : eta + t * estep,
                          W, b, ln_gamma, ln_beta, static_cast<char *>(o) + t * step};
        if (gated) {
            a.theta = theta;
            a.eta_base = eta_base;
        }
        if (ch) {
            a.Wc = Wc;
            a.bc = bc;
            a.mode = (pos + t) % mb == 0 ? 1 : 2;
        }
        if ((st = launched(ttt::launch_decode(a, stream)))) return st;
    }
    return ok();
}

}  // namespace

extern "C" {

int ttt_decode_steps(int T, int B, int H, int d, int io, float ln_eps, const void *xq,
                     const void *xk, const void *xv, const float *eta, float *W, float *b,
                     const float *ln_gamma, const float *ln_beta, void *o,
                     hipStream_t stream) {
    return decode_steps(T, B, H, d, io, ln_eps, 1, 0, xq, xk, xv, eta, nullptr, nullptr, W, b,
                        ln_gamma, ln_beta, o, stream);
}

int ttt_decode_steps_mb(int T, int B, int H, int d, int io, float ln_eps, int mb, int pos,
                        const void *xq, const void *xk, const void *xv, const float *eta,
                        float *W_chunk, float *b_chunk, float *W, float *b,
                        const float *ln_gamma, const float *ln_beta, void *o,
                        hipStream_t stream) {
    return decode_steps(T, B, H, d, io, ln_eps, mb, pos, xq, xk, xv, eta, W_chunk, b_chunk, W, b,
                        ln_gamma, ln_beta, o, stream);
}

int ttt_decode_steps_gated(int T, int B, int H, int d, int io, float ln_eps, int mb, int pos,
                           const void *xq, const void *xk, const void *xv,
                           const float *theta_lr, float eta_base, float *W_chunk,
                           float *b_chunk, float *W, float *b, const float *ln_gamma,
                           const float *ln_beta, void *o, hipStream_t stream) {
    return decode_steps(T, B, H, d, io, ln_eps, mb, pos, xq, xk, xv, nullptr, W_chunk, b_chunk, W,
                        b, ln_gamma, ln_beta, o, stream, theta_lr, eta_base, true);
}

}  // extern "C"
