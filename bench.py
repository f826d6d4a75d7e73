"""Benchmark: TTT-Linear dual-form prefill at L = 8192 (B=2, H=32, d=64, b=16,
bf16 inputs, fp32 state) through the C ABI on one MI355X.

A step is one ttt_linear_forward call over the whole workload with inputs
already resident in HBM. Prints ONE JSON line (metric, tokens/s, roofline of
the prefill kernel measured with HIP events on the launch stream, and the
fp64 CPU oracle timed on the host cores on the same workload).

Other workloads of the same hot path (--workload):
  2   TTT-Linear prefill, B=4, H=12, L=2048 (RMS-normalised inputs)
  5p  TTT-Linear prefill, B=1, H=32, L=32768
  4   TTT-MLP prefill, B=2, H=12, L=8192 (roofline: bf16 MFMA)
  4o  the MLP prefill through ttt_mlp_forward_opts (inner-product loss, weight
      decay 0.5 on W1 and W2)
  4g  the MLP prefill through ttt_mlp_forward_gated (eta from the gate in the
      kernel, theta_lr ~ N(0, 0.02^2), eta_base = 1/d)
  5d  TTT-Linear decode: one b=1 step on 64 x 32 states (roofline: state bytes)
  5r  TTT-Linear decode: 1024 b=1 steps on 64 x 32 states in one call, states
      resident in registers (roofline: fp32 vector ALU)
  5m  the same 1024 tokens under the mini-batch rule (b = 16) through
      ttt_decode_steps_mb: both states resident (roofline: fp32 vector ALU)
  5g  the same 1024 b=1 steps through ttt_decode_steps_gated (eta from the
      gate in the kernel; roofline: fp32 vector ALU)
  3b  TTT-Linear backward (ttt_linear_backward) on workload 3's shapes
      (roofline: fp32 vector ALU)
  4b  TTT-MLP backward (ttt_mlp_backward) on workload 4's shapes (roofline:
      fp32 MFMA)
  3g  workload 3 through ttt_linear_forward_gated: eta from the learning-rate
      gate evaluated in the kernel (theta_lr ~ N(0, 0.02^2), eta_base = 1/d)
  3gb ttt_eta_gate_backward on workload 3's keys (dXK += the path through
      eta, dtheta per sequence; roofline: HBM)
  3o  workload 3 through ttt_linear_forward_opts with the inner-product loss
      and weight decay 0.5 (the MFMA prefill's option instantiation; roofline: HBM)
  3p  the layer's Q/K/V input projections (ttt_qkv_project) at workload 3's
      shape, model width 2048 (roofline: bf16 MFMA); 2p at workload 2's (768)
  3L  the layer's inner path from its input at workload 3's shape: the Q/K/V
      projections, then the gated prefill, on one stream as one step
      (roofline: bf16 MFMA over the flops of both)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3]
                       [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, datasheet
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, datasheet
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector (packed FMA), datasheet
FP32_MFMA_PEAK_TFLOPS = 157.3    # MI355X dense fp32 MFMA, datasheet
WORKLOAD = 3
METRIC = "TTT layer tokens/s (dual-form prefill, L=8192) + % of roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_linear_prefill_workload3.json")


def alg_bytes_linear(B, H, L, d, s_in=2, s_out=2):
    """Algorithmic HBM bytes of one prefill launch: XQ, XK, XV and eta read,
    O written once per token-head, plus the fp32 state (W, b) read and
    written once per sequence."""
    per_token_head = 3 * d * s_in + 4 + d * s_out
    state = 2 * (d * d + d) * 4
    return B * H * L * per_token_head + B * H * state


def alg_flops_mlp(B, H, L, d, b=16):
    """Algorithmic flops of one TTT-MLP prefill launch (dual form, hidden 4d):
    56 d^2 + 20 b d per token-head."""
    return B * H * L * (56 * d * d + 20 * b * d)


def alg_flops_layer(B, L, dm, H, d, b=16):
    """Algorithmic flops of the layer's inner path from its input: the Q/K/V
    projections (2 B L d_model 3 H d) and the TTT-Linear dual-form prefill,
    6 d^2 + 4 b d per token-head (XK W, XQ W, the state update, the two
    token x token Grams and their products with E)."""
    return 2 * B * L * dm * 3 * H * d + B * H * L * (6 * d * d + 4 * b * d)


def alg_bytes_decode(B, H, d, s_in=2, s_out=2):
    """Algorithmic HBM bytes of one decode step: each fp32 state (W, b) read and
    written once, xq/xk/xv and eta read, o written."""
    return B * H * (2 * (d * d + d) * 4 + 3 * d * s_in + 4 + d * s_out)


def alg_flops_decode_step(B, H, d):
    """Algorithmic flops of one b=1 step on B x H states: xk W, xq W and the
    rank-one update, 2 d^2 each (the O(d) layer-norm work is left out)."""
    return B * H * 6 * d * d


def alg_flops_linear_backward(B, H, L, d, b=16):
    """Algorithmic flops of one ttt_linear_backward call per token-head:
    the forward pass that stores the chunk-start states (XK W and the state
    update, 4 d^2), the recomputed chunk (XK W, XQ W, T E: 4 d^2 + 2 b d),
    and the reverse products (dZb W^T, XK dW', E dW'^T, dZ W^T, XQ^T dZb,
    XK^T dZ: 12 d^2; dA, T^T dZb, dA XK, dA^T XQ: 8 b d; T: 2 b d)."""
    return B * H * L * (20 * d * d + 12 * b * d)


def alg_flops_mlp_backward(B, H, L, d, b=16):
    """Algorithmic flops of one ttt_mlp_backward call per token-head (hidden
    m = 4d, every product 2 flops per multiply-add):
      forward pass storing the chunk-start states: Z1, Z2, E2 W2^T and the two
      state updates, 5 x 2 d m = 40 d^2;
      recomputed chunk: Z1, XQ W1, Z2, E2 W2^T, Ab W2 (40 d^2), T1 and T2 E2
      (4 b d), T1 E1 and the Gram Ab A^T (16 b d);
      reverse products: dZb2 W2^T, A dW2', XK dW1', dQ W2, E2 dW2'^T, dZ2 W2^T,
      dZb1 W1^T, E1 dW1'^T, dZ1 W1^T and the five adjoint-state updates
      (Ab^T dZb2, dQ^T E2, A^T dZ2, XQ^T dZb1, XK^T dZ1): 14 x 8 d^2 = 112 d^2;
      dT2 A, dT2^T Ab, dZb1 E1^T, T1^T dZb1 (32 b d); dZb2 E2^T, T2^T dZb2,
      dT1 XK, dT1^T XQ (8 b d).
    Total 192 d^2 + 60 b d."""
    return B * H * L * (192 * d * d + 60 * b * d)


def kernel_sources_hash():
    from test_sequence_layer_ttt_amd import build as hb
    h = hashlib.sha256()
    # the sources that define the timed prefill kernel's code
    for name in ("linear_mfma.hip", "tile.hpp", "common.hpp"):
        p = os.path.join(hb.CSRC, name)
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(alg_bytes):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    counters, if they were taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("sources_hash") != kernel_sources_hash():
        return None
    return t.get("bytes_per_launch")


# host cores a one-GPU machine gives its job (whatever the host's own count is)
BOX_CPU_SHARE = 16


def cpu_threads(nseq: int) -> int:
    """Oracle threads: min(cores available, the box's share, sequences) -- the
    oracle parallelises over independent (n, h) sequences only."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(BOX_CPU_SHARE, n, int(nseq)))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_single_thread_small():
    """The oracle on one thread at the two small configs: workload 1 (B1 H1
    L64 d16, fp32, gated eta) and workload 2 (B4 H12 L2048 d64), in full."""
    import oracle
    from test_sequence_layer_ttt_amd import gen
    out = {}
    for num in (1, 2):
        x = gen.make_workload(num)
        t = time.perf_counter()
        eta = x.eta if x.eta is not None else oracle.eta_gate(x.XK, x.theta_lr, x.eta_base)
        oracle.linear_forward(x.XQ, x.XK, x.XV, eta, x.W0, x.b0, x.gamma, x.beta, x.eps, mb=16,
                              nthreads=1)
        dt = time.perf_counter() - t
        out[f"workload{num}"] = {"value": x.B * x.L / dt, "unit": "tokens/s", "seconds": dt,
                                 "cores": 1, "shape": f"B{x.B} H{x.H} L{x.L} d{x.d}"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="3", choices=["3", "2", "5p", "4", "4o", "4g", "5d", "5r", "5m", "5g", "3b", "4b",
                             "3g", "3gb", "3o", "3p", "2p", "3L"])
    ap.add_argument("--peaks", action="store_true",
                    help="measure achievable HBM copy bandwidth and bf16 GEMM throughput (context)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 256 MiB device-to-device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): the TTT inner "
              "loop shards over independent (batch, head) sequences with no exchange, so "
              "N GPUs run N independent copies of this measurement.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from test_sequence_layer_ttt_amd import gen, ttt

    if args.peaks:
        return bench_peaks(args)
    if args.copy_calibration:
        # Reference for the HBM byte counters: each launch reads and writes
        # exactly 256 MiB.
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n, "launches": max(1, args.steps)}))
        return

    if args.workload == "4":
        return bench_mlp(args)
    if args.workload == "4o":
        return bench_mlp(args, opts=True)
    if args.workload == "4g":
        return bench_mlp(args, gated=True)
    if args.workload == "5d":
        return bench_decode(args)
    if args.workload == "5r":
        return bench_decode_steps(args)
    if args.workload == "5m":
        return bench_decode_steps(args, mb=16)
    if args.workload == "5g":
        return bench_decode_steps(args, gated=True)
    if args.workload == "3b":
        return bench_backward(args)
    if args.workload == "4b":
        return bench_mlp_backward(args)
    if args.workload == "3gb":
        return bench_gate_backward(args)
    if args.workload in ("3p", "2p"):
        return bench_proj(args, int(args.workload[0]))
    if args.workload == "3L":
        return bench_layer(args)
    wl = {"3": 3, "3g": 3, "3o": 3, "2": 2, "5p": 5}[args.workload]
    gated = args.workload == "3g"
    opts = args.workload == "3o"  # inner-product loss, weight decay 0.5
    w = gen.WORKLOADS[wl]
    x = gen.make_workload(wl, decode_steps=0) if wl == 5 else gen.make_workload(wl)
    if wl == 5:
        x = x[0]
    B, H, L, d = x.B, x.H, x.L, x.d
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bf = torch.bfloat16
    T = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(dt)
    XQ, XK, XV = T(x.XQ, bf), T(x.XK, bf), T(x.XV, bf)
    eta, W0, b0, gam, bet = T(x.eta), T(x.W0), T(x.b0), T(x.gamma), T(x.beta)
    O = torch.empty_like(XQ)
    Wo = torch.empty((B, H, d, d), device=dev)
    bo = torch.empty((B, H, d), device=dev)
    stream = torch.cuda.current_stream()
    if gated:  # gate weights drawn on a stream of their own (seed 3 + 1000)
        theta_np = (0.02 * np.random.default_rng(1003).standard_normal((H, d))).astype(np.float32)
        theta, eta_base = T(theta_np), 1.0 / d

    def step():
        if gated:
            ttt.ttt_linear_forward_gated(XQ, XK, XV, theta, eta_base, W0, b0, gam, bet, O=O,
                                         W_out=Wo, b_out=bo, mb=16, ln_eps=x.eps, stream=stream)
        elif opts:
            ttt.ttt_linear_forward_opts(XQ, XK, XV, eta, W0, b0, gam, bet, "inner_product", 0.5,
                                        O=O, W_out=Wo, b_out=bo, mb=16, ln_eps=x.eps,
                                        stream=stream)
        else:
            ttt.ttt_linear_forward(XQ, XK, XV, eta, W0, b0, gam, bet, O=O, W_out=Wo, b_out=bo,
                                   mb=16, ln_eps=x.eps, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[2 * i].record(stream)
        step()
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(K)]
    kern_avg_s = float(np.mean(kern_ms)) / 1e3
    kern_med_s = float(np.median(kern_ms)) / 1e3
    ms_per_step = wall * 1e3 / K
    tokens = B * L
    value = tokens / (wall / K)

    ab = alg_bytes_linear(B, H, L, d)
    if gated:  # no eta array read; theta_lr [H,d] read once per sequence
        ab += B * H * (d * 4 - L * 4)
    achieved = ab / kern_avg_s / 1e9
    plain = not (gated or opts)
    traffic = measured_traffic(ab) if (wl == WORKLOAD and plain) else None
    tag = ", gated eta" if gated else (", inner-product loss, weight decay 0.5" if opts else "")
    out = {
        "metric": METRIC if wl == WORKLOAD and plain else f"TTT-Linear prefill tokens/s (L={L}{tag})",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name + ("+eta_gate" if gated else "") + ("+ip_loss+wd" if opts else ""), "B": B, "H": H, "L": L, "d": d, "mini_batch": 16,
                   "io": "bf16", "state": "fp32", "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "linear_prefill_mfma",
                     "kernel_avg_us": kern_avg_s * 1e6,
                     "kernel_median_us": kern_med_s * 1e6,
                     "frac_at_median": ab / kern_med_s / 1e9 / HBM_PEAK_GBS,
                     "alg_bytes_per_launch": ab},
    }

    if not args.no_cpu_baseline:
        import oracle
        nt = cpu_threads(B * H)
        xs = {k: np.ascontiguousarray(getattr(x, k), np.float64)
              for k in ("XQ", "XK", "XV", "eta", "W0", "b0", "gamma", "beta")}
        t1 = time.perf_counter()
        if gated:
            xs["eta"] = oracle.eta_gate(xs["XK"], theta_np, eta_base)
        run = (lambda *a, **k: oracle.linear_forward_opts(*a, loss="inner_product",
                                                          weight_decay=0.5, **k)) if opts \
            else oracle.linear_forward
        ro, rW, rb = run(xs["XQ"], xs["XK"], xs["XV"], xs["eta"], xs["W0"],
                                           xs["b0"], xs["gamma"], xs["beta"], x.eps, mb=16,
                                           nthreads=nt)
        tc = time.perf_counter() - t1
        out["cpu_baseline"] = {"value": tokens / tc, "unit": "tokens/s", "cores": nt,
                               "kind": "oracle", "cpu_model": cpu_model(),
                               "threads_rule": f"min(cores available, box share {BOX_CPU_SHARE}, "
                                               f"B*H = {B * H})",
                               "sample": f"full workload (B={B}, H={H}, L={L}), fp64 primal "
                                         f"form, {nt} threads over (n,h), {tc:.2f} s"}
        if wl == WORKLOAD and plain:
            out["cpu_baseline"]["single_thread"] = cpu_single_thread_small()
        if wl == 2:  # also one thread, on one sequence of the workload (scaled to tokens/s)
            one = {k: np.ascontiguousarray(v[:1, :1]) for k, v in xs.items()
                   if k in ("XQ", "XK", "XV", "eta")}
            t2 = time.perf_counter()
            oracle.linear_forward(one["XQ"], one["XK"], one["XV"], one["eta"], xs["W0"][:1],
                                  xs["b0"][:1], xs["gamma"][:1], xs["beta"][:1], x.eps, mb=16,
                                  nthreads=1)
            t1s = time.perf_counter() - t2
            out["cpu_baseline_single_thread"] = {
                "value": L / t1s, "unit": "token-heads/s", "cores": 1, "kind": "oracle",
                "sample": f"one sequence (L={L}), fp64 primal form, 1 thread, {t1s:.3f} s"}
        # parity of the timed launch's outputs against the oracle (S18 metric)
        def rel(g, r):
            g = g.detach().float().cpu().numpy().reshape(B * H, -1).astype(np.float64)
            r = r.reshape(B * H, -1)
            return float((np.abs(g - r).max(1) / np.abs(r).max(1)).max())
        out["parity_vs_oracle"] = {"O": rel(O, ro), "W_out": rel(Wo, rW), "b_out": rel(bo, rb),
                                   "tol": 2e-2}
    print(json.dumps(out), flush=True)


def _timed(step, stream, warmup, K):
    """Warm up, then time K steps: wall clock around all of them and HIP
    events around each launch on the launch stream."""
    import numpy as np
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * K)]
    t0 = time.perf_counter()
    for i in range(K):
        ev[2 * i].record(stream)
        step()
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = float(np.mean([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(K)])) / 1e3
    return wall / K, kern


def _line(metric, value, args, wall_step, dtype, config, roofline, extra=None):
    out = {"metric": metric, "value": value, "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall_step * 1e3,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
           "data": "synthetic", "config": config, "roofline": roofline}
    out.update(extra or {})
    print(json.dumps(out), flush=True)


def bench_mlp(args, opts=False, gated=False):
    """TTT-MLP prefill, workload 4 (B=2, H=12, L=8192, d=64, hidden 256); with
    opts, the inner-product loss and weight decay 0.5 on W1 and W2; with
    gated, eta from the learning-rate gate inside the kernel (theta_lr drawn
    N(0, 0.02^2) from seed 1004, eta_base = 1/d)."""
    import numpy as np
    import torch
    from test_sequence_layer_ttt_amd import gen, ttt
    x = gen.make_workload(4)
    B, H, L, d = x.B, x.H, x.L, x.d
    dev = torch.device("cuda:0")
    T = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(dt)
    bf = torch.bfloat16
    ins = [T(x.XQ, bf), T(x.XK, bf), T(x.XV, bf), T(x.eta), T(x.W1), T(x.b1), T(x.W2), T(x.b2),
           T(x.gamma), T(x.beta)]
    O = torch.empty_like(ins[0])
    kw = dict(device=dev, dtype=torch.float32)
    outs = (torch.empty((B, H, d, 4 * d), **kw), torch.empty((B, H, 4 * d), **kw),
            torch.empty((B, H, 4 * d, d), **kw), torch.empty((B, H, d), **kw))
    stream = torch.cuda.current_stream()
    if gated:
        theta_np = (0.02 * np.random.default_rng(1004).standard_normal((H, d))).astype(np.float32)
        theta, eta_base = T(theta_np), 1.0 / d
        gins = ins[:3] + [theta, eta_base] + ins[4:]
        step = lambda: ttt.ttt_mlp_forward_gated(*gins, O=O, outs=outs, ln_eps=x.eps,
                                                 stream=stream)
    elif opts:
        step = lambda: ttt.ttt_mlp_forward_opts(*ins, "inner_product", 0.5, O=O, outs=outs,
                                                ln_eps=x.eps, stream=stream)
    else:
        step = lambda: ttt.ttt_mlp_forward(*ins, O=O, outs=outs, ln_eps=x.eps, stream=stream)
    wall, kern = _timed(step, stream, args.warmup, args.steps)
    fl = alg_flops_mlp(B, H, L, d)
    roof = {"bound": "mfma", "achieved": fl / kern / 1e12, "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": fl / kern / 1e12 / BF16_PEAK_TFLOPS, "traffic": None,
            "kernel": "mlp_prefill", "kernel_avg_us": kern * 1e6, "alg_flops_per_launch": fl}
    extra = {}
    if not args.no_cpu_baseline:
        import oracle
        nt = cpu_threads(B * H)
        t1 = time.perf_counter()
        run = (lambda *a, **k: oracle.mlp_forward_opts(*a, loss="inner_product",
                                                       weight_decay=0.5, **k)) if opts \
            else oracle.mlp_forward
        eta = oracle.eta_gate(x.XK, theta_np, eta_base) if gated else x.eta
        run(x.XQ, x.XK, x.XV, eta, x.W1, x.b1, x.W2, x.b2, x.gamma, x.beta, x.eps, mb=16,
            nthreads=nt)
        tc = time.perf_counter() - t1
        extra["cpu_baseline"] = {"value": B * L / tc, "unit": "tokens/s", "cores": nt,
                                 "kind": "oracle",
                                 "sample": f"full workload (B={B}, H={H}, L={L}), fp64 primal "
                                           f"form, {nt} threads over (n,h), {tc:.2f} s"}
    tag = ", inner-product loss, weight decay 0.5" if opts else (", gated eta" if gated else "")
    _line(f"TTT-MLP prefill tokens/s (L={L}{tag})", B * L / wall, args, wall, "bf16",
          {"workload": gen.WORKLOADS[4].name + ("+ip_loss+wd" if opts else "")
           + ("+eta_gate" if gated else ""), "B": B, "H": H, "L": L, "d": d, "hidden": 4 * d,
           "mini_batch": 16, "io": "bf16", "state": "fp32", "parallelism": "none (1 GPU)"},
          roof, extra)


def bench_decode(args):
    """One b=1 decode step on the 64 x 32 states of workload 5, each started
    from the B=1, L=32768 prefill's final state."""
    import numpy as np
    import torch
    from test_sequence_layer_ttt_amd import gen, ttt
    nsteps = args.warmup + args.steps
    pre, dec = gen.make_workload(5, decode_steps=nsteps)
    dev = torch.device("cuda:0")
    T = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(dt)
    bf = torch.bfloat16
    _, Wp, bp = ttt.ttt_linear_forward(T(pre.XQ, bf), T(pre.XK, bf), T(pre.XV, bf), T(pre.eta),
                                       T(pre.W0), T(pre.b0), T(pre.gamma), T(pre.beta),
                                       ln_eps=pre.eps)
    B, H, d = dec.B, dec.H, dec.d
    W = Wp[0].expand(B, H, d, d).contiguous()
    b = bp[0].expand(B, H, d).contiguous()
    xq, xk, xv, et = T(dec.XQ, bf), T(dec.XK, bf), T(dec.XV, bf), T(dec.eta)
    g, be = T(pre.gamma), T(pre.beta)
    o = torch.empty((B, H, d), device=dev, dtype=bf)
    stream = torch.cuda.current_stream()
    it = [0]

    def step():
        i = it[0]
        it[0] += 1
        ttt.ttt_decode_step(xq[i], xk[i], xv[i], et[i], W, b, g, be, o=o, ln_eps=pre.eps,
                            stream=stream)
    wall, kern = _timed(step, stream, args.warmup, args.steps)
    ab = alg_bytes_decode(B, H, d)
    roof = {"bound": "hbm", "achieved": ab / kern / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": ab / kern / 1e9 / HBM_PEAK_GBS, "traffic": None, "kernel": "decode_step",
            "kernel_avg_us": kern * 1e6, "alg_bytes_per_launch": ab}
    extra = {}
    if not args.no_cpu_baseline:
        import oracle
        nt = cpu_threads(B * H)
        Wn = np.broadcast_to(Wp[0].cpu().numpy(), (B, H, d, d)).astype(np.float64)
        bn = np.broadcast_to(bp[0].cpu().numpy(), (B, H, d)).astype(np.float64)
        ns = 4  # bounded sample: four steps
        t1 = time.perf_counter()
        for s_ in range(ns):
            oracle.decode_step(dec.XQ[s_], dec.XK[s_], dec.XV[s_], dec.eta[s_], Wn, bn,
                               pre.gamma, pre.beta, pre.eps, nthreads=nt)
        tc = time.perf_counter() - t1
        extra["cpu_baseline"] = {"value": B * ns / tc, "unit": "tokens/s", "cores": nt,
                                 "kind": "oracle",
                                 "sample": f"{ns} steps on all {B}x{H} states, fp64, {nt} threads, "
                                           f"{tc:.2f} s"}
    _line("TTT-Linear decode tokens/s (64 sequences x 32 heads, b=1)", B / wall, args, wall,
          "bf16", {"workload": "ttt_linear_decode_bf16_B64_H32_d64", "B": B, "H": H, "d": d,
                   "io": "bf16", "state": "fp32", "parallelism": "none (1 GPU)"}, roof, extra)


def bench_decode_steps(args, mb: int = 1, gated: bool = False):
    """Workload 5's 1024 b=1 decode steps on 64 x 32 states in one
    ttt_decode_steps call (states resident in registers), each state started
    from the B=1, L=32768 prefill's final state. A bench step is one call;
    successive calls continue from the state the previous one left. With
    mb > 1 the same tokens go through ttt_decode_steps_mb (mini-batch rule,
    chunk-start state as a second resident copy). With gated, each step's
    eta comes from the learning-rate gate inside the kernel
    (ttt_decode_steps_gated, theta_lr ~ N(0, 0.02^2) from seed 1005,
    eta_base = 1/d) instead of the eta array."""
    import numpy as np
    import torch
    from test_sequence_layer_ttt_amd import gen, ttt
    pre, dec = gen.make_workload(5)
    dev = torch.device("cuda:0")
    T = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(dt)
    bf = torch.bfloat16
    _, Wp, bp = ttt.ttt_linear_forward(T(pre.XQ, bf), T(pre.XK, bf), T(pre.XV, bf), T(pre.eta),
                                       T(pre.W0), T(pre.b0), T(pre.gamma), T(pre.beta),
                                       ln_eps=pre.eps)
    S, B, H, d = dec.steps, dec.B, dec.H, dec.d
    W = Wp[0].expand(B, H, d, d).contiguous()
    b = bp[0].expand(B, H, d).contiguous()
    xq, xk, xv, et = T(dec.XQ, bf), T(dec.XK, bf), T(dec.XV, bf), T(dec.eta)
    g, be = T(pre.gamma), T(pre.beta)
    o = torch.empty((S, B, H, d), device=dev, dtype=bf)
    stream = torch.cuda.current_stream()
    if gated:
        theta_np = (0.02 * np.random.default_rng(1005).standard_normal((H, d))).astype(np.float32)
        th = T(theta_np)
        step = lambda: ttt.ttt_decode_steps_gated(xq, xk, xv, th, 1.0 / d, W, b, g, be, o=o,
                                                  ln_eps=pre.eps, stream=stream)
    elif mb == 1:
        step = lambda: ttt.ttt_decode_steps(xq, xk, xv, et, W, b, g, be, o=o, ln_eps=pre.eps,
                                            stream=stream)
    else:  # 1024 steps are 64 whole chunks, so every call starts a chunk (pos = 0)
        Wc, bc = torch.empty_like(W), torch.empty_like(b)
        step = lambda: ttt.ttt_decode_steps_mb(xq, xk, xv, et, Wc, bc, W, b, g, be, mb=mb, pos=0,
                                               o=o, ln_eps=pre.eps, stream=stream)
    wall, kern = _timed(step, stream, args.warmup, args.steps)
    fl = S * alg_flops_decode_step(B, H, d)
    roof = {"bound": "alu", "achieved": fl / kern / 1e12, "peak": FP32_VECTOR_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": fl / kern / 1e12 / FP32_VECTOR_PEAK_TFLOPS,
            "traffic": None, "kernel": "decode_steps_kernel", "kernel_avg_us": kern * 1e6,
            "alg_flops_per_launch": fl, "hbm_bytes_per_launch": S * B * H * (3 * d * 2 + 4 + d * 2)
            + 2 * B * H * (d * d + d) * 4}
    extra = {}
    if mb == 1 and not args.no_cpu_baseline:
        import oracle
        nt = cpu_threads(B * H)
        Wn = np.broadcast_to(Wp[0].cpu().numpy(), (B, H, d, d)).astype(np.float64)
        bn = np.broadcast_to(bp[0].cpu().numpy(), (B, H, d)).astype(np.float64)
        ns = 4  # bounded sample: four steps
        t1 = time.perf_counter()
        for s_ in range(ns):
            et_s = dec.eta[s_]
            if gated:  # the oracle's gate on this step's keys ([B,H,d] -> [B,H,1,d])
                et_s = oracle.eta_gate(dec.XK[s_][:, :, None], theta_np, 1.0 / d)[:, :, 0]
            oracle.decode_step(dec.XQ[s_], dec.XK[s_], dec.XV[s_], et_s, Wn, bn,
                               pre.gamma, pre.beta, pre.eps, nthreads=nt)
        tc = time.perf_counter() - t1
        extra["cpu_baseline"] = {"value": B * ns / tc, "unit": "tokens/s", "cores": nt,
                                 "kind": "oracle",
                                 "sample": f"{ns} steps on all {B}x{H} states, fp64, {nt} threads, "
                                           f"{tc:.2f} s"}
    if mb > 1 and not args.no_cpu_baseline:
        # the oracle's mini-batch rule over one chunk of mb tokens on all states
        import oracle
        nt = cpu_threads(B * H)
        Wn = np.broadcast_to(Wp[0].cpu().numpy(), (B, H, d, d)).astype(np.float64)
        bn = np.broadcast_to(bp[0].cpu().numpy(), (B, H, d)).astype(np.float64)
        tok = lambda a: np.ascontiguousarray(np.moveaxis(a[:mb], 0, 2))  # [T,B,H,..] -> [B,H,T,..]
        t1 = time.perf_counter()
        oracle.linear_forward(tok(dec.XQ), tok(dec.XK), tok(dec.XV), tok(dec.eta), Wn, bn,
                              pre.gamma, pre.beta, pre.eps, mb=mb, w0_batched=True, nthreads=nt)
        tc = time.perf_counter() - t1
        extra["cpu_baseline"] = {"value": B * mb / tc, "unit": "tokens/s", "cores": nt,
                                 "kind": "oracle",
                                 "sample": f"one chunk of {mb} tokens on all {B}x{H} states "
                                           f"(mini-batch rule), fp64, {nt} threads, {tc:.2f} s"}
    gtag = ", gated eta" if gated else ""
    _line(f"TTT-Linear decode tokens/s (64 sequences x 32 heads, b={mb}, 1024 steps per call{gtag})",
          B * S / wall, args, wall, "bf16",
          {"workload": "ttt_linear_decode_steps_bf16_T1024_B64_H32_d64" + (f"_mb{mb}" if mb > 1 else "")
           + ("+eta_gate" if gated else ""),
           "T": S, "B": B, "H": H, "d": d, "mini_batch": mb, "io": "bf16",
           "state": "fp32, resident in registers", "parallelism": "none (1 GPU)"}, roof, extra)


def bench_backward(args):
    """ttt_linear_backward on workload 3's shapes (B=2, H=32, L=8192, d=64,
    b=16, bf16 inputs), with a seeded dO and dW_out = db_out = 0."""
    import numpy as np
    import torch
    from test_sequence_layer_ttt_amd import gen, ttt
    x = gen.make_workload(3)
    B, H, L, d = x.B, x.H, x.L, x.d
    dev = torch.device("cuda:0")
    T = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(dt)
    bf = torch.bfloat16
    ins = [T(x.XQ, bf), T(x.XK, bf), T(x.XV, bf), T(x.eta), T(x.W0), T(x.b0), T(x.gamma), T(x.beta)]
    dO = torch.randn((B, H, L, d), generator=torch.Generator(device="cpu").manual_seed(3),
                     dtype=torch.float32).to(dev)
    ws = torch.empty(ttt.ttt_linear_backward_workspace(B, H, L, d, 16), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()
    step = lambda: ttt.ttt_linear_backward(*ins, dO, mb=16, ln_eps=x.eps, workspace=ws,
                                           stream=stream)
    wall, kern = _timed(step, stream, args.warmup, args.steps)
    fl = alg_flops_linear_backward(B, H, L, d)
    # one call is three launches of linear_backward_kernel (forward sweep, pre-pass, reverse
    # sweep); the events bracket the call, so kernel_avg_us is their sum
    roof = {"bound": "alu", "achieved": fl / kern / 1e12, "peak": FP32_VECTOR_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": fl / kern / 1e12 / FP32_VECTOR_PEAK_TFLOPS,
            "traffic": None, "kernel": "linear_backward_kernel (forward sweep + pre-pass + reverse sweep)",
            "kernel_avg_us": kern * 1e6, "alg_flops_per_launch": fl, "launches_per_call": 3}
    extra = {}
    if not args.no_cpu_baseline:
        from oracle import grad as OG
        # bounded sample: one sequence, the first 1024 tokens
        ns = 1024
        sl = lambda a: np.ascontiguousarray(a[:1, :1, :ns])
        t1 = time.perf_counter()
        OG.linear_backward(sl(x.XQ), sl(x.XK), sl(x.XV), sl(x.eta), x.W0[:1], x.b0[:1],
                           x.gamma[:1], x.beta[:1], x.eps, 16, dO[:1, :1, :ns].cpu().numpy())
        tc = time.perf_counter() - t1
        extra["cpu_baseline"] = {"value": ns / tc, "unit": "token-heads/s (one head)",
                                 "cores": torch.get_num_threads(), "kind": "oracle",
                                 "sample": f"autograd of the fp64 primal recurrence, one head, "
                                           f"{ns} tokens, {tc:.2f} s"}
    _line("TTT-Linear backward tokens/s (L=8192)", B * L / wall, args, wall, "bf16 in, fp32",
          {"workload": "ttt_linear_backward_bf16_B2_H32_L8192_d64", "B": B, "H": H, "L": L,
           "d": d, "mini_batch": 16, "io": "bf16", "grads": "fp32", "parallelism": "none (1 GPU)"},
          roof, extra)



def bench_mlp_backward(args):
    """ttt_mlp_backward on workload 4's shapes (B=2, H=12, L=8192, d=64,
    hidden 256, b=16, bf16 inputs), with a seeded dO and the state adjoints
    dW1_out ... db2_out = 0."""
    import numpy as np
    import torch
    from test_sequence_layer_ttt_amd import gen, ttt
    x = gen.make_workload(4)
    B, H, L, d = x.B, x.H, x.L, x.d
    dev = torch.device("cuda:0")
    T = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(dt)
    bf = torch.bfloat16
    ins = [T(x.XQ, bf), T(x.XK, bf), T(x.XV, bf), T(x.eta), T(x.W1), T(x.b1), T(x.W2), T(x.b2),
           T(x.gamma), T(x.beta)]
    dO = torch.randn((B, H, L, d), generator=torch.Generator(device="cpu").manual_seed(4),
                     dtype=torch.float32).to(dev)
    ws = torch.empty(ttt.ttt_mlp_backward_workspace(B, H, L, d, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    step = lambda: ttt.ttt_mlp_backward(*ins, dO, mb=16, ln_eps=x.eps, workspace=ws, stream=stream)
    wall, kern = _timed(step, stream, args.warmup, args.steps)
    fl = alg_flops_mlp_backward(B, H, L, d)
    # one call is three launches of mlp_backward_kernel on the stream: the forward sweep and the
    # reverse sweep (B*H workgroups each) and the pre-pass (one workgroup per chunk); the
    # events bracket the call, so kernel_avg_us is their sum
    roof = {"bound": "mfma", "achieved": fl / kern / 1e12, "peak": FP32_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": fl / kern / 1e12 / FP32_MFMA_PEAK_TFLOPS,
            "traffic": None, "kernel": "mlp_backward_kernel (forward sweep + pre-pass + reverse sweep)",
            "kernel_avg_us": kern * 1e6, "alg_flops_per_launch": fl,
            "launches_per_call": 3}
    extra = {}
    if not args.no_cpu_baseline:
        from oracle import grad as OG
        # bounded sample: one sequence, the first 2048 tokens
        ns = 2048
        sl = lambda a: np.ascontiguousarray(a[:1, :1, :ns])
        t1 = time.perf_counter()
        OG.mlp_backward(sl(x.XQ), sl(x.XK), sl(x.XV), sl(x.eta), x.W1[:1], x.b1[:1], x.W2[:1],
                        x.b2[:1], x.gamma[:1], x.beta[:1], x.eps, 16, dO[:1, :1, :ns].cpu().numpy())
        tc = time.perf_counter() - t1
        extra["cpu_baseline"] = {"value": ns / tc, "unit": "token-heads/s (one head)",
                                 "cores": torch.get_num_threads(), "kind": "oracle",
                                 "sample": f"autograd of the fp64 TTT-MLP primal recurrence, one head, "
                                           f"{ns} tokens, {tc:.2f} s"}
    _line("TTT-MLP backward tokens/s (L=8192)", B * L / wall, args, wall, "bf16 in, fp32",
          {"workload": "ttt_mlp_backward_bf16_B2_H12_L8192_d64", "B": B, "H": H, "L": L, "d": d,
           "hidden": 4 * d, "mini_batch": 16, "io": "bf16", "grads": "fp32",
           "parallelism": "none (1 GPU)"}, roof, extra)


def bench_gate_backward(args):
    """ttt_eta_gate_backward on workload 3's keys (B=2, H=32, L=8192, d=64,
    bf16): a seeded deta, theta_lr ~ N(0, 0.02^2), eta_base = 1/d. Algorithmic
    bytes per call: XK and deta read once, dXK read and written, per token-head."""
    import numpy as np
    import torch
    from test_sequence_layer_ttt_amd import gen, ttt
    x = gen.make_workload(3)
    B, H, L, d = x.B, x.H, x.L, x.d
    dev = torch.device("cuda:0")
    XK = torch.from_numpy(x.XK).to(dev).to(torch.bfloat16)
    rng = np.random.default_rng(1003)
    theta_np = (0.02 * rng.standard_normal((H, d))).astype(np.float32)
    deta_np = rng.standard_normal((B, H, L)).astype(np.float32)
    th, deta = torch.from_numpy(theta_np).to(dev), torch.from_numpy(deta_np).to(dev)
    dXK = torch.zeros((B, H, L, d), device=dev)
    dth = torch.empty((B, H, d), device=dev)
    stream = torch.cuda.current_stream()
    eta = torch.empty((B, H, L), device=dev)
    fwd = lambda: ttt.ttt_eta_gate(XK, th, 1.0 / d, eta=eta, stream=stream)
    _, kern_f = _timed(fwd, stream, args.warmup, args.steps)  # the forward gate, for reference
    fb = B * H * L * (d * 2 + 4) + H * d * 4
    step = lambda: ttt.ttt_eta_gate_backward(XK, th, 1.0 / d, deta, dXK, dtheta=dth, stream=stream)
    wall, kern = _timed(step, stream, args.warmup, args.steps)
    ab = B * H * L * (d * 2 + 4 + 2 * d * 4) + H * d * 4 + B * H * d * 4
    roof = {"bound": "hbm", "achieved": ab / kern / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": ab / kern / 1e9 / HBM_PEAK_GBS, "traffic": None,
            "kernel": "eta_gate_bwd_dx + eta_gate_bwd_dtheta (one call)",
            "kernel_avg_us": kern * 1e6, "alg_bytes_per_launch": ab}
    extra = {"eta_gate_fwd": {"kernel_avg_us": kern_f * 1e6, "alg_bytes_per_launch": fb,
                              "achieved_GBps": fb / kern_f / 1e9}}
    if not args.no_cpu_baseline:
        from oracle import grad as OG
        t1 = time.perf_counter()
        OG.eta_gate_backward(x.XK, theta_np, 1.0 / d, deta_np)
        tc = time.perf_counter() - t1
        extra["cpu_baseline"] = {"value": B * L / tc, "unit": "tokens/s",
                                 "cores": torch.get_num_threads(), "kind": "oracle",
                                 "sample": f"autograd of the fp64 gate over the whole workload, "
                                           f"{tc:.2f} s"}
    _line("learning-rate gate backward tokens/s (L=8192)", B * L / wall, args, wall, "bf16 in, fp32",
          {"workload": "ttt_eta_gate_backward_bf16_B2_H32_L8192_d64", "B": B, "H": H, "L": L,
           "d": d, "io": "bf16", "grads": "fp32", "parallelism": "none (1 GPU)"}, roof, extra)



def bench_proj(args, num: int):
    """The layer's Q/K/V input projections (ttt_qkv_project) at a Linear
    workload's shape (model width H*d), an MFMA-bound bf16 GEMM: the
    algorithmic flops are 2 * B*L * d_model * 3*H*d per launch."""
    import numpy as np
    import torch
    from test_sequence_layer_ttt_amd import gen, ttt
    x = gen.make_proj_workload(num)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    X = torch.from_numpy(x.X).to(dev).to(torch.bfloat16)
    th = torch.from_numpy(x.theta).to(dev).to(torch.bfloat16)
    out = tuple(torch.empty((x.B, x.H, x.L, x.d), device=dev, dtype=torch.bfloat16) for _ in range(3))
    stream = torch.cuda.current_stream()
    wall, kern = _timed(lambda: ttt.ttt_qkv_project(X, th, x.H, out=out, stream=stream), stream,
                        args.warmup, args.steps)
    fl = 2.0 * x.B * x.L * x.dm * 3 * x.H * x.d
    ach = fl / kern / 1e12
    extra = {}
    if not args.no_cpu_baseline:  # the oracle's sums at a bounded sample of outputs
        import oracle
        rng = np.random.default_rng(num)
        n = 20000
        idx = np.stack([rng.integers(0, 3, n), rng.integers(0, x.B, n), rng.integers(0, x.H, n),
                        rng.integers(0, x.L, n), rng.integers(0, x.d, n)], axis=1).astype(np.int32)
        t = time.perf_counter()
        oracle.qkv_project_at(x.X, x.theta, x.H, idx)
        tc = time.perf_counter() - t
        extra["cpu_baseline"] = {"value": n / tc / (3 * x.H * x.d) , "unit": "tokens/s", "cores": 1,
                                 "kind": "oracle", "cpu_model": cpu_model(),
                                 "sample": f"{n} outputs one by one (fp64 sums over d_model = {x.dm}), "
                                           f"1 thread, {tc:.2f} s, scaled to tokens of 3 H d outputs"}
    _line(f"Q/K/V projection tokens/s (d_model={x.dm})", x.B * x.L / wall, args, wall, "bf16",
          {"workload": f"qkv_project_B{x.B}_L{x.L}_dmodel{x.dm}_H{x.H}_d{x.d}", "B": x.B, "L": x.L,
           "d_model": x.dm, "H": x.H, "d": x.d, "parallelism": "none (1 GPU)"},
          {"bound": "mfma", "achieved": ach, "peak": 2500.0, "unit": "TFLOP/s", "frac": ach / 2500.0,
           "traffic": None, "kernel": "qkv_project_kernel", "kernel_avg_us": kern * 1e6,
           "alg_flops_per_launch": fl}, extra)


def bench_layer(args):
    """The TTT-Linear layer's inner path from its input at workload 3's shape
    (B=2, L=8192, model width 2048, H=32, d=64): the Q/K/V projections of X
    (ttt_qkv_project) and the prefill with the learning-rate gate inside the
    kernel (ttt_linear_forward_gated), launched back to back on one stream and
    timed as one step. X ~ N(0, 1) and theta ~ N(0, 0.02^2) as in the
    projection workload (seed 103); W0 ~ N(0, 0.02^2), b0 = 0, gamma = 1,
    beta = 0, theta_lr ~ N(0, 0.02^2), eta_base = 1/d (seed 1003)."""
    import numpy as np
    import torch
    from test_sequence_layer_ttt_amd import gen, ttt
    x = gen.make_proj_workload(3)
    B, L, dm, H, d = x.B, x.L, x.dm, x.H, x.d
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    X = torch.from_numpy(x.X).to(dev).to(torch.bfloat16)
    th = torch.from_numpy(x.theta).to(dev).to(torch.bfloat16)
    XQ, XK, XV, O = (torch.empty((B, H, L, d), device=dev, dtype=torch.bfloat16) for _ in range(4))
    rng = np.random.default_rng(1003)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    W0 = f32(0.02 * rng.standard_normal((H, d, d)))
    theta_lr = f32(0.02 * rng.standard_normal((H, d)))
    b0, gam, bet = f32(np.zeros((H, d))), f32(np.ones((H, d))), f32(np.zeros((H, d)))
    Wo = torch.empty((B, H, d, d), device=dev)
    bo = torch.empty((B, H, d), device=dev)
    stream = torch.cuda.current_stream()

    def step():
        ttt.ttt_qkv_project(X, th, H, out=(XQ, XK, XV), stream=stream)
        ttt.ttt_linear_forward_gated(XQ, XK, XV, theta_lr, 1.0 / d, W0, b0, gam, bet, O=O, W_out=Wo,
                                     b_out=bo, mb=16, ln_eps=gen.LN_EPS, stream=stream)

    wall, kern = _timed(step, stream, args.warmup, args.steps)
    fl = alg_flops_layer(B, L, dm, H, d)
    ach = fl / kern / 1e12
    _line("TTT-Linear layer tokens/s from its input (Q/K/V projections + gated dual-form prefill)",
          B * L / wall, args, wall, "bf16",
          {"workload": f"ttt_linear_layer_B{B}_L{L}_dmodel{dm}_H{H}_d{d}", "B": B, "L": L, "d_model": dm,
           "H": H, "d": d, "mini_batch": 16, "parallelism": "none (1 GPU)"},
          {"bound": "mfma", "achieved": ach, "peak": 2500.0, "unit": "TFLOP/s", "frac": ach / 2500.0,
           "traffic": None, "kernel": "qkv_project_kernel + linear_prefill_mfma (gated)",
           "kernel_avg_us": kern * 1e6, "alg_flops_per_launch": fl})


def bench_peaks(args):
    """Achievable peaks on this GPU, as context for the datasheet figures the
    roofline fractions use: a 1 GiB device-to-device copy (HBM read + write)
    and an 8192^3 bf16 matrix product through the vendor GEMM library."""
    import torch
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    _, kc = _timed(lambda: dst.copy_(src), stream, 3, 20)
    del src, dst
    m = 8192
    a = torch.randn(m, m, device=dev).to(torch.bfloat16)
    b = torch.randn(m, m, device=dev).to(torch.bfloat16)
    c = torch.empty(m, m, device=dev, dtype=torch.bfloat16)
    _, kg = _timed(lambda: torch.mm(a, b, out=c), stream, 3, 20)
    print(json.dumps({
        "copy": {"bytes_read_plus_written": 2 * n, "us": kc * 1e6, "GBps": 2 * n / kc / 1e9,
                 "frac_of_8000": 2 * n / kc / 1e9 / HBM_PEAK_GBS},
        "bf16_gemm": {"shape": [m, m, m], "us": kg * 1e6, "TFLOPs": 2 * m ** 3 / kg / 1e12,
                      "frac_of_2500": 2 * m ** 3 / kg / 1e12 / BF16_PEAK_TFLOPS}}), flush=True)


if __name__ == "__main__":
    main()
