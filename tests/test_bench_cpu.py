"""CPU checks of the benchmark script: the one-GPU contract and the roofline
arithmetic, pinned to figures computed independently from the method's
definition (bytes moved and flops of the dual form per token-head)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout == ""


def test_prefill_algorithmic_bytes():
    # per token-head: XQ, XK, XV in bf16 (3 x 64 x 2 B), eta (4 B), O in bf16
    # (64 x 2 B) = 516 B; per sequence the fp32 state (64 x 64 + 64) x 4 B read
    # and written: 2 x 16,640 B.  B = 2, H = 32, L = 8192.
    assert bench.alg_bytes_linear(2, 32, 8192, 64) == 2 * 32 * (8192 * 516 + 2 * 16640)
    assert bench.alg_bytes_linear(2, 32, 8192, 64) == 272_662_528
    # fp32 storage: 3 x 64 x 4 + 4 + 64 x 4 = 1,028 B per token-head
    assert bench.alg_bytes_linear(1, 1, 64, 16, 4, 4) == 64 * (3 * 16 * 4 + 4 + 16 * 4) + 2 * (256 + 16) * 4


def test_mlp_algorithmic_flops():
    # 56 d^2 + 20 b d = 249,856 flop per token-head at d = 64, b = 16
    assert bench.alg_flops_mlp(2, 12, 8192, 64) == 2 * 12 * 8192 * 249_856
    assert abs(bench.alg_flops_mlp(2, 12, 8192, 64) / 1e9 - 49.12) < 0.01


def test_decode_algorithmic_work():
    # one b = 1 step: 6 d^2 flops per state; state bytes 2 x (d^2 + d) x 4 each way
    assert bench.alg_flops_decode_step(64, 32, 64) == 64 * 32 * 6 * 4096
    assert bench.alg_bytes_decode(64, 32, 64) == 64 * 32 * (2 * 4160 * 4 + 3 * 128 + 4 + 128)


def test_layer_algorithmic_flops():
    # projections: 2 x (B L = 16,384) x d_model 2,048 x (3 H d = 6,144) = 412.3 GFLOP;
    # prefill: 6 d^2 + 4 b d = 28,672 flop per token-head over B H L = 524,288
    assert bench.alg_flops_layer(2, 8192, 2048, 32, 64) == 412_316_860_416 + 524_288 * 28_672
