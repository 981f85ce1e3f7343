"""Host logic of bench.py (no GPU): the algorithmic work behind every roofline fraction, and the
one-GPU contract of the command line.

The per-token byte counts are written out here tensor by tensor (what each step of the layer
must read and write once: "Jamba: A Hybrid Transformer-Mamba Language Model" §2, the Mamba layer
of citation [17]: in_proj -> causal conv + SiLU -> x_proj -> dt_proj + softplus -> selective scan
with the D skip and the SiLU(z) gate -> out_proj), at the Jamba-7B-class widths of the 128K
prefill workload, independently of bench.kernel_work's formulas.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

T, DM, DI, R, N = 131072, 4096, 8192, 256, 16
BF16, F32 = 2, 4


def per_token_bytes():
    """Activation bytes per token of each kernel (weights and per-launch constants excluded)."""
    return {
        # u in (d_model bf16); x and z out (2 d_inner bf16)
        "in_proj": DM * BF16 + 2 * DI * BF16,
        # x in, x_hat out (bf16 each)
        "conv1d_silu": DI * BF16 + DI * BF16,
        # x_hat in (bf16); delta out (dt_rank bf16), B and C out (16 fp32 each)
        "x_proj": DI * BF16 + R * BF16 + 2 * N * F32,
        # delta in (bf16); Delta out (d_inner fp32)
        "dt_proj": R * BF16 + DI * F32,
        # phase A: Delta (fp32) and x_hat (bf16) per channel, B (16 fp32)
        "scan_chunk_state": DI * (F32 + BF16) + N * F32,
        # phase C: Delta (fp32), x_hat, z in and g out (bf16) per channel, B and C
        "scan_chunk_output": DI * (F32 + 3 * BF16) + 2 * N * F32,
        # g in (d_inner bf16), out (d_model bf16)
        "out_proj": DI * BF16 + DM * BF16,
    }


def per_token_flops():
    """Multiply-adds x 2 per token of the projections; 4 taps x 2 per channel for the conv."""
    return {
        "in_proj": 2.0 * DM * 2 * DI,
        "conv1d_silu": 2.0 * 4 * DI,
        "x_proj": 2.0 * DI * (R + 2 * N),
        "dt_proj": 2.0 * R * DI,
        "out_proj": 2.0 * DI * DM,
    }


def test_kernel_work_bytes_per_token_match_the_tensor_counts():
    w1 = bench.kernel_work(1, DM, DI, R, N)
    w2 = bench.kernel_work(2, DM, DI, R, N)
    for k, b in per_token_bytes().items():
        # the slope in T is the per-token traffic; the rest is per launch (weights, biases)
        assert w2[k][1] - w1[k][1] == b, k


def test_kernel_work_weight_bytes_per_launch():
    w = bench.kernel_work(0, DM, DI, R, N)
    assert w["in_proj"][1] == 2 * DI * DM * BF16           # W_in (2 d_inner x d_model)
    assert w["x_proj"][1] == (R + 2 * N) * DI * BF16       # W_x
    assert w["dt_proj"][1] == DI * R * BF16 + DI * F32     # W_dt and the fp32 bias
    assert w["out_proj"][1] == DM * DI * BF16              # W_out
    assert w["conv1d_silu"][1] == DI * 5 * BF16            # 4 taps and a bias per channel


def test_kernel_work_flops_at_128k():
    w = bench.kernel_work(T, DM, DI, R, N)
    for k, f in per_token_flops().items():
        assert w[k][0] == f * T, k
    # the in_proj figure every roofline line of the prefill is quoted on
    assert w["in_proj"][0] == 2 * 131072 * 16384 * 4096


def test_staged_pipeline_bytes_per_token():
    # single-pass pipeline (the scan read once, in its output phase): 230,656 B per token;
    # the chunked scan's first phase re-reads Delta, x_hat and B: another 49,216
    b = per_token_bytes()
    assert sum(v for k, v in b.items() if k != "scan_chunk_state") == 230656
    assert b["scan_chunk_state"] == 49216


def test_bounds_of_kernels():
    assert bench.bound_of("in_proj") == "mfma" and bench.bound_of("out_proj") == "mfma"
    assert bench.bound_of("scan_chunk_state") == "alu"
    assert bench.bound_of("scan_chunk_output") == "alu"
    for k in ("conv1d_silu", "x_proj", "dt_proj", "scan_chunk_carry"):
        assert bench.bound_of(k) == "hbm"


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "4"})])
def test_bench_refuses_more_than_one_gpu(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], env=e,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
