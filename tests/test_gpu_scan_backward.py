"""Backward of the scan step on the GPU (jamba_mamba_scan_backward) against the fp64 backward
oracle (oracle/scan_backward.py, pinned by finite differences and autodiff), on identical
inputs: packed sequences of lengths that cross the 64-token chunk borders (including one-token
sequences and T below, at and just above one chunk), with initial states and a gradient on
the final states, fp32 and bf16 activations.

Bound: the gradients are fp32 sums along the recurrence and over up to 8192 channels (dB, dC)
or all tokens (dA_log, dD); each term carries a few ulp (2^-23 = 1.2e-7) from the hardware
exp2 and reciprocal, so 1e-4 norm-wise (the fp32 layer bound) holds with a wide margin
(measured values are printed).
"""
import numpy as np
import pytest

import oracle.scan_backward as sb
import synth
from jm_testutil import device_layer, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
jm = pytest.importorskip("mamba_selective_scan_mixer_amd")

TOL = 1e-4


def make_case(name, lengths, seed, with_states=True, d_inner=None):
    dims = None
    if d_inner is not None:
        base = synth.WORKLOADS[name]["dims"]
        dims = synth.LayerDims(d_model=base.d_model, d_inner=d_inner, d_state=16, d_conv=4,
                               dt_rank=base.dt_rank)
    wl = synth.make_workload(name, lengths=[4], dims=dims)
    rng = np.random.default_rng(seed)
    di = wl.dims.d_inner
    T = int(sum(lengths))
    n = len(lengths)

    def act(a):
        a = a.astype(np.float32)
        return (synth.round_bf16(a) if wl.dtype == "bf16" else a).astype(np.float64)

    f32 = lambda a: a.astype(np.float32).astype(np.float64)  # noqa: E731
    c = dict(
        x=act(rng.standard_normal((T, di))),
        dt=f32(np.exp(rng.uniform(np.log(1e-3), np.log(0.3), (T, di)))),
        B=f32(rng.standard_normal((T, 16))),
        C=f32(rng.standard_normal((T, 16))),
        z=act(rng.standard_normal((T, di))),
        dg=act(rng.standard_normal((T, di))),
        h0=f32(rng.standard_normal((n, di, 16)) * 0.3) if with_states else None,
        dh=f32(rng.standard_normal((n, di, 16))) if with_states else None,
    )
    wl.weights["D"] = rng.standard_normal(di).astype(np.float32)
    wl.weights["A_log"] = (wl.weights["A_log"] + 0.1 * rng.standard_normal((di, 16))).astype(np.float32)
    cu = np.zeros(n + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    return wl, c, cu


def run(wl, c, cu):
    layer = device_layer(wl)
    dev = lambda a, dt: None if a is None else to_dev(a, dt)  # noqa: E731
    cu_d = torch.as_tensor(cu).cuda()
    g = jm.jamba_mamba_scan_backward(
        layer, dev(c["x"], wl.dtype), dev(c["dt"], "f32"), dev(c["B"], "f32"), dev(c["C"], "f32"),
        dev(c["z"], wl.dtype), dev(c["dg"], wl.dtype), cu_d, [int(v) for v in cu],
        init_ssm_state=dev(c["h0"], "f32"), d_final_ssm_state=dev(c["dh"], "f32"))
    torch.cuda.synchronize()
    return g


def reference(wl, c, cu):
    w = wl.weights
    return sb.scan_gate_backward_packed(c["x"], c["dt"], w["A_log"].astype(np.float64), c["B"],
                                        c["C"], w["D"].astype(np.float64), c["z"], c["dg"], cu,
                                        c["h0"], c["dh"])


NAMES = {"dx_hat": "dx", "ddt": "ddt", "dz": "dz", "dB": "dB", "dC": "dC", "dA_log": "dA_log",
         "dD": "dD", "d_init_ssm_state": "dh0"}


@pytest.mark.parametrize("name,lengths", [
    ("tiny_fp32", [1, 3, 17, 64, 70, 5, 129]),
    ("tiny_fp32", [40]),           # one chunk, T < 64
    ("tiny_fp32", [64]),           # exactly one chunk
    ("tiny_fp32", [65, 63]),       # chunk borders inside both sequences
    ("prefill_4k", [200, 3, 97]),  # Jamba widths, bf16 activations
])
def test_scan_backward_matches_oracle(name, lengths):
    wl, c, cu = make_case(name, lengths, seed=sum(lengths))
    g = run(wl, c, cu)
    ref = reference(wl, c, cu)
    errs = {k: rel_err(to_np(g[k]), ref[v]) for k, v in NAMES.items()}
    print(f"scan backward {name} {lengths}: " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()),
          flush=True)
    assert max(errs.values()) < TOL, errs


# Lengths past the 64-token chunk of the backward: the carry kernels take eight chunks per
# step, so 18+ chunks run their loops three times. Borders of `BORDERS` fall on chunk edges
# (64, 704, 832, 1152) and inside chunks (65, 833), with one-token sequences on both sides.
BORDERS = [64, 1, 639, 128, 1, 319]


@pytest.mark.parametrize("name,lengths,d_inner", [
    ("tiny_fp32", BORDERS, 256),               # 1152 tokens, 18 chunks, fp32
    ("tiny_fp32", [1300], 512),               # one sequence over 21 chunks
    ("prefill_4k", [1, 1150, 3], 256),        # bf16 activations, 18 chunks
    ("prefill_4k", [300, 1, 299], None),      # Jamba widths (d_inner 8192), bf16, 10 chunks
])
def test_scan_backward_many_chunks(name, lengths, d_inner):
    wl, c, cu = make_case(name, lengths, seed=len(lengths) + sum(lengths), d_inner=d_inner)
    g = run(wl, c, cu)
    ref = reference(wl, c, cu)
    errs = {k: rel_err(to_np(g[k]), ref[v]) for k, v in NAMES.items()}
    print(f"scan backward {name} d_inner={wl.dims.d_inner} {lengths}: "
          + " ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
    assert max(errs.values()) < TOL, errs


def test_scan_backward_without_states_and_deterministic():
    wl, c, cu = make_case("tiny_fp32", [30, 100, 2], seed=9, with_states=False)
    g1 = run(wl, c, cu)
    g2 = run(wl, c, cu)
    ref = reference(wl, c, cu)
    for k, v in NAMES.items():
        assert rel_err(to_np(g1[k]), ref[v]) < TOL, k
        assert torch.equal(g1[k], g2[k]), k
