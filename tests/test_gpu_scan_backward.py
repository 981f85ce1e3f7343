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


# ---- the benchmark's length: one 131072-token sequence, 2048 backward chunks ----------------
FULL_T = 131072


def draw_full_length(d_inner, sample, seed, T=FULL_T, block=8192, width=512, sink=None):
    """One T-token sequence at Jamba widths with `d_inner` channels, bf16 activations. The
    per-channel inputs (x, Delta, z, dg) are drawn for `width` channels in `block`-token blocks
    (bounded host memory and time) and channel d takes those of channel d mod width: the
    channels of the scan are independent, and A_log, D and the states are drawn for every
    channel, so no two channels compute the same thing. sink(row0, arrays) receives every
    block (the device copy); returned are the oracle's inputs for the sampled channels (fp64)
    and the layer's weights. Distributions as in make_case."""
    base = synth.WORKLOADS["prefill_4k"]["dims"]
    dims = synth.LayerDims(d_model=base.d_model, d_inner=d_inner, d_state=16, d_conv=4,
                           dt_rank=base.dt_rank)
    wl = synth.make_workload("prefill_4k", lengths=[4], dims=dims)
    rng = np.random.default_rng(seed)
    width = min(width, d_inner)
    assert d_inner % width == 0
    S = np.asarray(sample)
    cols = {k: np.empty((T, len(S))) for k in ("x", "dt", "z", "dg")}
    BC = {k: np.empty((T, 16)) for k in ("B", "C")}
    for r0 in range(0, T, block):
        n = min(block, T - r0)
        blk = dict(
            x=synth.round_bf16(rng.standard_normal((n, width), dtype=np.float32)),
            dt=np.exp(rng.uniform(np.log(1e-3), np.log(0.3), (n, width))).astype(np.float32),
            B=rng.standard_normal((n, 16), dtype=np.float32),
            C=rng.standard_normal((n, 16), dtype=np.float32),
            z=synth.round_bf16(rng.standard_normal((n, width), dtype=np.float32)),
            dg=synth.round_bf16(rng.standard_normal((n, width), dtype=np.float32)),
        )
        for k in cols:
            cols[k][r0:r0 + n] = blk[k][:, S % width]
        for k in BC:
            BC[k][r0:r0 + n] = blk[k]
        if sink is not None:
            sink(r0, blk)
    h0 = (rng.standard_normal((1, d_inner, 16)) * 0.3).astype(np.float32)
    dh = rng.standard_normal((1, d_inner, 16)).astype(np.float32)
    wl.weights["D"] = rng.standard_normal(d_inner).astype(np.float32)
    wl.weights["A_log"] = (wl.weights["A_log"]
                           + 0.1 * rng.standard_normal((d_inner, 16))).astype(np.float32)
    ref_in = dict(x=cols["x"], dt=cols["dt"], z=cols["z"], dg=cols["dg"], B=BC["B"], C=BC["C"],
                  A_log=wl.weights["A_log"][S].astype(np.float64),
                  D=wl.weights["D"][S].astype(np.float64),
                  h0=h0[0][S].astype(np.float64), dh=dh[0][S].astype(np.float64))
    return wl, ref_in, h0, dh


def sampled_reference(ref_in):
    """The backward oracle on the sampled channels alone: every gradient but dB and dC is
    per channel (dB, dC sum over all channels), so these columns are exact references."""
    r = ref_in
    return sb.scan_gate_backward(r["x"], r["dt"], r["A_log"], r["B"], r["C"], r["D"], r["z"],
                                 r["dg"], r["h0"], r["dh"])


@pytest.mark.parametrize("d_inner,sample", [
    # the benchmark's configuration (d_inner 8192, 128 channel blocks x 2048 chunks): 16
    # channels from both ends and the middle of several 64-channel blocks, some sharing their
    # per-channel draws (d mod 512) with another sampled channel
    (8192, [0, 1, 63, 64, 511, 1000, 2047, 2048, 4095, 4096, 5000, 6143, 7000, 8126, 8190, 8191]),
    # 64 channels, all compared, so dB and dC (sums over channels) are exact references too
    (64, list(range(64))),
])
def test_scan_backward_full_length(d_inner, sample):
    T = FULL_T
    dev = {k: torch.empty((T, d_inner), dtype=torch.bfloat16, device="cuda")
           for k in ("x", "z", "dg")}
    dev["dt"] = torch.empty((T, d_inner), dtype=torch.float32, device="cuda")
    dev["B"] = torch.empty((T, 16), dtype=torch.float32, device="cuda")
    dev["C"] = torch.empty((T, 16), dtype=torch.float32, device="cuda")

    def sink(r0, blk):   # per-channel blocks tiled over d_inner on the device (bf16: exact)
        for k, v in blk.items():
            t = torch.from_numpy(v).cuda().to(dev[k].dtype)
            dev[k][r0:r0 + len(v)] = t if t.shape[1] == dev[k].shape[1] else \
                t.repeat(1, dev[k].shape[1] // t.shape[1])

    wl, ref_in, h0, dh = draw_full_length(d_inner, sample, seed=d_inner + 7, sink=sink)
    layer = device_layer(wl)
    cu = [0, T]
    g = jm.jamba_mamba_scan_backward(
        layer, dev["x"], dev["dt"], dev["B"], dev["C"], dev["z"], dev["dg"],
        torch.tensor(cu, dtype=torch.int32, device="cuda"), cu,
        init_ssm_state=torch.from_numpy(h0).cuda(), d_final_ssm_state=torch.from_numpy(dh).cuda())
    torch.cuda.synchronize()
    del dev
    S = torch.as_tensor(sample, dtype=torch.long, device="cuda")
    ref = sampled_reference(ref_in)
    got = {"dx": to_np(g["dx_hat"][:, S]), "ddt": to_np(g["ddt"][:, S]),
           "dz": to_np(g["dz"][:, S]), "dA_log": to_np(g["dA_log"][S]), "dD": to_np(g["dD"][S]),
           "dh0": to_np(g["d_init_ssm_state"][0][S])}
    if len(sample) == d_inner:
        got["dB"], got["dC"] = to_np(g["dB"]), to_np(g["dC"])
    errs = {k: rel_err(v, ref[k]) for k, v in got.items()}
    print(f"scan backward, one {T}-token sequence, d_inner {d_inner}, {len(sample)} channels compared: "
          + " ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
    assert max(errs.values()) < TOL, errs
