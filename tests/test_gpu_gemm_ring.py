"""The bf16 projection kernel's K pipeline at odd stage counts.

The projections cut K into 64-deep slices held in two LDS buffers; the prologue, the
branch-free steady loop and the peeled last two stages take different paths depending on
the slice count K / 64. The Jamba widths give 64 and 128 slices and the small test widths
1 and 2; these cases add 3, 4, 5 and 7 slices (layer widths d_model 192 / 448 and d_inner
320 / 256), with a token count that leaves a ragged last 256-row tile (300 = 256 + 44).
The dt_rank 256 case sends x_proj (288 outputs) to its dedicated 256 x 288 kernel.

Each projection is fed exactly the oracle's upstream tensor rounded to bf16 and compared
with the oracle's projection of that same tensor: the only difference left is the kernel's
fp32 accumulation and the final bf16 rounding of its output, whose bound is the unit
roundoff of an 8-bit significand (2^-8 = 3.9e-3 of an element), hence 4e-3 norm-wise.
The whole layer is also checked end to end at the layer bound (2e-2, bf16 activations).
"""
import numpy as np
import pytest

import oracle
import synth
from jm_testutil import TOL, device_layer, gpu_prefill, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
jm = pytest.importorskip("mamba_selective_scan_mixer_amd")

BF16_OUT = 4e-3

DIMS = {
    # in_proj K = d_model, x_proj / out_proj K = d_inner: slices K / 64
    "k3_k5": synth.LayerDims(d_model=192, d_inner=320, d_state=16, d_conv=4, dt_rank=16),
    "k7_k4": synth.LayerDims(d_model=448, d_inner=256, d_state=16, d_conv=4, dt_rank=16),
    # dt_rank 256: x_proj has 288 outputs and runs on its own 256 x 288 kernel (5 slices)
    "xp288_k5": synth.LayerDims(d_model=192, d_inner=320, d_state=16, d_conv=4, dt_rank=256),
}


def _bf16(a):
    return synth.round_bf16(np.asarray(a, np.float64)).astype(np.float64)


@pytest.fixture(params=list(DIMS))
def wl(request):
    return synth.make_workload("prefill_4k", lengths=[300], dims=DIMS[request.param],
                               dtype="bf16")


def test_projections_at_odd_slice_counts(wl):
    layer = device_layer(wl)
    w = oracle.as_f64(wl.weights)
    d = wl.dims
    x, z = jm.jm_stage_in_proj(layer, to_dev(wl.u, "bf16"))
    st = oracle.prefill(w, wl.u, wl.cu_seqlens, intermediates=True)["stages"]
    xh_in = _bf16(np.concatenate([s["x_hat"] for s in st]))
    g_in = _bf16(np.concatenate([s["g"] for s in st]))
    delta, B, C = jm.jm_stage_x_proj(layer, to_dev(xh_in, "bf16"))
    out = jm.jm_stage_out_proj(layer, to_dev(g_in, "bf16"))
    torch.cuda.synchronize()
    xr, zr = oracle.in_proj(wl.u, w["in_proj_w"], d.d_inner)
    dr, Br, Cr = oracle.x_proj(xh_in, w["x_proj_w"], d.dt_rank, d.d_state)
    e = dict(x=rel_err(to_np(x), xr), z=rel_err(to_np(z), zr), delta=rel_err(to_np(delta), dr),
             B=rel_err(to_np(B), Br), C=rel_err(to_np(C), Cr),
             out=rel_err(to_np(out), oracle.out_proj(g_in, w["out_proj_w"])))
    print(f"slices in_proj {d.d_model // 64}, x/out_proj {d.d_inner // 64}: "
          + " ".join(f"{k}={v:.1e}" for k, v in e.items()), flush=True)
    assert e["B"] < 1e-5 and e["C"] < 1e-5, e        # fp32 outputs
    assert max(e[k] for k in ("x", "z", "delta", "out")) < BF16_OUT, e


def test_layer_at_odd_slice_counts(wl):
    out, conv, ssm = gpu_prefill(wl)
    ref = oracle.prefill(wl.weights, wl.u, wl.cu_seqlens)
    e = dict(out=rel_err(out, ref["out"]), conv=rel_err(conv, ref["conv_state"]),
             ssm=rel_err(ssm, ref["ssm_state"]))
    print(f"layer d_model {wl.dims.d_model} d_inner {wl.dims.d_inner}: {e}", flush=True)
    assert max(e.values()) < TOL["bf16"], e


def test_persistent_tiles_with_a_ragged_row_block():
    """Jamba widths at 4196 tokens (17 row blocks, the last 100 rows): in_proj has 1088 tiles
    and out_proj 272, so the persistent workgroups take several tiles each and some follow a
    partial tile with a whole one (the wait that opens a tile then also covers the previous
    tile's stores). Both projections against the oracle at the bf16 rounding bound."""
    wl = synth.make_workload("prefill_4k", lengths=[4196], dtype="bf16")
    layer = device_layer(wl)
    w = oracle.as_f64(wl.weights)
    d = wl.dims
    x, z = jm.jm_stage_in_proj(layer, to_dev(wl.u, "bf16"))
    rng = np.random.default_rng(11)
    g_in = _bf16(rng.standard_normal((4196, d.d_inner)) * 0.05)
    out = jm.jm_stage_out_proj(layer, to_dev(g_in, "bf16"))
    torch.cuda.synchronize()
    xr, zr = oracle.in_proj(wl.u, w["in_proj_w"], d.d_inner)
    e = dict(x=rel_err(to_np(x), xr), z=rel_err(to_np(z), zr),
             out=rel_err(to_np(out), oracle.out_proj(g_in, w["out_proj_w"])))
    # the last (partial) row block on its own as well
    e["x_tail"] = rel_err(to_np(x)[4096:], xr[4096:])
    print(f"persistent 4196 tokens: {e}", flush=True)
    assert max(e.values()) < BF16_OUT, e
