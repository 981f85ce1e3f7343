"""The layer with its optional inner RMSNorm (delta, B and C normalised right after x_proj;
the Jamba paper's §2 Mamba-layer paragraph and §6.4 / Fig. 9 add RMSNorm to the layer's
internal activations). Same checks and bounds as the plain layer: prefill (fp32 and bf16,
packed, with initial states, several chunks) and decode (generic and fast bf16 paths)
against the fp64 oracle, each with D = 1 and the D = 0 twin; plus the x_proj step with its
norm fed the oracle's own input.

x_proj-stage bound in bf16: the normalised delta is rounded twice (x_proj's bf16 output,
then the normalised value), each step at most the unit roundoff 2^-8 = 3.9e-3 of the
element, and the normalisation is scale-invariant, so the norm-wise error stays below
2 x 3.9e-3 plus fp32 arithmetic error; bound 8e-3. B and C stay fp32 throughout: 1e-5.
"""
import numpy as np
import pytest

import oracle
import synth
from jm_testutil import TOL, device_layer, gpu_prefill, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
jm = pytest.importorskip("mamba_selective_scan_mixer_amd")


@pytest.fixture(autouse=True)
def _reset_chunk():
    jm.set_scan_chunk_len(0)
    yield
    jm.set_scan_chunk_len(0)


def _check(wl, tol, init_conv=None, init_ssm=None, label=""):
    assert "dt_norm_w" in wl.weights
    layer = device_layer(wl)
    assert layer.inner_norm
    out, conv, ssm = gpu_prefill(wl, layer, init_conv=init_conv, init_ssm=init_ssm)
    ref = oracle.prefill(wl.weights, wl.u, wl.cu_seqlens, init_conv, init_ssm)
    e = dict(out=rel_err(out, ref["out"]), conv=rel_err(conv, ref["conv_state"]),
             ssm=rel_err(ssm, ref["ssm_state"]))
    print(f"{label} {e}", flush=True)
    assert max(e.values()) < tol, e
    # the norm is really applied: the plain layer's output differs
    plain = {k: v for k, v in wl.weights.items() if k not in oracle.NORM_KEYS}
    ref_plain = oracle.prefill(plain, wl.u, wl.cu_seqlens, init_conv, init_ssm)
    assert rel_err(ref_plain["ssm_state"], ref["ssm_state"]) > 10 * tol


@pytest.mark.parametrize("D_value", [1.0, 0.0])
@pytest.mark.parametrize("chunk", [0, 16])
def test_inner_norm_tiny_fp32_packed(D_value, chunk):
    jm.set_scan_chunk_len(chunk)
    wl = synth.make_workload("tiny_fp32", seed=5, D_value=D_value, inner_norm=True,
                             lengths=[1, 3, 17, 64, 40])
    rng = np.random.default_rng(98)
    n, di = len(wl.lengths), wl.dims.d_inner
    init_conv = rng.standard_normal((n, di, 3)).astype(np.float32)
    init_ssm = (rng.standard_normal((n, di, 16)) * 1e-2).astype(np.float32)
    _check(wl, TOL["f32"], init_conv, init_ssm, label=f"norm tiny chunk={chunk} D={D_value}")


@pytest.mark.parametrize("D_value", [1.0, 0.0])
def test_inner_norm_jamba_bf16(D_value):
    jm.set_scan_chunk_len(64)
    wl = synth.make_workload("prefill_4k", D_value=D_value, inner_norm=True, lengths=[200, 3, 97])
    _check(wl, TOL["bf16"], label=f"norm jamba D={D_value}")


def _decode(wl, steps, tol):
    w64 = oracle.as_f64(wl.weights)
    ref = oracle.prefill(w64, wl.u, wl.cu_seqlens)
    layer = device_layer(wl)
    _, conv_g, ssm_g = gpu_prefill(wl, layer)
    conv_d = to_dev(conv_g, wl.dtype)
    ssm_d = torch.as_tensor(ssm_g.astype(np.float32)).cuda()
    conv_r, ssm_r = ref["conv_state"], ref["ssm_state"]
    for s in range(steps):
        tok = wl.next_decode_tokens()
        out_r, conv_r, ssm_r = oracle.decode_step(w64, tok, conv_r, ssm_r)
        out_g = jm.jamba_mamba_decode_step(layer, to_dev(tok, wl.dtype), conv_d, ssm_d)
        torch.cuda.synchronize()
        e = (rel_err(to_np(out_g), out_r), rel_err(to_np(conv_d), conv_r),
             rel_err(to_np(ssm_d), ssm_r))
        assert max(e) < tol, (s, e)


@pytest.mark.parametrize("D_value", [1.0, 0.0])
def test_inner_norm_decode_tiny_fp32(D_value):
    wl = synth.make_workload("decode_b64", dims=synth.TINY_DIMS, dtype="f32", batch=4,
                             prefill_len=6, steps=8, D_value=D_value, inner_norm=True)
    _decode(wl, 8, TOL["f32"])


@pytest.mark.parametrize("D_value", [1.0, 0.0])
def test_inner_norm_decode_jamba_bf16(D_value):
    wl = synth.make_workload("decode_b64", batch=3, prefill_len=12, steps=5, D_value=D_value,
                             inner_norm=True)
    _decode(wl, 5, TOL["bf16"])


@pytest.mark.parametrize("name", ["tiny_fp32", "prefill_4k"])
def test_inner_norm_x_proj_stage(name):
    wl = synth.make_workload(name, inner_norm=True, lengths=[150])
    layer = device_layer(wl)
    w = oracle.as_f64(wl.weights)
    st = oracle.prefill(w, wl.u, wl.cu_seqlens, intermediates=True)["stages"][0]
    xh = np.asarray(st["x_hat"])
    xh = (synth.round_bf16(xh) if wl.dtype == "bf16" else xh.astype(np.float32)).astype(np.float64)
    d, B, C = jm.jm_stage_x_proj(layer, to_dev(xh, wl.dtype))
    torch.cuda.synchronize()
    dr, Br, Cr = oracle.inner_norm(w, *oracle.x_proj(xh, w["x_proj_w"], wl.dims.dt_rank,
                                                     wl.dims.d_state))
    e = dict(delta=rel_err(to_np(d), dr), B=rel_err(to_np(B), Br), C=rel_err(to_np(C), Cr))
    print(f"x_proj+norm {wl.dtype}: {e}", flush=True)
    assert e["delta"] < (8e-3 if wl.dtype == "bf16" else 1e-5), e
    assert max(e["B"], e["C"]) < 1e-5, e


@pytest.mark.parametrize("dtype,dt_rank", [("bf16", 8), ("bf16", 24), ("f32", 264)])
def test_inner_norm_row_shapes(dtype, dt_rank):
    """The norm kernel's other row layouts: one 16-byte vector per delta row (64 rows per
    wave), three vectors padded to four lanes, and 66 vectors (more than one per lane, so
    the row loops); 150 tokens leave a ragged last wave. Bounds as above."""
    dims = synth.LayerDims(d_model=64, d_inner=128, dt_rank=dt_rank)
    wl = synth.make_workload("tiny_fp32", inner_norm=True, lengths=[150], dims=dims, dtype=dtype)
    layer = device_layer(wl)
    w = oracle.as_f64(wl.weights)
    st = oracle.prefill(w, wl.u, wl.cu_seqlens, intermediates=True)["stages"][0]
    xh = np.asarray(st["x_hat"])
    xh = (synth.round_bf16(xh) if dtype == "bf16" else xh.astype(np.float32)).astype(np.float64)
    d, B, C = jm.jm_stage_x_proj(layer, to_dev(xh, dtype))
    torch.cuda.synchronize()
    dr, Br, Cr = oracle.inner_norm(w, *oracle.x_proj(xh, w["x_proj_w"], dt_rank, wl.dims.d_state))
    e = dict(delta=rel_err(to_np(d), dr), B=rel_err(to_np(B), Br), C=rel_err(to_np(C), Cr))
    print(f"x_proj+norm {dtype} dt_rank {dt_rank}: {e}", flush=True)
    assert e["delta"] < (8e-3 if dtype == "bf16" else 1e-5), e
    assert max(e["B"], e["C"]) < 1e-5, e
