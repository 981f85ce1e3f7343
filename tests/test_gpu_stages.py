"""Stage-level parity: each step of the prefill (jm_stage_* entry points) fed the oracle's own
upstream tensors, rounded to the dtype the kernel reads, and compared with the oracle step
applied to exactly those inputs. With identical inputs the only differences left are the
kernel's arithmetic and its output rounding, so the bounds are far tighter than the
end-to-end ones:

  * outputs stored in bf16: one round-to-nearest-even step changes an element by at most the
    unit roundoff of an 8-bit significand, 2^-8 = 3.9e-3 of its size, so the norm-wise error
    is at most 3.9e-3 plus the fp32 arithmetic error (~1e-6 here); bound 4e-3;
  * fp32 outputs of a projection (B, C, Delta): fp32 accumulation over K <= 8192 terms and,
    for Delta, the hardware exp2 / log2 / reciprocal of the softplus (a few ulp each, an ulp
    being 2^-23 = 1.2e-7); bound 1e-5;
  * fp32 scan outputs (final state; g in the fp32 layer): each step's exp2 and FMAs carry a
    couple of ulp, and a state sums at most 203 steps here: 203 x 2 x 1.2e-7 = 4.9e-5 in the
    worst case; bound 5e-5.

The scan runs with D = 1 and with D = 0 (without the skip term, g is the scan alone), in
one chunk and in 32-token chunks (several chunks, sequences crossing chunk borders).
"""
import numpy as np
import pytest

import oracle
import synth
from jm_testutil import device_layer, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
jm = pytest.importorskip("mamba_selective_scan_mixer_amd")

BF16_OUT = 4e-3
F32_PROJ = 1e-5
F32_SCAN = 5e-5

CASES = {
    # name: (workload, lengths, layer sizes (None: the workload's own))
    "tiny_fp32": ("tiny_fp32", [37, 64, 3, 100], None),
    "jamba_bf16": ("prefill_4k", [150, 3, 203], None),
    # dt_rank 128: the dt_proj kernel's 8-slice form (half its waves load no token rows)
    "rank128_bf16": ("prefill_4k", [150, 3, 203],
                     synth.LayerDims(d_model=512, d_inner=1024, d_state=16, d_conv=4, dt_rank=128)),
    # fp32 matrix-core projections at odd widths: dt_proj K = 24 (one whole and one partial
    # 16-deep slice), x_proj 56 outputs (less than one 64-wide tile), 3 / 5 / 10 feature tiles
    # for out_proj / dt_proj / in_proj, 356 tokens (a ragged last 64-row tile)
    "odd_fp32": ("tiny_fp32", [150, 3, 203],
                 synth.LayerDims(d_model=192, d_inner=320, d_state=16, d_conv=4, dt_rank=24)),
}


def _round(a, dtype):
    """The values the kernel reads: dtype-rounded fp64 array."""
    a = np.asarray(a, dtype=np.float64)
    return synth.round_bf16(a).astype(np.float64) if dtype == "bf16" else a.astype(np.float32).astype(np.float64)


def _out_tol(dtype, kind):
    if kind == "proj":
        return BF16_OUT if dtype == "bf16" else F32_PROJ
    return BF16_OUT if dtype == "bf16" else F32_SCAN


@pytest.fixture(params=list(CASES))
def case(request):
    name, lengths, dims = CASES[request.param]
    wl = synth.make_workload(name, lengths=lengths, dims=dims)
    rng = np.random.default_rng(7)
    n = len(lengths)
    di = wl.dims.d_inner
    init_conv = _round(rng.standard_normal((n, di, 3)), wl.dtype)
    init_ssm = rng.standard_normal((n, di, 16)).astype(np.float32).astype(np.float64) * 0.01
    return wl, init_conv, init_ssm


def _cu(wl):
    return torch.as_tensor(np.asarray(wl.cu_seqlens, np.int32)).cuda(), [int(v) for v in wl.cu_seqlens]


def _seqs(wl):
    cu = wl.cu_seqlens
    return [(int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]


def test_stage_in_proj(case):
    wl, _, _ = case
    layer = device_layer(wl)
    x, z = jm.jm_stage_in_proj(layer, to_dev(wl.u, wl.dtype))
    torch.cuda.synchronize()
    w = oracle.as_f64(wl.weights)
    xr, zr = oracle.in_proj(wl.u, w["in_proj_w"], wl.dims.d_inner)
    e = dict(x=rel_err(to_np(x), xr), z=rel_err(to_np(z), zr))
    print(f"in_proj {wl.dtype}: {e}", flush=True)
    assert max(e.values()) < _out_tol(wl.dtype, "proj"), e


def test_stage_conv(case):
    wl, init_conv, _ = case
    layer = device_layer(wl)
    w = oracle.as_f64(wl.weights)
    x_ref, _ = oracle.in_proj(wl.u, w["in_proj_w"], wl.dims.d_inner)
    x_in = _round(x_ref, wl.dtype)
    cu_d, cu_h = _cu(wl)
    xh, fc = jm.jm_stage_conv(layer, to_dev(x_in, wl.dtype), cu_d, cu_h,
                              init_conv_state=to_dev(init_conv, wl.dtype))
    torch.cuda.synchronize()
    xh_ref = np.empty_like(x_in)
    fc_ref = np.empty_like(init_conv)
    for i, (s, e) in enumerate(_seqs(wl)):
        xh_ref[s:e], fc_ref[i] = oracle.causal_conv_silu(x_in[s:e], w["conv_w"], w["conv_b"],
                                                         init_conv[i])
    err = dict(x_hat=rel_err(to_np(xh), xh_ref))
    # the final conv state is a copy of (rounded) inputs: bit-exact
    assert np.array_equal(to_np(fc), fc_ref), "final conv state differs from the input rows"
    print(f"conv {wl.dtype}: {err}", flush=True)
    assert err["x_hat"] < _out_tol(wl.dtype, "proj"), err


def test_stage_x_proj(case):
    wl, _, _ = case
    layer = device_layer(wl)
    w = oracle.as_f64(wl.weights)
    st = oracle.prefill(w, wl.u, wl.cu_seqlens, intermediates=True)["stages"]
    xh_in = _round(np.concatenate([s["x_hat"] for s in st]), wl.dtype)
    d, B, C = jm.jm_stage_x_proj(layer, to_dev(xh_in, wl.dtype))
    torch.cuda.synchronize()
    dr, Br, Cr = oracle.x_proj(xh_in, w["x_proj_w"], wl.dims.dt_rank, wl.dims.d_state)
    e = dict(delta=rel_err(to_np(d), dr), B=rel_err(to_np(B), Br), C=rel_err(to_np(C), Cr))
    print(f"x_proj {wl.dtype}: {e}", flush=True)
    assert e["delta"] < _out_tol(wl.dtype, "proj"), e
    assert max(e["B"], e["C"]) < F32_PROJ, e


def test_stage_dt_proj(case):
    wl, _, _ = case
    layer = device_layer(wl)
    w = oracle.as_f64(wl.weights)
    st = oracle.prefill(w, wl.u, wl.cu_seqlens, intermediates=True)["stages"]
    d_in = _round(np.concatenate([s["delta"] for s in st]), wl.dtype)
    dt = jm.jm_stage_dt_proj(layer, to_dev(d_in, wl.dtype))
    torch.cuda.synchronize()
    ref = oracle.dt_proj(d_in, w["dt_proj_w"], w["dt_proj_b"])
    e = rel_err(to_np(dt), ref)
    print(f"dt_proj {wl.dtype}: {e:.2e}", flush=True)
    assert e < F32_PROJ, e


@pytest.mark.parametrize("chunk", [0, 32])
@pytest.mark.parametrize("D_value", [1.0, 0.0])
def test_stage_scan(case, chunk, D_value):
    wl, _, init_ssm = case
    wl.weights["D"] = np.full_like(wl.weights["D"], D_value)
    layer = device_layer(wl)
    w = oracle.as_f64(wl.weights)
    st = oracle.prefill(w, wl.u, wl.cu_seqlens, intermediates=True)["stages"]
    cat = lambda k: np.concatenate([s[k] for s in st])  # noqa: E731
    xh = _round(cat("x_hat"), wl.dtype)
    z = _round(cat("z"), wl.dtype)
    dt = cat("dt").astype(np.float32).astype(np.float64)
    B = cat("B").astype(np.float32).astype(np.float64)
    C = cat("C").astype(np.float32).astype(np.float64)
    cu_d, cu_h = _cu(wl)
    jm.set_scan_chunk_len(chunk)
    try:
        g, fs = jm.jm_stage_scan(layer, to_dev(xh, wl.dtype), to_dev(dt, "f32"),
                                 to_dev(B, "f32"), to_dev(C, "f32"), to_dev(z, wl.dtype), cu_d,
                                 cu_h, init_ssm_state=to_dev(init_ssm, "f32"))
        torch.cuda.synchronize()
    finally:
        jm.set_scan_chunk_len(0)
    A = -np.exp(w["A_log"])
    g_ref = np.empty_like(xh)
    fs_ref = np.empty_like(init_ssm)
    for i, (s, e) in enumerate(_seqs(wl)):
        y, fs_ref[i] = oracle.selective_scan(xh[s:e], dt[s:e], A, B[s:e], C[s:e], w["D"],
                                             init_ssm[i])
        g_ref[s:e] = oracle.gate(y, z[s:e])
    e = dict(g=rel_err(to_np(g), g_ref), state=rel_err(to_np(fs), fs_ref))
    print(f"scan {wl.dtype} D={D_value} chunk={chunk}: {e}", flush=True)
    assert e["g"] < _out_tol(wl.dtype, "scan"), e
    assert e["state"] < F32_SCAN, e


def test_stage_out_proj(case):
    wl, _, _ = case
    layer = device_layer(wl)
    w = oracle.as_f64(wl.weights)
    st = oracle.prefill(w, wl.u, wl.cu_seqlens, intermediates=True)["stages"]
    g_in = _round(np.concatenate([s["g"] for s in st]), wl.dtype)
    out = jm.jm_stage_out_proj(layer, to_dev(g_in, wl.dtype))
    torch.cuda.synchronize()
    e = rel_err(to_np(out), oracle.out_proj(g_in, w["out_proj_w"]))
    print(f"out_proj {wl.dtype}: {e:.2e}", flush=True)
    assert e < _out_tol(wl.dtype, "proj"), e


def test_stages_compose_to_prefill(case):
    """The six stages chained on the device give the prefill's output bit for bit."""
    wl, init_conv, init_ssm = case
    layer = device_layer(wl)
    u = to_dev(wl.u, wl.dtype)
    cu_d, cu_h = _cu(wl)
    ic = to_dev(init_conv, wl.dtype)
    isr = to_dev(init_ssm, "f32")
    out_ref, conv_ref, ssm_ref = jm.jamba_mamba_prefill(layer, u, cu_d, cu_h, ic, isr)
    x, z = jm.jm_stage_in_proj(layer, u)
    xh, fc = jm.jm_stage_conv(layer, x, cu_d, cu_h, init_conv_state=ic)
    d, B, C = jm.jm_stage_x_proj(layer, xh)
    dt = jm.jm_stage_dt_proj(layer, d)
    g, fs = jm.jm_stage_scan(layer, xh, dt, B, C, z, cu_d, cu_h, init_ssm_state=isr)
    out = jm.jm_stage_out_proj(layer, g)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref)
    assert torch.equal(fc, conv_ref)
    assert torch.equal(fs, ssm_ref)


def _decode_update_inputs(wl, w):
    """The decode update's upstream tensors for one step, from the oracle's own steps: states
    from the oracle's prefill of the workload, then in_proj, conv + SiLU (each sequence from its
    carried window) and x_proj of the step's tokens; rounded to the dtypes the kernel reads."""
    di, R, N = wl.dims.d_inner, wl.dims.dt_rank, wl.dims.d_state
    ref = oracle.prefill(w, wl.u, wl.cu_seqlens)
    tok = wl.next_decode_tokens()
    x, z = oracle.in_proj(tok, w["in_proj_w"], di)
    xh = np.empty_like(x)
    for b in range(wl.n_seqs):
        xh[b:b + 1], _ = oracle.causal_conv_silu(x[b:b + 1], w["conv_w"], w["conv_b"],
                                                 ref["conv_state"][b])
    delta, B, C = oracle.x_proj(xh, w["x_proj_w"], R, N)
    f32 = lambda a: a.astype(np.float32).astype(np.float64)  # noqa: E731
    return dict(xh=_round(xh, wl.dtype), z=_round(z, wl.dtype), delta=_round(delta, wl.dtype),
                B=f32(B), C=f32(C), h0=f32(ref["ssm_state"]))


def _decode_update_reference(w, c):
    """dt_proj + softplus, one step of the recurrence from each sequence's state, D skip and
    gate: the oracle's own step functions with T = 1 per sequence."""
    dt = oracle.dt_proj(c["delta"], w["dt_proj_w"], w["dt_proj_b"])
    A = -np.exp(w["A_log"])
    g = np.empty_like(c["xh"])
    h = np.empty_like(c["h0"])
    for b in range(c["xh"].shape[0]):
        y, h[b] = oracle.selective_scan(c["xh"][b:b + 1], dt[b:b + 1], A, c["B"][b:b + 1],
                                        c["C"][b:b + 1], w["D"], c["h0"][b])
        g[b:b + 1] = oracle.gate(y, c["z"][b:b + 1])
    return g, h


@pytest.mark.parametrize("batch,use_slots,D_value", [
    (64, False, 0.0), (64, False, 1.0), (70, True, 0.0), (70, False, 1.0), (5, True, 1.0)])
def test_stage_decode_update(batch, use_slots, D_value):
    """jm_stage_decode_update (the fused decode kernel: dt_proj on MFMA, softplus, in-place state
    update, D skip, gate) at Jamba widths, one and two 64-row tiles, with and without a slot map
    (slots outside the batch must stay bit-for-bit unchanged)."""
    wl = synth.make_workload("decode_b64", batch=batch, prefill_len=6, steps=1, D_value=D_value)
    _check_decode_update(wl, use_slots)


def test_stage_decode_update_generic_fp32():
    """The fp32 layer's decode update (generic kernel), tiny widths."""
    wl = synth.make_workload("decode_b64", dims=synth.TINY_DIMS, dtype="f32", batch=5,
                             prefill_len=7, steps=1, D_value=0.0)
    _check_decode_update(wl, use_slots=True)


def _check_decode_update(wl, use_slots):
    layer = device_layer(wl)
    w = oracle.as_f64(wl.weights)
    c = _decode_update_inputs(wl, w)
    g_ref, h_ref = _decode_update_reference(w, c)
    b, di = c["xh"].shape
    dev = lambda k, dt: to_dev(c[k], dt)  # noqa: E731
    args = (layer, dev("xh", wl.dtype), dev("z", wl.dtype), dev("delta", wl.dtype),
            dev("B", "f32"), dev("C", "f32"))
    if use_slots:
        n_slots = 2 * b + 3
        rng = np.random.default_rng(b)
        slots = [int(v) for v in rng.permutation(n_slots)[:b]]
        cache = torch.as_tensor((rng.standard_normal((n_slots, di, 16)) * 0.01).astype(np.float32)).cuda()
        cache[torch.as_tensor(slots, dtype=torch.long).cuda()] = to_dev(c["h0"], "f32")
        before = cache.clone()
        g = jm.jm_stage_decode_update(*args, cache, slots=slots)
        torch.cuda.synchronize()
        h = to_np(cache[torch.as_tensor(slots, dtype=torch.long).cuda()])
        others = sorted(set(range(n_slots)) - set(slots))
        idx = torch.as_tensor(others, dtype=torch.long).cuda()
        assert torch.equal(cache[idx], before[idx]), "a slot outside the batch changed"
    else:
        state = to_dev(c["h0"], "f32")
        g = jm.jm_stage_decode_update(*args, state)
        torch.cuda.synchronize()
        h = to_np(state)
    e = dict(g=rel_err(to_np(g), g_ref), state=rel_err(h, h_ref))
    print(f"decode update {wl.dtype} batch={b} slots={use_slots}: {e}", flush=True)
    assert e["g"] < _out_tol(wl.dtype, "scan"), e
    assert e["state"] < F32_SCAN, e
