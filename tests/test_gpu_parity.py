"""GPU parity: the HIP library (through its C ABI) against the fp64 CPU oracle.

Tolerances: norm-wise relative error (max|gpu-ref| / max|ref| per tensor) below
1e-4 for the fp32 layer and 2e-2 for bf16 activations with fp32 state. Every
case also runs with D = 0, because with D = 1 the skip term dominates `out` and
would hide the scan. Bitwise checks cover packing, state resets and causality.
"""
import numpy as np
import pytest

import oracle
import synth
from jm_testutil import TOL, device_layer, gpu_prefill, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
jm = pytest.importorskip("mamba_selective_scan_mixer_amd")

JAMBA_SMALL_T = 300


@pytest.fixture(autouse=True)
def _reset_chunk():
    jm.set_scan_chunk_len(0)
    yield
    jm.set_scan_chunk_len(0)


def check_against_oracle(wl, tol, init_conv=None, init_ssm=None, label=""):
    out, conv, ssm = gpu_prefill(wl, init_conv=init_conv, init_ssm=init_ssm)
    ref = oracle.prefill(wl.weights, wl.u, wl.cu_seqlens, init_conv, init_ssm)
    e = (rel_err(out, ref["out"]), rel_err(conv, ref["conv_state"]), rel_err(ssm, ref["ssm_state"]))
    print(f"{label} errors out={e[0]:.2e} conv={e[1]:.2e} ssm={e[2]:.2e}", flush=True)
    assert e[0] < tol and e[1] < tol and e[2] < tol, e
    return out, conv, ssm, ref


@pytest.mark.parametrize("D_value", [1.0, 0.0])
def test_tiny_fp32(D_value):
    wl = synth.make_workload("tiny_fp32", D_value=D_value)
    check_against_oracle(wl, TOL["f32"], label=f"tiny D={D_value}")


@pytest.mark.parametrize("D_value", [1.0, 0.0])
@pytest.mark.parametrize("chunk", [0, 16, 48])
def test_tiny_fp32_packed_with_initial_states(D_value, chunk):
    jm.set_scan_chunk_len(chunk)
    wl = synth.make_workload("tiny_fp32", seed=3, D_value=D_value, lengths=[1, 2, 3, 5, 17, 64, 40, 9])
    rng = np.random.default_rng(99)
    n, di = wl.n_seqs, wl.dims.d_inner
    init_conv = rng.standard_normal((n, di, 3)).astype(np.float32)
    init_ssm = (rng.standard_normal((n, di, 16)) * 1e-2).astype(np.float32)
    check_against_oracle(wl, TOL["f32"], init_conv, init_ssm, label=f"packed chunk={chunk}")
    check_against_oracle(wl, TOL["f32"], label=f"packed zero-init chunk={chunk}")


@pytest.fixture(scope="module")
def jamba_small():
    """Jamba-7B-class layer widths, bf16, a ragged 300-token sequence (tiles of 128)."""
    return {D: synth.make_workload("prefill_4k", lengths=[JAMBA_SMALL_T], D_value=D)
            for D in (1.0, 0.0)}


@pytest.mark.parametrize("D_value", [1.0, 0.0])
def test_jamba_bf16_single_sequence(jamba_small, D_value):
    check_against_oracle(jamba_small[D_value], TOL["bf16"], label=f"jamba300 D={D_value}")


@pytest.mark.parametrize("D_value", [1.0, 0.0])
def test_jamba_bf16_packed(D_value):
    jm.set_scan_chunk_len(32)   # sequence starts land inside chunks
    wl = synth.make_workload("packed_varlen", seed=4, D_value=D_value, n_seqs=5,
                             lengths=[1, 2, 3, 130, 70])
    check_against_oracle(wl, TOL["bf16"], label=f"jamba packed D={D_value}")


def test_chunk_count_invariance(jamba_small):
    wl = jamba_small[0.0]
    layer = device_layer(wl)
    res = {}
    for chunk in (0, 16, 64, 1 << 20):
        jm.set_scan_chunk_len(chunk)
        res[chunk] = gpu_prefill(wl, layer)
    base = res[1 << 20]   # one chunk: no carry across chunks at all
    for chunk, (o, c, s) in res.items():
        # fp32 state: only rounding order differs. out: the same plus the bf16
        # rounding of the gate output, which can flip by one bf16 ulp (2^-8 rel.).
        eo, es = rel_err(o, base[0]), rel_err(s, base[2])
        print(f"chunk={chunk}: out {eo:.2e} ssm {es:.2e}", flush=True)
        assert es < 1e-4 and eo < 1e-2, (chunk, eo, es)
        assert np.array_equal(c, base[1])


def test_zero_input_gives_exact_zero_output(jamba_small):
    wl = jamba_small[1.0]
    out, conv, ssm = gpu_prefill(wl, u=np.zeros_like(wl.u))
    assert np.all(out == 0.0)
    assert np.all(conv == 0.0)
    ref = oracle.prefill(wl.weights, np.zeros_like(wl.u), wl.cu_seqlens)
    assert rel_err(ssm, ref["ssm_state"]) < TOL["bf16"]


def test_deterministic(jamba_small):
    wl = jamba_small[0.0]
    layer = device_layer(wl)
    a = gpu_prefill(wl, layer)
    b = gpu_prefill(wl, layer)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_concurrent_calls_on_two_streams(jamba_small):
    """Two host threads call the prefill at the same time, each on its own stream with its own
    workspace and input (the boundary allows concurrent calls that share nothing writable);
    each result equals the same call made alone, bit for bit."""
    import threading
    wl = jamba_small[0.0]
    layer = device_layer(wl)
    rng = np.random.default_rng(21)
    us = [wl.u, synth.round_bf16(rng.standard_normal(wl.u.shape))]
    alone = [gpu_prefill(wl, layer, u=u) for u in us]
    cu_d = torch.as_tensor(wl.cu_seqlens, dtype=torch.int32).cuda()
    u_d = [to_dev(u, wl.dtype) for u in us]
    streams = [torch.cuda.Stream() for _ in us]
    torch.cuda.synchronize()
    res, errs = [None] * len(us), []

    def run(i):
        try:
            with torch.cuda.stream(streams[i]):
                res[i] = jm.jamba_mamba_prefill(layer, u_d[i], cu_d, wl.cu_seqlens,
                                                stream=streams[i])
        except Exception as e:   # reported below, from the main thread
            errs.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(us))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errs, errs
    for i in range(len(us)):
        for x, y in zip(alone[i], res[i]):
            assert np.array_equal(x, to_np(y)), i


def test_sequences_are_isolated_bitwise():
    jm.set_scan_chunk_len(32)
    wl = synth.make_workload("packed_varlen", seed=5, D_value=0.0, n_seqs=4, lengths=[50, 3, 77, 40])
    layer = device_layer(wl)
    base = gpu_prefill(wl, layer)
    cu = wl.cu_seqlens
    rng = np.random.default_rng(7)
    for j in range(4):
        u2 = wl.u.copy()
        for i in range(4):
            if i != j:
                u2[cu[i]:cu[i + 1]] = synth.round_bf16(rng.standard_normal((cu[i + 1] - cu[i], u2.shape[1])))
        got = gpu_prefill(wl, layer, u=u2)
        assert np.array_equal(got[0][cu[j]:cu[j + 1]], base[0][cu[j]:cu[j + 1]]), j
        assert np.array_equal(got[1][j], base[1][j]) and np.array_equal(got[2][j], base[2][j]), j


def test_causal_bitwise():
    jm.set_scan_chunk_len(32)
    wl = synth.make_workload("prefill_4k", seed=6, lengths=[200], D_value=0.0)
    layer = device_layer(wl)
    base = gpu_prefill(wl, layer)
    for t in (0, 31, 32, 150):
        u2 = wl.u.copy()
        u2[t + 1:] = synth.round_bf16(-u2[t + 1:] * 3.0 + 0.5)
        got = gpu_prefill(wl, layer, u=u2)
        assert np.array_equal(got[0][:t + 1], base[0][:t + 1]), t


def _decode_case(wl, steps, tol, state_tol=None):
    """Prefill (oracle and GPU each from their own prefill), then decode steps."""
    state_tol = tol if state_tol is None else state_tol
    w64 = oracle.as_f64(wl.weights)
    ref = oracle.prefill(w64, wl.u, wl.cu_seqlens)
    layer = device_layer(wl)
    _, conv_g, ssm_g = gpu_prefill(wl, layer)
    conv_d = to_dev(conv_g, wl.dtype)
    ssm_d = torch.as_tensor(ssm_g.astype(np.float32)).cuda()
    conv_r, ssm_r = ref["conv_state"], ref["ssm_state"]
    worst = 0.0
    for s in range(steps):
        tok = wl.next_decode_tokens()
        out_r, conv_r, ssm_r = oracle.decode_step(w64, tok, conv_r, ssm_r)
        out_g = jm.jamba_mamba_decode_step(layer, to_dev(tok, wl.dtype), conv_d, ssm_d)
        torch.cuda.synchronize()
        e = (rel_err(to_np(out_g), out_r), rel_err(to_np(conv_d), conv_r), rel_err(to_np(ssm_d), ssm_r))
        worst = max(worst, *e)
        assert e[0] < tol and e[1] < state_tol and e[2] < state_tol, (s, e)
    print(f"decode worst error {worst:.2e}", flush=True)


@pytest.mark.parametrize("D_value", [1.0, 0.0])
def test_decode_tiny_fp32(D_value):
    wl = synth.make_workload("decode_b64", dims=synth.TINY_DIMS, dtype="f32", batch=5,
                             prefill_len=7, steps=12, D_value=D_value)
    _decode_case(wl, 12, TOL["f32"])


@pytest.mark.parametrize("D_value", [1.0, 0.0])
def test_decode_jamba_bf16(D_value):
    wl = synth.make_workload("decode_b64", batch=3, prefill_len=20, steps=6, D_value=D_value)
    _decode_case(wl, 6, TOL["bf16"])


def test_decode_tiny_bf16_generic_path():
    """bf16 at widths the fast decode kernels do not take (generic kernels).

    Not one of the Jamba-width workloads the 2e-2 bound is stated for: at 128
    channels with D = 0 the output is a short, cancelling sum C.h, and a numpy
    model that only rounds x, z, x^, delta, g and out to bf16 (everything else
    fp64) already reaches 2.4e-2 at step 2 of this very input. So `out` is held to
    5e-2 here and the carried states to the usual 2e-2."""
    wl = synth.make_workload("decode_b64", dims=synth.TINY_DIMS, dtype="bf16", batch=4,
                             prefill_len=9, steps=5, D_value=0.0)
    _decode_case(wl, 5, 5e-2, state_tol=TOL["bf16"])


def test_decode_jamba_bf16_two_batch_tiles():
    """Batch 70 > 64: the fast path runs two row tiles per step."""
    wl = synth.make_workload("decode_b64", batch=70, prefill_len=3, steps=2, D_value=0.0)
    _decode_case(wl, 2, TOL["bf16"])


def test_decode_rows_are_independent_bitwise():
    """Batch 129 = three 64-row tiles (the last holds one row): every row of a decode step is
    computed exactly as when it is decoded alone (the projections and the update add in a fixed
    order per element, whatever the row's place in its tile), so rows on each side of the tile
    borders match single-row decodes bit for bit: outputs and both states. This also runs the
    out_proj split-K sum once per tile with counters reused across the tiles of a step."""
    wl = synth.make_workload("decode_b64", batch=129, prefill_len=2, steps=1, D_value=1.0)
    layer = device_layer(wl)
    d = wl.dims
    rng = np.random.default_rng(21)
    conv0 = to_dev(synth.round_bf16(rng.standard_normal((129, d.d_inner, 3)) * 0.5), "bf16")
    ssm0 = torch.as_tensor((rng.standard_normal((129, d.d_inner, 16)) * 0.1).astype(np.float32)).cuda()
    tok = to_dev(synth.round_bf16(rng.standard_normal((129, d.d_model))), "bf16")
    conv, ssm = conv0.clone(), ssm0.clone()
    out = jm.jamba_mamba_decode_step(layer, tok, conv, ssm)
    torch.cuda.synchronize()
    for r in (0, 63, 64, 100, 127, 128):
        c1, s1 = conv0[r:r + 1].clone(), ssm0[r:r + 1].clone()
        o1 = jm.jamba_mamba_decode_step(layer, tok[r:r + 1].contiguous(), c1, s1)
        torch.cuda.synchronize()
        assert torch.equal(o1[0], out[r]), r
        assert torch.equal(c1[0], conv[r]) and torch.equal(s1[0], ssm[r]), r


def test_prefill_state_equals_repeated_decode_fp32():
    wl = synth.make_workload("tiny_fp32", seed=8, lengths=[23], D_value=0.0)
    layer = device_layer(wl)
    out_p, conv_p, ssm_p = gpu_prefill(wl, layer)
    di = wl.dims.d_inner
    conv = torch.zeros((1, di, 3), dtype=torch.float32, device="cuda")
    ssm = torch.zeros((1, di, 16), dtype=torch.float32, device="cuda")
    for t in range(23):
        o = jm.jamba_mamba_decode_step(layer, to_dev(wl.u[t:t + 1], "f32"), conv, ssm)
        assert rel_err(to_np(o)[0], out_p[t]) < 1e-5
    torch.cuda.synchronize()
    assert np.array_equal(to_np(conv), conv_p)
    assert rel_err(to_np(ssm), ssm_p) < 1e-5


@pytest.mark.parametrize("widths,batch,D_value", [
    ((512, 1024, 128), 5, 0.0),     # out_proj: one 64-wide K block per wave
    ((512, 1024, 128), 70, 1.0),
    ((768, 3072, 128), 5, 1.0),     # in_proj and out_proj: three K blocks per wave
    ((768, 3072, 128), 70, 0.0),    # and two 64-row tiles
])
def test_decode_bf16_odd_k_blocks(widths, batch, D_value):
    """Widths at which a wave of the fast decode GEMM owns an odd number of 64-wide K blocks
    (d_model / 256 or d_inner / 1024 odd): every block must enter the sum exactly once."""
    dm, di, R = widths
    dims = synth.LayerDims(d_model=dm, d_inner=di, d_state=16, d_conv=4, dt_rank=R)
    wl = synth.make_workload("decode_b64", dims=dims, batch=batch, prefill_len=5, steps=3,
                             D_value=D_value)
    _decode_case(wl, 3, TOL["bf16"])


def test_stream_argument_without_context_manager(jamba_small):
    """stream= given while another stream is current: the result equals the same call on the
    current stream, bit for bit (outputs and workspace belong to the call's stream)."""
    wl = jamba_small[0.0]
    layer = device_layer(wl)
    base = gpu_prefill(wl, layer)
    side = torch.cuda.Stream()
    u = to_dev(wl.u, wl.dtype)
    cu_d = torch.as_tensor(wl.cu_seqlens, dtype=torch.int32).cuda()
    torch.cuda.synchronize()
    res = []
    for _ in range(3):   # later calls reuse memory the allocator gave earlier ones
        res.append(jm.jamba_mamba_prefill(layer, u, cu_d, wl.cu_seqlens, stream=side))
        junk = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
        junk.fill_(0xAB)          # current-stream work that would clobber a shared workspace
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for out, conv, ssm in res:
        assert np.array_equal(to_np(out), base[0])
        assert np.array_equal(to_np(conv), base[1]) and np.array_equal(to_np(ssm), base[2])
