"""Property test on the GPU (hypothesis, derandomized): random fp32 layer widths, packed
sequence lengths, initial states or zeros, D = 0 or 1 and forced scan chunk lengths, the
library's prefill against the fp64 oracle (bound 1e-4, the fp32 layer bound)."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import synth
from jm_testutil import TOL, gpu_prefill, rel_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
jm = pytest.importorskip("mamba_selective_scan_mixer_amd")


@settings(max_examples=12, deadline=None, derandomize=True)
@given(st.sampled_from([64, 128, 192]), st.sampled_from([64, 128, 192, 320]),
       st.sampled_from([8, 16, 24]), st.lists(st.integers(1, 70), min_size=1, max_size=5),
       st.integers(0, 2**31 - 1), st.sampled_from([0.0, 1.0]), st.booleans(),
       st.sampled_from([0, 16, 32, 48]))
def test_prefill_random_layers_against_oracle(dm, di, R, lengths, seed, D_value, states, chunk):
    dims = synth.LayerDims(d_model=dm, d_inner=di, d_state=16, d_conv=4, dt_rank=R)
    wl = synth.make_workload("tiny_fp32", seed=seed % 1000, lengths=lengths, dims=dims,
                             D_value=D_value)
    rng = np.random.default_rng(seed)
    n = len(lengths)
    ic = rng.standard_normal((n, di, 3)).astype(np.float32) if states else None
    isr = (rng.standard_normal((n, di, 16)) * 0.1).astype(np.float32) if states else None
    jm.set_scan_chunk_len(chunk)
    try:
        out, conv, ssm = gpu_prefill(wl, init_conv=ic, init_ssm=isr)
    finally:
        jm.set_scan_chunk_len(0)
    ref = oracle.prefill(wl.weights, wl.u, wl.cu_seqlens, ic, isr)
    e = (rel_err(out, ref["out"]), rel_err(conv, ref["conv_state"]), rel_err(ssm, ref["ssm_state"]))
    print(f"widths {dm}/{di}/{R} lengths {lengths} D={D_value} states={states} chunk={chunk}: "
          f"out {e[0]:.1e} conv {e[1]:.1e} ssm {e[2]:.1e}", flush=True)
    assert max(e) < TOL["f32"], e
