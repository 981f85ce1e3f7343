"""The seeded input generator: determinism, draw order and the initialisation recipe."""
import numpy as np

import synth


def test_deterministic_and_seeded():
    a = synth.make_workload("tiny_fp32", seed=0)
    b = synth.make_workload("tiny_fp32", seed=0)
    c = synth.make_workload("tiny_fp32", seed=1)
    for k in a.weights:
        assert np.array_equal(a.weights[k], b.weights[k])
    assert np.array_equal(a.u, b.u)
    assert not np.array_equal(a.u, c.u)


def test_init_recipe():
    wl = synth.make_workload("tiny_fp32")
    w = wl.weights
    assert np.array_equal(w["A_log"][5], np.log(np.arange(1, 17)).astype(np.float32))
    assert np.all(w["D"] == 1.0)
    assert 1e-3 <= w["dt0"].min() and w["dt0"].max() <= 1e-1
    assert abs(np.std(w["in_proj_w"]) - 0.02) < 0.002
    assert wl.u.shape == (64, 64)
    assert synth.make_workload("tiny_fp32", D_value=0.0).weights["D"].max() == 0.0


def test_bf16_rounding_and_bits():
    v = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3], dtype=np.float32)
    r = synth.round_bf16(v)
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == 1.015625 and r[3] == -2.5
    assert np.all(r.view(np.uint32) & 0xFFFF == 0)
    bits = synth.bf16_bits(r)
    assert bits.dtype == np.uint16 and bits[0] == 0x3F80
    wl = synth.make_workload("packed_varlen", dims=synth.TINY_DIMS, n_seqs=3)
    assert np.all(wl.u.view(np.uint32) & 0xFFFF == 0)
    assert np.all(wl.weights["in_proj_w"].view(np.uint32) & 0xFFFF == 0)


def test_packed_lengths_and_decode_stream():
    wl = synth.make_workload("packed_varlen", dims=synth.TINY_DIMS)
    assert len(wl.lengths) == 16 and all(1024 <= n <= 8192 for n in wl.lengths)
    assert wl.cu_seqlens[0] == 0 and wl.cu_seqlens[-1] == sum(wl.lengths)
    d1 = synth.make_workload("decode_b64", dims=synth.TINY_DIMS, batch=4, prefill_len=8, steps=3)
    d2 = synth.make_workload("decode_b64", dims=synth.TINY_DIMS, batch=4, prefill_len=8, steps=3)
    s1 = [d1.next_decode_tokens() for _ in range(3)]
    s2 = [d2.next_decode_tokens() for _ in range(3)]
    assert all(np.array_equal(p, q) for p, q in zip(s1, s2))
    assert s1[0].shape == (4, 64) and not np.array_equal(s1[0], s1[1])
