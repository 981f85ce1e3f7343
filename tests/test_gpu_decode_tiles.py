"""Decode from the tiled copies of in_proj_w / out_proj_w (jm_tile_decode_weights): the tile
layout against an independent re-layout of the matrices, decode steps bit for bit equal to those
from the row-major matrices (plain, slot-indexed and no-workspace entry points, one and two
64-row tiles, the odd K-block widths), the prefill unaffected, and one run against the oracle.
"""
import numpy as np
import pytest

import oracle
import synth
from jm_testutil import TOL, device_layer, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
jm = pytest.importorskip("mamba_selective_scan_mixer_amd")

WIDTHS = {"jamba": (4096, 8192, 256), "small": (512, 1024, 128), "odd": (768, 3072, 128)}


def layer_for(widths, seed=0):
    dm, di, R = widths
    dims = synth.LayerDims(d_model=dm, d_inner=di, d_state=16, d_conv=4, dt_rank=R)
    wl = synth.make_workload("decode_b64", seed=seed, dims=dims, batch=2, prefill_len=2, steps=1)
    return wl, device_layer(wl)


def blocked(W):
    """Independent re-layout: 64 x 64 tiles, tile (b, s) = rows 64b.., columns 64s.., tiles in
    order of b then s, each tile row-major."""
    N, K = W.shape
    return W.view(N // 64, 64, K // 64, 64).permute(0, 2, 1, 3).contiguous().view(-1)


@pytest.mark.parametrize("name", ["jamba", "odd"])
def test_tile_layout(name):
    _, layer = layer_for(WIDTHS[name])
    layer.tile_for_decode()
    torch.cuda.synchronize()
    ti, to = layer.tiles
    assert torch.equal(ti.view(-1), blocked(layer.tensors["in_proj_w"]))
    assert torch.equal(to.view(-1), blocked(layer.tensors["out_proj_w"]))


def random_states(d, batch, rng, rows=None):
    rows = batch if rows is None else rows
    conv = to_dev(synth.round_bf16(rng.standard_normal((rows, d.d_inner, 3)) * 0.5), "bf16")
    ssm = torch.as_tensor((rng.standard_normal((rows, d.d_inner, 16)) * 0.1).astype(np.float32)).cuda()
    return conv, ssm


@pytest.mark.parametrize("name,batch", [("jamba", 64), ("jamba", 70), ("small", 5),
                                        ("odd", 70)])
def test_tiled_decode_equals_row_major_bitwise(name, batch):
    wl, plain = layer_for(WIDTHS[name], seed=batch)
    _, tiled = layer_for(WIDTHS[name], seed=batch)
    tiled.tile_for_decode()
    d = wl.dims
    rng = np.random.default_rng(batch)
    conv0, ssm0 = random_states(d, batch, rng)
    c1, s1, c2, s2 = conv0.clone(), ssm0.clone(), conv0.clone(), ssm0.clone()
    for step in range(3):
        tok = to_dev(synth.round_bf16(rng.standard_normal((batch, d.d_model))), "bf16")
        o1 = jm.jamba_mamba_decode_step(plain, tok, c1, s1)
        o2 = jm.jamba_mamba_decode_step(tiled, tok, c2, s2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), step
        assert torch.equal(c1, c2) and torch.equal(s1, s2), step
    # the no-workspace entry point reads the tiles too
    o3 = jm.jamba_mamba_decode_step_noalloc(tiled, tok, c2, s2, torch.empty_like(o2))
    o4 = jm.jamba_mamba_decode_step(plain, tok, c1, s1)
    torch.cuda.synchronize()
    assert torch.equal(o3, o4) and torch.equal(c1, c2) and torch.equal(s1, s2)


def test_tiled_slot_decode_equals_row_major_bitwise():
    wl, plain = layer_for(WIDTHS["jamba"], seed=3)
    _, tiled = layer_for(WIDTHS["jamba"], seed=3)
    tiled.tile_for_decode()
    d = wl.dims
    rng = np.random.default_rng(5)
    n_slots, batch = 96, 70
    slots = [int(v) for v in rng.permutation(n_slots)[:batch]]
    caches = [jm.StateCache(plain.dims, n_slots, device="cuda") for _ in range(2)]
    conv0, ssm0 = random_states(d, batch, rng, rows=n_slots)
    for c in caches:
        c.conv.copy_(conv0)
        c.ssm.copy_(ssm0)
    tok = to_dev(synth.round_bf16(rng.standard_normal((batch, d.d_model))), "bf16")
    o1 = jm.jamba_mamba_decode_step_slots(plain, tok, caches[0], slots)
    o2 = jm.jamba_mamba_decode_step_slots(tiled, tok, caches[1], slots)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(caches[0].conv, caches[1].conv) and torch.equal(caches[0].ssm, caches[1].ssm)


def test_prefill_ignores_tiles():
    wl = synth.make_workload("prefill_4k", seed=2, lengths=[70, 1, 33])
    plain = device_layer(wl)
    tiled = device_layer(wl).tile_for_decode()
    u = to_dev(wl.u, wl.dtype)
    cu = torch.as_tensor(wl.cu_seqlens, dtype=torch.int32).cuda()
    r1 = jm.jamba_mamba_prefill(plain, u, cu, wl.cu_seqlens)
    r2 = jm.jamba_mamba_prefill(tiled, u, cu, wl.cu_seqlens)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


def test_tiled_decode_against_oracle():
    """Prefill (oracle and GPU each their own), then decode steps from the tiled weights."""
    wl = synth.make_workload("decode_b64", batch=3, prefill_len=20, steps=4, D_value=0.0)
    w64 = oracle.as_f64(wl.weights)
    ref = oracle.prefill(w64, wl.u, wl.cu_seqlens)
    layer = device_layer(wl).tile_for_decode()
    cu = torch.as_tensor(wl.cu_seqlens, dtype=torch.int32).cuda()
    _, conv, ssm = jm.jamba_mamba_prefill(layer, to_dev(wl.u, "bf16"), cu, wl.cu_seqlens)
    conv_r, ssm_r = ref["conv_state"], ref["ssm_state"]
    for s in range(4):
        tok = wl.next_decode_tokens()
        out_r, conv_r, ssm_r = oracle.decode_step(w64, tok, conv_r, ssm_r)
        out = jm.jamba_mamba_decode_step(layer, to_dev(tok, "bf16"), conv, ssm)
        torch.cuda.synchronize()
        e = (rel_err(to_np(out), out_r), rel_err(to_np(conv), conv_r), rel_err(to_np(ssm), ssm_r))
        assert max(e) < TOL["bf16"], (s, e)
