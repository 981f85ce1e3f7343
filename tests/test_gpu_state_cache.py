"""State cache (serving): prefill and decode against a cache of slots.

  * a prompt prefilled in three chunks, each continuing from the slot the previous one
    left, equals the one-shot prefill and the oracle;
  * a serving script with two prompts, then a mixed call (a new prompt plus one decode
    token for each running sequence, all in one packed prefill), decode steps over a
    permuted subset of slots and a fork (continue a sequence into a new slot): every
    output and every slot against the oracle run per sequence;
  * slot-indexed decode equals the plain decode on the same states gathered into a
    contiguous batch, bit for bit, for the fast bf16 path (two 64-row tiles) and the
    generic path; slots outside the batch are left untouched, bit for bit.
Bounds are the layer's (1e-4 fp32, 2e-2 bf16).
"""
import numpy as np
import pytest

import oracle
import synth
from jm_testutil import TOL, device_layer, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
jm = pytest.importorskip("mamba_selective_scan_mixer_amd")

CASES = ["tiny_fp32", "prefill_4k"]   # fp32 generic paths / bf16 Jamba widths (fast decode)


@pytest.fixture(autouse=True)
def _reset_chunk():
    jm.set_scan_chunk_len(0)
    yield
    jm.set_scan_chunk_len(0)


def _cu(lengths):
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    return torch.as_tensor(cu).cuda(), [int(v) for v in cu]


def _tokens(wl, rng, n):
    u = rng.standard_normal((n, wl.dims.d_model)).astype(np.float32)
    return synth.round_bf16(u) if wl.dtype == "bf16" else u


class RefSeq:
    """One sequence's oracle state (fp64)."""

    def __init__(self, di):
        self.conv = np.zeros((di, 3))
        self.ssm = np.zeros((di, 16))

    def prefill(self, w64, u):
        r = oracle.prefill(w64, u, [0, len(u)], init_conv=self.conv[None], init_ssm=self.ssm[None])
        self.conv, self.ssm = r["conv_state"][0], r["ssm_state"][0]
        return r["out"]

    def decode(self, w64, tok):
        o, c, s = oracle.decode_step(w64, tok[None], self.conv[None], self.ssm[None])
        self.conv, self.ssm = c[0], s[0]
        return o[0]


@pytest.mark.parametrize("name", CASES)
def test_chunked_prefill_continues_through_a_slot(name):
    wl = synth.make_workload(name, lengths=[150])
    tol = TOL[wl.dtype]
    layer = device_layer(wl)
    cache = jm.StateCache(layer.dims, 4)
    outs = []
    for a, b in ((0, 61), (61, 62), (62, 150)):      # includes a one-token chunk
        cu_d, cu_h = _cu([b - a])
        outs.append(jm.jamba_mamba_prefill_slots(layer, to_dev(wl.u[a:b], wl.dtype), cu_d, cu_h,
                                                 cache, init_slots=[-1 if a == 0 else 2],
                                                 final_slots=[2]))
    torch.cuda.synchronize()
    out = np.concatenate([to_np(o) for o in outs])
    ref = oracle.prefill(wl.weights, wl.u, wl.cu_seqlens)
    e = dict(out=rel_err(out, ref["out"]), conv=rel_err(to_np(cache.conv[2]), ref["conv_state"][0]),
             ssm=rel_err(to_np(cache.ssm[2]), ref["ssm_state"][0]))
    print(f"chunked prefill {wl.dtype}: {e}", flush=True)
    assert max(e.values()) < tol, e
    # the other slots were never written
    for s in (0, 1, 3):
        assert not torch.any(cache.conv[s]) and not torch.any(cache.ssm[s])
    # and the one-shot prefill agrees with the chunked one
    one, conv1, ssm1 = jm.jamba_mamba_prefill(layer, to_dev(wl.u, wl.dtype),
                                              *_cu([150]))
    torch.cuda.synchronize()
    assert rel_err(to_np(cache.ssm[2]), to_np(ssm1)[0]) < tol


@pytest.mark.parametrize("name", CASES)
def test_serving_script_mixed_batches(name):
    wl = synth.make_workload(name, lengths=[8])
    tol = TOL[wl.dtype]
    w64 = oracle.as_f64(wl.weights)
    di = wl.dims.d_inner
    layer = device_layer(wl)
    cache = jm.StateCache(layer.dims, 6)
    rng = np.random.default_rng(21)
    ref = {k: RefSeq(di) for k in "ABCD"}
    slot = {"A": 4, "B": 1, "C": 0}

    def check(label, got, want):
        e = rel_err(to_np(got), want)
        assert e < tol, (label, e)

    # 1: two prompts
    uA, uB = _tokens(wl, rng, 37), _tokens(wl, rng, 20)
    cu_d, cu_h = _cu([37, 20])
    o = jm.jamba_mamba_prefill_slots(layer, to_dev(np.concatenate([uA, uB]), wl.dtype), cu_d, cu_h,
                                     cache, init_slots=[-1, -1], final_slots=[slot["A"], slot["B"]])
    check("prefill A", o[:37], ref["A"].prefill(w64, uA))
    check("prefill B", o[37:], ref["B"].prefill(w64, uB))
    # 2: mixed: a new prompt C, one decode token each for A and B, one packed call
    uC, tA, tB = _tokens(wl, rng, 25), _tokens(wl, rng, 1), _tokens(wl, rng, 1)
    cu_d, cu_h = _cu([25, 1, 1])
    o = jm.jamba_mamba_prefill_slots(layer, to_dev(np.concatenate([uC, tA, tB]), wl.dtype), cu_d,
                                     cu_h, cache, init_slots=[-1, slot["A"], slot["B"]],
                                     final_slots=[slot["C"], slot["A"], slot["B"]])
    check("prefill C", o[:25], ref["C"].prefill(w64, uC))
    check("mixed decode A", o[25:26], ref["A"].decode(w64, tA[0])[None])
    check("mixed decode B", o[26:27], ref["B"].decode(w64, tB[0])[None])
    # 3: decode steps over a permuted subset of slots
    for order in (["C", "A", "B"], ["B"], ["A", "C"]):
        toks = _tokens(wl, rng, len(order))
        o = jm.jamba_mamba_decode_step_slots(layer, to_dev(toks, wl.dtype), cache,
                                             [slot[k] for k in order])
        for i, k in enumerate(order):
            check(f"decode {k}", o[i], ref[k].decode(w64, toks[i]))
    # 4: fork A into slot 5 (slot 4 keeps A's state)
    uD = _tokens(wl, rng, 5)
    ref["D"].conv, ref["D"].ssm = ref["A"].conv.copy(), ref["A"].ssm.copy()
    cu_d, cu_h = _cu([5])
    o = jm.jamba_mamba_prefill_slots(layer, to_dev(uD, wl.dtype), cu_d, cu_h, cache,
                                     init_slots=[slot["A"]], final_slots=[5])
    check("fork D", o, ref["D"].prefill(w64, uD))
    torch.cuda.synchronize()
    slot["D"] = 5
    for k, s in slot.items():
        e = (rel_err(to_np(cache.conv[s]), ref[k].conv), rel_err(to_np(cache.ssm[s]), ref[k].ssm))
        assert max(e) < tol, (k, e)
    assert not torch.any(cache.conv[2]) and not torch.any(cache.ssm[3])


@pytest.mark.parametrize("name,batch", [("tiny_fp32", 5), ("prefill_4k", 70)])
def test_decode_slots_equal_contiguous_decode_bitwise(name, batch):
    wl = synth.make_workload(name, lengths=[4])
    layer = device_layer(wl)
    d = layer.dims
    n_slots = batch + 13
    rng = np.random.default_rng(5)
    cache = jm.StateCache(d, n_slots)
    cache.conv.copy_(to_dev(rng.standard_normal((n_slots, d.d_inner, 3)), wl.dtype))
    cache.ssm.copy_(torch.as_tensor(rng.standard_normal((n_slots, d.d_inner, 16)) * 0.05,
                                    dtype=torch.float32))
    slots = [int(v) for v in rng.permutation(n_slots)[:batch]]
    idx = torch.tensor(slots, dtype=torch.long, device="cuda")
    conv_c = cache.conv[idx].contiguous()
    ssm_c = cache.ssm[idx].contiguous()
    before_conv, before_ssm = cache.conv.clone(), cache.ssm.clone()
    for step in range(2):
        u = to_dev(_tokens(wl, rng, batch), wl.dtype)
        o_c = jm.jamba_mamba_decode_step(layer, u, conv_c, ssm_c)
        o_s = jm.jamba_mamba_decode_step_slots(layer, u, cache, slots)
        torch.cuda.synchronize()
        assert torch.equal(o_c, o_s), step
    assert torch.equal(cache.conv[idx], conv_c) and torch.equal(cache.ssm[idx], ssm_c)
    rest = torch.tensor(sorted(set(range(n_slots)) - set(slots)), dtype=torch.long, device="cuda")
    assert torch.equal(cache.conv[rest], before_conv[rest])
    assert torch.equal(cache.ssm[rest], before_ssm[rest])
