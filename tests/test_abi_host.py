"""Host-side checks of the C-ABI library: it loads, exports what the header declares,
validates arguments before touching the GPU, and plans packed sequences exactly.
No test here launches a kernel (this suite runs without a GPU)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import mamba_selective_scan_mixer_amd as jm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
           if f.endswith(".h")]


def declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                             text, flags=re.M):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(jm.LIB_PATH):
        from mamba_selective_scan_mixer_amd import build
        build.build()
    return jm.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"jamba_mamba_prefill", "jamba_mamba_decode_step", "jm_prefill_workspace_size"} <= names
    out = subprocess.run(["nm", "-D", "--defined-only", jm.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = names - exported
    assert not missing, f"declared but not exported: {missing}"
    for n in names:
        assert hasattr(L, n)


def test_status_strings(L):
    for i, n in enumerate(jm._STATUS):
        assert L.jm_status_string(i).decode() == n
    assert L.jm_status_string(99).decode() == "JM_ERR_UNKNOWN"


JAMBA = dict(d_model=4096, d_inner=8192, d_state=16, d_conv=4, dt_rank=256)


def dims(**kw):
    p = dict(JAMBA)
    p.update(kw)
    return jm.LayerDims(p["d_model"], p["d_inner"], p["d_state"], p["d_conv"], p["dt_rank"],
                        p.get("act", jm.JM_BF16), p.get("wt", jm.JM_BF16))


@pytest.mark.parametrize("kw,status", [
    (dict(d_state=8), jm.JMError), (dict(d_conv=3), jm.JMError), (dict(d_model=100), jm.JMError),
    (dict(dt_rank=12), jm.JMError), (dict(act=jm.JM_F32), jm.JMError), (dict(act=7), jm.JMError),
])
def test_dims_rejected(kw, status):
    with pytest.raises(status) as ei:
        jm.prefill_workspace_size(dims(**kw), 1, 10)
    assert ei.value.status_name in ("JM_ERR_UNSUPPORTED", "JM_ERR_INVALID_ARG")


def test_workspace_sizes():
    d = dims()
    T = 4096
    ws = jm.prefill_workspace_size(d, 1, T)
    # x, z, x^ (bf16) + delta (bf16) + B, C (fp32) + Delta (fp32) at least
    assert ws >= T * (3 * 8192 * 2 + 256 * 2 + 2 * 16 * 4 + 8192 * 4)
    assert jm.prefill_workspace_size(d, 0, 0) == 0
    assert jm.decode_workspace_size(d, 64) >= 64 * 8192 * 2 * 4
    assert jm.decode_workspace_size(d, 0) == 0
    big = jm.prefill_workspace_size(d, 1, 131072)
    assert big > 8 * 2**30   # > 4 GiB tensors at 128K tokens are carved correctly (64-bit sizes)
    with pytest.raises(jm.JMError):
        jm.prefill_workspace_size(d, 1, 2**31)


class _Fake:
    """Distinct, 16-byte aligned fake device addresses; never dereferenced (validation fails first)."""
    def __init__(self):
        self.next = 0x10000000

    def __call__(self):
        self.next += 0x100000
        return self.next


def _weights(fake, **override):
    w = jm.LayerWeights(*[fake() for _ in jm.MambaLayer.WEIGHT_KEYS])
    for k, v in override.items():
        setattr(w, k, v)
    return w


def _prefill(L, d, w, cu, T=None, u=1, out=1, ws_bytes=None, ws=1, fake=None, **kw):
    fake = fake or _Fake()
    host = (ctypes.c_int32 * len(cu))(*cu)
    n = len(cu) - 1
    T = cu[-1] if T is None else T
    args = dict(u=fake() if u else None, cu=fake(), init_conv=None, init_ssm=None,
                out=fake() if out else None, fconv=None, fssm=None, ws=fake() if ws else None)
    args.update(kw)
    if ws_bytes is None:
        ws_bytes = jm.prefill_workspace_size(d, n, T) if T > 0 else 0
    return L.jamba_mamba_prefill(ctypes.byref(d), ctypes.byref(w), args["u"], args["cu"], host, n,
                                 T, args["init_conv"], args["init_ssm"], args["out"],
                                 args["fconv"], args["fssm"], args["ws"], ws_bytes, None)


def test_prefill_validation_paths(L):
    f = _Fake()
    d = dims()
    w = _weights(f)
    S = {n: i for i, n in enumerate(jm._STATUS)}
    assert _prefill(L, d, w, [0, 5, 4], fake=f) == S["JM_ERR_SHAPE"]          # decreasing
    assert _prefill(L, d, w, [0, 5, 5], fake=f) == S["JM_ERR_SHAPE"]          # empty sequence
    assert _prefill(L, d, w, [1, 5], T=4, fake=f) == S["JM_ERR_SHAPE"]        # cu[0] != 0
    assert _prefill(L, d, w, [0, 5], T=6, fake=f) == S["JM_ERR_SHAPE"]        # total mismatch
    assert _prefill(L, d, w, [0, 5], u=0, fake=f) == S["JM_ERR_INVALID_ARG"]  # null input
    assert _prefill(L, d, w, [0, 5], ws=0, fake=f) == S["JM_ERR_WORKSPACE"]
    assert _prefill(L, d, w, [0, 5], ws_bytes=100, fake=f) == S["JM_ERR_WORKSPACE"]
    assert _prefill(L, d, w, [0, 5], fake=f, init_ssm=0x20000000, fssm=0x20000040) == S["JM_ERR_INVALID_ARG"]
    assert _prefill(L, d, w, [0, 5], fake=f, out=None) == S["JM_ERR_INVALID_ARG"]
    wb = _weights(f, A_log=None)
    assert _prefill(L, d, wb, [0, 5], fake=f) == S["JM_ERR_INVALID_ARG"]
    assert "A_log" in L.jm_last_error().decode()
    wa = _weights(f, D=0x30000004)
    assert _prefill(L, d, wa, [0, 5], fake=f) == S["JM_ERR_ALIGNMENT"]
    assert _prefill(L, d, w, [0, 5], fake=f, u=1, init_conv=0x40000008) == S["JM_ERR_ALIGNMENT"]
    # empty input: no sequences, no tokens -> nothing to do
    assert _prefill(L, d, w, [0], fake=f, u=0, out=0, ws=0) == S["JM_OK"]
    # inner norm: all three gains or none; eps finite and > 0; gains aligned
    wn = _weights(f, dt_norm_w=f(), B_norm_w=f(), C_norm_w=None, norm_eps=1e-6)
    assert _prefill(L, d, wn, [0, 5], fake=f) == S["JM_ERR_INVALID_ARG"]
    assert "all" in L.jm_last_error().decode()
    for eps in (0.0, -1.0, float("inf"), float("nan")):
        we = _weights(f, dt_norm_w=f(), B_norm_w=f(), C_norm_w=f(), norm_eps=eps)
        assert _prefill(L, d, we, [0, 5], fake=f) == S["JM_ERR_INVALID_ARG"], eps
    wa = _weights(f, dt_norm_w=f(), B_norm_w=f() + 4, C_norm_w=f(), norm_eps=1e-6)
    assert _prefill(L, d, wa, [0, 5], fake=f) == S["JM_ERR_ALIGNMENT"]


def test_decode_validation_paths(L):
    f = _Fake()
    d = dims()
    w = _weights(f)
    S = {n: i for i, n in enumerate(jm._STATUS)}
    need = jm.decode_workspace_size(d, 4)
    call = lambda b, u, cs, ss, o, ws, nb: L.jamba_mamba_decode_step(  # noqa: E731
        ctypes.byref(d), ctypes.byref(w), u, b, cs, ss, o, ws, nb, None)
    assert call(4, f(), f(), f(), f(), f(), need - 1) == S["JM_ERR_WORKSPACE"]
    assert call(4, None, f(), f(), f(), f(), need) == S["JM_ERR_INVALID_ARG"]
    assert call(-1, f(), f(), f(), f(), f(), need) == S["JM_ERR_INVALID_ARG"]
    assert call(4, f() + 8, f(), f(), f(), f(), need) == S["JM_ERR_ALIGNMENT"]
    assert call(0, None, None, None, None, None, 0) == S["JM_OK"]


def test_noalloc_decode_validation_paths(L):
    """The no-workspace decode step validates like the decode step and rejects a batch whose
    workspace would not fit the fixed scratch, all before touching the GPU."""
    f = _Fake()
    d = dims()
    w = _weights(f)
    S = {n: i for i, n in enumerate(jm._STATUS)}
    call = lambda b, u=None: L.jamba_mamba_decode_step_noalloc(  # noqa: E731
        ctypes.byref(d), ctypes.byref(w), f() if u is None else u, b, f(), f(), f(), None)
    fits = max(b for b in range(1, 1024) if jm.decode_workspace_size(d, b) <= jm.NOALLOC_SCRATCH_BYTES)
    assert 400 < fits < 1024
    assert call(fits + 1) == S["JM_ERR_WORKSPACE"]
    assert call(4096) == S["JM_ERR_WORKSPACE"]
    assert call(-1) == S["JM_ERR_INVALID_ARG"]
    assert call(4, u=f() + 8) == S["JM_ERR_ALIGNMENT"]
    assert L.jamba_mamba_decode_step_noalloc(ctypes.byref(d), ctypes.byref(w), None, 4, f(), f(),
                                             f(), None) == S["JM_ERR_INVALID_ARG"]
    assert L.jamba_mamba_decode_step_noalloc(ctypes.byref(d), ctypes.byref(w), None, 0, None,
                                             None, None, None) == S["JM_OK"]


def test_decode_tiles_validation_paths(L):
    """Tiled decode weights: jm_tile_decode_weights and the decode entry points reject
    unsupported widths, half-set, misaligned or overlapping tiles before touching the GPU."""
    f = _Fake()
    d = dims()
    S = {n: i for i, n in enumerate(jm._STATUS)}
    tile = lambda dd, a, b, c, e: L.jm_tile_decode_weights(ctypes.byref(dd), a, b, c, e, None)  # noqa: E731
    tiny = jm.make_dims(64, 128, 16, 4, 8, jm.torch.float32)
    odd = jm.make_dims(4096, 8192, 16, 4, 64, jm.torch.bfloat16)   # dt_rank 64: generic decode
    assert tile(tiny, f(), f(), f(), f()) == S["JM_ERR_UNSUPPORTED"]
    assert tile(odd, f(), f(), f(), f()) == S["JM_ERR_UNSUPPORTED"]
    assert tile(d, f(), f(), None, f()) == S["JM_ERR_INVALID_ARG"]
    assert tile(d, f(), f(), f() + 8, f()) == S["JM_ERR_ALIGNMENT"]
    a, b = f(), f() + 0x10000000
    assert tile(d, a, b, a + 256, b + 2 * 0x10000000) == S["JM_ERR_INVALID_ARG"]   # tiles over W_in
    assert tile(d, a, b, a + 0x20000000, a + 0x20000000 + 4096) == S["JM_ERR_INVALID_ARG"]
    need = jm.decode_workspace_size(d, 4)
    call = lambda dd, w: L.jamba_mamba_decode_step(  # noqa: E731
        ctypes.byref(dd), ctypes.byref(w), f(), 4, f(), f(), f(), f(), need, None)
    assert call(d, _weights(f, in_proj_w_tiles=f())) == S["JM_ERR_INVALID_ARG"]
    assert call(d, _weights(f, in_proj_w_tiles=f(), out_proj_w_tiles=f() + 8)) == S["JM_ERR_ALIGNMENT"]
    assert call(odd, _weights(f, in_proj_w_tiles=f(), out_proj_w_tiles=f())) == S["JM_ERR_UNSUPPORTED"]
    assert L.jamba_mamba_decode_step_noalloc(
        ctypes.byref(odd), ctypes.byref(_weights(f, in_proj_w_tiles=f(), out_proj_w_tiles=f())),
        f(), 4, f(), f(), f(), None) == S["JM_ERR_UNSUPPORTED"]


def test_stage_validation_paths(L):
    """Every stage entry point rejects bad arguments on the host (nothing is launched)."""
    f = _Fake()
    d = dims()
    w = _weights(f)
    S = {n: i for i, n in enumerate(jm._STATUS)}
    D, W = ctypes.byref(d), ctypes.byref(w)
    cu = [0, 5, 9]
    host = (ctypes.c_int32 * 3)(*cu)
    bad = (ctypes.c_int32 * 3)(0, 5, 5)
    # in_proj / x_proj / dt_proj / out_proj: null, misaligned, token count
    assert L.jm_stage_in_proj(D, W, f(), 9, f(), None, None) == S["JM_ERR_INVALID_ARG"]
    assert L.jm_stage_in_proj(D, W, f() + 4, 9, f(), f(), None) == S["JM_ERR_ALIGNMENT"]
    assert L.jm_stage_in_proj(D, W, f(), 0, f(), f(), None) == S["JM_ERR_SHAPE"]
    assert L.jm_stage_x_proj(D, W, f(), 9, f(), f(), None, None) == S["JM_ERR_INVALID_ARG"]
    assert L.jm_stage_dt_proj(D, W, f(), -1, f(), None) == S["JM_ERR_SHAPE"]
    assert L.jm_stage_out_proj(D, W, None, 9, f(), None) == S["JM_ERR_INVALID_ARG"]
    wb = _weights(f, out_proj_w=None)
    assert L.jm_stage_out_proj(D, ctypes.byref(wb), f(), 9, f(), None) == S["JM_ERR_INVALID_ARG"]
    # conv: cu_seqlens checks, optional states aligned
    assert L.jm_stage_conv(D, W, f(), f(), bad, 2, 9, None, f(), None, None) == S["JM_ERR_SHAPE"]
    assert L.jm_stage_conv(D, W, f(), f(), host, 2, 10, None, f(), None, None) == S["JM_ERR_SHAPE"]
    assert L.jm_stage_conv(D, W, f(), None, host, 2, 9, None, f(), None, None) == S["JM_ERR_INVALID_ARG"]
    assert L.jm_stage_conv(D, W, f(), f(), host, 2, 9, f() + 8, f(), None, None) == S["JM_ERR_ALIGNMENT"]
    # scan: overlap of the two states, workspace size
    need = ctypes.c_size_t(0)
    assert L.jm_stage_scan_workspace_size(D, 100000, ctypes.byref(need)) == S["JM_OK"]
    assert need.value > 0
    big = (ctypes.c_int32 * 2)(0, 100000)
    args = lambda st_in, st_out, ws, nb, h=big, n=1, T=100000: (  # noqa: E731
        D, W, f(), f(), f(), f(), f(), f(), h, n, T, st_in, f(), st_out, ws, nb, None)
    assert L.jm_stage_scan(*args(None, None, f(), need.value - 1)) == S["JM_ERR_WORKSPACE"]
    assert L.jm_stage_scan(*args(None, None, None, need.value)) == S["JM_ERR_WORKSPACE"]
    assert L.jm_stage_scan(*args(0x50000000, 0x50000100, f(), need.value)) == S["JM_ERR_INVALID_ARG"]
    assert L.jm_stage_scan(*args(None, None, f(), need.value, h=bad, n=2, T=9)) == S["JM_ERR_SHAPE"]
    # decode update: required pointers, alignment, batch, and the optional slot map
    arr = lambda *v: (ctypes.c_int32 * len(v))(*v)  # noqa: E731

    def upd(b, xh, slots=None, slots_host=None, n_slots=0, B=None):
        return L.jm_stage_decode_update(D, W, xh, f(), f(), f() if B is None else B, f(), b,
                                        slots, slots_host, n_slots, f(), f(), None)

    assert upd(4, None) == S["JM_ERR_INVALID_ARG"]
    assert upd(4, f() + 4) == S["JM_ERR_ALIGNMENT"]
    assert upd(4, f(), B=f() + 8) == S["JM_ERR_ALIGNMENT"]
    assert upd(-1, f()) == S["JM_ERR_INVALID_ARG"]
    assert upd(0, None) == S["JM_OK"]
    assert upd(3, f(), f(), arr(0, 8, 1), 8) == S["JM_ERR_SHAPE"]          # slot 8 of 8
    assert upd(3, f(), f(), arr(2, 5, 2), 8) == S["JM_ERR_INVALID_ARG"]    # slot twice
    assert upd(3, f(), None, arr(2, 5, 3), 8) == S["JM_ERR_INVALID_ARG"]   # no device copy
    assert upd(3, f(), f(), None, 8) == S["JM_ERR_INVALID_ARG"]            # no host copy
    assert upd(3, f(), f(), arr(2, 5, 3), 0) == S["JM_ERR_INVALID_ARG"]    # n_slots < 1


def test_state_cache_validation_paths(L):
    """Slot arrays of the state-cache entry points are checked on the host."""
    f = _Fake()
    d = dims()
    w = _weights(f)
    S = {n: i for i, n in enumerate(jm._STATUS)}
    D, W = ctypes.byref(d), ctypes.byref(w)
    cu = [0, 5, 9, 10]
    host = (ctypes.c_int32 * 4)(*cu)
    arr = lambda *v: (ctypes.c_int32 * len(v))(*v)  # noqa: E731
    need = jm.prefill_slots_workspace_size(d, 3, 10)
    assert need > jm.prefill_workspace_size(d, 3, 10)

    def pre(init, fin, n_slots=8, init_dev=True, fin_dev=True, nb=need):
        return L.jamba_mamba_prefill_slots(
            D, W, f(), f(), host, 3, 10, f() if (init is not None and init_dev) else None, init,
            f() if (fin is not None and fin_dev) else None, fin, f(), f(), n_slots, f(), f(), nb,
            None)

    assert pre(arr(0, 1, 8), arr(0, 1, 2)) == S["JM_ERR_SHAPE"]           # slot 8 of 8
    assert pre(arr(0, -2, 1), None) == S["JM_ERR_SHAPE"]                  # below -1
    assert pre(None, arr(3, 4, 3)) == S["JM_ERR_INVALID_ARG"]             # final slot twice
    assert pre(arr(3, -1, -1), arr(4, 3, -1)) == S["JM_ERR_INVALID_ARG"]  # another's init slot
    assert pre(arr(3, 4, 5), arr(3, 4, 5), init_dev=False) == S["JM_ERR_INVALID_ARG"]
    assert pre(arr(3, 4, 5), arr(3, 4, 5), n_slots=0) == S["JM_ERR_INVALID_ARG"]
    assert pre(arr(3, 4, 5), arr(3, 4, 5), nb=need - 1) == S["JM_ERR_WORKSPACE"]
    dneed = jm.decode_workspace_size(d, 3)

    def dec(slots, n_slots=8, dev=True):
        return L.jamba_mamba_decode_step_slots(D, W, f(), 3, f() if dev else None, slots, f(),
                                               f(), n_slots, f(), f(), dneed, None)

    assert dec(arr(0, 8, 1)) == S["JM_ERR_SHAPE"]
    assert dec(arr(0, -1, 1)) == S["JM_ERR_SHAPE"]
    assert dec(arr(2, 5, 2)) == S["JM_ERR_INVALID_ARG"]
    assert dec(arr(2, 5, 3), dev=False) == S["JM_ERR_INVALID_ARG"]


def expected_segments(cu, chunk_len):
    """Independent statement of the chunking: chunk c covers [c*L, min((c+1)*L, T))."""
    T = cu[-1]
    segs = []
    n_chunks = -(-T // chunk_len)
    for c in range(n_chunks):
        a, b = c * chunk_len, min((c + 1) * chunk_len, T)
        for s in range(len(cu) - 1):
            lo, hi = max(a, cu[s]), min(b, cu[s + 1])
            if lo < hi:
                segs.append(dict(chunk=c, seq=s, begin=lo, end=hi, starts_seq=int(lo == cu[s]),
                                 ends_seq=int(hi == cu[s + 1])))
    return n_chunks, segs


@pytest.mark.parametrize("lengths", [[4096], [131072], [1, 2, 3, 1000, 64, 65, 7],
                                     [5000] * 16, [1] * 300])
@pytest.mark.parametrize("chunk_override", [0, 16, 1000])
def test_plan_matches_independent_chunking(lengths, chunk_override):
    cu = [0] + list(np.cumsum(lengths))
    d = dims()
    jm.set_scan_chunk_len(chunk_override)
    try:
        cl, nc, segs = jm.prefill_plan(d, cu)
    finally:
        jm.set_scan_chunk_len(0)
    if chunk_override:
        assert cl == chunk_override
    n_exp, segs_exp = expected_segments(cu, cl)
    assert nc == n_exp
    assert segs == segs_exp
    # every token is covered exactly once, every sequence starts and ends exactly once
    assert sum(s["end"] - s["begin"] for s in segs) == cu[-1]
    assert sum(s["starts_seq"] for s in segs) == len(lengths)
    assert sum(s["ends_seq"] for s in segs) == len(lengths)


@settings(max_examples=60, deadline=None, derandomize=True)
@given(st.lists(st.integers(1, 3000), min_size=1, max_size=12), st.sampled_from([0, 1, 7, 64, 256, 1000]))
def test_plan_property(lengths, chunk_override):
    """Random packings and chunk lengths: the library's plan equals the independent chunking,
    and the chunks tile the tokens exactly once."""
    test_plan_matches_independent_chunking(lengths, chunk_override)


def test_plan_rejects_bad_cu():
    d = dims()
    with pytest.raises(jm.JMError):
        jm.prefill_plan(d, [0, 3, 3])
    with pytest.raises(jm.JMError):
        jm.set_scan_chunk_len(-1)
