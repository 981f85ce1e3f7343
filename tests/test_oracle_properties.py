"""Property tests of the CPU oracle (hypothesis): random tiny layer widths, packed sequence
lengths, initial states, D and the optional inner norm, each compared with the independent
pure-Python brute force of test_oracle_pins (products of decays written out, plain loops for
every projection, the conv and the gate); and the backward oracle over random packings against
fp64 autograd of a forward written in torch ops. Examples are derandomized, so the suite is
repeatable.
"""
import numpy as np
from hypothesis import given, settings, strategies as st

import oracle
from test_oracle_pins import brute_layer, brute_scan, rel_err, tiny_weights, with_norm

SETTINGS = settings(max_examples=30, deadline=None, derandomize=True)


@st.composite
def layer_case(draw):
    dm = draw(st.integers(1, 5))
    di = draw(st.integers(1, 4))
    N = draw(st.integers(1, 4))
    R = draw(st.integers(1, 3))
    lengths = draw(st.lists(st.integers(1, 9), min_size=1, max_size=4))
    seed = draw(st.integers(0, 2**31 - 1))
    D_value = draw(st.sampled_from([0.0, 1.0]))
    states = draw(st.booleans())
    norm = draw(st.booleans())
    return dm, di, N, R, lengths, seed, D_value, states, norm


@SETTINGS
@given(layer_case())
def test_packed_layer_matches_brute_force(case):
    """Each packed sequence, from its own initial states or zeros, equals the brute-force layer
    run on that sequence alone: outputs and both final states."""
    dm, di, N, R, lengths, seed, D_value, states, norm = case
    rng = np.random.default_rng(seed)
    w = tiny_weights(rng, dm=dm, di=di, N=N, R=R, D_value=D_value)
    if norm:
        w = with_norm(w, rng)
    n = len(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    u = rng.standard_normal((int(cu[-1]), dm))
    hist = rng.standard_normal((n, di, 3)) if states else None
    h0 = rng.standard_normal((n, di, N)) * 0.3 if states else None
    r = oracle.prefill(w, u, cu, init_conv=hist, init_ssm=h0)
    for i in range(n):
        s, e = int(cu[i]), int(cu[i + 1])
        ob, cb, hb = brute_layer(w, u[s:e], None if hist is None else hist[i],
                                 None if h0 is None else h0[i])
        assert rel_err(r["out"][s:e], ob) < 1e-10, (i, case)
        assert rel_err(r["conv_state"][i], cb) < 1e-12, (i, case)
        assert rel_err(r["ssm_state"][i], hb) < 1e-10, (i, case)


@SETTINGS
@given(layer_case(), st.integers(1, 4))
def test_decode_steps_continue_the_prefill(case, steps):
    """Decoding `steps` more tokens from a prefill's final states equals the prefill of the
    longer sequences (every sequence of the batch at once)."""
    dm, di, N, R, lengths, seed, D_value, states, norm = case
    rng = np.random.default_rng(seed)
    w = tiny_weights(rng, dm=dm, di=di, N=N, R=R, D_value=D_value)
    if norm:
        w = with_norm(w, rng)
    n = len(lengths)
    seqs = [rng.standard_normal((L + steps, dm)) for L in lengths]
    head = np.concatenate([q[:-steps] for q in seqs])
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    r = oracle.prefill(w, head, cu)
    conv, ssm = r["conv_state"], r["ssm_state"]
    outs = []
    for k in range(steps):
        tok = np.stack([q[len(q) - steps + k] for q in seqs])
        o, conv, ssm = oracle.decode_step(w, tok, conv, ssm)
        outs.append(o)
    full_cu = np.concatenate([[0], np.cumsum([L + steps for L in lengths])]).astype(np.int64)
    full = oracle.prefill(w, np.concatenate(seqs), full_cu)
    for i in range(n):
        tail = full["out"][int(full_cu[i + 1]) - steps:int(full_cu[i + 1])]
        assert rel_err(np.stack([o[i] for o in outs]), tail) < 1e-10, (i, case, steps)
    assert rel_err(conv, full["conv_state"]) < 1e-12
    assert rel_err(ssm, full["ssm_state"]) < 1e-10


@SETTINGS
@given(st.integers(1, 10), st.integers(1, 3), st.integers(1, 4), st.integers(0, 2**31 - 1),
       st.floats(0.0, 1.0))
def test_scan_matches_brute_force(T, di, N, seed, h0_scale):
    """The oracle's recurrence against the O(T^2) product-of-decays form."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, di))
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(2.0), (T, di)))
    A = -np.exp(rng.standard_normal((di, N)))
    B = rng.standard_normal((T, N))
    C = rng.standard_normal((T, N))
    D = rng.standard_normal(di)
    h0 = rng.standard_normal((di, N)) * h0_scale
    y, h = oracle.selective_scan(x, dt, A, B, C, D, h0)
    yb, hb = brute_scan(x, dt, A, B, C, D, h0)
    assert rel_err(y, yb) < 1e-11 and rel_err(h, hb) < 1e-11


@SETTINGS
@given(st.lists(st.integers(1, 8), min_size=1, max_size=3), st.integers(1, 4), st.integers(1, 5),
       st.integers(0, 2**31 - 1), st.booleans())
def test_backward_matches_autograd(lengths, di, N, seed, states):
    """The backward oracle over packed sequences against fp64 autograd of a forward written in
    torch ops (per sequence: the state restarts, the loss adds sum(R * g) and sum(R2 * h_last))."""
    import torch
    import oracle.scan_backward as sb
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    n = len(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    c = dict(x=rng.standard_normal((T, di)),
             dt=np.exp(rng.uniform(np.log(0.02), np.log(0.8), (T, di))),
             A_log=rng.standard_normal((di, N)) * 0.5, B=rng.standard_normal((T, N)),
             C=rng.standard_normal((T, N)), D=rng.standard_normal(di), z=rng.standard_normal((T, di)),
             h0=rng.standard_normal((n, di, N)) * 0.5 if states else np.zeros((n, di, N)))
    R = rng.standard_normal((T, di))
    R2 = rng.standard_normal((n, di, N)) if states else np.zeros((n, di, N))
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in c.items()}
    A = -torch.exp(t["A_log"])
    loss = torch.zeros((), dtype=torch.float64)
    for i in range(n):
        h = t["h0"][i]
        for j in range(int(cu[i]), int(cu[i + 1])):
            h = torch.exp(t["dt"][j][:, None] * A) * h + (t["dt"][j] * t["x"][j])[:, None] * t["B"][j][None, :]
            y = (h * t["C"][j][None, :]).sum(1) + t["D"] * t["x"][j]
            loss = loss + (torch.tensor(R[j]) * y * t["z"][j] * torch.sigmoid(t["z"][j])).sum()
        loss = loss + (torch.tensor(R2[i]) * h).sum()
    loss.backward()
    g = sb.scan_gate_backward_packed(c["x"], c["dt"], c["A_log"], c["B"], c["C"], c["D"], c["z"], R,
                                     cu, c["h0"] if states else None, R2 if states else None)
    for k, gk in {"x": "dx", "dt": "ddt", "A_log": "dA_log", "B": "dB", "C": "dC", "D": "dD",
                  "z": "dz", "h0": "dh0"}.items():
        assert rel_err(g[gk], t[k].grad.numpy()) < 1e-11, (k, lengths, di, N)
