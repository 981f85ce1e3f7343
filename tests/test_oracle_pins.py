"""Pins for the CPU oracle, independent of the oracle's own code.

Each check uses a different route to the same number: brute force (materialised
products of decays, pure-Python loops), closed forms (geometric series), a library
routine for a special case (scipy.signal.lfilter), invariants (zero input, split,
packing, linearity, prefill vs. repeated decode) and hand sums on small integers.
The mutation tests at the bottom plant plausible mistakes in the oracle and check
that at least one pin fails for each.
"""
import math

import numpy as np
import pytest
import scipy.signal

import oracle
import oracle.mamba_ref as ref
import synth

TOL = 1e-12


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.max(np.abs(b))
    if den == 0:
        return float(np.max(np.abs(a)))
    return float(np.max(np.abs(a - b)) / den)


# ----------------------------------------------------------------------------------
# Independent brute-force building blocks (no oracle code used)
# ----------------------------------------------------------------------------------

def brute_scan(x, dt, A, B, C, D, h0):
    """h_t = (prod_{r<=t} a_r) h0 + sum_{s<=t} (prod_{r=s+1..t} a_r) dt_s B_s x_s, O(T^2)."""
    T, di = x.shape
    N = A.shape[1]
    y = np.zeros((T, di))
    h_last = np.zeros((di, N))
    for d in range(di):
        for n in range(N):
            a = [math.exp(dt[r, d] * A[d, n]) for r in range(T)]
            for t in range(T):
                p = 1.0
                for r in range(t + 1):
                    p *= a[r]
                h = p * h0[d, n]
                for s in range(t + 1):
                    q = 1.0
                    for r in range(s + 1, t + 1):
                        q *= a[r]
                    h += q * dt[s, d] * B[s, n] * x[s, d]
                y[t, d] += C[t, n] * h
                if t == T - 1:
                    h_last[d, n] = h
        for t in range(T):
            y[t, d] += D[d] * x[t, d]
    return y, h_last


def brute_layer(w, u, conv_hist=None, h0=None):
    """The whole layer in pure-Python loops for tiny sizes (one sequence)."""
    W_in, cw, cb = w["in_proj_w"], w["conv_w"], w["conv_b"]
    W_x, W_dt, b_dt = w["x_proj_w"], w["dt_proj_w"], w["dt_proj_b"]
    A_log, Dv, W_out = w["A_log"], w["D"], w["out_proj_w"]
    T, dm = u.shape
    di, K = cw.shape
    N = A_log.shape[1]
    R = W_dt.shape[1]
    x = [[sum(float(W_in[j, k]) * float(u[t, k]) for k in range(dm)) for j in range(di)] for t in range(T)]
    z = [[sum(float(W_in[di + j, k]) * float(u[t, k]) for k in range(dm)) for j in range(di)] for t in range(T)]

    def xval(t, d):  # pre-conv value at local time t (t<0 -> history)
        if t >= 0:
            return x[t][d]
        if conv_hist is None:
            return 0.0
        return float(conv_hist[d, K - 1 + t])

    sig = lambda v: 1.0 / (1.0 + math.exp(-v))  # noqa: E731
    xh = np.zeros((T, di))
    for t in range(T):
        for d in range(di):
            c = float(cb[d])
            for j in range(K):   # tap j looks back K-1-j tokens
                c += float(cw[d, j]) * xval(t - (K - 1 - j), d)
            xh[t, d] = c * sig(c)
    dbc = np.array([[sum(float(W_x[r, d]) * xh[t, d] for d in range(di)) for r in range(R + 2 * N)]
                    for t in range(T)])
    delta, Bm, Cm = dbc[:, :R], dbc[:, R:R + N], dbc[:, R + N:]
    if w.get("dt_norm_w") is not None:   # inner RMSNorm, row by row in plain loops
        eps = float(w.get("norm_eps", 1e-6))

        def rms_rows(M, gain):
            out_rows = []
            for row in M:
                r = math.sqrt(sum(float(v) * float(v) for v in row) / len(row) + eps)
                out_rows.append([float(v) / r * float(g) for v, g in zip(row, gain)])
            return np.array(out_rows)

        delta, Bm, Cm = (rms_rows(delta, w["dt_norm_w"]), rms_rows(Bm, w["B_norm_w"]),
                         rms_rows(Cm, w["C_norm_w"]))
    dt = np.zeros((T, di))
    for t in range(T):
        for d in range(di):
            v = sum(float(W_dt[d, r]) * delta[t, r] for r in range(R)) + float(b_dt[d])
            dt[t, d] = math.log(1.0 + math.exp(v))
    A = -np.exp(A_log.astype(np.float64))
    hz = np.zeros((di, N)) if h0 is None else np.asarray(h0, dtype=np.float64)
    y, h_last = brute_scan(xh, dt, A, Bm, Cm, Dv.astype(np.float64), hz)
    out = np.zeros((T, W_out.shape[0]))
    for t in range(T):
        g = [y[t, d] * z[t][d] * sig(z[t][d]) for d in range(di)]
        for m in range(W_out.shape[0]):
            out[t, m] = sum(float(W_out[m, d]) * g[d] for d in range(di))
    conv_new = np.array([[xval(T - (K - 1) + j, d) for j in range(K - 1)] for d in range(di)])
    return out, conv_new, h_last


def tiny_weights(rng, dm=4, di=4, N=3, K=4, R=2, D_value=1.0, scale=0.5):
    w = {
        "in_proj_w": rng.standard_normal((2 * di, dm)) * scale,
        "conv_w": rng.standard_normal((di, K)) * scale,
        "conv_b": rng.standard_normal(di) * scale,
        "x_proj_w": rng.standard_normal((R + 2 * N, di)) * scale,
        "dt_proj_w": rng.standard_normal((di, R)) * scale,
        "dt_proj_b": rng.standard_normal(di) * 0.5 - 2.0,
        "A_log": np.log(np.tile(np.arange(1, N + 1, dtype=np.float64), (di, 1))) + rng.standard_normal((di, N)) * 0.1,
        "D": np.full(di, D_value),
        "out_proj_w": rng.standard_normal((dm, di)) * scale,
    }
    return w


def with_norm(w, rng, eps=1e-6):
    """The same tiny layer with inner-RMSNorm gains (not close to 1, so they matter)."""
    w = dict(w)
    R = w["dt_proj_w"].shape[1]
    N = w["A_log"].shape[1]
    w["dt_norm_w"] = 1.0 + 0.5 * rng.standard_normal(R)
    w["B_norm_w"] = 1.0 + 0.5 * rng.standard_normal(N)
    w["C_norm_w"] = 1.0 + 0.5 * rng.standard_normal(N)
    w["norm_eps"] = eps
    return w


def rand_scan_inputs(rng, T, di, N):
    x = rng.standard_normal((T, di))
    dt = np.exp(rng.uniform(np.log(1e-2), np.log(1.0), (T, di)))
    A = -np.exp(rng.standard_normal((di, N)) * 0.5)
    B = rng.standard_normal((T, N))
    C = rng.standard_normal((T, N))
    D = rng.standard_normal(di)
    h0 = rng.standard_normal((di, N))
    return x, dt, A, B, C, D, h0


# ----------------------------------------------------------------------------------
# Pin checks (raise AssertionError on mismatch); the mutation tests reuse them.
# ----------------------------------------------------------------------------------

def check_scan_bruteforce():
    rng = np.random.default_rng(11)
    for T, di, N in [(1, 1, 1), (5, 3, 4), (8, 4, 4), (7, 2, 3)]:
        args = rand_scan_inputs(rng, T, di, N)
        y, h = oracle.selective_scan(*args)
        yb, hb = brute_scan(*args)
        assert rel_err(y, yb) < TOL and rel_err(h, hb) < TOL, (T, di, N)


def check_scan_geometric():
    rng = np.random.default_rng(12)
    T, di, N = 50, 3, 4
    dt_c = np.array([0.01, 0.2, 1.3])
    A = -np.exp(rng.standard_normal((di, N)))
    Bv = rng.standard_normal(N)
    Cv = rng.standard_normal(N)
    xv = rng.standard_normal(di)
    D = rng.standard_normal(di)
    x = np.tile(xv, (T, 1))
    dt = np.tile(dt_c, (T, 1))
    B = np.tile(Bv, (T, 1))
    C = np.tile(Cv, (T, 1))
    y, h_last = oracle.selective_scan(x, dt, A, B, C, D, None)
    t = np.arange(T)[:, None, None]
    a = np.exp(dt_c[:, None] * A)                       # (di, N)
    b = dt_c[:, None] * Bv[None, :] * xv[:, None]       # (di, N)
    h = b[None] * (1.0 - a[None] ** (t + 1)) / (1.0 - a[None])   # (T, di, N)
    y_cf = np.einsum("tdn,n->td", h, Cv) + D[None, :] * xv[None, :]
    assert rel_err(y, y_cf) < TOL
    assert rel_err(h_last, h[-1]) < TOL


def check_scan_lfilter():
    rng = np.random.default_rng(13)
    T, di, N = 200, 2, 3
    dt_c = np.array([0.05, 0.7])
    A = -np.exp(rng.standard_normal((di, N)))
    x = rng.standard_normal((T, di))
    B = rng.standard_normal((T, N))
    C = np.zeros((T, N))
    D = np.zeros(di)
    dt = np.tile(dt_c, (T, 1))
    # read h through y with C = e_n (one state at a time)
    for n in range(N):
        Cn = C.copy()
        Cn[:, n] = 1.0
        y, _ = oracle.selective_scan(x, dt, A, B, Cn, D, None)
        for d in range(di):
            ref_h = scipy.signal.lfilter([dt_c[d]], [1.0, -math.exp(dt_c[d] * A[d, n])], B[:, n] * x[:, d])
            assert rel_err(y[:, d], ref_h) < TOL, (n, d)


def check_zero_input():
    rng = np.random.default_rng(14)
    x, dt, A, B, C, D, _ = rand_scan_inputs(rng, 30, 4, 5)
    y, h = oracle.selective_scan(np.zeros_like(x), dt, A, B, C, D, None)
    assert np.all(y == 0.0) and np.all(h == 0.0)
    wl = synth.make_workload("tiny_fp32", lengths=[5, 17, 1])
    r = oracle.prefill(wl.weights, np.zeros_like(wl.u), wl.cu_seqlens)
    assert np.all(r["out"] == 0.0)


def check_prefill_vs_decode():
    for seed, T in [(0, 1), (1, 2), (2, 3), (3, 7), (4, 20)]:
        wl = synth.make_workload("tiny_fp32", seed=seed, lengths=[T])
        w = oracle.as_f64(wl.weights)
        r = oracle.prefill(w, wl.u, wl.cu_seqlens)
        di = w["D"].shape[0]
        conv = np.zeros((1, di, 3))
        ssm = np.zeros((1, di, 16))
        for t in range(T):
            o, conv, ssm = oracle.decode_step(w, wl.u[t:t + 1], conv, ssm)
            assert rel_err(o[0], r["out"][t]) < 1e-11, (T, t)
        assert rel_err(conv, r["conv_state"]) < TOL, T
        assert rel_err(ssm, r["ssm_state"]) < 1e-11, T


def check_split_invariance():
    wl = synth.make_workload("tiny_fp32", seed=5, lengths=[40])
    w = oracle.as_f64(wl.weights)
    full = oracle.prefill(w, wl.u, [0, 40])
    for L1 in (1, 2, 3, 17, 39):
        a = oracle.prefill(w, wl.u[:L1], [0, L1])
        b = oracle.prefill(w, wl.u[L1:], [0, 40 - L1], init_conv=a["conv_state"], init_ssm=a["ssm_state"])
        assert rel_err(np.concatenate([a["out"], b["out"]]), full["out"]) < 1e-11, L1
        assert rel_err(b["conv_state"], full["conv_state"]) < TOL, L1
        assert rel_err(b["ssm_state"], full["ssm_state"]) < 1e-11, L1


def check_packing():
    wl = synth.make_workload("tiny_fp32", seed=6, lengths=[3, 1, 9, 2, 12])
    w = oracle.as_f64(wl.weights)
    packed = oracle.prefill(w, wl.u, wl.cu_seqlens)
    cu = wl.cu_seqlens
    for i in range(len(cu) - 1):
        s, e = cu[i], cu[i + 1]
        single = oracle.prefill(w, wl.u[s:e], [0, e - s])
        assert np.array_equal(single["out"], packed["out"][s:e])
        assert np.array_equal(single["conv_state"][0], packed["conv_state"][i])
        assert np.array_equal(single["ssm_state"][0], packed["ssm_state"][i])


def check_special_cases():
    rng = np.random.default_rng(15)
    T, di, N = 25, 3, 4
    x, dt, A, B, C, D, h0 = rand_scan_inputs(rng, T, di, N)
    # B = 0: the state only decays
    Cn = np.zeros((T, N)); Cn[:, 1] = 1.0
    y, h = oracle.selective_scan(x, dt, A, np.zeros((T, N)), Cn, np.zeros(di), h0)
    decay = np.exp(np.cumsum(dt, axis=0)[:, :, None] * A[None])       # (T, di, N)
    assert rel_err(h, decay[-1] * h0) < TOL
    assert rel_err(y, (decay * h0[None])[:, :, 1]) < TOL
    # A = 0: running sum of dt*B*x
    y, h = oracle.selective_scan(x, dt, np.zeros((di, N)), B, C, np.zeros(di), h0)
    hs = h0[None] + np.cumsum(dt[:, :, None] * B[:, None, :] * x[:, :, None], axis=0)
    assert rel_err(h, hs[-1]) < TOL
    assert rel_err(y, np.einsum("tdn,tn->td", hs, C)) < TOL
    # C = 0: only the skip term
    y, _ = oracle.selective_scan(x, dt, A, B, np.zeros((T, N)), D, h0)
    assert rel_err(y, D[None, :] * x) < TOL


def check_linearity():
    rng = np.random.default_rng(16)
    T, di, N = 30, 3, 4
    x, dt, A, B, C, D, h0 = rand_scan_inputs(rng, T, di, N)
    x2 = rng.standard_normal((T, di))
    h02 = rng.standard_normal((di, N))
    al, be = 0.7, -1.9
    y1, h1 = oracle.selective_scan(x, dt, A, B, C, D, h0)
    y2, h2 = oracle.selective_scan(x2, dt, A, B, C, D, h02)
    y3, h3 = oracle.selective_scan(al * x + be * x2, dt, A, B, C, D, al * h0 + be * h02)
    assert rel_err(y3, al * y1 + be * y2) < TOL
    assert rel_err(h3, al * h1 + be * h2) < TOL


def check_small_integer_stages():
    # in_proj: x rows first, then z; hand sums of small integers are exact
    rng = np.random.default_rng(17)
    u = rng.integers(-3, 4, (3, 5)).astype(np.float64)
    W = rng.integers(-2, 3, (8, 5)).astype(np.float64)
    x, z = oracle.in_proj(u, W, 4)
    for t in range(3):
        for j in range(4):
            assert x[t, j] == sum(W[j, k] * u[t, k] for k in range(5))
            assert z[t, j] == sum(W[4 + j, k] * u[t, k] for k in range(5))
    # x_proj split: delta | B | C
    xh = rng.integers(-3, 4, (2, 6)).astype(np.float64)
    Wx = rng.integers(-2, 3, (2 + 2 * 3, 6)).astype(np.float64)
    dl, Bm, Cm = oracle.x_proj(xh, Wx, 2, 3)
    full = [[sum(Wx[r, d] * xh[t, d] for d in range(6)) for r in range(8)] for t in range(2)]
    assert np.array_equal(dl, np.array(full)[:, :2])
    assert np.array_equal(Bm, np.array(full)[:, 2:5])
    assert np.array_equal(Cm, np.array(full)[:, 5:8])
    # out_proj
    g = rng.integers(-3, 4, (2, 4)).astype(np.float64)
    Wo = rng.integers(-2, 3, (3, 4)).astype(np.float64)
    o = oracle.out_proj(g, Wo)
    assert np.array_equal(o, np.array([[sum(Wo[m, d] * g[t, d] for d in range(4)) for m in range(3)] for t in range(2)]))
    # conv impulse response: unit impulse at t0 gives silu(b + w[d, K-1-(t-t0)]) for t0 <= t < t0+K
    di, K, T, t0 = 3, 4, 9, 2
    cw = rng.integers(-3, 4, (di, K)).astype(np.float64)
    cb = np.array([0.0, 1.0, -2.0])
    xin = np.zeros((T, di)); xin[t0, :] = 1.0
    xh, hist = oracle.causal_conv_silu(xin, cw, cb, None)
    for t in range(T):
        for d in range(di):
            c = cb[d] + (cw[d, K - 1 - (t - t0)] if 0 <= t - t0 < K else 0.0)
            assert abs(xh[t, d] - c / (1.0 + math.exp(-c))) < 1e-15
    assert np.array_equal(hist, xin[T - 3:].T)
    # conv history: values before the first token enter oldest first
    hist_in = rng.integers(-3, 4, (di, K - 1)).astype(np.float64)
    xh, hist2 = oracle.causal_conv_silu(np.zeros((1, di)), cw, np.zeros(di), hist_in)
    c = np.array([sum(cw[d, j] * hist_in[d, j] for j in range(K - 1)) for d in range(di)])
    assert np.allclose(xh[0], c / (1.0 + np.exp(-c)), rtol=0, atol=1e-15)
    assert np.array_equal(hist2, np.concatenate([hist_in[:, 1:], np.zeros((di, 1))], axis=1))
    # activations
    assert oracle.softplus(0.0) == math.log(2.0)
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(oracle.softplus(50.0) - 50.0) < 1e-15
    assert abs(oracle.softplus(-50.0) - math.exp(-50.0)) < 1e-30
    assert abs(oracle.softplus(1.5) - math.log(1.0 + math.exp(1.5))) < 1e-15
    wts = synth.make_weights(synth.TINY_DIMS, "f32", np.random.default_rng(0))
    back = oracle.softplus(wts["dt_proj_b"].astype(np.float64))
    assert np.max(np.abs(back / wts["dt0"] - 1.0)) < 1e-6     # fp32 bias storage
    # dt_proj: softplus(W delta + b)
    dl = np.array([[1.0, -2.0]])
    Wd = np.array([[1.0, 1.0], [0.5, 0.0], [0.0, 2.0]])
    bd = np.array([0.0, 1.0, 4.0])
    dtv = oracle.dt_proj(dl, Wd, bd)
    assert np.allclose(dtv[0], [math.log1p(math.exp(-1.0)), math.log1p(math.exp(1.5)), math.log1p(math.exp(0.0))],
                       rtol=1e-15, atol=0)
    # gate
    assert np.allclose(oracle.gate(np.array([2.0, -1.0]), np.array([0.0, 3.0])),
                       [0.0, -3.0 / (1.0 + math.exp(-3.0))], rtol=1e-15, atol=0)


def check_layer_bruteforce():
    rng = np.random.default_rng(18)
    for D_value in (1.0, 0.0):
        w = tiny_weights(rng, D_value=D_value)
        T = 6
        u = rng.standard_normal((T, 4))
        hist = rng.standard_normal((4, 3))
        h0 = rng.standard_normal((4, 3)) * 0.3
        r = oracle.prefill(w, u, [0, T], init_conv=hist[None], init_ssm=h0[None])
        ob, cb_, hb = brute_layer(w, u, hist, h0)
        assert rel_err(r["out"], ob) < 1e-11
        assert rel_err(r["conv_state"][0], cb_) < TOL
        assert rel_err(r["ssm_state"][0], hb) < 1e-11
        # and from zero state, T < K-1
        r = oracle.prefill(w, u[:2], [0, 2])
        ob, cb_, hb = brute_layer(w, u[:2])
        assert rel_err(r["out"], ob) < 1e-11 and rel_err(r["conv_state"][0], cb_) < TOL


def check_rmsnorm_closed_form():
    # v / sqrt(mean(v^2) + eps) * gain on hand values
    s = math.sqrt(12.5)
    assert np.allclose(oracle.rmsnorm([[3.0, 4.0]], [1.0, 1.0], 0.0), [[3 / s, 4 / s]], rtol=0, atol=1e-15)
    assert np.allclose(oracle.rmsnorm([[3.0, 4.0]], [2.0, -1.0], 0.0), [[6 / s, -4 / s]], rtol=0, atol=1e-15)
    # eps sits inside the root, added to the mean square: 1e-3 / sqrt(1e-6 + 1e-6) = 1/sqrt(2)
    assert abs(oracle.rmsnorm([[1e-3]], [1.0], 1e-6)[0, 0] - 1 / math.sqrt(2)) < 1e-15
    # a mean, not a sum; rows are independent; an all-zero row stays zero
    r = oracle.rmsnorm([[1.0, 1.0, 1.0, 1.0], [0.0, 0.0, 0.0, 0.0]], [1.0] * 4, 1e-6)
    assert abs(r[0, 0] - 1 / math.sqrt(1 + 1e-6)) < 1e-15 and np.all(r[1] == 0.0)


def check_rmsnorm_invariants():
    rng = np.random.default_rng(21)
    v = rng.standard_normal((5, 256))
    g = np.ones(256)
    r = oracle.rmsnorm(v, g, 0.0)
    assert rel_err(oracle.rmsnorm(7.3 * v, g, 0.0), r) < TOL          # scale invariance
    assert np.max(np.abs(np.mean(r * r, axis=1) - 1.0)) < TOL          # unit mean square


def check_layer_bruteforce_inner_norm():
    rng = np.random.default_rng(22)
    for D_value in (1.0, 0.0):
        w_plain = tiny_weights(rng, D_value=D_value)
        w = with_norm(w_plain, rng)
        T = 6
        u = rng.standard_normal((T, 4))
        hist = rng.standard_normal((4, 3))
        h0 = rng.standard_normal((4, 3)) * 0.3
        r = oracle.prefill(w, u, [0, T], init_conv=hist[None], init_ssm=h0[None])
        ob, cb_, hb = brute_layer(w, u, hist, h0)
        assert rel_err(r["out"], ob) < 1e-11
        assert rel_err(r["ssm_state"][0], hb) < 1e-11
        # the norm changes the result (the step is not a no-op on this layer)
        plain = oracle.prefill(w_plain, u, [0, T], init_conv=hist[None], init_ssm=h0[None])
        assert rel_err(r["out"], plain["out"]) > 1e-3


def check_prefill_vs_decode_inner_norm():
    """The decode step (its own code) agrees with the prefill when the norm is on."""
    rng = np.random.default_rng(23)
    w = with_norm(tiny_weights(rng), rng)
    T = 7
    u = rng.standard_normal((T, 4))
    r = oracle.prefill(w, u, [0, T])
    conv = np.zeros((1, 4, 3))
    ssm = np.zeros((1, 4, 3))
    outs = []
    for t in range(T):
        o, conv, ssm = oracle.decode_step(w, u[t:t + 1], conv, ssm)
        outs.append(o[0])
    assert rel_err(np.array(outs), r["out"]) < 1e-12
    assert rel_err(ssm, r["ssm_state"]) < 1e-12


PINS = {
    "scan_bruteforce": check_scan_bruteforce,
    "scan_geometric": check_scan_geometric,
    "scan_lfilter": check_scan_lfilter,
    "zero_input": check_zero_input,
    "prefill_vs_decode": check_prefill_vs_decode,
    "split_invariance": check_split_invariance,
    "packing": check_packing,
    "special_cases": check_special_cases,
    "linearity": check_linearity,
    "small_integer_stages": check_small_integer_stages,
    "layer_bruteforce": check_layer_bruteforce,
    "rmsnorm_closed_form": check_rmsnorm_closed_form,
    "rmsnorm_invariants": check_rmsnorm_invariants,
    "layer_bruteforce_inner_norm": check_layer_bruteforce_inner_norm,
    "prefill_vs_decode_inner_norm": check_prefill_vs_decode_inner_norm,
}


@pytest.mark.parametrize("name", list(PINS))
def test_pin(name):
    PINS[name]()


# ----------------------------------------------------------------------------------
# Mutation tests: a plausible mistake planted in the oracle must fail some pin.
# ----------------------------------------------------------------------------------

def _fails_some_pin():
    for fn in PINS.values():
        try:
            fn()
        except AssertionError:
            return True
    return False


def _mut_conv_reversed(x, conv_w, conv_b, history=None):
    return _orig["causal_conv_silu"](x, np.asarray(conv_w)[:, ::-1], conv_b, history)


def _mut_xz_swapped(u, in_proj_w, d_inner):
    x, z = _orig["in_proj"](u, in_proj_w, d_inner)
    return z, x


def _mut_softplus_plain_exp(v):
    return np.exp(np.asarray(v, dtype=np.float64))


def _mut_gate_swapped(y, z):
    return _orig["silu"](y) * np.asarray(z, dtype=np.float64)


def _mut_xproj_order(x_hat, x_proj_w, dt_rank, d_state):
    d, B, C = _orig["x_proj"](x_hat, x_proj_w, dt_rank, d_state)
    return d, C, B


def _mut_scan_no_skip(x, dt, A, B, C, D, h0=None):
    return _orig["selective_scan"](x, dt, A, B, C, np.zeros_like(np.asarray(D, dtype=np.float64)), h0)


def _mut_scan_sign(x, dt, A, B, C, D, h0=None):
    return _orig["selective_scan"](x, dt, -np.asarray(A, dtype=np.float64), B, C, D, h0)


def _mut_scan_ignores_h0(x, dt, A, B, C, D, h0=None):
    return _orig["selective_scan"](x, dt, A, B, C, D, None)


def _mut_rms_eps_outside(v, gain, eps):
    v = np.asarray(v, dtype=np.float64)
    return v / (np.sqrt(np.mean(v * v, axis=-1, keepdims=True)) + eps) * np.asarray(gain)


def _mut_rms_sum(v, gain, eps):
    v = np.asarray(v, dtype=np.float64)
    return v / np.sqrt(np.sum(v * v, axis=-1, keepdims=True) + eps) * np.asarray(gain)


def _mut_rms_no_gain(v, gain, eps):
    return _orig["rmsnorm"](v, np.ones_like(np.asarray(gain, dtype=np.float64)), eps)


def _mut_inner_norm_skips_B(w, delta, B, C):
    d, _, c = _orig["inner_norm"](w, delta, B, C)
    return d, B, c


_orig = {k: getattr(ref, k) for k in ("causal_conv_silu", "in_proj", "softplus", "silu", "gate",
                                      "x_proj", "selective_scan", "rmsnorm", "inner_norm")}

MUTATIONS = [
    ("causal_conv_silu", _mut_conv_reversed),
    ("in_proj", _mut_xz_swapped),
    ("softplus", _mut_softplus_plain_exp),
    ("gate", _mut_gate_swapped),
    ("x_proj", _mut_xproj_order),
    ("selective_scan", _mut_scan_no_skip),
    ("selective_scan", _mut_scan_sign),
    ("selective_scan", _mut_scan_ignores_h0),
    ("rmsnorm", _mut_rms_eps_outside),
    ("rmsnorm", _mut_rms_sum),
    ("rmsnorm", _mut_rms_no_gain),
    ("inner_norm", _mut_inner_norm_skips_B),
]


@pytest.mark.parametrize("target,mutant", MUTATIONS, ids=[m[1].__name__ for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(ref, target, mutant)
    monkeypatch.setattr(oracle, target, mutant)
    assert _fails_some_pin()


def test_planted_scan_kernel_mistake_is_caught(monkeypatch):
    """A wrong recurrence in the C loop itself (decay applied after the input term)."""
    def wrong(x, dt, A, B, C, D, h0=None):
        x, dt, A, B, C, D = (np.asarray(v, dtype=np.float64) for v in (x, dt, A, B, C, D))
        T, di = x.shape
        h = np.zeros((di, A.shape[1])) if h0 is None else np.array(h0, dtype=np.float64)
        y = np.empty((T, di))
        for t in range(T):
            h = np.exp(dt[t][:, None] * A) * (h + dt[t][:, None] * B[t][None, :] * x[t][:, None])
            y[t] = h @ C[t] + D * x[t]
        return y, h
    monkeypatch.setattr(ref, "selective_scan", wrong)
    monkeypatch.setattr(oracle, "selective_scan", wrong)
    assert _fails_some_pin()


def test_blocked_prefill_equals_one_call():
    """The test helper that streams the oracle's prefill in token blocks (carrying each
    sequence's states between blocks) gives the one-call prefill: outputs and final states."""
    from jm_testutil import oracle_prefill_blocked
    wl = synth.make_workload("tiny_fp32", seed=11, lengths=[20, 3, 9, 1])
    w = oracle.as_f64(wl.weights)
    rng = np.random.default_rng(12)
    ic = rng.standard_normal((4, 128, 3))
    ih = rng.standard_normal((4, 128, 16)) * 0.1
    ref = oracle.prefill(w, wl.u, wl.cu_seqlens, ic, ih)
    got = np.full_like(ref["out"], np.nan)

    def put(r0, rows):
        got[r0:r0 + len(rows)] = rows

    conv, ssm = oracle_prefill_blocked(oracle, w, wl.u, wl.cu_seqlens, 7, put, ic, ih)
    assert np.max(np.abs(got - ref["out"])) <= 1e-12 * np.max(np.abs(ref["out"]))
    # conv state: copies of x, whose in_proj products BLAS may round differently for a
    # different number of rows, so the same 1e-12 bound as the other tensors
    assert np.max(np.abs(conv - ref["conv_state"])) <= 1e-12 * np.max(np.abs(ref["conv_state"]))
    assert np.max(np.abs(ssm - ref["ssm_state"])) <= 1e-12 * np.max(np.abs(ref["ssm_state"]))
