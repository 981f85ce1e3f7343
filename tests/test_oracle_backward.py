"""Pins for the backward oracle of the scan step (oracle/scan_backward.py), independent of
its code:

  * central finite differences of the forward oracle (selective_scan + gate) for every
    input element of small random cases, including h0 and a loss term on the final state;
  * reverse-mode autodiff (PyTorch on the CPU, fp64) of a forward written here in plain
    torch ops;
  * zero upstream gradients give exactly zero gradients; packed sequences equal the
    per-sequence results.
Planted mistakes in the oracle's pieces (SiLU' replaced by SiLU, the adjoint not decayed
towards h_{t-1}, dt dropped from dB) must each fail a pin.
"""
import numpy as np
import pytest

import oracle
import oracle.scan_backward as sb

torch = pytest.importorskip("torch")


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    den = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / den) if den > 0 else float(np.max(np.abs(a)))


def case(rng, T=5, di=3, N=4):
    return dict(
        x=rng.standard_normal((T, di)),
        dt=np.exp(rng.uniform(np.log(0.02), np.log(0.8), (T, di))),
        A_log=rng.standard_normal((di, N)) * 0.5,
        B=rng.standard_normal((T, N)),
        C=rng.standard_normal((T, N)),
        D=rng.standard_normal(di),
        z=rng.standard_normal((T, di)),
        h0=rng.standard_normal((di, N)) * 0.5,
    )


def loss_forward(c, R, R2):
    A = -np.exp(c["A_log"])
    y, h_last = oracle.selective_scan(c["x"], c["dt"], A, c["B"], c["C"], c["D"], c["h0"])
    g = oracle.gate(y, c["z"])
    return float(np.sum(R * g) + np.sum(R2 * h_last))


def check_finite_differences():
    rng = np.random.default_rng(31)
    for T, di, N in [(5, 3, 4), (1, 2, 2), (7, 1, 3)]:
        c = case(rng, T, di, N)
        R = rng.standard_normal((T, di))
        R2 = rng.standard_normal((di, N))
        g = sb.scan_gate_backward(c["x"], c["dt"], c["A_log"], c["B"], c["C"], c["D"], c["z"], R,
                                  c["h0"], R2)
        names = {"x": "dx", "dt": "ddt", "A_log": "dA_log", "B": "dB", "C": "dC", "D": "dD",
                 "z": "dz", "h0": "dh0"}
        for k, gk in names.items():
            fd = np.zeros_like(c[k])
            for idx in np.ndindex(c[k].shape):
                v = c[k][idx]
                eps = 1e-6 * max(1.0, abs(v))
                c[k][idx] = v + eps
                lp = loss_forward(c, R, R2)
                c[k][idx] = v - eps
                lm = loss_forward(c, R, R2)
                c[k][idx] = v
                fd[idx] = (lp - lm) / (2 * eps)
            assert rel(g[gk], fd) < 1e-7, (T, di, N, k, rel(g[gk], fd))


def torch_forward_loss(t, R, R2):
    """Independent forward in torch ops (fp64): returns the scalar loss."""
    A = -torch.exp(t["A_log"])
    h = t["h0"]
    loss = torch.zeros((), dtype=torch.float64)
    for i in range(t["x"].shape[0]):
        a = torch.exp(t["dt"][i][:, None] * A)
        h = a * h + (t["dt"][i] * t["x"][i])[:, None] * t["B"][i][None, :]
        y = (h * t["C"][i][None, :]).sum(1) + t["D"] * t["x"][i]
        g = y * t["z"][i] * torch.sigmoid(t["z"][i])
        loss = loss + (R[i] * g).sum()
    return loss + (R2 * h).sum()


def check_autograd():
    rng = np.random.default_rng(32)
    for T, di, N in [(6, 4, 5), (12, 2, 16)]:
        c = case(rng, T, di, N)
        R = rng.standard_normal((T, di))
        R2 = rng.standard_normal((di, N))
        t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in c.items()}
        torch_forward_loss(t, torch.tensor(R), torch.tensor(R2)).backward()
        g = sb.scan_gate_backward(c["x"], c["dt"], c["A_log"], c["B"], c["C"], c["D"], c["z"], R,
                                  c["h0"], R2)
        for k, gk in {"x": "dx", "dt": "ddt", "A_log": "dA_log", "B": "dB", "C": "dC", "D": "dD",
                      "z": "dz", "h0": "dh0"}.items():
            assert rel(g[gk], t[k].grad.numpy()) < 1e-12, (k, rel(g[gk], t[k].grad.numpy()))


def check_zero_upstream_and_packing():
    rng = np.random.default_rng(33)
    c = case(rng, 9, 3, 4)
    z0 = sb.scan_gate_backward(c["x"], c["dt"], c["A_log"], c["B"], c["C"], c["D"], c["z"],
                               np.zeros((9, 3)), c["h0"], None)
    assert all(np.all(v == 0.0) for v in z0.values())
    cu = [0, 2, 3, 9]
    R = rng.standard_normal((9, 3))
    h0 = rng.standard_normal((3, 3, 4))
    dh = rng.standard_normal((3, 3, 4))
    p = sb.scan_gate_backward_packed(c["x"], c["dt"], c["A_log"], c["B"], c["C"], c["D"], c["z"],
                                     R, cu, h0, dh)
    dD = np.zeros(3)
    for i in range(3):
        s, e = cu[i], cu[i + 1]
        r = sb.scan_gate_backward(c["x"][s:e], c["dt"][s:e], c["A_log"], c["B"][s:e],
                                  c["C"][s:e], c["D"], c["z"][s:e], R[s:e], h0[i], dh[i])
        for k in ("dx", "ddt", "dz", "dB", "dC"):
            assert np.array_equal(p[k][s:e], r[k])
        assert np.array_equal(p["dh0"][i], r["dh0"])
        dD += r["dD"]
    assert rel(p["dD"], dD) < 1e-15


PINS = {"finite_differences": check_finite_differences, "autograd": check_autograd,
        "zero_upstream_and_packing": check_zero_upstream_and_packing}


@pytest.mark.parametrize("name", list(PINS))
def test_backward_pin(name):
    PINS[name]()


_orig = {k: getattr(sb, k) for k in ("silu_prime", "adjoint_to_previous", "input_term_grads")}


def _mut_silu_prime(z):
    z = np.asarray(z, np.float64)
    return z * sb.sigmoid(z)


def _mut_adjoint_not_decayed(lam, a_t):
    return lam


def _mut_dB_without_dt(lam, dt_t, B_t, x_t):
    ddt, _, dx = _orig["input_term_grads"](lam, dt_t, B_t, x_t)
    return ddt, np.sum(lam * x_t[:, None], axis=0), dx


MUTATIONS = [("silu_prime", _mut_silu_prime), ("adjoint_to_previous", _mut_adjoint_not_decayed),
             ("input_term_grads", _mut_dB_without_dt)]


@pytest.mark.parametrize("target,mutant", MUTATIONS, ids=[m[1].__name__ for m in MUTATIONS])
def test_planted_backward_mistake_is_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(sb, target, mutant)
    failed = False
    for fn in PINS.values():
        try:
            fn()
        except AssertionError:
            failed = True
            break
    assert failed
