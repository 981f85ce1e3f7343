"""CPU oracle (fp64) for the backward pass of the scan step -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may use it; the HIP
library never does. Pinned in tests/test_oracle_backward.py by central finite differences
of the forward oracle and by reverse-mode autodiff of an independently written forward.

Training is how the paper reaches its results (Jamba: A Hybrid Transformer-Mamba Language
Model, §3.1: trained up to 1M-token contexts; §6.4: training stability at scale), and the
backward of the layer's recurrence is what a training step adds on top of the forward. The
step differentiated here is the forward oracle's `selective_scan` followed by `gate`, per
sequence:

    a_t = exp(dt_t A),  A = -exp(A_log)          (per channel d and state n)
    h_t = a_t h_{t-1} + dt_t B_t x_t,  h_{-1} = h0 (or 0)
    y_t = C_t . h_t + D x_t
    g_t = y_t SiLU(z_t)

Given dL/dg (dg) and optionally dL/dh_{T-1} (dh_last), reverse mode gives the adjoint
lam_t = dL/dh_t through lam_t = a_{t+1} lam_{t+1} + dy_t C_t (dy = dg SiLU(z)), starting
from dh_last, and then every input's gradient from lam_t and h_{t-1}:

    dz_t  = dg_t y_t SiLU'(z_t)           dD   = sum_t dy_t x_t
    dC_t  = sum_d dy_t h_t                 dh0  = a_0 lam_0
    dx_t  = dy_t D + sum_n lam_t dt_t B_t
    ddt_t = sum_n lam_t (h_{t-1} a_t A + B_t x_t)
    dB_t  = sum_d lam_t dt_t x_t
    dA    = sum_t lam_t h_{t-1} a_t dt_t,  dA_log = dA * A
All arithmetic fp64; h is kept for every token (small test sizes).
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-_f64(z)))


def silu_prime(z):
    """d/dz [z sigmoid(z)] = sigmoid(z) (1 + z (1 - sigmoid(z)))."""
    z = _f64(z)
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def adjoint_to_previous(lam, a_t):
    """The part of lam_t that reaches h_{t-1}: dh_{t-1} receives a_t lam_t."""
    return a_t * lam


def input_term_grads(lam, dt_t, B_t, x_t):
    """Gradients through u_t = dt_t B_t x_t: (ddt_t part, dB_t, dx_t part)."""
    ddt = np.sum(lam * B_t[None, :], axis=1) * x_t
    dB = np.sum(lam * (dt_t * x_t)[:, None], axis=0)
    dx = np.sum(lam * B_t[None, :], axis=1) * dt_t
    return ddt, dB, dx


def scan_gate_backward(x, dt, A_log, B, C, D, z, dg, h0=None, dh_last=None) -> Dict[str, np.ndarray]:
    """Gradients of one sequence's scan + skip + gate step (see the module docstring).

    x, dt, z, dg: (T, d_inner); A_log: (d_inner, N); B, C: (T, N); D: (d_inner,);
    h0, dh_last: (d_inner, N) or None. Returns dx, ddt, dz (T, d_inner), dB, dC (T, N),
    dD (d_inner,), dA_log (d_inner, N), dh0 (d_inner, N).
    """
    x, dt, A_log, B, C, D, z, dg = (_f64(v) for v in (x, dt, A_log, B, C, D, z, dg))
    T, di = x.shape
    N = A_log.shape[1]
    A = -np.exp(A_log)
    hz = np.zeros((di, N)) if h0 is None else _f64(h0)
    # forward, keeping every state
    a = np.exp(dt[:, :, None] * A[None])                      # (T, di, N)
    h = np.empty((T, di, N))
    hp = hz
    for t in range(T):
        hp = a[t] * hp + (dt[t] * x[t])[:, None] * B[t][None, :]
        h[t] = hp
    y = np.einsum("tdn,tn->td", h, C) + D[None, :] * x
    s = z * sigmoid(z)
    dy = dg * s
    out = {
        "dz": dg * y * silu_prime(z),
        "dD": np.sum(dy * x, axis=0),
        "dC": np.einsum("td,tdn->tn", dy, h),
        "dx": dy * D[None, :],
        "ddt": np.zeros((T, di)),
        "dB": np.zeros((T, N)),
    }
    dA = np.zeros((di, N))
    lam = np.zeros((di, N)) if dh_last is None else _f64(dh_last).copy()
    for t in range(T - 1, -1, -1):
        lam = lam + dy[t][:, None] * C[t][None, :]            # lam_t
        h_prev = h[t - 1] if t > 0 else hz
        da = lam * h_prev
        ddt_u, dB_t, dx_u = input_term_grads(lam, dt[t], B[t], x[t])
        out["ddt"][t] = np.sum(da * a[t] * A, axis=1) + ddt_u
        out["dB"][t] = dB_t
        out["dx"][t] += dx_u
        dA += da * a[t] * dt[t][:, None]
        lam = adjoint_to_previous(lam, a[t])                   # towards h_{t-1}
    out["dA_log"] = dA * A
    out["dh0"] = lam
    return out


def scan_gate_backward_packed(x, dt, A_log, B, C, D, z, dg, cu_seqlens, h0=None,
                              dh_last=None) -> Dict[str, np.ndarray]:
    """Packed sequences (rows cu[i]..cu[i+1]-1): each sequence on its own; dD and dA_log
    summed over sequences, dh0 per sequence. h0, dh_last: (n, d_inner, N) or None."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    n = len(cu) - 1
    T, di = np.shape(x)
    N = np.shape(A_log)[1]
    res = {"dx": np.zeros((T, di)), "ddt": np.zeros((T, di)), "dz": np.zeros((T, di)),
           "dB": np.zeros((T, N)), "dC": np.zeros((T, N)), "dD": np.zeros(di),
           "dA_log": np.zeros((di, N)), "dh0": np.zeros((n, di, N))}
    for i in range(n):
        s, e = int(cu[i]), int(cu[i + 1])
        r = scan_gate_backward(np.asarray(x)[s:e], np.asarray(dt)[s:e], A_log,
                               np.asarray(B)[s:e], np.asarray(C)[s:e], D, np.asarray(z)[s:e],
                               np.asarray(dg)[s:e], None if h0 is None else h0[i],
                               None if dh_last is None else dh_last[i])
        for k in ("dx", "ddt", "dz", "dB", "dC"):
            res[k][s:e] = r[k]
        res["dD"] += r["dD"]
        res["dA_log"] += r["dA_log"]
        res["dh0"][i] = r["dh0"]
    return res
