"""CPU oracle (fp64) for the Mamba selective-state-space mixer layer.

TEST INFRASTRUCTURE ONLY -- imported by tests, the smoke check and the benchmark's
CPU-baseline leg; never by the HIP library. Parity of functions here is pinned by
the `-m "not gpu"` tests in tests/test_oracle_pins.py (brute force, closed forms,
scipy special case, invariants); every function below has at least one pin.

The layer is the Mamba block the Jamba paper interleaves with attention (Jamba: A
Hybrid Transformer-Mamba Language Model, §2 "Model architecture": Mamba layer from
citation [17], no explicit positional information (§6.5), a fixed-size summary
state per sequence instead of a KV cache (A1 and §2 on the KV cache)). The pages
give no equations for it; the steps below are the standard selective-SSM block
with these readings (each listed in the design notes):
  * in_proj output rows: x first (d_inner rows), then z;
  * causal depthwise conv1d over the *pre-conv* x with kernel d_conv, tap d_conv-1
    on the current token, bias added, history per sequence = caller's initial
    conv state (oldest first) or zeros, then SiLU;
  * x_proj output rows: delta (dt_rank), then B (d_state), then C (d_state);
  * dt = softplus(dt_proj(delta) + dt_bias);
  * A = -exp(A_log); h_t = exp(dt*A) h_{t-1} + dt*B_t*x_t; y_t = C_t.h_t + D*x_t;
  * gate: g = y * SiLU(z); out = out_proj(g); no bias on in/x/out projections;
  * inner normalisation (optional): the paper applies RMSNorm inside the Mamba layer
    (§2, the paragraph on the Mamba layer's implementation; §6.4 and Fig. 9: added to
    internal activations after loss spikes at scale) without saying where. When the
    layer has norm gains, delta, B and C are each RMS-normalised over their own
    feature axis right after x_proj; without gains the step is absent.
All arithmetic is fp64 from the exact values of the (bf16 or fp32) inputs, with no
intermediate rounding. Matrix products use numpy's matmul (a library primitive);
the recurrence is a plain sequential C loop (scan_ref.c).
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libjm_oracle.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        f = lib.jm_oracle_scan
        f.restype = None
        f.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 9
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


NORM_KEYS = ("dt_norm_w", "B_norm_w", "C_norm_w")
DEFAULT_NORM_EPS = 1e-6


def as_f64(weights: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """fp64 copies of the layer parameters (exact: inputs are fp32 or bf16 values)."""
    keys = ("in_proj_w", "conv_w", "conv_b", "x_proj_w", "dt_proj_w", "dt_proj_b",
            "A_log", "D", "out_proj_w")
    w = {k: _f64(weights[k]) for k in keys}
    if weights.get("dt_norm_w") is not None:
        for k in NORM_KEYS:
            w[k] = _f64(weights[k])
        w["norm_eps"] = float(weights.get("norm_eps", DEFAULT_NORM_EPS))
    return w


def rmsnorm(v, gain, eps):
    """Root-mean-square normalisation of each row (the paper's citation [53], Root mean
    square layer normalization): v / sqrt(mean(v^2) + eps) * gain, over the last axis."""
    v = _f64(v)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps) * _f64(gain)


def inner_norm(w, delta, B, C):
    """The layer's inner RMSNorm when it has gains (else the identity): delta, B and C
    each normalised over its own feature axis, right after x_proj."""
    if w.get("dt_norm_w") is None:
        return delta, B, C
    eps = w.get("norm_eps", DEFAULT_NORM_EPS)
    return (rmsnorm(delta, w["dt_norm_w"], eps), rmsnorm(B, w["B_norm_w"], eps),
            rmsnorm(C, w["C_norm_w"], eps))


def silu(v):
    """SiLU(v) = v * sigmoid(v) = v / (1 + e^-v)."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def softplus(v):
    """softplus(v) = ln(1 + e^v), in the overflow-free form max(v,0) + ln(1 + e^-|v|)."""
    v = np.asarray(v, dtype=np.float64)
    return np.maximum(v, 0.0) + np.log1p(np.exp(-np.abs(v)))


def in_proj(u, in_proj_w, d_inner: int):
    """[x ; z] = W_in u_t for every token; returns (x, z), each (T, d_inner)."""
    xz = _f64(u) @ _f64(in_proj_w).T
    return xz[:, :d_inner], xz[:, d_inner:]


def causal_conv_silu(x, conv_w, conv_b, history=None):
    """Causal depthwise conv1d + bias + SiLU over one sequence.

    x: (T, d_inner) pre-conv values of one sequence. conv_w: (d_inner, K);
    tap K-1 multiplies the current token, tap k the token K-1-k steps back.
    history: (d_inner, K-1) values before the first token, oldest first, or None
    (zeros). Returns (x_hat (T, d_inner), new_history (d_inner, K-1)), where the new
    history is the last K-1 pre-conv values (again oldest first).
    """
    x = _f64(x)
    w = _f64(conv_w)
    T, di = x.shape
    K = w.shape[1]
    hist = np.zeros((K - 1, di)) if history is None else _f64(history).T
    # padded row j holds the value at time j - (K-1)
    padded = np.concatenate([hist, x], axis=0)
    c = np.broadcast_to(_f64(conv_b)[None, :], (T, di)).copy()
    for k in range(K):
        c += w[:, k][None, :] * padded[k:k + T]
    new_hist = padded[T:T + K - 1].T.copy()
    return silu(c), new_hist


def x_proj(x_hat, x_proj_w, dt_rank: int, d_state: int):
    """[delta ; B ; C] = W_x x_hat_t; returns (delta (T,R), B (T,N), C (T,N))."""
    dbc = _f64(x_hat) @ _f64(x_proj_w).T
    return dbc[:, :dt_rank], dbc[:, dt_rank:dt_rank + d_state], dbc[:, dt_rank + d_state:]


def dt_proj(delta, dt_proj_w, dt_proj_b):
    """Delta_t = softplus(W_dt delta_t + b_dt), (T, d_inner)."""
    return softplus(_f64(delta) @ _f64(dt_proj_w).T + _f64(dt_proj_b)[None, :])


def selective_scan(x, dt, A, B, C, D, h0=None):
    """Sequential recurrence h_t = exp(dt A) h_{t-1} + dt B_t x_t, y_t = C_t.h_t + D x_t.

    x, dt: (T, d_inner); A: (d_inner, N) (the negative matrix, not A_log);
    B, C: (T, N); D: (d_inner,); h0: (d_inner, N) or None. Returns (y, h_last).
    """
    x, dt, A, B, C, D = (_f64(v) for v in (x, dt, A, B, C, D))
    T, di = x.shape
    N = A.shape[1]
    h0 = None if h0 is None else _f64(h0)
    y = np.empty((T, di))
    h_last = np.empty((di, N))
    lib = _load()
    p = lambda a: None if a is None else a.ctypes.data  # noqa: E731
    lib.jm_oracle_scan(T, di, N, p(x), p(dt), p(A), p(B), p(C), p(D), p(h0), p(y), p(h_last))
    return y, h_last


def gate(y, z):
    """g = y * SiLU(z)."""
    return _f64(y) * silu(z)


def out_proj(g, out_proj_w):
    """out_t = W_out g_t."""
    return _f64(g) @ _f64(out_proj_w).T


def _layer_one_sequence(w, u, conv_hist, h0, keep):
    di = w["D"].shape[0]
    N = w["A_log"].shape[1]
    R = w["dt_proj_w"].shape[1]
    x, z = in_proj(u, w["in_proj_w"], di)
    x_hat, conv_new = causal_conv_silu(x, w["conv_w"], w["conv_b"], conv_hist)
    delta_raw, B_raw, C_raw = x_proj(x_hat, w["x_proj_w"], R, N)
    delta, B, C = inner_norm(w, delta_raw, B_raw, C_raw)
    dt = dt_proj(delta, w["dt_proj_w"], w["dt_proj_b"])
    A = -np.exp(w["A_log"])
    y, h_last = selective_scan(x_hat, dt, A, B, C, w["D"], h0)
    g = gate(y, z)
    out = out_proj(g, w["out_proj_w"])
    stages = None
    if keep:
        stages = dict(x=x, z=z, x_hat=x_hat, delta_raw=delta_raw, B_raw=B_raw, C_raw=C_raw,
                      delta=delta, B=B, C=C, dt=dt, y=y, g=g)
    return out, conv_new, h_last, stages


def prefill(weights, u, cu_seqlens, init_conv=None, init_ssm=None, intermediates=False):
    """Mamba layer over packed sequences: sequence i is rows cu[i]..cu[i+1]-1 of u.

    Every sequence starts from its own initial state (init_conv[i]: (d_inner, K-1),
    init_ssm[i]: (d_inner, N)) or from zeros, and is computed on its own.
    Returns dict(out (T, d_model), conv_state (n, d_inner, K-1), ssm_state
    (n, d_inner, N)[, stages: per-sequence list of intermediates]).
    """
    w = weights if weights["D"].dtype == np.float64 else as_f64(weights)
    u = _f64(u)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    n = len(cu) - 1
    di = w["D"].shape[0]
    N = w["A_log"].shape[1]
    K = w["conv_w"].shape[1]
    out = np.empty((u.shape[0], w["out_proj_w"].shape[0]))
    conv_state = np.empty((n, di, K - 1))
    ssm_state = np.empty((n, di, N))
    stages = []
    for i in range(n):
        s, e = int(cu[i]), int(cu[i + 1])
        ch = None if init_conv is None else init_conv[i]
        h0 = None if init_ssm is None else init_ssm[i]
        o, cs, hs, st = _layer_one_sequence(w, u[s:e], ch, h0, intermediates)
        out[s:e] = o
        conv_state[i] = cs
        ssm_state[i] = hs
        stages.append(st)
    res = dict(out=out, conv_state=conv_state, ssm_state=ssm_state)
    if intermediates:
        res["stages"] = stages
    return res


def decode_step(weights, u, conv_state, ssm_state):
    """One token per sequence, written on its own (not via prefill).

    u: (batch, d_model); conv_state: (batch, d_inner, K-1) pre-conv history, oldest
    first; ssm_state: (batch, d_inner, N). Returns (out (batch, d_model),
    new_conv_state, new_ssm_state); the inputs are not modified.
    """
    w = weights if weights["D"].dtype == np.float64 else as_f64(weights)
    u = _f64(u)
    di = w["D"].shape[0]
    N = w["A_log"].shape[1]
    R = w["dt_proj_w"].shape[1]
    xz = u @ w["in_proj_w"].T                       # (b, 2 di)
    x, z = xz[:, :di], xz[:, di:]
    window = np.concatenate([_f64(conv_state), x[:, :, None]], axis=2)   # (b, di, K)
    conv = w["conv_b"][None, :] + np.sum(window * w["conv_w"][None, :, :], axis=2)
    x_hat = conv / (1.0 + np.exp(-conv))
    dbc = x_hat @ w["x_proj_w"].T
    delta, Bm, Cm = dbc[:, :R], dbc[:, R:R + N], dbc[:, R + N:]
    if w.get("dt_norm_w") is not None:      # inner RMSNorm of delta, B and C
        e = w.get("norm_eps", DEFAULT_NORM_EPS)
        delta = delta * w["dt_norm_w"][None, :] / np.sqrt((delta ** 2).mean(axis=1)[:, None] + e)
        Bm = Bm * w["B_norm_w"][None, :] / np.sqrt((Bm ** 2).mean(axis=1)[:, None] + e)
        Cm = Cm * w["C_norm_w"][None, :] / np.sqrt((Cm ** 2).mean(axis=1)[:, None] + e)
    pre = delta @ w["dt_proj_w"].T + w["dt_proj_b"][None, :]
    dt = np.maximum(pre, 0.0) + np.log1p(np.exp(-np.abs(pre)))
    A = -np.exp(w["A_log"])                         # (di, N)
    h = np.exp(dt[:, :, None] * A[None]) * _f64(ssm_state) \
        + dt[:, :, None] * Bm[:, None, :] * x_hat[:, :, None]
    y = np.einsum("bdn,bn->bd", h, Cm) + w["D"][None, :] * x_hat
    with np.errstate(over="ignore"):
        g = y * (z / (1.0 + np.exp(-z)))
    out = g @ w["out_proj_w"].T
    return out, window[:, :, 1:].copy(), h
