"""Shared helpers for the tests: error metric, workload -> device tensors, oracle runs."""
from __future__ import annotations

import numpy as np

import synth

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(got, ref) -> float:
    """Norm-wise relative error max|got - ref| / max|ref| (0 when both are all zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den


def torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def dims_of(wl: synth.Workload):
    import mamba_selective_scan_mixer_amd as jm
    d = wl.dims
    return jm.make_dims(d.d_model, d.d_inner, d.d_state, d.d_conv, d.dt_rank, torch_dtype(wl.dtype))


def device_layer(wl: synth.Workload):
    import mamba_selective_scan_mixer_amd as jm
    return jm.MambaLayer.from_arrays(dims_of(wl), wl.weights)


def to_dev(a, dtype: str):
    import torch
    return torch.as_tensor(np.ascontiguousarray(a)).to("cuda", torch_dtype(dtype)).contiguous()


def to_np(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def gpu_prefill(wl: synth.Workload, layer=None, u=None, init_conv=None, init_ssm=None):
    """Run the library's prefill on the workload; returns numpy (out, conv, ssm)."""
    import torch
    import mamba_selective_scan_mixer_amd as jm
    layer = layer or device_layer(wl)
    u_d = to_dev(wl.u if u is None else u, wl.dtype)
    cu_d = torch.as_tensor(wl.cu_seqlens, dtype=torch.int32).cuda()
    ic = None if init_conv is None else to_dev(init_conv, wl.dtype)
    isr = None if init_ssm is None else torch.as_tensor(np.asarray(init_ssm, np.float32)).cuda()
    out, conv, ssm = jm.jamba_mamba_prefill(layer, u_d, cu_d, wl.cu_seqlens, ic, isr)
    torch.cuda.synchronize()
    return to_np(out), to_np(conv), to_np(ssm)


class NormErr:
    """Running norm-wise relative error, max|got - ref| / max|ref|, of one tensor whose parts
    arrive in blocks (the same value rel_err gives on the whole tensor)."""

    def __init__(self):
        self.num = 0.0
        self.den = 0.0

    def add(self, got, ref) -> None:
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        if ref.size:
            self.num = max(self.num, float(np.max(np.abs(got - ref))))
            self.den = max(self.den, float(np.max(np.abs(ref))))

    @property
    def value(self) -> float:
        return self.num / self.den if self.den else self.num


def oracle_prefill_blocked(oracle, w64, u, cu_seqlens, block, on_block, init_conv=None,
                           init_ssm=None):
    """The oracle's prefill of packed sequences, run one sequence and at most `block` tokens at a
    time: each block starts from the conv and SSM states the previous block of its sequence left
    (splitting a sequence this way leaves the result unchanged; the CPU suite pins that split
    invariance). Keeps host memory bounded at full workload sizes. on_block(row0, out_rows) gets
    each block's output rows as they are computed; returns (conv_state, ssm_state) of every
    sequence."""
    cu = [int(v) for v in cu_seqlens]
    n = len(cu) - 1
    di = w64["D"].shape[0]
    K = w64["conv_w"].shape[1]
    N = w64["A_log"].shape[1]
    conv = np.empty((n, di, K - 1))
    ssm = np.empty((n, di, N))
    for i in range(n):
        c = None if init_conv is None else np.asarray(init_conv[i:i + 1], np.float64)
        h = None if init_ssm is None else np.asarray(init_ssm[i:i + 1], np.float64)
        for s in range(cu[i], cu[i + 1], block):
            e = min(s + block, cu[i + 1])
            r = oracle.prefill(w64, u[s:e], [0, e - s], c, h)
            on_block(s, r["out"])
            c, h = r["conv_state"], r["ssm_state"]
        conv[i], ssm[i] = c[0], h[0]
    return conv, ssm


def oracle_threads() -> int:
    """Host threads the oracle may use: the OpenMP thread count the machine was given (all
    cores when unset), at most 16."""
    import os
    n = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    return max(1, min(16, n))
