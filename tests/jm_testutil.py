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
