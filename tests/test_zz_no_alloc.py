"""The decode step without a workspace (jamba_mamba_decode_step_noalloc: the library's fixed
per-GPU scratch array instead of a caller workspace) against jamba_mamba_decode_step with a
caller workspace. Both run the same kernels on the same inputs, so out and the updated states
must agree bit for bit (stricter than the 2e-2 / 1e-4 layer bounds). Two calls in a row, the
second with a smaller batch, so the second runs over scratch the first left filled; on the
fast bf16 path (two 64-row tiles, then one) and on the generic fp32 path."""
import numpy as np
import pytest

import synth
from jm_testutil import device_layer, gpu_prefill, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
jm = pytest.importorskip("mamba_selective_scan_mixer_amd")


@pytest.mark.parametrize("name,dims,dtype,batches", [
    ("jamba_bf16", None, "bf16", (70, 9)),
    ("tiny_fp32", synth.TINY_DIMS, "f32", (6, 2)),
])
def test_noalloc_decode_equals_workspace_decode(name, dims, dtype, batches):
    kw = {} if dims is None else dict(dims=dims, dtype=dtype)
    wl = synth.make_workload("decode_b64", batch=batches[0], prefill_len=5, steps=len(batches),
                             D_value=0.0, **kw)
    layer = device_layer(wl)
    _, conv0, ssm0 = gpu_prefill(wl, layer)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for call, b in enumerate(batches):
        tok = to_dev(wl.next_decode_tokens()[:b], dtype)
        conv_a = to_dev(conv0[:b], dtype)
        ssm_a = torch.as_tensor(ssm0[:b].astype(np.float32)).cuda()
        conv_b, ssm_b = conv_a.clone(), ssm_a.clone()
        out_a = jm.jamba_mamba_decode_step(layer, tok, conv_a, ssm_a)
        out_b = torch.full((b, wl.dims.d_model), float("nan"), dtype=tdt, device="cuda")
        jm.jamba_mamba_decode_step_noalloc(layer, tok, conv_b, ssm_b, out_b)
        torch.cuda.synchronize()
        print(f"noalloc {name} call {call} batch {b}: max |out diff| "
              f"{float((out_a.float() - out_b.float()).abs().max()):.3e}", flush=True)
        assert torch.equal(out_a, out_b), (name, call, b)
        assert torch.equal(conv_a, conv_b), (name, call, b)
        assert torch.equal(ssm_a, ssm_b), (name, call, b)
        conv0 = conv0.copy()
        ssm0 = ssm0.copy()
        conv0[:b] = conv_a.float().cpu().numpy()
        ssm0[:b] = ssm_a.cpu().numpy()
