"""Full-size parity: every workload at its full size, in the launch configuration the
benchmark uses (automatic chunk plan, 64-row decode tiles), compared with the fp64 CPU
oracle on every output, with D = 1 and with the D = 0 twin:

  prefill_4k     (4096 tokens) out and both final states;
  prefill_128k   (one 131072-token sequence) every row of out and both final states of the
                 real input; the oracle runs in 8192-token blocks that carry the conv and
                 SSM states (split invariance, pinned on the CPU), so its memory stays
                 bounded; plus a constructed input - random first and last 512 tokens,
                 zeros in between - where every middle row must be exactly 0 (z = 0 so the
                 gate is 0) and the last rows and final states must match the oracle started
                 from the closed-form fixed point of the zero-input recurrence,
                 h* = Delta B x^ / (1 - exp(Delta A)); and one sequence past 2^19 tokens;
  decode_b64     2048-token prefill for 64 sequences, then 1024 decode steps: out of all 64
                 sequences at every step, both states at steps 1, 32 and 1024; the oracle
                 decodes from its own prefill states;
  packed_varlen  16 sequences of 1024..8192 tokens: out of every sequence, all 16 final
                 conv and SSM states.
Errors are norm-wise per tensor (max|gpu - ref| / max|ref|), bound 2e-2 (bf16 activations,
fp32 state).
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import synth
from jm_testutil import (TOL, NormErr, device_layer, oracle_prefill_blocked, oracle_threads,
                         rel_err, to_dev, to_np)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
jm = pytest.importorskip("mamba_selective_scan_mixer_amd")

ORACLE_BLOCK = 8192


@pytest.fixture(autouse=True)
def _auto_chunk():
    jm.set_scan_chunk_len(0)
    yield


def run_prefill(layer, u_np, cu, dtype="bf16"):
    u = to_dev(u_np, dtype)
    cu_d = torch.as_tensor(np.asarray(cu, np.int32)).cuda()
    out, conv, ssm = jm.jamba_mamba_prefill(layer, u, cu_d, [int(v) for v in cu])
    torch.cuda.synchronize()
    del u
    return out, conv, ssm


def report(label, **errs):
    print(label + " " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)


def compare_prefill(wl, out, conv, ssm, label):
    """Every output row and both final states of a prefill against the block-streamed oracle."""
    w64 = oracle.as_f64(wl.weights)
    e_out = NormErr()

    def check_block(r0, ref_rows):
        e_out.add(to_np(out[r0:r0 + len(ref_rows)]), ref_rows)

    conv_r, ssm_r = oracle_prefill_blocked(oracle, w64, wl.u, wl.cu_seqlens, ORACLE_BLOCK,
                                           check_block)
    e = dict(out=e_out.value, conv=rel_err(to_np(conv), conv_r), ssm=rel_err(to_np(ssm), ssm_r))
    report(label, **e)
    assert max(e.values()) < TOL["bf16"], e


@pytest.mark.parametrize("D_value", [1.0, 0.0])
def test_prefill_4k_full(D_value):
    wl = synth.make_workload("prefill_4k", D_value=D_value)
    out, conv, ssm = run_prefill(device_layer(wl), wl.u, wl.cu_seqlens)
    compare_prefill(wl, out, conv, ssm, f"prefill_4k D={D_value}")


@pytest.mark.parametrize("D_value", [1.0, 0.0])
def test_prefill_128k_full(D_value):
    wl = synth.make_workload("prefill_128k", D_value=D_value)
    out, conv, ssm = run_prefill(device_layer(wl), wl.u, wl.cu_seqlens)
    compare_prefill(wl, out, conv, ssm, f"prefill_128k all 131072 rows D={D_value}")


def zero_input_fixed_point(w64):
    """Closed-form limit of the SSM state under a long run of zero input tokens."""
    di = w64["D"].shape[0]
    N = w64["A_log"].shape[1]
    R = w64["dt_proj_w"].shape[1]
    x_hat0, _ = oracle.causal_conv_silu(np.zeros((1, di)), w64["conv_w"], w64["conv_b"], None)
    delta0, B0, _ = oracle.x_proj(x_hat0, w64["x_proj_w"], R, N)
    dt0 = oracle.dt_proj(delta0, w64["dt_proj_w"], w64["dt_proj_b"])[0]       # (di,)
    a = np.exp(dt0[:, None] * (-np.exp(w64["A_log"])))                       # (di, N)
    b = dt0[:, None] * B0[0][None, :] * x_hat0[0][:, None]
    return b / (1.0 - a), a


@pytest.mark.parametrize("D_value", [1.0, 0.0])
def test_prefill_128k_constructed_input(D_value):
    wl = synth.make_workload("prefill_128k", D_value=D_value)
    T = wl.total_tokens
    P = 512
    u = wl.u.copy()
    u[P:T - P] = 0.0
    layer = device_layer(wl)
    out, conv, ssm = run_prefill(layer, u, wl.cu_seqlens)
    w64 = oracle.as_f64(wl.weights)
    # (a) head rows
    ref_head = oracle.prefill(w64, u[:P], [0, P])
    e_head = rel_err(to_np(out[:P]), ref_head["out"])
    # (b) the zero stretch gives exactly zero output rows
    mid = out[P:T - P]
    n_nonzero = int(torch.count_nonzero(mid).item())
    # (c) tail rows and final states from the fixed point
    h_star, a = zero_input_fixed_point(w64)
    assert np.max(a) ** (T - 2 * P) < 1e-40      # the head is forgotten
    di = w64["D"].shape[0]
    ref_tail = oracle.prefill(w64, u[T - P:], [0, P], init_conv=np.zeros((1, di, 3)),
                              init_ssm=h_star[None])
    e = dict(head=e_head, tail=rel_err(to_np(out[T - P:]), ref_tail["out"]),
             conv=rel_err(to_np(conv), ref_tail["conv_state"]),
             ssm=rel_err(to_np(ssm), ref_tail["ssm_state"]))
    report(f"prefill_128k constructed D={D_value} nonzero_mid={n_nonzero}", **e)
    assert n_nonzero == 0
    assert max(e.values()) < TOL["bf16"], e


def test_prefill_past_32bit_offsets():
    """One sequence of 2^19 + 300 tokens: every activation buffer passes 2^32 bytes (x, z,
    x_hat and g are 8.6 GB each, Delta 17 GB) and token x channel indexes pass 2^31, so a
    32-bit byte offset or element index anywhere on the path would show. The input is built
    as in the 128K constructed case: random head and tail of 512 tokens around zeros, checked
    against the oracle at both ends and for exact zeros between."""
    P = 512
    base = synth.make_workload("prefill_4k", D_value=1.0, lengths=[2 * P])
    T = (1 << 19) + 300
    layer = device_layer(base)
    u = torch.zeros((T, base.dims.d_model), dtype=torch.bfloat16, device="cuda")
    u[:P] = to_dev(base.u[:P], "bf16")
    u[T - P:] = to_dev(base.u[P:], "bf16")
    cu_d = torch.as_tensor(np.asarray([0, T], np.int32)).cuda()
    out, conv, ssm = jm.jamba_mamba_prefill(layer, u, cu_d, [0, T])
    torch.cuda.synchronize()
    del u
    n_nonzero = int(torch.count_nonzero(out[P:T - P]).item())
    w64 = oracle.as_f64(base.weights)
    ref_head = oracle.prefill(w64, base.u[:P], [0, P])
    h_star, a = zero_input_fixed_point(w64)
    assert np.max(a) ** (T - 2 * P) < 1e-40
    di = w64["D"].shape[0]
    ref_tail = oracle.prefill(w64, base.u[P:], [0, P], init_conv=np.zeros((1, di, 3)),
                              init_ssm=h_star[None])
    e = dict(head=rel_err(to_np(out[:P]), ref_head["out"]),
             tail=rel_err(to_np(out[T - P:]), ref_tail["out"]),
             conv=rel_err(to_np(conv), ref_tail["conv_state"]),
             ssm=rel_err(to_np(ssm), ref_tail["ssm_state"]))
    report(f"prefill {T} tokens constructed nonzero_mid={n_nonzero}", **e)
    assert n_nonzero == 0
    assert max(e.values()) < TOL["bf16"], e


@pytest.fixture(scope="module")
def decode_prefill_states():
    """The oracle's states after the decode workload's 2048-token prefill of each of the 64
    sequences. D enters only y, never the states, so one oracle run serves both twins."""
    wl = synth.make_workload("decode_b64", D_value=1.0, steps=0)
    w64 = oracle.as_f64(wl.weights)
    conv, ssm = oracle_prefill_blocked(oracle, w64, wl.u, wl.cu_seqlens, ORACLE_BLOCK,
                                       lambda r0, rows: None)
    return conv, ssm


@pytest.mark.parametrize("D_value", [0.0, 1.0])
def test_decode_b64_full(decode_prefill_states, D_value):
    import threadpoolctl
    steps = 1024
    wl = synth.make_workload("decode_b64", D_value=D_value, steps=steps)
    B = wl.n_seqs
    layer = device_layer(wl)
    _, conv, ssm = run_prefill(layer, wl.u, wl.cu_seqlens)
    conv_r, ssm_r = decode_prefill_states
    e_c, e_s = rel_err(to_np(conv), conv_r), rel_err(to_np(ssm), ssm_r)
    report(f"decode_b64 D={D_value} after prefill", conv=e_c, ssm=e_s)
    assert e_c < TOL["bf16"] and e_s < TOL["bf16"], (e_c, e_s)
    w64 = oracle.as_f64(wl.weights)
    out = torch.empty((B, wl.dims.d_model), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(jm.decode_workspace_size(layer.dims, B), dtype=torch.uint8, device="cuda")
    # the oracle's step runs on sub-batches in threads (its sequences are independent), two
    # BLAS threads each, while the GPU computes the same step
    n_par = max(1, oracle_threads() // 2)
    parts = [(i * B // n_par, (i + 1) * B // n_par) for i in range(n_par)]
    worst = {"out": 0.0, "conv": 0.0, "ssm": 0.0}
    with ThreadPoolExecutor(n_par) as pool, threadpoolctl.threadpool_limits(2, "blas"):
        for s in range(1, steps + 1):
            tok = wl.next_decode_tokens()
            jm.jamba_mamba_decode_step(layer, to_dev(tok, "bf16"), conv, ssm, out=out,
                                       workspace=ws)
            res = list(pool.map(lambda p: oracle.decode_step(w64, tok[p[0]:p[1]],
                                                             conv_r[p[0]:p[1]],
                                                             ssm_r[p[0]:p[1]]), parts))
            out_r = np.concatenate([r[0] for r in res])
            conv_r = np.concatenate([r[1] for r in res])
            ssm_r = np.concatenate([r[2] for r in res])
            e_out = rel_err(to_np(out), out_r)
            worst["out"] = max(worst["out"], e_out)
            assert e_out < TOL["bf16"], (s, e_out)
            if s % 256 == 0:
                print(f"decode_b64 D={D_value}: step {s}/{steps} worst out so far "
                      f"{worst['out']:.2e}", flush=True)
            if s in (1, 32, steps):
                e_c = rel_err(to_np(conv), conv_r)
                e_s = rel_err(to_np(ssm), ssm_r)
                worst["conv"] = max(worst["conv"], e_c)
                worst["ssm"] = max(worst["ssm"], e_s)
                report(f"decode_b64 D={D_value} step {s}", out=e_out, conv=e_c, ssm=e_s)
                assert e_c < TOL["bf16"] and e_s < TOL["bf16"], (s, e_c, e_s)
    report(f"decode_b64 D={D_value} worst over {steps} steps, all {B} sequences", **worst)


@pytest.mark.parametrize("D_value", [1.0, 0.0])
def test_packed_varlen_full(D_value):
    wl = synth.make_workload("packed_varlen", D_value=D_value)
    out, conv, ssm = run_prefill(device_layer(wl), wl.u, wl.cu_seqlens)
    compare_prefill(wl, out, conv, ssm,
                    f"packed_varlen all {wl.n_seqs} sequences D={D_value} lengths={wl.lengths}")
