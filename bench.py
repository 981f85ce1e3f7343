"""Benchmark: Mamba mixer layer prefill at 128K tokens (and decode at batch 64) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode] [--no-cpu]

One step = one jamba_mamba_prefill call over a single 131072-token sequence at the
Jamba-7B-class layer sizes (d_model 4096, d_inner 8192, d_state 16, d_conv 4,
dt_rank 256), bf16 activations and weights, fp32 state, inputs resident in HBM.
Prints ONE JSON line: value = prefill tokens/s of the layer; per-kernel durations
come from HIP events the library records around each kernel on the call's stream
during the timed steps. The decode figure (64 sequences, one token per step,
carried state from a 2048-token prefill each) is reported alongside. The CPU
oracle is timed on a bounded sample of the same workload as a reported baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
# fp32 VALU issue rate without packed math: 256 CU x 4 SIMD x 16 lanes x 2.4 GHz
VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9
# issue slots per SSM state update when no counter record applies (a model: mul, exp2, mul, fma,
# + fma for y; the exp counted as two slots)
SCAN_SLOTS = {"scan_chunk_state": 5.0, "scan_chunk_output": 6.0}
METRIC = "Mamba-layer prefill tok/s @128K, decode tok/s @B=64; % HBM/MFMA peak"


def kernel_work(T: int, dm: int, di: int, R: int, N: int = 16):
    """Algorithmic FLOPs and HBM bytes per launch for T tokens (bf16 activations,
    fp32 Delta/B/C/state): what each kernel must read and write, counted once."""
    a = 2  # bf16 bytes
    w = {
        "in_proj": (2.0 * T * 2 * di * dm, T * dm * a + 2 * di * dm * a + T * 2 * di * a),
        "conv1d_silu": (8.0 * T * di, T * di * a * 2 + di * 5 * a),
        "conv_final": (0.0, 3 * di * a * 2),
        "x_proj": (2.0 * T * (R + 2 * N) * di, T * di * a + (R + 2 * N) * di * a + T * (R * a + 2 * N * 4)),
        "dt_proj": (2.0 * T * di * R, T * R * a + di * R * a + di * 4 + T * di * 4),
        "scan_chunk_state": (0.0, T * di * (4 + a) + T * N * 4),
        "scan_chunk_carry": (0.0, 0.0),   # filled in by the caller (depends on the chunk count)
        "scan_chunk_output": (0.0, T * di * (4 + a + a + a) + T * 2 * N * 4 + di * N * 4),
        "out_proj": (2.0 * T * dm * di, T * di * a + dm * di * a + T * dm * a),
    }
    return w


def bound_of(name: str) -> str:
    if name in ("in_proj", "out_proj"):
        return "mfma"
    return "alu" if name in SCAN_SLOTS else "hbm"


def recorded_traffic(kernel: str):
    """HBM-side bytes per launch of `kernel` from the committed rocprofv3 counter summary,
    or None when the GEMM sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "prefill_128k_hbm_traffic.md")
    srcs = [os.path.join(ROOT, "mamba_selective_scan_mixer_amd", "csrc", f)
            for f in ("jm_gemm.hip", "jm_internal.h")]
    try:
        rec = None
        for line in open(path):
            if line.startswith("traffic-record:"):
                kv = dict(t.split("=", 1) for t in line.split()[1:])
                if kv.get("kernel") == kernel:
                    rec = kv
        if rec is None:
            return None
        h = hashlib.sha256(b"".join(open(f, "rb").read() for f in srcs)).hexdigest()[:16]
        if h != rec["source_sha256"]:
            return None
        return (float(rec["fetch_kib"]) * float(rec["fetch_factor"])
                + float(rec["write_kib"]) * float(rec["write_factor"])) * 1024.0
    except OSError:
        return None


def recorded_valu(kernel: str, profile: str = "prefill_128k_mfma_valu_counters.md",
                  sources=("jm_scan.hip", "jm_internal.h")):
    """Measured wave-level VALU instructions per lane state update of a scan kernel, from a
    committed rocprofv3 counter summary (SQ_INSTS_VALU x 64 / updates), or None when the
    kernel's sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    srcs = [os.path.join(ROOT, "mamba_selective_scan_mixer_amd", "csrc", f) for f in sources]
    try:
        rec = None
        for line in open(path):
            if line.startswith("valu-record:"):
                kv = dict(t.split("=", 1) for t in line.split()[1:])
                if kv.get("kernel") == kernel:
                    rec = kv
        if rec is None:
            return None
        h = hashlib.sha256(b"".join(open(f, "rb").read() for f in srcs)).hexdigest()[:16]
        if h != rec["source_sha256"]:
            return None
        return float(rec["valu_insts_per_update"])
    except OSError:
        return None


def make_inputs(seed: int = 0):
    import synth
    wl = synth.make_workload("prefill_128k", seed=seed)
    return wl


def cpu_baseline(wl, target_s: float = 15.0):
    """Time the fp64 oracle on the first tokens of the same sequence (bounded sample)."""
    import oracle
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        blas_threads = max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:
        blas_threads = os.cpu_count() or 1
    omp = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    w64 = oracle.as_f64(wl.weights)
    # calibrate on a small sample, then size the timed sample for ~target_s (at most 48K
    # tokens: the fp64 intermediates take ~0.5 MB per token)
    n0 = 512
    t = time.perf_counter()
    oracle.prefill(w64, wl.u[:n0], [0, n0])
    dt0 = time.perf_counter() - t
    n = int(min(49152, max(n0, n0 * target_s / max(dt0, 1e-3))))
    t = time.perf_counter()
    oracle.prefill(w64, wl.u[:n], [0, n])
    el = time.perf_counter() - t
    return {"value": n / el, "unit": "tokens/s", "cores": int(max(blas_threads, omp)),
            "kind": "oracle", "cpu_model": cpu_model(), "cpu_count": os.cpu_count(),
            "sample": f"first {n} tokens of the 131072-token sequence, fp64 oracle (numpy matmul "
                      f"+ C recurrence), {el:.1f} s wall; BLAS threads {blas_threads}, OpenMP {omp}"}


def cpu_model() -> str:
    """The host CPU's model name (what lscpu reports), from /proc/cpuinfo."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the scan-backward measurement")
    ap.add_argument("--no-inner-norm", action="store_true",
                    help="skip the prefill measurement with the inner RMSNorm on")
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the timed prefill (profiling runs of the other legs; the line's "
                         "value is then null)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB device copy first (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this layer's path has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import mamba_selective_scan_mixer_amd as jm

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    t_gen = time.perf_counter()
    wl = make_inputs()
    d = wl.dims
    T = wl.total_tokens
    dims = jm.make_dims(d.d_model, d.d_inner, d.d_state, d.d_conv, d.dt_rank, torch.bfloat16)
    layer = jm.MambaLayer.from_arrays(dims, wl.weights)
    u = torch.as_tensor(wl.u).to(dev, torch.bfloat16)
    cu = torch.as_tensor(wl.cu_seqlens, dtype=torch.int32).to(dev)
    out = torch.empty((T, d.d_model), dtype=torch.bfloat16, device=dev)
    fconv = torch.empty((1, d.d_inner, 3), dtype=torch.bfloat16, device=dev)
    fssm = torch.empty((1, d.d_inner, 16), dtype=torch.float32, device=dev)
    ws = torch.empty(jm.prefill_workspace_size(dims, 1, T), dtype=torch.uint8, device=dev)
    print(f"[bench] inputs ready in {time.perf_counter() - t_gen:.1f} s; workspace "
          f"{ws.numel() / 2**30:.2f} GiB", file=sys.stderr, flush=True)

    if args.copy_calibration:
        a = torch.ones(2**30, dtype=torch.uint8, device=dev)   # written first, so the copy reads HBM
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    value = ms_per_step = roof = None
    kernels = {}
    cl, nc, _ = jm.prefill_plan(dims, wl.cu_seqlens)
    if not args.no_prefill:
        def step():
            jm.jamba_mamba_prefill(layer, u, cu, wl.cu_seqlens, out=out, final_conv_state=fconv,
                                   final_ssm_state=fssm, workspace=ws)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        jm.profile_reset()
        jm.profile_enable(True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        jm.profile_enable(False)
        prof = jm.profile_read()
        jm.profile_reset()
        ms_per_step = elapsed * 1e3 / args.steps
        value = T * args.steps / elapsed
        print(f"[bench] prefill {ms_per_step:.2f} ms/step, {value / 1e6:.3f} M tok/s", file=sys.stderr,
              flush=True)

        work = kernel_work(T, d.d_model, d.d_inner, d.dt_rank)
        work["scan_chunk_carry"] = (0.0, 3.0 * nc * d.d_inner * 16 * 4)
        for name, (launches, total_ms) in prof.items():
            avg = total_ms / max(launches, 1)
            flops, nbytes = work.get(name, (0.0, 0.0))
            k = {"launches": launches, "avg_ms": round(avg, 4),
                 "gbs": round(nbytes / (avg * 1e-3) / 1e9, 1) if nbytes else None,
                 "tflops": round(flops / (avg * 1e-3) / 1e12, 1) if flops else None}
            b = bound_of(name)
            k["bound"] = b
            if name in SCAN_SLOTS:
                updates = float(T) * d.d_inner * 16
                if name == "scan_chunk_state":
                    updates *= (nc - 1) / nc      # the last chunk needs no aggregate
                per = recorded_valu(name)
                k["alu_basis"] = ("measured VALU instructions per update (rocprofv3 SQ_INSTS_VALU, "
                                  "profiles/prefill_128k_mfma_valu_counters.md)" if per is not None
                                  else "slot model")
                per = SCAN_SLOTS[name] if per is None else per
                k["valu_per_update"] = per
                k["alu_frac"] = round(updates * per / VALU_LANE_OPS / (avg * 1e-3), 4)
            if b == "mfma":
                k["frac"] = round(k["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)
            elif b == "alu":
                k["frac"] = k["alu_frac"]
            elif k["gbs"] is not None:
                k["frac"] = round(k["gbs"] / HBM_PEAK_GBS, 4)
            kernels[name] = k
        dom = max(kernels, key=lambda n: kernels[n]["avg_ms"]) if kernels else None
        if dom:
            kd = kernels[dom]
            if kd["bound"] == "mfma":
                roof = {"kernel": dom, "bound": "mfma", "achieved": kd["tflops"],
                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": kd["frac"],
                        "traffic": recorded_traffic(dom),
                        "traffic_note": "HBM-side bytes per launch = 2 x FETCH_SIZE + WRITE_SIZE "
                                        "(calibrated on a 1 GiB copy); algorithmic bytes "
                                        f"{kernel_work(T, d.d_model, d.d_inner, d.dt_rank)[dom][1]:.4g}"}
            elif kd["bound"] == "alu":
                roof = {"kernel": dom, "bound": "alu", "achieved": kd["alu_frac"] * VALU_LANE_OPS / 1e12,
                        "peak": VALU_LANE_OPS / 1e12, "unit": "T VALU lane-slots/s",
                        "frac": kd["alu_frac"], "traffic": None}
            else:
                roof = {"kernel": dom, "bound": "hbm", "achieved": kd["gbs"], "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": kd["frac"], "traffic": None}

    inner = None
    if not args.no_inner_norm and not args.no_prefill:
        inner = run_inner_norm(jm, torch, wl, dims, u, cu, out, fconv, fssm, ws, T)
        print(f"[bench] prefill with inner norm {inner['ms_per_step']:.2f} ms/step "
              f"(norm kernel {inner['norm_kernel']['avg_ms']:.3f} ms)", file=sys.stderr, flush=True)

    backward = None
    if not args.no_backward:
        backward = run_scan_backward(jm, torch, wl, layer, dims, u, cu, T)
        print(f"[bench] scan backward {backward['ms_per_call']:.2f} ms/call "
              f"({backward['tokens_per_s'] / 1e6:.3f} M tok/s)", file=sys.stderr, flush=True)

    decode = None
    if not args.no_decode:
        decode = run_decode(jm, torch, dev, layer, dims, wl, args.decode_steps)
        print(f"[bench] decode {decode['us_per_step']:.1f} us/step, "
              f"{decode['tokens_per_s'] / 1e6:.3f} M tok/s (cold {decode['us_per_step_cold']:.1f}; "
              f"tiled weights {decode['us_per_step_tiled']:.1f}, cold "
              f"{decode['us_per_step_cold_tiled']:.1f})", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl)
        print(f"[bench] cpu oracle {cpu['value']:.1f} tok/s ({cpu['sample']})", file=sys.stderr,
              flush=True)

    rec = {
        "metric": METRIC, "value": None if value is None else round(value, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": None if ms_per_step is None else round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill_128k: one 131072-token sequence, Mamba layer d_model 4096, "
                               "d_inner 8192, d_state 16, d_conv 4, dt_rank 256; bf16, fp32 state",
                   "global_batch": 1, "seq_len": T, "scan_chunk_len": cl, "scan_chunks": nc,
                   "parallelism": "none (one GPU)"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "decode": decode,
        "inner_norm": inner,
        "scan_backward": backward,
        "kernels": kernels,
    }
    print(json.dumps(rec), flush=True)


def run_scan_backward(jm, torch, wl, layer, dims, u, cu, T, steps: int = 3):
    """Backward of the scan step (training) over the same 131072-token sequence: inputs from
    the stage entry points on the benchmark's tokens, a seeded N(0,1) upstream gradient dg."""
    x, z = jm.jm_stage_in_proj(layer, u)
    xh, _ = jm.jm_stage_conv(layer, x, cu, wl.cu_seqlens, want_final_state=False)
    del x
    delta, B, C = jm.jm_stage_x_proj(layer, xh)
    dt = jm.jm_stage_dt_proj(layer, delta)
    del delta
    gen = torch.Generator(device=u.device)
    gen.manual_seed(5)
    dg = torch.randn(tuple(xh.shape), generator=gen, device=u.device).to(torch.bfloat16)
    ws = torch.empty(jm.jm_scan_backward_workspace_size(dims, T), dtype=torch.uint8,
                     device=u.device)

    def call():
        return jm.jamba_mamba_scan_backward(layer, xh, dt, B, C, z, dg, cu, wl.cu_seqlens,
                                            want_d_init=False, workspace=ws)

    g = call()
    del g
    torch.cuda.synchronize()
    jm.profile_reset()
    jm.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        g = call()
        del g
    torch.cuda.synchronize()
    el = (time.perf_counter() - t0) / steps
    jm.profile_enable(False)
    prof = jm.profile_read()
    jm.profile_reset()
    del xh, z, dt, dg, ws
    torch.cuda.empty_cache()
    di = dims.d_inner
    # algorithmic bytes: inputs x_hat, z, dg (bf16), dt (fp32), B, C read once; dx, ddt, dz
    # (fp32) written once; dB, dC written once
    nbytes = T * di * (2 + 2 + 2 + 4 + 3 * 4) + T * 16 * 4 * 4
    kernels_ms = {k: round(v[1] / max(v[0], 1), 4) for k, v in prof.items()}
    out = {"ms_per_call": round(el * 1e3, 3), "tokens_per_s": round(T / el, 1), "steps": steps,
           "algorithmic_bytes": nbytes,
           "hbm_frac": round(nbytes / el / 1e9 / HBM_PEAK_GBS, 4),
           "kernels_ms": kernels_ms,
           "note": "gradients of the scan + D skip + gate step w.r.t. x_hat, Delta, B, C, z, "
                   "A_log, D (fp32), 64-token chunks; bound by VALU work, not HBM"}
    # the main kernel against the VALU issue rate, with its measured instructions per update
    per = recorded_valu("bwd_main", "scan_backward_128k_counters.md",
                        ("jm_scan_bwd.hip", "jm_internal.h"))
    if per is not None and kernels_ms.get("bwd_main"):
        updates = T * di * 16
        out["bwd_main"] = {"bound": "alu", "valu_per_update": per,
                           "alu_frac": round(updates * per / VALU_LANE_OPS
                                             / (kernels_ms["bwd_main"] * 1e-3), 4),
                           "alu_basis": "measured VALU instructions per state update (rocprofv3 "
                                        "SQ_INSTS_VALU, profiles/scan_backward_128k_counters.md)"}
    return out


def run_inner_norm(jm, torch, wl, dims, u, cu, out, fconv, fssm, ws, T, steps: int = 5):
    """The same prefill with the optional inner RMSNorm on (synthetic gains, seed 1)."""
    import synth
    gains = synth.make_norm_gains(wl.dims, np.random.default_rng(1))
    arrays = dict(wl.weights)
    arrays.update(gains)
    layer = jm.MambaLayer.from_arrays(dims, arrays)

    def step():
        jm.jamba_mamba_prefill(layer, u, cu, wl.cu_seqlens, out=out, final_conv_state=fconv,
                               final_ssm_state=fssm, workspace=ws)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    jm.profile_reset()
    jm.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    jm.profile_enable(False)
    prof = jm.profile_read()
    jm.profile_reset()
    n, ms = prof.get("inner_norm", (0, 0.0))
    avg = ms / max(n, 1)
    R, N = wl.dims.dt_rank, wl.dims.d_state
    nbytes = T * (2 * R * 2 + 2 * 2 * N * 4)      # delta bf16, B and C fp32: read + write
    return {"ms_per_step": round(el * 1e3 / steps, 3), "tokens_per_s": round(T * steps / el, 1),
            "steps": steps,
            "placement": "RMSNorm of delta, B and C right after x_proj (gains 1 + N(0, 0.01))",
            "norm_kernel": {"avg_ms": round(avg, 4), "bytes": nbytes,
                            "gbs": round(nbytes / (avg * 1e-3) / 1e9, 1) if avg else None,
                            "bound": "hbm",
                            "frac": round(nbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4) if avg else None}}


def run_decode(jm, torch, dev, layer, dims, wl_prefill, steps: int):
    """Decode at batch 64: states from a 2048-token prefill per sequence (not timed),
    then `steps` single-token steps, timed back to back."""
    import synth
    B, L0 = 64, 2048
    wl = synth.make_workload("decode_b64", seed=0, steps=steps)
    d = wl.dims
    u0 = torch.as_tensor(wl.u).to(dev, torch.bfloat16)
    cu = torch.as_tensor(wl.cu_seqlens, dtype=torch.int32).to(dev)
    dec_layer = jm.MambaLayer.from_arrays(dims, wl.weights)
    _, conv, ssm = jm.jamba_mamba_prefill(dec_layer, u0, cu, wl.cu_seqlens)
    del u0
    toks = torch.empty((steps, B, d.d_model), dtype=torch.bfloat16)
    for s in range(steps):
        toks[s] = torch.as_tensor(wl.next_decode_tokens()).to(torch.bfloat16)
    toks = toks.to(dev)
    out = torch.empty((B, d.d_model), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(jm.decode_workspace_size(dims, B), dtype=torch.uint8, device=dev)
    for s in range(min(8, steps)):   # warm-up on copies of the state
        jm.jamba_mamba_decode_step(dec_layer, toks[s], conv.clone(), ssm.clone(), out=out,
                                   workspace=ws)
    torch.cuda.synchronize()
    # eager: one library call per step from Python
    t0 = time.perf_counter()
    for s in range(steps):
        jm.jamba_mamba_decode_step(dec_layer, toks[s], conv, ssm, out=out, workspace=ws)
    torch.cuda.synchronize()
    el_eager = time.perf_counter() - t0
    # graph: G consecutive steps (each with its own tokens) captured once, replayed
    G = 16
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for s in range(G):
            jm.jamba_mamba_decode_step(dec_layer, toks[s], conv, ssm, out=out, workspace=ws)
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // G)
    t0 = time.perf_counter()
    for _ in range(reps):
        graph.replay()
    torch.cuda.synchronize()
    el = (time.perf_counter() - t0) * steps / (reps * G)
    # cold: a 1 GiB read before each timed step evicts weights and state from the 256 MB
    # Infinity Cache; events bracket the step only
    scrub = torch.ones(2**28, dtype=torch.float32, device=dev)
    cold = []
    for s in range(min(32, steps)):
        _ = scrub.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        jm.jamba_mamba_decode_step(dec_layer, toks[s], conv, ssm, out=out, workspace=ws)
        e1.record()
        e1.synchronize()
        cold.append(e0.elapsed_time(e1) * 1e3)
    # the same steps from the decode copies of in_proj_w / out_proj_w in 64 x 64 tiles
    # (jm_tile_decode_weights; bit-identical results): graph replay and cold, as above
    dec_layer.tile_for_decode()
    tgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(tgraph):
        for s in range(G):
            jm.jamba_mamba_decode_step(dec_layer, toks[s], conv, ssm, out=out, workspace=ws)
    tgraph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        tgraph.replay()
    torch.cuda.synchronize()
    el_tiled = (time.perf_counter() - t0) * steps / (reps * G)
    cold_tiled = []
    for s in range(min(32, steps)):
        _ = scrub.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        jm.jamba_mamba_decode_step(dec_layer, toks[s], conv, ssm, out=out, workspace=ws)
        e1.record()
        e1.synchronize()
        cold_tiled.append(e0.elapsed_time(e1) * 1e3)
    del tgraph
    dec_layer.drop_decode_tiles()
    del scrub
    # state cache: the same 64 sequences scattered over a 256-slot cache (random slot map),
    # decoded in place through the slot-indexed entry point, 16-step graph replayed
    n_slots = 256
    cache = jm.StateCache(dims, n_slots, device=dev)
    slot_ids = [int(v) for v in np.random.default_rng(3).permutation(n_slots)[:B]]
    sidx = torch.tensor(slot_ids, dtype=torch.long, device=dev)
    cache.conv[sidx] = conv
    cache.ssm[sidx] = ssm
    slots_dev = torch.tensor(slot_ids, dtype=torch.int32, device=dev)
    for s in range(min(4, steps)):
        jm.jamba_mamba_decode_step_slots(dec_layer, toks[s], cache, slot_ids, out=out, workspace=ws,
                                         slots_device=slots_dev)
    torch.cuda.synchronize()
    sgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(sgraph):
        for s in range(G):
            jm.jamba_mamba_decode_step_slots(dec_layer, toks[s], cache, slot_ids, out=out,
                                             workspace=ws, slots_device=slots_dev)
    sgraph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        sgraph.replay()
    torch.cuda.synchronize()
    el_slots = (time.perf_counter() - t0) * steps / (reps * G)
    del cache
    # per-kernel breakdown in a separate eager pass (events between kernels perturb short steps)
    jm.profile_reset()
    jm.profile_enable(True)
    for s in range(min(64, steps)):
        jm.jamba_mamba_decode_step(dec_layer, toks[s], conv, ssm, out=out, workspace=ws)
    torch.cuda.synchronize()
    jm.profile_enable(False)
    prof = jm.profile_read()
    jm.profile_reset()
    di, dm, R = d.d_inner, d.d_model, d.dt_rank
    wbytes = (2 * di * dm + (R + 32) * di + di * R + dm * di) * 2
    state_bytes = B * di * 16 * 4 * 2 + B * di * 3 * 2 * 2
    per_step = wbytes + state_bytes + B * dm * 2 * 2
    return {"batch": B, "context": L0, "steps": steps, "us_per_step": el * 1e6 / steps,
            "tokens_per_s": B * steps / el, "timing": "HIP graph of 16 steps, replayed",
            "us_per_step_eager": el_eager * 1e6 / steps,
            "us_per_step_cold": round(float(np.median(cold)), 2),
            "us_per_step_state_cache": round(el_slots * 1e6 / steps, 2),
            "us_per_step_tiled": round(el_tiled * 1e6 / steps, 2),
            "us_per_step_cold_tiled": round(float(np.median(cold_tiled)), 2),
            "tiled_note": "decode copies of in_proj_w / out_proj_w in 64 x 64 tiles "
                          "(jm_tile_decode_weights, +201 MB; same outputs bit for bit), graph "
                          "replay and cold as above",
            "state_cache_note": "the 64 states in random slots of a 256-slot cache, slot-indexed "
                                "in-place decode (jamba_mamba_decode_step_slots), graph replay",
            "cold_note": "median of 32 single steps, each after a 1 GiB read (Infinity Cache "
                         "flushed), HIP events around the step",
            "algorithmic_bytes_per_step": per_step,
            "hbm_frac": per_step / (el / steps) / 1e9 / HBM_PEAK_GBS,
            "kernels_us": {k: round(v[1] * 1e3 / max(v[0], 1), 2) for k, v in prof.items()},
            "kernels_note": "eager steps with a HIP event pair around each launch (x_proj and "
                            "out_proj include their split-K sums); the events add a few us per "
                            "launch, so these sum to more than the graph-replayed step"}


if __name__ == "__main__":
    main()
