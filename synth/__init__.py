"""Seeded synthetic inputs for the Mamba (selective state-space) mixer layer.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark. It holds no arithmetic of the layer itself: only random draws, the
parameter initialisation recipe, and round-to-nearest-even to bfloat16 of the
draws (so that both sides consume bit-identical values).

Workloads (shapes, dtypes, value distributions) follow the layer the Jamba paper
builds on (Jamba: A Hybrid Transformer-Mamba Language Model, §2 "Model
architecture": Mamba layers interleaved with attention, no positional
information, a constant-size state per sequence instead of a KV cache):

  tiny_fp32      batch 1, L=64, d_model 64, d_inner 128, N 16, d_conv 4, dt_rank 8, fp32
  prefill_4k     batch 1, L=4096, d_model 4096, d_inner 8192, N 16, d_conv 4, dt_rank 256, bf16
  prefill_128k   same layer, one 131072-token sequence
  decode_b64     same layer, 64 sequences: 2048-token prefill each, then 1024 single-token steps
  packed_varlen  same layer, 16 sequences of lengths uniform in [1024, 8192], packed

Initialisation: weights N(0, 0.02); A_log[d, n] = ln(n + 1); D = 1 (or 0 for the
"D=0 twin" that makes the scan's contribution visible in the output);
dt bias = inverse softplus of dt0, dt0 log-uniform in [1e-3, 1e-1]; inputs N(0, 1).
Random stream: numpy PCG64 seeded per workload; draws are fp64, cast to fp32,
then rounded to bf16 for bf16 workloads. Fixed draw order:
[packed lengths] -> in_proj -> conv_w -> conv_b -> x_proj -> dt_proj -> U(dt) ->
out_proj -> [inner-norm gains: delta, B, C] -> inputs (decode: prefill tokens, then each
step's tokens in order).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "LayerDims", "Workload", "JAMBA_DIMS", "TINY_DIMS", "WORKLOADS",
    "round_bf16", "bf16_bits", "make_weights", "make_workload",
]


@dataclasses.dataclass(frozen=True)
class LayerDims:
    d_model: int
    d_inner: int
    d_state: int = 16
    d_conv: int = 4
    dt_rank: int = 8


TINY_DIMS = LayerDims(d_model=64, d_inner=128, d_state=16, d_conv=4, dt_rank=8)
JAMBA_DIMS = LayerDims(d_model=4096, d_inner=8192, d_state=16, d_conv=4, dt_rank=256)

# name -> dict(dims, dtype, lengths | n_seqs/len_range | batch/prefill_len/steps)
WORKLOADS: Dict[str, dict] = {
    "tiny_fp32": dict(dims=TINY_DIMS, dtype="f32", lengths=[64]),
    "prefill_4k": dict(dims=JAMBA_DIMS, dtype="bf16", lengths=[4096]),
    "prefill_128k": dict(dims=JAMBA_DIMS, dtype="bf16", lengths=[131072]),
    "decode_b64": dict(dims=JAMBA_DIMS, dtype="bf16", batch=64, prefill_len=2048, steps=1024),
    "packed_varlen": dict(dims=JAMBA_DIMS, dtype="bf16", n_seqs=16, len_range=(1024, 8192)),
}

WEIGHT_STD = 0.02
DT_MIN, DT_MAX = 1e-3, 1e-1


def round_bf16(a) -> np.ndarray:
    """Round fp32 values to the nearest bfloat16 (ties to even); returns fp32.

    Works on the IEEE-754 bit pattern: add 0x7FFF plus the lowest kept bit, then
    clear the 16 dropped bits. Inputs are finite draws (no NaN handling needed).
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    keep_lsb = (bits >> np.uint64(16)) & np.uint64(1)
    r = ((bits + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).reshape(a.shape)


def bf16_bits(a) -> np.ndarray:
    """uint16 bit patterns of fp32 values that are exactly bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    if np.any(bits & np.uint32(0xFFFF)):
        raise ValueError("values are not bf16-representable; call round_bf16 first")
    return (bits >> np.uint32(16)).astype(np.uint16)


def _cast(a: np.ndarray, dtype: str) -> np.ndarray:
    a32 = np.asarray(a, dtype=np.float32)
    return round_bf16(a32) if dtype == "bf16" else np.ascontiguousarray(a32)


def _normal(rng: np.random.Generator, shape, dtype: str, std: float = 1.0,
            block_rows: int = 8192) -> np.ndarray:
    """N(0, std^2) draws in fp64, cast to fp32 (then bf16), drawn in row blocks.

    Drawing a 2-D array in consecutive row blocks consumes the generator exactly
    as one draw of the whole array would, so block size does not change values.
    """
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.float32)
    if len(shape) == 0 or shape[0] == 0:
        return out
    flat = out.reshape(shape[0], -1)
    for r0 in range(0, shape[0], block_rows):
        r1 = min(shape[0], r0 + block_rows)
        blk = rng.standard_normal((r1 - r0, flat.shape[1]))
        if std != 1.0:
            blk *= std
        flat[r0:r1] = _cast(blk, dtype)
    return out


NORM_GAIN_STD = 0.1
NORM_EPS = 1e-6


def make_norm_gains(dims: LayerDims, rng: np.random.Generator) -> Dict[str, np.ndarray]:
    """Inner-RMSNorm gains (fp32): delta (dt_rank), B and C (d_state), each 1 + N(0, 0.1^2),
    drawn in that order; plus norm_eps."""
    g = {}
    for k, n in (("dt_norm_w", dims.dt_rank), ("B_norm_w", dims.d_state),
                 ("C_norm_w", dims.d_state)):
        g[k] = (1.0 + NORM_GAIN_STD * rng.standard_normal(n)).astype(np.float32)
    g["norm_eps"] = NORM_EPS
    return g


def make_weights(dims: LayerDims, dtype: str, rng: np.random.Generator,
                 D_value: float = 1.0, inner_norm: bool = False) -> Dict[str, np.ndarray]:
    """Layer parameters, drawn in the fixed order documented in the module docstring.

    Layouts (row-major): in_proj_w (2*d_inner, d_model) with x rows first, then z;
    conv_w (d_inner, d_conv), tap d_conv-1 multiplies the current token; conv_b (d_inner);
    x_proj_w (dt_rank + 2*d_state, d_inner) with rows delta | B | C; dt_proj_w
    (d_inner, dt_rank); dt_proj_b (d_inner) fp32; A_log (d_inner, d_state) fp32;
    D (d_inner) fp32; out_proj_w (d_model, d_inner).
    Weight matrices are fp32 arrays holding `dtype` values; A_log, D and dt_proj_b
    are fp32 in every workload (they parameterise the fp32 recurrence).
    With inner_norm, three fp32 RMSNorm gain vectors follow, drawn after out_proj_w
    (so every other parameter is the same as without): dt_norm_w (dt_rank), B_norm_w and
    C_norm_w (d_state), each 1 + N(0, 0.1^2) so that a dropped gain is visible, and
    norm_eps = 1e-6.
    """
    di, dm, N, K, R = dims.d_inner, dims.d_model, dims.d_state, dims.d_conv, dims.dt_rank
    w = {}
    w["in_proj_w"] = _normal(rng, (2 * di, dm), dtype, WEIGHT_STD)
    w["conv_w"] = _normal(rng, (di, K), dtype, WEIGHT_STD)
    w["conv_b"] = _normal(rng, (di,), dtype, WEIGHT_STD)
    w["x_proj_w"] = _normal(rng, (R + 2 * N, di), dtype, WEIGHT_STD)
    w["dt_proj_w"] = _normal(rng, (di, R), dtype, WEIGHT_STD)
    U = rng.random(di)
    dt0 = np.exp(np.log(DT_MIN) + U * (np.log(DT_MAX) - np.log(DT_MIN)))
    w["dt_proj_b"] = np.log(np.expm1(dt0)).astype(np.float32)   # softplus^{-1}(dt0)
    w["out_proj_w"] = _normal(rng, (dm, di), dtype, WEIGHT_STD)
    if inner_norm:
        w.update(make_norm_gains(dims, rng))
    w["A_log"] = np.tile(np.log(np.arange(1, N + 1, dtype=np.float64)), (di, 1)).astype(np.float32)
    w["D"] = np.full(di, D_value, dtype=np.float32)
    w["dt0"] = dt0   # fp64, kept for the softplus round-trip pin (not a layer weight)
    return w


@dataclasses.dataclass
class Workload:
    name: str
    dims: LayerDims
    dtype: str
    weights: Dict[str, np.ndarray]
    lengths: List[int]
    u: np.ndarray                      # (total_tokens, d_model) fp32 holding dtype values
    cu_seqlens: np.ndarray             # int32 (n_seqs + 1,)
    steps: int = 0                     # decode steps (decode workloads only)
    _rng: Optional[np.random.Generator] = None
    _steps_drawn: int = 0

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def n_seqs(self) -> int:
        return len(self.lengths)

    def next_decode_tokens(self) -> np.ndarray:
        """The next decode step's (batch, d_model) tokens, in stream order."""
        if self._rng is None or self._steps_drawn >= self.steps:
            raise RuntimeError("no decode steps left in this workload")
        self._steps_drawn += 1
        return _normal(self._rng, (self.n_seqs, self.dims.d_model), self.dtype)


def make_workload(name: str, seed: int = 0, D_value: float = 1.0, *,
                  lengths: Optional[List[int]] = None, n_seqs: Optional[int] = None,
                  batch: Optional[int] = None, prefill_len: Optional[int] = None,
                  steps: Optional[int] = None, dims: Optional[LayerDims] = None,
                  dtype: Optional[str] = None, inner_norm: bool = False) -> Workload:
    """Build a named workload; keyword overrides give scaled-down variants for tests.

    Overrides keep the draw order, so e.g. a packed workload with n_seqs=3 draws
    3 lengths first, then the weights, then the tokens.
    """
    spec = dict(WORKLOADS[name])
    dims = dims or spec["dims"]
    dtype = dtype or spec["dtype"]
    rng = np.random.default_rng(seed)
    n_steps = 0
    if "len_range" in spec and lengths is None:
        lo, hi = spec["len_range"]
        ns = n_seqs if n_seqs is not None else spec["n_seqs"]
        lengths = [int(v) for v in rng.integers(lo, hi + 1, ns)]
    elif "batch" in spec:
        b = batch if batch is not None else spec["batch"]
        pl = prefill_len if prefill_len is not None else spec["prefill_len"]
        lengths = lengths or [pl] * b
        n_steps = steps if steps is not None else spec["steps"]
    elif lengths is None:
        lengths = list(spec["lengths"])
    lengths = [int(v) for v in lengths]
    w = make_weights(dims, dtype, rng, D_value, inner_norm)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    u = _normal(rng, (int(cu[-1]), dims.d_model), dtype)
    return Workload(name=name, dims=dims, dtype=dtype, weights=w, lengths=lengths, u=u,
                    cu_seqlens=cu, steps=n_steps, _rng=rng if n_steps else None)
