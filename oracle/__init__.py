"""CPU oracle for the Mamba mixer layer -- TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 reference used to check the HIP library. Only `tests/`, the
smoke check in `__graft_entry__.py` and the CPU-baseline leg of `bench.py` may
import it. It shares no code with the HIP path (the library under
`mamba_selective_scan_mixer_amd/` never imports or links anything here).
"""
from . import scan_backward  # noqa: F401  (backward of the scan step, row f4)
from .mamba_ref import (  # noqa: F401
    as_f64, silu, softplus, in_proj, causal_conv_silu, x_proj, dt_proj,
    selective_scan, gate, out_proj, prefill, decode_step, rmsnorm, inner_norm, NORM_KEYS,
    DEFAULT_NORM_EPS,
)
