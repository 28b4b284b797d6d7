"""CPU oracle for the ragged dot (grouped GEMM) of MoE expert FFNs and its GLU.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
statement of what the GPU library computes.  Only the test suite, the smoke
check in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP path (no kernels, headers, helpers
or constants), and the HIP path never imports it.

Floating point: GEMM-type results are exact bf16 -> float64 conversions
accumulated in float64 per group; the GLU is evaluated in float32 in the op
order the MaxText page fixes, rounding only the final result to bf16; the
weighted unsort backward forms its product in float32 and rounds it once to
bf16, and its row dot is a float64 sum of exact products.

Pins (what fixes each function independently of itself) live in
``tests/test_oracle_*.py``; every public function here is pinned.
"""

from .bf16 import bf16_bits_to_f32, bf16_bits_to_f64, f32_to_bf16_bits
from .ragged import boundaries, ragged_dot, trans_ragged_dot
from .glu import glu_fwd, glu_bwd
from .unsort import unsort_bwd_rows
from .fp8 import e4m3_to_f64, e4m3_to_bf16_bits, ragged_dot_fp8, trans_ragged_dot_fp8

__all__ = [
    "bf16_bits_to_f32",
    "bf16_bits_to_f64",
    "f32_to_bf16_bits",
    "boundaries",
    "ragged_dot",
    "trans_ragged_dot",
    "glu_fwd",
    "glu_bwd",
    "unsort_bwd_rows",
    "e4m3_to_f64",
    "e4m3_to_bf16_bits",
    "ragged_dot_fp8",
    "trans_ragged_dot_fp8",
]
