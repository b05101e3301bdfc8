"""fp64 CPU oracle for the attention forward pass (fp16 and fp8 inputs) and its gradients.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the product library never does.
It shares no code with the HIP path.  See ``oracle/fa_oracle.c`` for the
definition it follows and ``oracle/oracle.py`` for the Python wrapper.
"""
from .oracle import (  # noqa: F401
    backward, build, build_variant, default_scale, e4m3_to_double, forward, forward_fp8,
    half_to_double, library_path, row_probs, rows, rows_fp8, source_text)
