"""CPU oracle for the KV-cached decode step (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  It wraps the plain-C f64 reference in kvdec_oracle.c through
ctypes; it shares no code with the HIP library.
"""
from .oracle import (attend, prefill_causal, append, append_slide, seed, rope, bf16_to_f32,  # noqa: F401
                     load, SCALE_HEAD_DIM_64)
