"""CPU oracle for the tensorwise-scaled Float8Linear forward + backward.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package; the product path (the
HIP library and its Python binding) never does, and shares no code with it.

The element-wise steps (amax, scale, fp8 encode/decode, cast + transposed
copy, amax history) live in plain C (f8ref.c, built by oracle/build.py into
liboracle.so); this module loads it with ctypes and adds the three GEMM
references, which follow the plain definition of a dequantised matrix
product: every fp8 code is decoded to its exact value in fp64, products of
two fp8 values are exact in fp64, and the dequantisation divides by both
tensor scales; and the bias terms (Y + b, and the bias gradient as the fp64
column sum of dY).

Parity status: every function here is pinned by tests/test_oracle_pins.py
against brute force, closed forms of the OCP 8-bit formats, exact rational
arithmetic or torch's own float8 conversions; none is "parity unpinned".
"""
from .reference import (  # noqa: F401
    E4M3, E5M2, FMAX, HIST_LEN, EPS,
    amax, scale, cast, encode_f32, encode_bits_range, decode, decode_table,
    bf16_bits_to_f32, fp8_encode_scalar, fp8_decode_scalar,
    gemm_ref, forward_ref, dgrad_ref, wgrad_ref, forward_ref_at, dgrad_ref_at, wgrad_ref_at,
    bf16_to_f64, dbias_ref,
    DelayedHistory, linear_step, lib_path,
)
