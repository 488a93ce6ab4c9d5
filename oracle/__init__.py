"""CPU oracle for the small-batch MoE decode layer (warp-decode form).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import, call or link anything in this
package.  The product (the HIP library and its Python binding) never does, and
this package never imports the product.  The two share no code: the only
module both sides use is the seeded input generator, which holds none of the
layer's arithmetic.

Contents
  oracle.c   plain FP64 C implementation of the layer (see its header)
  ref.py     ctypes loader for liboracle.so plus NumPy-level conveniences
  brute.py   pure-Python expert-centric brute force for tiny shapes (a pin)
  build.py   gcc build of liboracle.so
"""
from .ref import (  # noqa: F401
    e4m3_table, e8m0_table, dequant, bf16_value, bf16_rne, round_f32, silu,
    gate_up, down, moe_decode, route, max_threads, lib_path,
    e4m3_encode, mxfp8_quantize, moe_decode_exact, moe_decode_conventional,
    moe_decode_dense_weights,
)
