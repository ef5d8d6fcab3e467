"""Exact decoding of stored cache elements to fp64 (oracle; test infrastructure only).

The attention result must be compared on the values the kernels actually read,
so the oracle decodes the stored bits itself, from the format definitions:

* fp32 is IEEE binary32; every value is exact in fp64.
* bf16 is the upper 16 bits of an IEEE binary32 word (sign, 8-bit exponent,
  7-bit fraction).  Shifting the 16-bit pattern into the top half of a 32-bit
  word gives that binary32 value exactly.
* int8 with a per-(block, KV head) fp32 scale is dequantised by Lecture 10's
  affine rule ("Quantization 量化 / 基本概念"): x = (x_q - zero_point) * scale,
  here with zero_point = 0.  x_q * scale is an 8-bit times a 24-bit significand,
  so the fp64 product is exact.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """Decode bf16 bit patterns (any integer dtype of 16 bits) to fp64, exactly."""
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def decode(stored, kind, scale=None):
    """Decode a stored array to fp64.

    ``kind`` is ``"f32"`` (float32 array), ``"bf16"`` (16-bit integer array
    holding bf16 bit patterns) or ``"i8"`` (int8 array; ``scale`` must broadcast
    against it).
    """
    if kind == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if kind == "bf16":
        return bf16_bits_to_f64(stored)
    if kind == "i8":
        if scale is None:
            raise ValueError("int8 storage needs a scale")
        q = np.asarray(stored, dtype=np.int8).astype(np.float64)
        return q * np.asarray(scale, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown storage kind {kind!r}")
