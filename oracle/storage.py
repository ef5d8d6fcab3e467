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
* fp8 e4m3 (the OCP 8-bit floating-point format "E4M3": 1 sign bit, 4 exponent bits
  with bias 7, 3 mantissa bits, subnormals, no infinities, S.1111.111 is NaN) with the
  same per-(block, KV head) fp32 scale: x = value(code) * scale.  value(code) is
  (-1)^s * 2^(e - 7) * (1 + m / 8) for e > 0 and (-1)^s * 2^-6 * (m / 8) for e = 0;
  every such value times an fp32 scale is exact in fp64.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """Decode bf16 bit patterns (any integer dtype of 16 bits) to fp64, exactly."""
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def fp8_e4m3_to_f64(codes):
    """Decode e4m3 bytes (any 8-bit integer dtype) to fp64, from the format definition."""
    b = np.asarray(codes).astype(np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    val = np.where(e > 0, np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32)),
                   np.ldexp(m / 8.0, -6))
    val = np.where((e == 0xF) & ((b & 0x7) == 0x7), np.nan, val)
    return sign * val


def decode(stored, kind, scale=None):
    """Decode a stored array to fp64.

    ``kind`` is ``"f32"`` (float32 array), ``"bf16"`` (16-bit integer array
    holding bf16 bit patterns), ``"i8"`` (int8 array) or ``"fp8"`` (8-bit array of
    e4m3 codes); for the last two ``scale`` must broadcast against the array.
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
    if kind == "fp8":
        if scale is None:
            raise ValueError("fp8 storage needs a scale")
        return fp8_e4m3_to_f64(stored) * np.asarray(scale, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown storage kind {kind!r}")
