"""Exact decoding of the stored number formats to fp64 (oracle; test infrastructure only).

* bf16: the upper 16 bits of an IEEE fp32 word, so decoding is a 16-bit left
  shift into fp32, then widening to fp64 (exact).
* fp16: IEEE binary16, widened exactly by numpy.
* e4m3fn: the fp8 format of an fp8 KV cache (page
  vllm.v1.attention.backends.flashinfer_ts, ``_kv_kernel_dtype``: one-byte
  storage whose bytes the kernel reads as e4m3 values; ``_ts_output_dtype``
  names torch.float8_e4m3fn).
  The table below is built from the format's definition, not from any
  library: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
  exponent field 0 is subnormal (m/8 * 2^-6); there are no infinities and
  only S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
"""

from __future__ import annotations

import math

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns widen to NaN, quietly
        return b.view(np.float32).astype(np.float64)


def fp16_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE half bit patterns (uint16) -> exact fp64 values."""
    return np.asarray(bits).astype(np.uint16).view(np.float16).astype(np.float64)


def e4m3fn_value(byte: int) -> float:
    """Value of one e4m3fn byte, from the format definition."""
    byte = int(byte) & 0xFF
    sign = -1.0 if byte & 0x80 else 1.0
    exp_field = (byte >> 3) & 0xF
    mant = byte & 0x7
    if exp_field == 0xF and mant == 0x7:
        return math.nan
    if exp_field == 0:
        return sign * (mant / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)


E4M3FN_TABLE = np.array([e4m3fn_value(b) for b in range(256)], dtype=np.float64)
E4M3FN_TABLE.setflags(write=False)


def e4m3fn_to_f64(data: np.ndarray) -> np.ndarray:
    """e4m3fn bytes (uint8) -> exact fp64 values."""
    return E4M3FN_TABLE[np.asarray(data).astype(np.uint8)]


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Decode stored elements of the named format ("bf16", "fp16", "fp8_e4m3", "f32", "f64")."""
    if dtype == "bf16":
        return bf16_to_f64(bits)
    if dtype == "fp16":
        return fp16_to_f64(bits)
    if dtype == "fp8_e4m3":
        return e4m3fn_to_f64(bits)
    if dtype in ("f32", "f64"):
        return np.asarray(bits, dtype=np.float64)
    raise ValueError(f"unknown format {dtype!r}")
