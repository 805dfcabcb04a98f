"""Decode stored element bits to float64 (oracle side; test infrastructure only).

The oracle consumes exactly the values the device tensors hold, so it decodes
the raw bits itself from each format's definition rather than trusting a
framework cast:

  fp32   IEEE-754 binary32.
  fp16   IEEE-754 binary16.
  bf16   the upper 16 bits of a binary32 (1 sign, 8 exponent, 7 mantissa bits).
  e4m3fn OCP 8-bit float, E4M3 "fn" variant: 1 sign, 4 exponent (bias 7),
         3 mantissa bits; exponent 0 is subnormal (m * 2^-9); the all-ones
         exponent is a normal binade except mantissa 7, which is NaN; there
         is no infinity. Largest finite magnitude: 1.75 * 2^8 = 448.
         (FP8 is the precision the "FlashAttention" dictionary entry credits
         to FlashAttention-3.)
"""
from __future__ import annotations

import numpy as np


def decode_f32(bits: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)


def decode_f16(bits: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    wide = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return wide.view(np.float32).astype(np.float64)


def decode_e4m3fn(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = m * 2.0 ** -9
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((e == 0xF) & ((b & 0x7) == 0x7), np.nan, mag)
    return sign * mag


def decode(bits: np.ndarray, fmt: str, descale: float = 1.0) -> np.ndarray:
    """Decode ``bits`` of storage format ``fmt`` and multiply by ``descale``.

    ``descale`` is the per-tensor fp32 factor of the fp8 encoding (1.0 for
    the other formats); the product is formed in float64, exactly.
    """
    fn = {"f32": decode_f32, "f16": decode_f16, "bf16": decode_bf16, "fp8": decode_e4m3fn}[fmt]
    x = fn(bits)
    if descale != 1.0:
        x = x * float(np.float32(descale))
    return x
