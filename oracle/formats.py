"""Exact decoders for the number formats the path reads (oracle side).

Each decoder is written from the format's definition and returns float64,
where every value of these formats is exact.

* e4m3fn (OCP 8-bit float, "E4M3"): 1 sign, 4 exponent bits (bias 7),
  3 mantissa bits; exponent field 0 is subnormal (m * 2^-9); the all-ones
  pattern S.1111.111 is NaN; there are no infinities; max finite 448.
  The fp8 index cache of the DeepSeek-V3.2 indexer page stores these codes.
* e2m1 (OCP MX FP4): 1 sign, 2 exponent bits (bias 1), 1 mantissa bit;
  exponent field 0 is subnormal (m * 0.5); values 0, .5, 1, 1.5, 2, 3, 4, 6.
* ue8m0 (OCP MX scale): unsigned 8-bit exponent, value 2^(e - 127); 255 is NaN.
* bfloat16: the upper 16 bits of an IEEE binary32.
* fp32 scales are 4 little-endian bytes (IEEE binary32).

Pins (tests/test_oracle_formats.py): all 256 e4m3 codes against torch's
float8_e4m3fn -> float cast; all 16 e2m1 codes against the OCP value table;
ue8m0 against 2^(e-127); bf16 against torch's bfloat16 -> float cast.
"""

from __future__ import annotations

import numpy as np


def e4m3(codes) -> np.ndarray:
    """uint8 e4m3fn codes -> float64 values (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, out)


def e2m1(nibbles) -> np.ndarray:
    """4-bit e2m1 codes (0..15) -> float64 values."""
    n = np.asarray(nibbles, dtype=np.uint8).astype(np.int64) & 0xF
    sign = np.where(n & 0x8, -1.0, 1.0)
    e = (n >> 1) & 0x3
    m = n & 0x1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1.0))
    return sign * mag


def ue8m0(codes) -> np.ndarray:
    """uint8 ue8m0 exponents -> float64 2^(e-127) (NaN for 255)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def bf16(bits) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f32le(four_bytes) -> np.ndarray:
    """[..., 4] uint8 little-endian bytes -> float64."""
    a = np.ascontiguousarray(np.asarray(four_bytes, dtype=np.uint8))
    return a.view("<f4")[..., 0].astype(np.float64)
