"""Decoding of stored values to fp64 (oracle; test infrastructure only).

Storage: f32 as float32, f16 as IEEE binary16 (numpy float16), bf16 as the
upper 16 bits of a binary32 pattern held in uint16.  Each decode is exact:
every value of the three formats is representable in fp64.
"""
import numpy as np


def decode(raw, dtype: str) -> np.ndarray:
    with np.errstate(invalid="ignore"):     # signalling-NaN patterns widen to NaN
        return _decode(raw, dtype)


def _decode(raw, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(raw, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        hi = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return hi.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# 8-bit floating point, OCP E4M3 ("fn": finite, no infinities) for a KV cache
# stored in 8 bits ("pagedattention vllm" glossary, Comparison with
# Alternatives > vs Compression: paging combines with quantization).
# Code bits S EEEE MMM, exponent bias 7; exponent field 0 holds subnormals
# m/8 * 2^-6; S 1111 111 is NaN; the largest finite magnitude is
# 1.75 * 2^8 = 448.  A stored code c with scale s stands for e4m3(c) * s.
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0


def decode_e4m3(codes) -> np.ndarray:
    """fp64 value of every code (exact)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag
    out[(e == 15) & (c & 7 == 7)] = np.nan
    return out


# The finite non-negative codes 0x00 .. 0x7E, whose values increase with the code.
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = decode_e4m3(_POS_CODES)


def quantize_e4m3(y) -> np.ndarray:
    """uint8 code of each fp32 value y: the nearest finite E4M3 value, a tie
    going to the code with an even last bit; |y| above 448 gives +-448
    (saturation); NaN gives 0x7F.  The sign of y (-0.0 included) is kept."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = np.abs(a - _POS_VALUES[lo])
    d_hi = np.abs(_POS_VALUES[hi] - a)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(a >= E4M3_MAX, np.uint8(0x7E), code)
    code = np.where(np.signbit(y), code | np.uint8(0x80), code).astype(np.uint8)
    return np.where(np.isnan(y), np.uint8(0x7F), code).astype(np.uint8)
