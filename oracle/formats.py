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
