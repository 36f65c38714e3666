"""Seeded N(0, 1) input values for a decode step, on the host (numpy) or on a
GPU (torch's generator).

Storage conventions shared by every consumer:
  f32  -> numpy float32 / torch.float32
  f16  -> numpy float16 / torch.float16
  bf16 -> numpy uint16 bit patterns / torch.bfloat16
  fp8  -> numpy uint8 E4M3 codes / torch.uint8 (8-bit caches only)

Pool slots that hold no token before the step are poisoned with all-ones bit
patterns (a NaN in every format), so a read of a slot outside a sequence shows
up as a NaN.  Copy-on-write copies hold the same leading rows as their shared
source, as they would after the copy.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .layout import Layout

_NP_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8": np.uint8}
POISON_BITS = {"f32": 0xFFFFFFFF, "f16": 0xFFFF, "bf16": 0xFFFF, "fp8": 0xFF}
_BITS = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8}


def to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 data to the storage format (round to nearest even)."""
    if dtype == "f32":
        return x64.astype(np.float32)
    if dtype == "f16":
        return x64.astype(np.float16)
    if dtype == "bf16":
        bits = x64.astype(np.float32).view(np.uint32)
        bias = ((bits >> 16) & 1) + np.uint32(0x7FFF)
        return ((bits + bias) >> 16).astype(np.uint16)
    raise ValueError(dtype)


def _poison(shape, dtype):
    bits = np.full(shape, POISON_BITS[dtype], dtype=_BITS[dtype])
    return bits.view(_NP_STORAGE[dtype])


def e4m3_codes(rng: np.random.Generator, shape) -> np.ndarray:
    """Random finite E4M3 codes for an 8-bit cache: random sign, exponent
    field uniform in 1..12 (magnitudes 2^-6 .. 60, a wide dynamic range),
    mantissa uniform.  Integers only: nothing is rounded."""
    sign = rng.integers(0, 2, size=shape).astype(np.uint8) << 7
    exp = rng.integers(1, 13, size=shape).astype(np.uint8) << 3
    man = rng.integers(0, 8, size=shape).astype(np.uint8)
    return (sign | exp | man).astype(np.uint8)


@dataclass
class HostStep:
    q: np.ndarray        # [S, Hq, D]
    k_cache: np.ndarray  # [N, Hkv, B, D]
    v_cache: np.ndarray
    k_new: np.ndarray    # [S, Hkv, D], token appended at position L-1
    v_new: np.ndarray


def _normal(seed: int, stream: int, shape) -> np.ndarray:
    return np.random.default_rng([seed, stream]).standard_normal(shape)


def host_values(layout: Layout) -> HostStep:
    cfg, seed = layout.cfg, layout.seed
    S, Hq, Hkv, D, B = cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    S = len(layout.context_lens)
    N, dt = layout.num_blocks, cfg.dtype
    q = to_storage(_normal(seed, 1, (S, Hq, D)), dt)
    kvdt = cfg.kv_dtype
    caches = []
    for stream in (2, 3):
        if kvdt == "fp8":
            full = e4m3_codes(np.random.default_rng([seed, stream]), (N, Hkv, B, D))
        else:
            full = to_storage(_normal(seed, stream, (N, Hkv, B, D)), dt)
        cache = _poison((N, Hkv, B, D), kvdt)
        blk, off = np.nonzero(layout.live)
        cache[blk, :, off, :] = full[blk, :, off, :]
        r = layout.cow_rows
        for src, dst in layout.cow_pairs:
            cache[dst, :, :r, :] = cache[src, :, :r, :]
        caches.append(cache)
    k_new = to_storage(_normal(seed, 4, (S, Hkv, D)), dt)
    v_new = to_storage(_normal(seed, 5, (S, Hkv, D)), dt)
    return HostStep(q=q, k_cache=caches[0], v_cache=caches[1], k_new=k_new, v_new=v_new)


def device_values(layout: Layout, device="cuda"):
    """The same kind of data drawn on the GPU with torch's seeded generator.

    Used where the host would take minutes to draw the pool (tens of GB).
    Returns torch tensors (q, k_cache, v_cache, k_new, v_new)."""
    import torch

    cfg, seed = layout.cfg, layout.seed
    Hq, Hkv, D, B = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    S = len(layout.context_lens)
    N = layout.num_blocks
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[cfg.dtype]

    def gen(stream):
        g = torch.Generator(device=device)
        g.manual_seed(seed * 64 + stream)
        return g

    def normal(shape, stream, chunk_rows=4096):
        out = torch.empty(shape, dtype=tdt, device=device)
        g = gen(stream)
        flat = out.view(shape[0], -1)
        for r0 in range(0, shape[0], chunk_rows):
            r1 = min(shape[0], r0 + chunk_rows)
            flat[r0:r1] = torch.randn((r1 - r0, flat.shape[1]), generator=g, device=device,
                                      dtype=torch.float32).to(tdt)
        return out

    q = normal((S, Hq, D), 1)
    dead = torch.from_numpy(~layout.live).to(device)
    caches = []
    for stream in (2, 3):
        if cfg.kv_dtype == "fp8":
            g = gen(stream)
            sign = torch.randint(0, 2, (N, Hkv, B, D), generator=g, device=device, dtype=torch.uint8) << 7
            expo = torch.randint(1, 13, (N, Hkv, B, D), generator=g, device=device, dtype=torch.uint8) << 3
            cache = sign | expo | torch.randint(0, 8, (N, Hkv, B, D), generator=g, device=device, dtype=torch.uint8)
            cache.masked_fill_(dead[:, None, :, None], 0xFF)
        else:
            cache = normal((N, Hkv, B, D), stream)
            view = cache.view(torch.int16) if tdt != torch.float32 else cache.view(torch.int32)
            view.masked_fill_(dead[:, None, :, None], -1)
        if len(layout.cow_pairs):
            r = layout.cow_rows
            src = torch.from_numpy(layout.cow_pairs[:, 0].astype(np.int64)).to(device)
            dst = torch.from_numpy(layout.cow_pairs[:, 1].astype(np.int64)).to(device)
            cache[dst, :, :r, :] = cache[src, :, :r, :]
        caches.append(cache)
    k_new = normal((S, Hkv, D), 4)
    v_new = normal((S, Hkv, D), 5)
    return q, caches[0], caches[1], k_new, v_new
