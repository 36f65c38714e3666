"""Paged KV-cache decode attention for AMD Instinct MI355X (gfx950).

Thin Python binding of libpkv.so (C ABI declared in include/pkv.h).  The
functions here only marshal arguments: every step of the decode path runs in
the library's HIP kernels.  torch is used for device memory and streams.

If libpkv.so has not been built, importing this package raises: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

from ._lib import LIB_PATH, PkvError, check, lib
from .beam import BeamSearchCache
from .ops import (
    BlockManager,
    copy_blocks,
    decode_step,
    gather_kv,
    paged_attention_decode,
    paged_attention_decode_noalloc,
    paged_attention_decode_shared_prefix,
    plan_info,
    reshape_and_cache,
    reshape_and_cache_fp8,
    shared_prefix_workspace_bytes,
    swap_blocks,
    workspace_bytes,
)

__all__ = [
    "BeamSearchCache", "LIB_PATH", "PkvError", "lib", "check", "BlockManager", "copy_blocks", "decode_step", "gather_kv",
    "paged_attention_decode", "paged_attention_decode_noalloc", "paged_attention_decode_shared_prefix", "plan_info", "reshape_and_cache", "reshape_and_cache_fp8", "swap_blocks", "workspace_bytes",
    "shared_prefix_workspace_bytes",
]
