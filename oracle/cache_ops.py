"""Cache scatter and block copy, bitwise (oracle; test infrastructure only).

* reshape_and_cache: the new token's key and value are stored into the cache
  block the block table names ("What is PagedAttention" (tecyfy), "How it
  works"): token i goes to block slot_mapping[i] // B at offset
  slot_mapping[i] % B, all KV heads; a negative slot means "do not store".
* reshape_and_cache_fp8: the same store into a cache of 8-bit E4M3 codes with
  a per-tensor scale (paging combined with quantization, "pagedattention
  vllm" glossary, "Comparison with Alternatives > vs Compression").
* copy_blocks: the copy made before a shared block is modified
  ("pagedattention vllm" glossary, "Copy-on-Write Sharing > Divergence
  Handling"): for each (src, dst) pair, block dst of both caches becomes a
  copy of block src, all heads and offsets.

Both move bit patterns only.  Pairs must have distinct destinations and no
destination may also be a source in the same call; then the result does not
depend on the order pairs are applied in.
"""
from __future__ import annotations

import numpy as np

from .formats import decode, quantize_e4m3


def _bits(a: np.ndarray) -> np.ndarray:
    return a.view({1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[a.dtype.itemsize])


def reshape_and_cache(k, v, k_cache, v_cache, slot_mapping, block_size: int) -> None:
    """In place.  k, v: [T, Hkv, D]; caches [N, Hkv, B, D]; slot_mapping [T]."""
    kc, vc, kb, vb = _bits(k_cache), _bits(v_cache), _bits(k), _bits(v)
    num_blocks = kc.shape[0]
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        block, offset = divmod(slot, block_size)
        if block >= num_blocks:
            raise ValueError(f"slot {slot} outside the pool")
        kc[block, :, offset, :] = kb[i]
        vc[block, :, offset, :] = vb[i]


def copy_blocks(k_cache, v_cache, pairs) -> None:
    """In place.  pairs: iterable of (src, dst) physical block ids."""
    pairs = [tuple(map(int, p)) for p in np.asarray(pairs).reshape(-1, 2)]
    dsts = [d for _, d in pairs]
    if len(set(dsts)) != len(dsts) or set(dsts) & {s for s, _ in pairs}:
        raise ValueError("copy pairs need distinct destinations that are not sources")
    kc, vc = _bits(k_cache), _bits(v_cache)
    num_blocks = kc.shape[0]
    for src, dst in pairs:
        if not (0 <= src < num_blocks and 0 <= dst < num_blocks):
            raise ValueError("block id outside the pool")
        kc[dst] = kc[src]
        vc[dst] = vc[src]


def reshape_and_cache_fp8(k, v, k_cache, v_cache, slot_mapping, block_size: int, k_scale: float,
                          v_scale: float, dtype: str) -> None:
    """In place, into caches of E4M3 codes (uint8 [N, Hkv, B, D]).  Each new
    value x (storage format `dtype`) is stored as the code of
    fp32(x) / fp32(scale), the division in fp32 (the precision the decision
    is taken in on both sides), rounded by quantize_e4m3; negative slots
    are skipped."""
    kq = quantize_e4m3(decode(k, dtype).astype(np.float32) / np.float32(k_scale))
    vq = quantize_e4m3(decode(v, dtype).astype(np.float32) / np.float32(v_scale))
    num_blocks = k_cache.shape[0]
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        block, offset = divmod(slot, block_size)
        if block >= num_blocks:
            raise ValueError(f"slot {slot} outside the pool")
        k_cache[block, :, offset, :] = kq[i]
        v_cache[block, :, offset, :] = vq[i]


def swap_blocks(src_k, src_v, dst_k, dst_v, pairs) -> None:
    """In place: block dst of the destination pools becomes a bitwise copy of
    block src of the source pools, for each (src, dst) pair ("pagedattention
    vllm" glossary, "Memory Management > Swapping": blocks move between GPU
    memory and CPU memory to serve more sequences than the GPU holds).  The
    two pools are different arrays, so any pair order gives one result as
    long as destinations are distinct."""
    pairs = [tuple(map(int, p)) for p in np.asarray(pairs).reshape(-1, 2)]
    dsts = [d for _, d in pairs]
    if len(set(dsts)) != len(dsts):
        raise ValueError("swap pairs need distinct destinations")
    sk, sv, dk, dv = _bits(src_k), _bits(src_v), _bits(dst_k), _bits(dst_v)
    for src, dst in pairs:
        if not (0 <= src < sk.shape[0] and 0 <= dst < dk.shape[0]):
            raise ValueError("block id outside a pool")
        dk[dst] = sk[src]
        dv[dst] = sv[src]
