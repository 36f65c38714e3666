"""Paged decode attention, fp64 (oracle; test infrastructure only).

Definition followed:
* Address translation ("pagedattention vllm" glossary, chipfoundryservices,
  "Attention Computation > Address Translation"; "PagedAttention",
  lastdictionary): logical token t of sequence s lives in physical block
  block_tables[s, t // B] at in-block offset t % B.  Cache layout
  [num_blocks, num_kv_heads, B, head_dim] for both keys and values.
* Block-wise attention (same glossary, "Attention Computation > Block-Wise
  Attention"; systemdesign.academy glossary "Paged Attention"): the blocks are
  gathered and attention is computed as if they were contiguous, which is
  mathematically standard attention.  So the oracle gathers each sequence
  into contiguous fp64 arrays and evaluates

      x_t = scale * <q, K_t>,   p = softmax(x),   out = sum_t p_t V_t

  over the L = context_lens[s] tokens of the sequence, all in fp64.
* Query head j reads key/value head j // (num_q_heads / num_kv_heads) (heads
  sharing one set of keys and values, systemdesign.academy glossary; the
  grouping into contiguous runs of query heads is a reading, not on the pages).
* The scale is taken as the fp32 value the library receives, widened to fp64.
* A sequence of length 0 has an all-zero output row (the pages are silent).
* 8-bit cache ("pagedattention vllm" glossary, "Comparison with Alternatives
  > vs Compression"): with kv_format "fp8_e4m3" the caches hold E4M3 codes
  and a key or value is e4m3(code) * k_scale (or v_scale), the scales taken
  as the fp32 values the library receives; q keeps its own format.
* Sliding window ("pagedattention vllm" glossary, "Advanced Features >
  Sliding Window": models with sliding-window attention keep only recent
  blocks): with a window of W > 0 tokens, only the last W of the L tokens
  are attended, t in [max(0, L - W), L); W = 0 means no window.  Blocks that
  hold no attended token are never read, so their table entries may be -1.
"""
from __future__ import annotations

import numpy as np

from .formats import decode, decode_e4m3


def gather_sequence(cache, table_row, length: int, kv_head: int, block_size: int, start: int = 0) -> np.ndarray:
    """Contiguous [length - start, head_dim] copy of tokens start .. length-1
    of one sequence's cached rows for one KV head.

    `cache` is an array (or anything that supports cache[int_array, int]
    indexing and returns a numpy array) laid out [num_blocks, Hkv, B, D]."""
    first = int(start) // block_size
    n_blocks = -(-int(length) // block_size)
    phys = np.asarray(table_row[first:n_blocks], dtype=np.int64)
    num_blocks = cache.shape[0]
    if phys.size and (phys.min() < 0 or phys.max() >= num_blocks):
        raise ValueError("block table entry outside the pool")
    tiles = np.asarray(cache[phys, kv_head])            # [n_blocks - first, B, D]
    rows = tiles.reshape((n_blocks - first) * block_size, tiles.shape[-1])
    return rows[int(start) - first * block_size:int(length) - first * block_size]


def paged_attention_decode(q, k_cache, v_cache, block_tables, context_lens, scale: float,
                           block_size: int, num_kv_heads: int, dtype: str, rows=None,
                           sliding_window: int = 0, kv_format: str = "same", k_scale: float = 1.0,
                           v_scale: float = 1.0) -> np.ndarray:
    """fp64 decode attention through the block tables.

    q: [S, Hq, D] in storage format; caches [N, Hkv, B, D]; block_tables int
    [S, M]; context_lens int [S].  Returns fp64 [S, Hq, D], or, when `rows`
    lists (s, j) pairs, an fp64 [len(rows), D] array in that order.
    sliding_window > 0 attends to the last sliding_window tokens only."""
    S, Hq, D = q.shape
    if Hq % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    group = Hq // num_kv_heads
    scale64 = float(np.float32(scale))
    wanted = [(s, j) for s in range(S) for j in range(Hq)] if rows is None else [tuple(map(int, r)) for r in rows]

    by_kv = {}
    for idx, (s, j) in enumerate(wanted):
        by_kv.setdefault((s, j // group), []).append((idx, j))

    result = np.zeros((len(wanted), D), dtype=np.float64)
    for (s, h), members in by_kv.items():
        L = int(context_lens[s])
        if L <= 0:
            continue
        t0 = max(0, L - sliding_window) if sliding_window > 0 else 0
        Kraw = gather_sequence(k_cache, block_tables[s], L, h, block_size, t0)
        Vraw = gather_sequence(v_cache, block_tables[s], L, h, block_size, t0)
        if kv_format == "fp8_e4m3":
            K = decode_e4m3(Kraw) * float(np.float32(k_scale))
            V = decode_e4m3(Vraw) * float(np.float32(v_scale))
        elif kv_format == "same":
            K, V = decode(Kraw, dtype), decode(Vraw, dtype)
        else:
            raise ValueError(f"unknown kv_format {kv_format!r}")
        for idx, j in members:
            qv = decode(q[s, j], dtype)
            x = scale64 * (K @ qv)
            e = np.exp(x - x.max())
            p = e / e.sum()
            result[idx] = p @ V
    if rows is None:
        return result.reshape(S, Hq, D)
    return result
