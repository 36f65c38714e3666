"""Seeded block placement for a decode step (integers only, numpy).

`make_layout` decides, for one workload:

* the context length L of every sequence, counting the token this step
  appends (so the step writes position L-1 and then attends over L tokens);
* the size of the physical block pool and a seeded random order of its blocks
  (or the identity order, for measuring what scattering the blocks costs);
* each sequence's block table (int32, -1 padded), filled sequence by sequence
  from the front of that random order;
* for shared-prefix workloads, the prompt blocks that the samples of one
  prompt share, and the copy-on-write copies of the prompt's partial last
  block that every sample but the last one owns;
* the slot (block * B + offset) of the token each sequence appends this step,
  and which pool slots hold a token before the step.

The draw order is fixed: lengths first, then the pool order.
"""
from __future__ import annotations

from dataclasses import dataclass
import math

import numpy as np

from .configs import DecodeConfig


@dataclass
class Layout:
    cfg: DecodeConfig
    seed: int
    context_lens: np.ndarray   # int32 [S]
    block_tables: np.ndarray   # int32 [S, M], -1 = no block
    num_blocks: int            # pool size N
    pool_order: np.ndarray     # int64 [N], the seeded order blocks are handed out in
    used_blocks: int           # how many blocks of pool_order the tables use
    new_slots: np.ndarray      # int32 [S], slot of position L-1 of each sequence
    live: np.ndarray           # bool [N, B], slot holds a token before the step
    cow_pairs: np.ndarray      # int32 [P, 2], (shared source, private copy)
    cow_rows: int              # leading slots of each copy that mirror its source

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if len(self.context_lens) else 0


def draw_lengths(cfg: DecodeConfig, rng: np.random.Generator) -> np.ndarray:
    S = cfg.num_seqs
    if cfg.lengths == "fixed":
        lens = np.array(cfg.fixed_lengths, dtype=np.int64)
        assert len(lens) == S
    elif cfg.lengths == "uniform":
        lens = rng.integers(cfg.len_lo, cfg.len_hi + 1, size=S)
    elif cfg.lengths == "lognormal":
        raw = rng.lognormal(mean=math.log(cfg.lognormal_median), sigma=cfg.lognormal_sigma, size=S)
        lens = np.clip(np.rint(raw), cfg.len_lo, cfg.len_hi).astype(np.int64)
    elif cfg.lengths == "shared_prefix":
        tails = rng.integers(cfg.len_lo, cfg.len_hi + 1, size=S)
        lens = cfg.prompt_len + tails
    else:
        raise ValueError(cfg.lengths)
    return lens.astype(np.int32)


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def make_layout(cfg: DecodeConfig, seed: int, lengths=None) -> Layout:
    """Seeded placement.  `lengths` overrides the drawn lengths (edge-case tests)."""
    rng = np.random.default_rng(seed)
    lens = draw_lengths(cfg, rng) if lengths is None else np.asarray(lengths, dtype=np.int32)
    S, B = len(lens), cfg.block_size
    nblk = [_ceil_div(int(L), B) for L in lens]
    # With a sliding window, blocks wholly before the last W tokens are
    # released: their table entries stay -1 and take no pool block.
    W = cfg.sliding_window
    skip = [max(0, int(L) - W) // B if W > 0 else 0 for L in lens]

    shared = cfg.lengths == "shared_prefix"
    if shared:
        spp = cfg.samples_per_prompt
        assert S % spp == 0
        pb = _ceil_div(cfg.prompt_len, B)
        rem = cfg.prompt_len % B
        copies = (spp - 1) if rem else 0
        need = 0
        for p in range(S // spp):
            need += pb + copies
            for k in range(spp):
                need += nblk[p * spp + k] - pb
    else:
        need = sum(n - k for n, k in zip(nblk, skip))
    N = cfg.pool_blocks if cfg.pool_blocks else int(math.ceil(cfg.pool_factor * need))
    if N < need:
        raise ValueError(f"pool of {N} blocks cannot hold {need}")
    order = rng.permutation(N)
    if cfg.placement == "contiguous":
        # Each sequence's blocks adjacent and in order (the permutation is
        # still drawn, so every later draw is unchanged).
        order = np.arange(N)
    elif cfg.placement != "shuffled":
        raise ValueError(f"unknown placement {cfg.placement!r}")

    M = max(1, max(nblk) if nblk else 1)
    tables = np.full((S, M), -1, dtype=np.int32)
    pairs = []
    cursor = 0

    def take(n):
        nonlocal cursor
        out = order[cursor:cursor + n]
        cursor += n
        return out

    if shared:
        for p in range(S // spp):
            prompt_blocks = take(pb)
            for k in range(spp):
                s = p * spp + k
                row = list(prompt_blocks)
                if rem and k < spp - 1:
                    (copy,) = take(1)
                    pairs.append((prompt_blocks[-1], copy))
                    row[-1] = copy
                row += list(take(nblk[s] - pb))
                tables[s, :nblk[s]] = row
    else:
        for s in range(S):
            tables[s, skip[s]:nblk[s]] = take(nblk[s] - skip[s])

    live = np.zeros((N, B), dtype=bool)
    new_slots = np.full(S, -1, dtype=np.int32)
    for s in range(S):
        L = int(lens[s])
        if L == 0:
            continue
        t = np.arange(skip[s] * B, L - 1)
        live[tables[s, t // B], t % B] = True
        last = L - 1
        new_slots[s] = tables[s, last // B] * B + last % B

    return Layout(cfg=cfg, seed=seed, context_lens=lens, block_tables=tables, num_blocks=N,
                  pool_order=order, used_blocks=cursor, new_slots=new_slots, live=live,
                  cow_pairs=np.array(pairs, dtype=np.int32).reshape(-1, 2),
                  cow_rows=(cfg.prompt_len % B) if shared else 0)


def shared_prefix_groups(layout: Layout):
    """Groups of a shared-prefix layout and their shared tokens.

    Returns (members int32 [prompts, samples], prefix_lens int32 [S]): the
    samples of each prompt, and for every sequence the prompt tokens held in
    whole blocks that all samples of the prompt share (the partial last
    prompt block is a private copy after the copy-on-write)."""
    cfg = layout.cfg
    S = len(layout.context_lens)
    spp = cfg.samples_per_prompt
    members = np.arange(S, dtype=np.int32).reshape(S // spp, spp)
    prefix = np.full(S, (cfg.prompt_len // cfg.block_size) * cfg.block_size, dtype=np.int32)
    return members, prefix
