"""Host control plane of beam search over the paged KV cache.

Parallel sampling and beam search share a prompt's blocks by reference
instead of copying them ("pagedattention vllm" glossary, "Copy-on-Write
Sharing > Use Cases" and "Use Cases > Beam Search"; "PagedAttention",
lastdictionary).  At every step each new beam continues one old beam: it
forks the parent's block table (one more reference per block), the old
beams are released, and one token is appended to every new beam, which
copies a shared last block first ("Copy-on-Write Sharing > Divergence
Handling").  Everything here runs on the host through the library's C++
block manager; the copies, token stores and attention are the caller's
pkv_copy_blocks and pkv_decode_step calls with the arrays returned (or
pkv_paged_attention_decode_shared_prefix with shared_prefix(), which reads
each request's prompt blocks once for all its beams).

Sequence ids alternate between two banks of R*W ids so that a step's new
beams never collide with the old ones they fork from.
"""
from __future__ import annotations

import numpy as np

from .ops import BlockManager


class BeamSearchCache:
    def __init__(self, num_requests: int, beam_width: int, num_blocks: int, block_size: int,
                 free_order=None):
        self.R, self.W, self.B = num_requests, beam_width, block_size
        self.bm = BlockManager(num_blocks, block_size, 2 * num_requests * beam_width, free_order)
        self.bank = 0
        self.started = False
        self.prompt_len = 0

    def seq_ids(self, bank=None) -> np.ndarray:
        """Ids of the live beams, request-major: [R * W]."""
        bank = self.bank if bank is None else bank
        n = self.R * self.W
        return np.arange(bank * n, (bank + 1) * n, dtype=np.int32)

    def prefill(self, prompt_len: int) -> np.ndarray:
        """Beam 0 of every request takes the prompt.  Returns the slots of the
        prompt tokens, [R, prompt_len] (request r's keys and values go there)."""
        self.prompt_len = prompt_len
        ids = self.seq_ids()
        slots = np.zeros((self.R, prompt_len), dtype=np.int32)
        for r in range(self.R):
            seq = int(ids[r * self.W])
            self.bm.add_seq(seq)
            for t in range(prompt_len):
                slots[r, t], cow = self.bm.append(seq)
                assert cow is None
        return slots

    def step(self, parents: np.ndarray):
        """One decode step.  parents: int [R, W], new beam b of request r
        continues old beam parents[r, b] (on the first step every new beam
        continues beam 0, the prompt).  Returns (seqs, slots, pairs): the new
        beams' ids [R*W], the slot of each one's new token [R*W], and the
        copy-on-write pairs [P, 2] to copy before those tokens are stored."""
        old = self.seq_ids()
        new = self.seq_ids(1 - self.bank)
        chosen = np.zeros((self.R, self.W), dtype=np.int64) if not self.started else np.asarray(parents)
        rows = np.arange(self.R)[:, None] * self.W
        self.bm.fork_batch(old[(rows + chosen).ravel()], new)
        self.bm.free_batch(old if self.started else old[::self.W])
        self.started = True
        self.bank = 1 - self.bank
        slots, pairs = self.bm.append_batch(new)
        return new, slots, pairs

    def shared_prefix(self):
        """Groups for pkv_paged_attention_decode_shared_prefix over the rows of
        tables(): the beams of each request [R, W] (rows, request-major), and
        for every beam the prompt tokens held in whole blocks.  Every beam
        descends from its request's prompt, so those blocks stay shared by all
        W beams; a partial last prompt block is copied on divergence and is
        read with each beam's own tokens."""
        members = np.arange(self.R * self.W, dtype=np.int32).reshape(self.R, self.W)
        prefix = np.full(self.R * self.W, self.prompt_len // self.B * self.B, dtype=np.int32)
        return members, prefix

    def tables(self, max_blocks: int):
        """Block tables [R*W, max_blocks] (-1 padded) and lengths of the live beams."""
        return self.bm.export(self.seq_ids(), max_blocks)

    def close(self):
        self.bm.close()
