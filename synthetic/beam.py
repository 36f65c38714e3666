"""Seeded beam-search workloads: which parent each new beam continues at every
step, and the N(0, 1) values of prompts, new tokens and queries.

Integers and values only: no block manager, scatter or attention here.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
import math

import numpy as np

from .configs import DTYPE_BYTES
from .values import to_storage


@dataclass(frozen=True)
class BeamConfig:
    name: str
    num_requests: int
    beam_width: int
    prompt_len: int
    steps: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    block_size: int
    pool_factor: float = 1.25
    cache_policy: str = "keep"   # the beams of a request share their prompt blocks

    @property
    def num_seqs(self) -> int:
        return self.num_requests * self.beam_width

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def dtype_bytes(self) -> int:
        return DTYPE_BYTES[self.dtype]

    def pool_blocks(self) -> int:
        """Blocks enough for every request's prompt plus every beam holding
        private blocks for all generated tokens (an upper bound), times the
        pool factor."""
        B = self.block_size
        prompt = -(-self.prompt_len // B)
        own = self.beam_width * (-(-(self.steps + 1) // B) + 1)
        return int(math.ceil(self.pool_factor * self.num_requests * (prompt + own)))

    def scaled(self, **kw) -> "BeamConfig":
        return replace(self, **kw)


# Beam search over a Llama-2-7B-shaped layer: 16 requests x 8 beams, a
# 1024-token prompt shared by the beams of a request, 32 decode steps.
BEAM_CONFIGS = {
    7: BeamConfig("beam8_llama2_7b_layer_f16", num_requests=16, beam_width=8, prompt_len=1024, steps=32,
                  num_q_heads=32, num_kv_heads=32, head_dim=128, dtype="f16", block_size=16),
}


def beam_parents(cfg: BeamConfig, seed: int) -> np.ndarray:
    """int32 [steps, R, W]: new beam b of request r at step t continues old
    beam parents[t, r, b].  Parents are drawn from the best half of the beams
    with a bias towards the first (beams collapse onto a few survivors, as in
    a real search), so some beams are forked several times and others die."""
    rng = np.random.default_rng([seed, 100])
    W = cfg.beam_width
    top = max(1, W // 2)
    weights = np.array([2.0 ** -i for i in range(top)])
    weights /= weights.sum()
    return rng.choice(top, size=(cfg.steps, cfg.num_requests, W), p=weights).astype(np.int32)


def prompt_values(cfg: BeamConfig, seed: int):
    """k, v of every request's prompt: [R, prompt_len, Hkv, D] in storage format."""
    shape = (cfg.num_requests, cfg.prompt_len, cfg.num_kv_heads, cfg.head_dim)
    k = to_storage(np.random.default_rng([seed, 101]).standard_normal(shape), cfg.dtype)
    v = to_storage(np.random.default_rng([seed, 102]).standard_normal(shape), cfg.dtype)
    return k, v


def step_values(cfg: BeamConfig, seed: int, step: int):
    """q [S, Hq, D], k_new, v_new [S, Hkv, D] of one decode step (S = R * W)."""
    rng = np.random.default_rng([seed, 103, step])
    S = cfg.num_seqs
    q = to_storage(rng.standard_normal((S, cfg.num_q_heads, cfg.head_dim)), cfg.dtype)
    k = to_storage(rng.standard_normal((S, cfg.num_kv_heads, cfg.head_dim)), cfg.dtype)
    v = to_storage(rng.standard_normal((S, cfg.num_kv_heads, cfg.head_dim)), cfg.dtype)
    return q, k, v
