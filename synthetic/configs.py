"""Decode workloads for paged attention, as plain data.

Each workload is one decode step over a batch of sequences whose keys and
values sit in fixed-size blocks of a shared physical pool.  The shapes are
those of single attention layers of well-known models (no weights are
involved); every value is drawn from N(0, 1).

Nothing in this package computes attention, scatters a token or copies a
block: it only decides lengths, block placement and input values, so that the
CPU oracle and the GPU library can be fed identical bits.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
import math

DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str              # "f32" | "f16" | "bf16"
    block_size: int
    lengths: str            # "fixed" | "uniform" | "lognormal" | "shared_prefix"
    fixed_lengths: tuple = ()
    len_lo: int = 1
    len_hi: int = 1
    lognormal_median: float = 0.0
    lognormal_sigma: float = 1.0
    pool_blocks: int = 0    # explicit pool size; 0 = ceil(pool_factor * need)
    pool_factor: float = 1.2
    partition_size: int = 0  # split-K partition in tokens; 0 = library default
    prompt_len: int = 0      # shared-prefix workloads only
    samples_per_prompt: int = 0
    sliding_window: int = 0  # attend to the last W tokens; blocks wholly before them are released
    kv_format: str = "same"  # "same" (caches in `dtype`) or "fp8_e4m3" (8-bit codes with scales)
    k_scale: float = 1.0
    v_scale: float = 1.0
    placement: str = "shuffled"  # pool order: "shuffled" (seeded permutation) or "contiguous" (identity)
    cache_policy: str = "stream"  # attention loads: "stream" (nontemporal) or "keep" (shared blocks re-read)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def dtype_bytes(self) -> int:
        return DTYPE_BYTES[self.dtype]

    @property
    def kv_dtype(self) -> str:
        """Storage format of the caches: `dtype`, or "fp8" (E4M3 codes)."""
        return "fp8" if self.kv_format == "fp8_e4m3" else self.dtype

    def scaled(self, **kw) -> "DecodeConfig":
        return replace(self, **kw)


# The decode workloads.  Shapes: Llama-2-7B (32 heads), Llama-2-13B
# (40 heads) and a 70B-class grouped-query layer (64 query heads over 8 KV
# heads); block size 16 is the default the glossary pages give, 32 the size
# one of them recommends for balance.
CONFIGS = {
    1: DecodeConfig("tiny_mha_f32", num_seqs=4, num_q_heads=2, num_kv_heads=2,
                    head_dim=64, dtype="f32", block_size=16, lengths="fixed",
                    fixed_lengths=(5, 17, 33, 64), pool_blocks=32),
    2: DecodeConfig("llama2_7b_layer_f16", num_seqs=64, num_q_heads=32, num_kv_heads=32,
                    head_dim=128, dtype="f16", block_size=16, lengths="uniform",
                    len_lo=128, len_hi=2048),
    3: DecodeConfig("llama2_13b_layer_bf16", num_seqs=128, num_q_heads=40, num_kv_heads=40,
                    head_dim=128, dtype="bf16", block_size=16, lengths="lognormal",
                    lognormal_median=400.0, lognormal_sigma=1.0, len_lo=1, len_hi=4096),
    4: DecodeConfig("gqa70b_layer_bf16", num_seqs=256, num_q_heads=64, num_kv_heads=8,
                    head_dim=128, dtype="bf16", block_size=32, lengths="uniform",
                    len_lo=1024, len_hi=32768, partition_size=512),
    5: DecodeConfig("shared_prefix_sampling_bf16", num_seqs=512, num_q_heads=40, num_kv_heads=40,
                    head_dim=128, dtype="bf16", block_size=16, lengths="shared_prefix",
                    len_lo=1, len_hi=512, prompt_len=1000, samples_per_prompt=8,
                    partition_size=1024, cache_policy="keep"),
    # A sliding-window grouped-query layer (Mistral-7B-like: 32 query heads
    # over 8 KV heads, 4096-token window): only the blocks the window touches
    # hold data; table entries before them are -1.
    6: DecodeConfig("swa_mistral7b_layer_bf16", num_seqs=64, num_q_heads=32, num_kv_heads=8,
                    head_dim=128, dtype="bf16", block_size=16, lengths="uniform",
                    len_lo=1024, len_hi=16384, sliding_window=4096),
    # The Llama-2-7B-shaped layer with an 8-bit E4M3 KV cache (per-tensor
    # scales 1/32; paging combined with quantization).
    8: DecodeConfig("llama2_7b_layer_fp8kv", num_seqs=64, num_q_heads=32, num_kv_heads=32,
                    head_dim=128, dtype="f16", block_size=16, lengths="uniform",
                    len_lo=128, len_hi=2048, kv_format="fp8_e4m3", k_scale=1.0 / 32, v_scale=1.0 / 32),
    # The 70B-style grouped-query layer with the same 8-bit cache: quantized
    # pages shared by 8 query heads each, on the matrix cores.
    9: DecodeConfig("gqa70b_layer_fp8kv", num_seqs=256, num_q_heads=64, num_kv_heads=8,
                    head_dim=128, dtype="bf16", block_size=32, lengths="uniform",
                    len_lo=1024, len_hi=32768, kv_format="fp8_e4m3", k_scale=1.0 / 32, v_scale=1.0 / 32),
    # A multi-query layer (Falcon-7B-like: 71 query heads over one KV head,
    # head_dim 64): the group is larger than one workgroup computes, so each
    # (sequence, partition) is served by 5 workgroups of 15, 15, 15, 15 and
    # 11 heads that read the same key/value tiles.
    10: DecodeConfig("mqa_falcon7b_layer_bf16", num_seqs=256, num_q_heads=71, num_kv_heads=1,
                     head_dim=64, dtype="bf16", block_size=16, lengths="uniform",
                     len_lo=1024, len_hi=8192),
}


def kv_bytes(context_lens, num_kv_heads: int, head_dim: int, dtype: str, sliding_window: int = 0) -> int:
    """Logical K+V bytes one decode step reads: sum(L) * Hkv * D * 2 * bytes,
    with L capped at the window when there is one."""
    lens = [min(int(x), sliding_window) if sliding_window > 0 else int(x) for x in context_lens]
    return sum(lens) * num_kv_heads * head_dim * 2 * DTYPE_BYTES[dtype]
