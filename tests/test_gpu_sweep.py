"""Seeded sweep over combinations the hand-picked GPU cases may miss: for
each of 40 draws, a format, head counts, head_dim, block size, kernel,
window, partition size and ragged lengths (edge lengths included), checked
against the oracle for the plain decode call; every other draw also groups
the batch into shared-prefix groups and checks the shared-prefix call."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_339_amd as pkv
from synthetic import DecodeConfig, host_values, make_layout
from tests.gpu_util import DeviceStep, assert_rows_close, ints, oracle_step, say, widen

pytestmark = pytest.mark.gpu


def draw_case(i):
    rng = np.random.default_rng(1000 + i)
    dtype = ["f32", "f16", "bf16"][i % 3]
    Hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16]))
    D = int(rng.choice([64, 128]))
    B = int(rng.choice([8, 16, 32, 64]))
    kernel = "valu" if dtype == "f32" else str(rng.choice(["auto", "valu", "mfma"]))
    S = int(rng.integers(1, 9))
    lens = rng.integers(1, 700, size=S)
    edges = [1, B - 1, B, B + 1, 31, 32, 33, 511, 512, 513]
    for k in range(S):
        if rng.random() < 0.3:
            lens[k] = max(1, edges[int(rng.integers(len(edges)))])
    window = int(rng.choice([0, 0, 1, 40, 300]))
    align = max(B, 32) if kernel != "valu" else B
    part = int(rng.choice([0, 0, align, 4 * align]))
    cfg = DecodeConfig(f"sweep{i}", num_seqs=S, num_q_heads=g * Hkv, num_kv_heads=Hkv, head_dim=D, dtype=dtype,
                       block_size=B, lengths="fixed", fixed_lengths=tuple(int(x) for x in lens),
                       sliding_window=window)
    return cfg, kernel, part


@pytest.mark.parametrize("i", range(40))
def test_random_combinations_match_the_oracle(i):
    cfg, kernel, part = draw_case(i)
    lay = make_layout(cfg, seed=2000 + i)
    host = host_values(lay)
    say(f"sweep {i}: {cfg.dtype} Hq={cfg.num_q_heads} Hkv={cfg.num_kv_heads} D={cfg.head_dim} B={cfg.block_size} "
        f"{kernel} window={cfg.sliding_window} partition={part} lens={list(cfg.fixed_lengths)}")
    step = DeviceStep.from_host(lay, host)
    step.scatter()
    got = widen(step.attend(partition_size=part, kernel=kernel))
    want, _, _ = oracle_step(lay, host)
    assert_rows_close(got, want, cfg.dtype, f"sweep {i}")

    if i % 2 == 0 and cfg.sliding_window == 0 and len(lay.context_lens) >= 2:
        # Pairs of consecutive sequences share nothing in this layout, so a
        # group's prefix is 0 tokens; groups still change the launches (the
        # grouped pass sees empty prefixes) and must not change the rows.
        S = len(lay.context_lens)
        members = np.full(((S + 1) // 2, 2), -1, dtype=np.int32)
        members.ravel()[:S] = np.arange(S)
        prefix = np.zeros(S, dtype=np.int32)
        out = torch.empty_like(step.q)
        pkv.paged_attention_decode_shared_prefix(out, step.q, step.k_cache, step.v_cache, step.tables, step.lens,
                                                 ints(prefix), ints(members), 0, cfg.scale, cfg.block_size,
                                                 cfg.num_kv_heads, lay.max_context_len, partition_size=part,
                                                 kernel=kernel)
        torch.cuda.synchronize()
        assert_rows_close(widen(out), want, cfg.dtype, f"sweep {i}, shared-prefix call")
