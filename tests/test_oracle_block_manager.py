"""Pins of the oracle's block manager: structural invariants under random
operation sequences, the pages' worked numbers, and the shared-prefix workload
structure."""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import BlockManager, BlockManagerError, NoFreeBlocks
from synthetic import CONFIGS, kv_bytes, make_layout

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_worked_numbers.json")))


def check_invariants(bm: BlockManager):
    N, B = bm.num_blocks, bm.block_size
    counted = [0] * N
    for seq, table in bm.tables.items():
        L = bm.lengths[seq]
        assert len(table) == -(-L // B), "a sequence holds exactly ceil(L/B) blocks"
        released = sum(1 for b in table if b < 0)
        assert all(b < 0 for b in table[:released]), "only a leading run of blocks is released"
        assert released == 0 or released * B < L, "the last token's block is never released"
        for b in table:
            if b >= 0:
                counted[b] += 1
    assert counted == bm.refcount, "reference count = number of tables naming the block"
    free = list(bm.free)
    assert len(set(free)) == len(free), "free list holds a block twice"
    used = {b for b in range(N) if bm.refcount[b] > 0}
    assert used.isdisjoint(free) and used | set(free) == set(range(N)), "free + used = pool"


def _snapshot(bm):
    return ({s: list(t) for s, t in bm.tables.items()}, dict(bm.lengths), list(bm.refcount), list(bm.free))


ops = st.lists(st.tuples(st.sampled_from(["add", "fork", "append", "append", "append", "free", "slide"]),
                         st.integers(0, 7), st.integers(0, 7), st.integers(1, 40)), max_size=60)


@settings(max_examples=200, deadline=None)
@given(ops=ops, N=st.integers(1, 24), B=st.sampled_from([1, 2, 4, 16]), seed=st.integers(0, 2**16))
def test_invariants_hold_under_random_operations(ops, N, B, seed):
    bm = BlockManager(N, B, np.random.default_rng(seed).permutation(N))
    for op, a, b, n in ops:
        before = _snapshot(bm)
        try:
            if op == "add":
                bm.add_seq(a)
            elif op == "fork":
                bm.fork(a, b)
            elif op == "free":
                bm.free_seq(a)
            elif op == "slide":
                L = bm.lengths.get(a, 0)
                n_rel = bm.slide_window(a, n)
                first = L - n
                assert all(b < 0 for b in bm.tables[a][:max(0, first) // B]), "blocks before the window released"
                assert all(b >= 0 for b in bm.tables[a][max(0, first) // B:]), "window blocks kept"
                assert n_rel <= max(0, first) // B
            else:
                for _ in range(n):
                    others = {s: list(t) for s, t in bm.tables.items() if s != a}
                    slot, cow = bm.append(a)
                    blk = slot // B
                    assert bm.refcount[blk] == 1, "the written block is owned by the writer alone"
                    assert bm.tables[a][(bm.lengths[a] - 1) // B] == blk
                    if cow is not None:
                        src, dst = cow
                        assert dst == blk and bm.refcount[src] >= 1
                    for s, t in others.items():
                        assert bm.tables[s] == t, "copy-on-write must leave other sequences alone"
                    before = _snapshot(bm)
        except NoFreeBlocks:
            assert _snapshot(bm) == before, "a failed allocation must not change state"
        except BlockManagerError:
            assert _snapshot(bm) == before
        check_invariants(bm)


def test_exhaustion_and_release():
    bm = BlockManager(2, 4)
    bm.add_seq(0)
    for _ in range(8):
        bm.append(0)
    with pytest.raises(NoFreeBlocks):
        bm.append(0)
    assert bm.seq_len(0) == 8
    bm.free_seq(0)
    assert bm.num_free() == 2
    bm.add_seq(1)
    bm.append(1)


def test_fork_then_divergence_copies_once_per_writer():
    bm = BlockManager(10, 4, list(range(10)))
    bm.add_seq(0)
    for _ in range(6):              # blocks 0 (full) and 1 (2 of 4 used)
        bm.append(0)
    bm.fork(0, 1)
    bm.fork(0, 2)
    assert bm.refcount[:2] == [3, 3]
    slot, cow = bm.append(1)
    assert cow == (1, 2) and slot == 2 * 4 + 2
    slot, cow = bm.append(2)
    assert cow == (1, 3) and slot == 3 * 4 + 2
    slot, cow = bm.append(0)        # last holder writes in place
    assert cow is None and slot == 1 * 4 + 2
    assert bm.refcount[:4] == [3, 1, 1, 1]
    bm.free_seq(1)
    assert list(bm.free)[0] == 2 and bm.refcount[0] == 2


def test_naive_allocation_example_and_paged_waste():
    ex, bound = GOLDEN["naive_allocation_example"], GOLDEN["paged_waste_bound"]
    S, max_len, avg = ex["num_seqs"], ex["max_len"], ex["avg_len"]
    naive = S * max_len
    used = S * avg
    assert naive // 1000 == 65 and naive == 65536               # printed, truncated, as "65K"
    assert used == 6400                                          # printed as "6.4K"
    assert round(100 * (1 - used / naive)) == ex["naive_waste_as_printed_percent"]
    B = bound["block_size_example"]
    bm = BlockManager(S * math.ceil(max_len / B), B)
    for s in range(S):
        bm.add_seq(s)
        for _ in range(avg):
            bm.append(s)
    held = sum(len(t) for t in bm.tables.values()) * B
    assert (held - used) / held < bound["max_waste_fraction"]
    assert held - used <= S * (B - 1), "waste is under one block per sequence"


def test_block_table_metadata_overhead():
    g = GOLDEN["block_table_size"]
    for idx in (2, 3, 4, 5):
        cfg = CONFIGS[idx]
        lay = make_layout(cfg, seed=idx)
        S, M = lay.block_tables.shape
        assert lay.block_tables.nbytes == S * M * g["bytes_per_entry"]
        pool = 2 * lay.num_blocks * cfg.num_kv_heads * cfg.block_size * cfg.head_dim * cfg.dtype_bytes
        assert lay.block_tables.nbytes / pool < g["max_fraction_of_memory"]


def test_kv_bytes_per_token_order_of_magnitude():
    g = GOLDEN["kv_bytes_per_token_13b"]
    per_token = g["layers"] * kv_bytes([1], g["kv_heads"], g["head_dim"], g["dtype"])
    assert 0.5 * g["per_token_order_bytes"] < per_token < 2 * g["per_token_order_bytes"]
    per_user = per_token * g["context"]
    assert 0.5 * g["per_user_approx_bytes"] < per_user < 1.5 * g["per_user_approx_bytes"]


def test_shared_prefix_workload_is_what_the_block_manager_builds():
    """Driving the twin through prompt, forks and sample tails reproduces the
    shared-prefix workload's tables and copy-on-write pairs exactly."""
    cfg = CONFIGS[5].scaled(num_seqs=16)
    lay = make_layout(cfg, seed=5)
    bm = BlockManager(lay.num_blocks, cfg.block_size, lay.pool_order)
    spp, P = cfg.samples_per_prompt, cfg.prompt_len
    pairs = []
    for p in range(cfg.num_seqs // spp):
        root = p * spp
        bm.add_seq(root)
        for _ in range(P):
            bm.append(root)
        for k in range(1, spp):
            bm.fork(root, root + k)
        for k in range(spp):
            s = root + k
            for _ in range(int(lay.context_lens[s]) - P):
                slot, cow = bm.append(s)
                if cow:
                    pairs.append(cow)
    for s in range(cfg.num_seqs):
        t = bm.block_table(s)
        assert t == list(lay.block_tables[s, :len(t)])
        assert bm.seq_len(s) == lay.context_lens[s]
        last = int(lay.context_lens[s]) - 1
        assert t[last // cfg.block_size] * cfg.block_size + last % cfg.block_size == lay.new_slots[s]
    assert pairs == [tuple(p) for p in lay.cow_pairs.tolist()]
    assert len(pairs) == (spp - 1) * (cfg.num_seqs // spp)
    check_invariants(bm)


def test_swap_out_and_back_leaves_attention_bitwise_equal():
    """A sequence moved to a host pool (blocks copied there) and back to the
    device pool reads the same keys and values: attention is bit-identical,
    and a move that finds too few free blocks changes nothing."""
    import oracle
    from synthetic import to_storage
    rng = np.random.default_rng(12)
    N, Nh, B, Hkv, D = 24, 16, 4, 2, 8
    kc = to_storage(rng.standard_normal((N, Hkv, B, D)), "f16")
    vc = to_storage(rng.standard_normal((N, Hkv, B, D)), "f16")
    hk = np.zeros((Nh, Hkv, B, D), dtype=np.float16)
    hv = np.zeros_like(hk)
    dev, host = BlockManager(N, B, rng.permutation(N)), BlockManager(Nh, B, rng.permutation(Nh))
    for s, L in enumerate([13, 6]):
        dev.add_seq(s)
        for _ in range(L):
            dev.append(s)
    dev.fork(0, 2)
    q = to_storage(rng.standard_normal((1, 2, D)), "f16")

    def attend(bm, k, v, s):
        t = np.array([bm.block_table(s)], dtype=np.int32)
        return oracle.paged_attention_decode(q, k, v, t, [bm.seq_len(s)], 0.3, B, Hkv, "f16")

    before = attend(dev, kc, vc, 0)
    oracle.swap_blocks(kc, vc, hk, hv, dev.move_seq(host, 0))
    assert 0 not in dev.tables and np.array_equal(attend(host, hk, hv, 0), before)
    assert dev.block_table(2) and all(dev.refcount[b] == 1 for b in dev.block_table(2)), "shared blocks keep fork 2"
    pairs = host.move_seq(dev, 0)
    oracle.swap_blocks(hk, hv, kc, vc, pairs)
    assert np.array_equal(attend(dev, kc, vc, 0), before)
    small = BlockManager(2, B)
    snap = (dict(dev.tables), list(dev.refcount), list(dev.free))
    with pytest.raises(NoFreeBlocks):
        dev.move_seq(small, 0)
    assert (dict(dev.tables), list(dev.refcount), list(dev.free)) == snap
