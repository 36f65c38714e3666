"""Beam search on the GPU under block churn: every step forks beams, frees
the losers, copies shared last blocks and appends a token to every beam
(pkv_copy_blocks + pkv_decode_step).  The oracle runs the same steps on a
host pool with its own block manager, scatter, copy and attention; the
attention rows of every step must agree to the tolerance, and the whole
device pool must equal the host pool byte for byte at the end."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_339_amd as pkv
from synthetic import BEAM_CONFIGS, POISON_BITS, beam_parents, prompt_values, step_values
from tests.gpu_util import assert_rows_close, ints, say, to_device, to_storage_np, widen

pytestmark = pytest.mark.gpu

NP_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


@pytest.mark.parametrize("R,W,P,steps,B,dtype,Hq,Hkv", [
    (2, 4, 37, 12, 8, "f16", 4, 4),
    (3, 2, 16, 20, 16, "bf16", 16, 2),
])
def test_beam_search_steps_match_the_oracle(R, W, P, steps, B, dtype, Hq, Hkv):
    cfg = BEAM_CONFIGS[7].scaled(num_requests=R, beam_width=W, prompt_len=P, steps=steps, block_size=B,
                                 dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv)
    seed = 11
    parents = beam_parents(cfg, seed)
    N = cfg.pool_blocks()
    D = cfg.head_dim
    width = np.uint32 if dtype == "f32" else np.uint16
    host_k = np.full((N, Hkv, B, D), POISON_BITS[dtype], dtype=width).view(NP_STORAGE[dtype])
    host_v = host_k.copy()
    dev_k, dev_v = to_device(host_k, dtype), to_device(host_v, dtype)
    order = np.random.default_rng(seed).permutation(N)
    cache = pkv.BeamSearchCache(R, W, N, B, order)
    twin = oracle.BlockManager(N, B, order)

    pk, pv = prompt_values(cfg, seed)
    slots = cache.prefill(P)
    for r in range(R):
        twin.add_seq(r * W)
        for _ in range(P):
            twin.append(r * W)
        kk, vv = pk[r], pv[r]
        pkv.reshape_and_cache(to_device(kk, dtype), to_device(vv, dtype), dev_k, dev_v, ints(slots[r]))
        oracle.reshape_and_cache(kk, vv, host_k, host_v, slots[r], B)

    bank = 0
    for t in range(steps):
        seqs, slots, pairs = cache.step(parents[t])
        # The oracle's own block manager takes the same decisions.
        old = list(range(bank * R * W, (bank + 1) * R * W))
        new = list(range((1 - bank) * R * W, (2 - bank) * R * W))
        for r in range(R):
            for b in range(W):
                twin.fork(old[r * W + (0 if t == 0 else int(parents[t, r, b]))], new[r * W + b])
        for r in range(R):
            for b in range(W):
                if t > 0 or b == 0:
                    twin.free_seq(old[r * W + b])
        bank = 1 - bank
        t_slots, t_pairs = [], []
        for s in new:
            slot, cow = twin.append(s)
            t_slots.append(slot)
            if cow is not None:
                t_pairs.append(cow)
        assert slots.tolist() == t_slots and pairs.tolist() == [list(p) for p in t_pairs]

        M = max(len(twin.block_table(s)) for s in new)
        tables, lens = cache.tables(M)
        q, kn, vn = step_values(cfg, seed, t)
        say(f"beam step {t}: {len(pairs)} copies, lengths {lens.min()}..{lens.max()}")
        if len(pairs):
            pkv.copy_blocks(dev_k, dev_v, ints(pairs))
            oracle.copy_blocks(host_k, host_v, pairs)
        out = torch.empty_like(to_device(q, dtype))
        pkv.decode_step(out, to_device(q, dtype), to_device(kn, dtype), to_device(vn, dtype), dev_k, dev_v,
                        ints(slots), ints(tables), ints(lens), cfg.scale, B, Hkv, int(lens.max()))
        torch.cuda.synchronize()
        oracle.reshape_and_cache(kn, vn, host_k, host_v, slots, B)
        want = oracle.paged_attention_decode(q, host_k, host_v, tables, lens, cfg.scale, B, Hkv, dtype)
        assert_rows_close(widen(out), want, dtype, f"beam step {t}")
        # The same attention with each request's prompt blocks read once for its beams.
        members, prefix = cache.shared_prefix()
        out2 = torch.empty_like(out)
        pkv.paged_attention_decode_shared_prefix(out2, to_device(q, dtype), dev_k, dev_v, ints(tables), ints(lens),
                                                 ints(prefix), ints(members), int(prefix.max()), cfg.scale, B,
                                                 Hkv, int(lens.max()))
        torch.cuda.synchronize()
        assert_rows_close(widen(out2), want, dtype, f"beam step {t}, shared-prefix call")
    assert to_storage_np(dev_k, dtype).tobytes() == host_k.tobytes(), "key pool differs after the search"
    assert to_storage_np(dev_v, dtype).tobytes() == host_v.tobytes(), "value pool differs after the search"
    cache.close()
