"""Pins of the oracle's cache scatter and block copy: whole-pool byte
comparisons against expectations built by other means, and consistency of the
scatter's addressing with the attention's gather."""
import numpy as np
import pytest

import oracle
from synthetic import POISON_BITS, to_storage


def _pool(rng, N, Hkv, B, D, dtype):
    return to_storage(rng.standard_normal((N, Hkv, B, D)), dtype)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_scatter_changes_exactly_the_named_slots(dtype):
    rng = np.random.default_rng(3)
    N, Hkv, B, D, T = 9, 3, 8, 16, 20
    kc, vc = _pool(rng, N, Hkv, B, D, dtype), _pool(rng, N, Hkv, B, D, dtype)
    k, v = _pool(rng, T, Hkv, 1, D, dtype)[:, :, 0], _pool(rng, T, Hkv, 1, D, dtype)[:, :, 0]
    slots = rng.choice(N * B, size=T, replace=False).astype(np.int32)
    slots[[2, 7]] = -1                                  # skipped tokens
    k0, v0 = kc.copy(), vc.copy()
    oracle.reshape_and_cache(k, v, kc, vc, slots, B)
    # Expected pool: flatten (block, offset) with numpy's own index arithmetic.
    want_k = k0.transpose(0, 2, 1, 3).reshape(N * B, Hkv, D).copy()
    want_v = v0.transpose(0, 2, 1, 3).reshape(N * B, Hkv, D).copy()
    for i, s in enumerate(slots):
        if s >= 0:
            blk, off = np.unravel_index(s, (N, B))
            want_k[blk * B + off] = k[i]
            want_v[blk * B + off] = v[i]
    got_k = kc.transpose(0, 2, 1, 3).reshape(N * B, Hkv, D)
    got_v = vc.transpose(0, 2, 1, 3).reshape(N * B, Hkv, D)
    assert got_k.tobytes() == want_k.tobytes()
    assert got_v.tobytes() == want_v.tobytes()


def test_scatter_then_gather_round_trip():
    """Tokens scattered to the slots a block table implies come back, in
    order, from the gather the attention uses."""
    rng = np.random.default_rng(4)
    N, Hkv, B, D, L = 12, 2, 16, 8, 41
    table = rng.permutation(N)[: -(-L // B)].astype(np.int32)
    kc = np.full((N, Hkv, B, D), POISON_BITS["bf16"], dtype=np.uint16)
    vc = kc.copy()
    k = to_storage(rng.standard_normal((L, Hkv, D)), "bf16")
    v = to_storage(rng.standard_normal((L, Hkv, D)), "bf16")
    t = np.arange(L)
    slots = (table[t // B] * B + t % B).astype(np.int32)
    oracle.reshape_and_cache(k, v, kc, vc, slots, B)
    for h in range(Hkv):
        assert np.array_equal(oracle.gather_sequence(kc, table, L, h, B), k[:, h])
        assert np.array_equal(oracle.gather_sequence(vc, table, L, h, B), v[:, h])


def test_scatter_rejects_slot_outside_pool():
    kc = np.zeros((2, 1, 4, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.reshape_and_cache(np.zeros((1, 1, 4), np.float32), np.zeros((1, 1, 4), np.float32),
                                 kc, kc.copy(), np.array([8], np.int32), 4)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_copy_blocks_is_a_bitwise_copy_and_order_free(dtype):
    rng = np.random.default_rng(5)
    N, Hkv, B, D = 16, 2, 8, 8
    kc, vc = _pool(rng, N, Hkv, B, D, dtype), _pool(rng, N, Hkv, B, D, dtype)
    kc.view(np.uint8)[0, 0, 0, :4] = 0xFF                 # a NaN pattern must copy as is
    perm = rng.permutation(N)
    pairs = np.stack([perm[:5], perm[5:10]], axis=1).astype(np.int32)
    k0, v0 = kc.copy(), vc.copy()
    oracle.copy_blocks(kc, vc, pairs)
    for blk in range(N):
        srcs = [s for s, d in pairs if d == blk]
        ek = k0[srcs[0]] if srcs else k0[blk]
        ev = v0[srcs[0]] if srcs else v0[blk]
        assert kc[blk].tobytes() == ek.tobytes()
        assert vc[blk].tobytes() == ev.tobytes()
    kr, vr = k0.copy(), v0.copy()
    oracle.copy_blocks(kr, vr, pairs[::-1])
    assert kr.tobytes() == kc.tobytes() and vr.tobytes() == vc.tobytes()


def test_copy_blocks_rejects_ambiguous_pairs():
    kc = np.zeros((4, 1, 2, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.copy_blocks(kc, kc.copy(), [(0, 1), (2, 1)])     # duplicate destination
    with pytest.raises(ValueError):
        oracle.copy_blocks(kc, kc.copy(), [(0, 1), (1, 2)])     # destination is a source


def test_fp8_store_changes_only_the_slots_and_rounds_to_nearest():
    """Quantized store: only the target slots change, and each stored code is
    a nearest E4M3 value of x / scale (within half a code step of it)."""
    from oracle import decode_e4m3, reshape_and_cache_fp8
    from synthetic import to_storage
    rng = np.random.default_rng(4)
    N, Hkv, B, D, T = 12, 3, 8, 16, 20
    kc = rng.integers(0, 256, size=(N, Hkv, B, D)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(N, Hkv, B, D)).astype(np.uint8)
    k = to_storage(rng.standard_normal((T, Hkv, D)) * 3, "bf16")
    v = to_storage(rng.standard_normal((T, Hkv, D)) * 3, "bf16")
    slots = rng.choice(N * B, size=T, replace=False).astype(np.int32)
    slots[[2, 7]] = -1
    k2, v2 = kc.copy(), vc.copy()
    reshape_and_cache_fp8(k, v, k2, v2, slots, B, 0.05, 0.02, "bf16")
    touched = np.zeros((N, B), dtype=bool)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        touched[s // B, s % B] = True
        x = oracle.decode(k[i], "bf16").astype(np.float32) / np.float32(0.05)
        got = decode_e4m3(k2[s // B, :, s % B, :])
        step = np.where(np.abs(got) < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(got), 2.0 ** -6))) - 3))
        assert np.all(np.abs(got - x) <= step / 2 + 1e-12)
    untouched = ~np.broadcast_to(touched[:, None, :, None], kc.shape)
    assert np.array_equal(k2[untouched], kc[untouched])
    assert np.array_equal(v2[untouched], vc[untouched])
