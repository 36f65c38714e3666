"""Pins of the oracle's paged decode attention, and proof that the pins bite:
each planted mistake in a copy of the oracle fails at least one of them."""
import numpy as np
import pytest

import oracle
import oracle.attention as oa
from oracle.formats import decode
from tests import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_passes_pin(check):
    check(oracle.paged_attention_decode)


def test_oracle_rejects_table_entries_outside_pool():
    rng = np.random.default_rng(0)
    K, V, q = pins.draw(rng, [20], 1, 1, 8, "f32")
    p = pins.Paged(K, V, q, 8, "f32", 0)
    p.table[0, 1] = -1
    with pytest.raises(ValueError):
        p.run(oracle.paged_attention_decode, 0.5, 1)


def test_zero_length_sequence_gives_zero_row():
    rng = np.random.default_rng(1)
    K, V, q = pins.draw(rng, [4, 3], 2, 2, 8, "f16")
    p = pins.Paged(K, V, q, 8, "f16", 0)
    p.lens[1] = 0
    out = p.run(oracle.paged_attention_decode, 0.5, 2)
    assert np.all(out[1] == 0)


# ---------------------------------------------------------------------------
# Planted mistakes.  Each is a small change to the oracle; the pins above must
# reject every one of them.
# ---------------------------------------------------------------------------

def _with_gather(fake_gather):
    def impl(*args, **kw):
        saved = oa.gather_sequence
        oa.gather_sequence = fake_gather
        try:
            return oa.paged_attention_decode(*args, **kw)
        finally:
            oa.gather_sequence = saved
    return impl


def _with_decode(fake_decode):
    def impl(*args, **kw):
        saved = oa.decode
        oa.decode = fake_decode
        try:
            return oa.paged_attention_decode(*args, **kw)
        finally:
            oa.decode = saved
    return impl


def _gather_offset_off_by_one(cache, row, length, h, B, start=0):
    n = -(-length // B)
    tiles = np.asarray(cache[np.asarray(row[:n], dtype=np.int64), h])
    tiles = np.roll(tiles, 1, axis=1)                  # in-block offset shifted
    return tiles.reshape(n * B, -1)[start:length]


def _gather_block_order_reversed(cache, row, length, h, B, start=0):
    n = -(-length // B)
    tiles = np.asarray(cache[np.asarray(row[:n], dtype=np.int64)[::-1], h])
    return tiles.reshape(n * B, -1)[start:length]


def _gather_head_and_offset_swapped(cache, row, length, h, B, start=0):
    # reads the pool as if it were laid out [N, B, Hkv, D]
    n = -(-length // B)
    arr = np.asarray(cache)
    N, Hkv, _, D = arr.shape
    tiles = arr.reshape(N, B, Hkv, D)[np.asarray(row[:n], dtype=np.int64)][:, :, h, :]
    return tiles.reshape(n * B, -1)[start:length]


def _gather_drops_last_token(cache, row, length, h, B, start=0):
    return oracle.gather_sequence(cache, row, max(1, length - 1), h, B, min(start, max(0, length - 2)))


def _gather_whole_last_block(cache, row, length, h, B, start=0):
    n = -(-length // B)
    tiles = np.asarray(cache[np.asarray(row[:n], dtype=np.int64), h])
    return tiles.reshape(n * B, -1)[start:]


def _decode_bf16_shift_15(raw, dtype):
    if dtype == "bf16":
        return (np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
    return decode(raw, dtype)


def _decode_f16_as_bf16(raw, dtype):
    if dtype == "f16":
        return decode(np.asarray(raw).view(np.uint16), "bf16")
    return decode(raw, dtype)


def _fnuz_like_decode(codes):
    """E4M3 decoded with exponent bias 8 (another 8-bit format's convention)."""
    return oracle.decode_e4m3(codes) / 2.0


def _mutant_body(head_of=None, drop_scale=False, no_normalise=False, no_max=False, scale_twice=False,
                 window_shift=0, window_from_start=False, ignore_k_scale=False, ignore_v_scale=False,
                 fp8_decode=None):
    def impl(q, k_cache, v_cache, block_tables, context_lens, scale, block_size, num_kv_heads, dtype, rows=None,
             sliding_window=0, kv_format="same", k_scale=1.0, v_scale=1.0):
        S, Hq, D = q.shape
        g = Hq // num_kv_heads
        out = np.zeros((S, Hq, D))
        for s in range(S):
            L = int(context_lens[s])
            if L <= 0:
                continue
            for j in range(Hq):
                h = head_of(j, g, num_kv_heads) if head_of else j // g
                lo, hi = 0, L
                if sliding_window > 0:
                    W = min(L, max(1, sliding_window + window_shift))
                    lo, hi = (0, W) if window_from_start else (L - W, L)
                Kr = oracle.gather_sequence(k_cache, block_tables[s], hi, h, block_size, lo)
                Vr = oracle.gather_sequence(v_cache, block_tables[s], hi, h, block_size, lo)
                if kv_format == "fp8_e4m3":
                    dec = fp8_decode or oracle.decode_e4m3
                    K = dec(Kr) * (1.0 if ignore_k_scale else float(np.float32(k_scale)))
                    V = dec(Vr) * (1.0 if ignore_v_scale else float(np.float32(v_scale)))
                else:
                    K, V = decode(Kr, dtype), decode(Vr, dtype)
                x = (K @ decode(q[s, j], dtype))
                if not drop_scale:
                    x = float(np.float32(scale)) * x
                if scale_twice:
                    x = float(np.float32(scale)) * x
                e = np.exp(x - (0.0 if no_max else x.max()))
                p = e if no_normalise else e / e.sum()
                out[s, j] = p @ V
        if rows is not None:
            return np.stack([out[s, j] for s, j in rows])
        return out
    return impl


MUTANTS = {
    "offset_off_by_one": _with_gather(_gather_offset_off_by_one),
    "block_order_reversed": _with_gather(_gather_block_order_reversed),
    "layout_head_offset_swapped": _with_gather(_gather_head_and_offset_swapped),
    "drops_last_token": _with_gather(_gather_drops_last_token),
    "reads_whole_last_block": _with_gather(_gather_whole_last_block),
    "bf16_decode_wrong_shift": _with_decode(_decode_bf16_shift_15),
    "f16_decoded_as_bf16": _with_decode(_decode_f16_as_bf16),
    "kv_head_is_j_mod_hkv": _mutant_body(head_of=lambda j, g, hkv: j % hkv),
    "scale_dropped": _mutant_body(drop_scale=True),
    "scale_applied_twice": _mutant_body(scale_twice=True),
    "softmax_not_normalised": _mutant_body(no_normalise=True),
    "window_one_token_too_long": _mutant_body(window_shift=1),
    "window_one_token_too_short": _mutant_body(window_shift=-1),
    "window_counted_from_the_start": _mutant_body(window_from_start=True),
    "fp8_k_scale_ignored": _mutant_body(ignore_k_scale=True),
    "fp8_v_scale_ignored": _mutant_body(ignore_v_scale=True),
    "fp8_decoded_with_bias_8": _mutant_body(fp8_decode=_fnuz_like_decode),
}


def test_reference_body_itself_passes():
    """The re-typed body used for mutants is correct when nothing is planted."""
    for check in pins.ALL_CHECKS:
        check(_mutant_body())


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name):
    impl = MUTANTS[name]
    failures = 0
    for check in pins.ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(impl)
        except (AssertionError, ValueError, IndexError):
            failures += 1
    assert failures > 0, f"no pin caught the planted mistake {name}"
