"""8-bit E4M3 KV cache on the GPU: the quantizing store is bit-exact against
the oracle on every tie, overflow, NaN, signed zero and subnormal, for each
input format and several scales; every code decodes exactly through the
attention kernel (a one-token sequence returns its value row); copies of
8-bit blocks are bitwise."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_339_amd as pkv
from synthetic import to_storage
from tests.gpu_util import ints, say, to_device, to_storage_np

pytestmark = pytest.mark.gpu


def special_values():
    v = oracle.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    mids = (v[1:] + v[:-1]) / 2
    extra = [448.0, 464.0, 480.0, 1e4, np.inf, -np.inf, np.nan, 0.0, -0.0, 2.0 ** -10, 3 * 2.0 ** -10, 1e-6]
    rng = np.random.default_rng(8)
    return np.concatenate([v, -v, mids, -mids, extra, rng.standard_normal(700) * 60])


@pytest.mark.parametrize("in_dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("k_scale,v_scale", [(1.0, 1.0), (1.0 / 32, 1.0 / 64), (0.37, 3.1)])
def test_fp8_store_is_bit_exact(in_dtype, k_scale, v_scale):
    Hkv, D, B, N = 2, 128, 16, 24
    vals = special_values()
    T = -(-len(vals) // (Hkv * D))
    flat = np.resize(vals, T * Hkv * D)
    k = to_storage(flat.reshape(T, Hkv, D), in_dtype)
    v = to_storage(flat[::-1].copy().reshape(T, Hkv, D), in_dtype)
    rng = np.random.default_rng(1)
    kc = rng.integers(0, 256, size=(N, Hkv, B, D)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(N, Hkv, B, D)).astype(np.uint8)
    slots = rng.choice(N * B, size=T, replace=False).astype(np.int32)
    say(f"fp8 store {in_dtype} scales {k_scale}, {v_scale} ({T} tokens)")
    dk, dv = to_device(kc, "fp8"), to_device(vc, "fp8")
    pkv.reshape_and_cache_fp8(to_device(k, in_dtype), to_device(v, in_dtype), dk, dv, ints(slots), k_scale, v_scale)
    torch.cuda.synchronize()
    oracle.reshape_and_cache_fp8(k, v, kc, vc, slots, B, k_scale, v_scale, in_dtype)
    assert to_storage_np(dk, "fp8").tobytes() == kc.tobytes()
    assert to_storage_np(dv, "fp8").tobytes() == vc.tobytes()


@pytest.mark.parametrize("q_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("kernel,group,B", [("valu", 2, 16), ("mfma", 4, 16), ("mfma", 16, 32)])
def test_every_code_decodes_exactly_through_attention(q_dtype, kernel, group, B):
    """A one-token sequence returns v_scale * e4m3(code) for each code of its
    value row: all 256 codes over 2 KV heads x 128, `group` query heads
    each, through either kernel."""
    Hkv, D = 2, 128
    codes = np.arange(256, dtype=np.uint8).reshape(Hkv, D)
    kc = np.zeros((3, Hkv, B, D), dtype=np.uint8)
    vc = np.full((3, Hkv, B, D), 0xFF, dtype=np.uint8)
    vc[1, :, 0, :] = codes
    kc[1, :, 0, :] = 0x38                                   # key 1.0 everywhere
    q = to_storage(np.random.default_rng(2).standard_normal((1, group * Hkv, D)), q_dtype)
    say(f"fp8 decode of all codes, q {q_dtype}, {kernel} kernel, group {group}, B {B}")
    out = torch.empty((1, group * Hkv, D), dtype={"f16": torch.float16, "bf16": torch.bfloat16}[q_dtype],
                      device="cuda")
    pkv.paged_attention_decode(out, to_device(q, q_dtype), to_device(kc, "fp8"), to_device(vc, "fp8"),
                               ints([[1]]), ints([1]), 0.1, B, Hkv, 1, kv_format="fp8_e4m3", k_scale=1.0,
                               v_scale=0.5, kernel=kernel)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()[0]
    want = np.repeat(oracle.decode_e4m3(codes) * 0.5, group, axis=0)
    assert np.array_equal(got, want, equal_nan=True)


def test_fp8_blocks_copy_bitwise():
    rng = np.random.default_rng(5)
    kc = rng.integers(0, 256, size=(40, 8, 16, 128)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(40, 8, 16, 128)).astype(np.uint8)
    perm = rng.permutation(40)
    pairs = np.stack([perm[:12], perm[12:24]], axis=1).astype(np.int32)
    dk, dv = to_device(kc, "fp8"), to_device(vc, "fp8")
    pkv.copy_blocks(dk, dv, ints(pairs))
    torch.cuda.synchronize()
    oracle.copy_blocks(kc, vc, pairs)
    assert to_storage_np(dk, "fp8").tobytes() == kc.tobytes()
    assert to_storage_np(dv, "fp8").tobytes() == vc.tobytes()


FP8_CASES = [
    # q dtype, head_dim, block size, Hq, Hkv, kernel
    ("f16", 64, 16, 4, 4, "valu"), ("bf16", 64, 32, 8, 4, "valu"), ("bf16", 128, 32, 2, 2, "valu"),
    ("bf16", 64, 16, 16, 4, "mfma"), ("f16", 64, 32, 32, 4, "mfma"), ("f16", 128, 16, 16, 1, "mfma"),
    ("bf16", 128, 32, 64, 4, "mfma"),
]


@pytest.mark.parametrize("q_dtype,D,B,Hq,Hkv,kernel", FP8_CASES)
@pytest.mark.parametrize("window", [0, 300])
def test_fp8_attention_matches_the_oracle(q_dtype, D, B, Hq, Hkv, kernel, window):
    """8-bit caches through both kernels at head_dim 64 and 128, 16- and
    32-token blocks, group sizes 1-16, with and without a sliding window
    and split-K: every row against the oracle (same stored codes)."""
    from synthetic import DecodeConfig, host_values, make_layout
    from tests.gpu_util import DeviceStep, assert_rows_close, oracle_step, widen

    lens = [1, B - 1, B + 1, 77, 300, 301, 640, 1000]
    cfg = DecodeConfig(f"fp8_{q_dtype}_{D}", num_seqs=len(lens), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                       dtype=q_dtype, block_size=B, lengths="fixed", fixed_lengths=(1,), pool_factor=1.5,
                       sliding_window=window, kv_format="fp8_e4m3", k_scale=1.0 / 16, v_scale=1.0 / 8)
    lay = make_layout(cfg, 21, lengths=lens)
    host = host_values(lay)
    step = DeviceStep.from_host(lay, host)
    step.scatter()
    want, kc, vc = oracle_step(lay, host)
    assert to_storage_np(step.k_cache, "fp8").tobytes() == kc.tobytes()
    for part in (0, 128):
        say(f"fp8 attention {q_dtype} D{D} B{B} G{Hq // Hkv} {kernel} window={window} partition={part}")
        out = step.attend(partition_size=part, kernel=kernel)
        torch.cuda.synchronize()
        assert_rows_close(widen(out), want, q_dtype, f"fp8 {q_dtype} D{D} B{B} {kernel} w{window} p{part}")
