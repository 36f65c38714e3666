"""GPU parity for any number G of query heads per KV head: groups that are no
power of two (3, 5, 6, 7), single heads on the matrix cores, several 16-head
column tiles per workgroup, and groups larger than one workgroup computes
(multi-query layers up to G = 128), cut into head chunks; both kernels, 16-
and 8-bit caches, split-K and sliding windows, every row against the
oracle."""
import pytest
import torch

import paged_kv_cache_339_amd as pkv
from synthetic import DecodeConfig, host_values, make_layout
from tests.gpu_util import DeviceStep, assert_rows_close, oracle_step, say, to_storage_np, widen

pytestmark = pytest.mark.gpu

GROUP_CASES = [
    # q dtype, cache format, D, B, Hq, Hkv, kernel          G: chunks x heads
    ("f32", "same", 64, 16, 6, 2, "valu"),                  # 3: one chunk
    ("f32", "same", 128, 16, 12, 1, "valu"),                # 12: 2 x 6
    ("f32", "same", 64, 32, 32, 2, "valu"),                 # 16: 2 x 8
    ("bf16", "same", 128, 16, 10, 2, "auto"),               # 5 (matrix cores)
    ("f16", "same", 128, 32, 12, 2, "auto"),                # 6
    ("bf16", "same", 128, 16, 28, 4, "auto"),               # 7
    ("f16", "same", 64, 16, 3, 1, "auto"),                  # 3
    ("bf16", "same", 128, 16, 2, 2, "mfma"),                # 1
    ("f16", "same", 128, 8, 4, 2, "mfma"),                  # 2
    ("bf16", "same", 128, 32, 48, 2, "auto"),               # 24: 2 column tiles
    ("f16", "same", 128, 16, 32, 1, "auto"),                # 32: 2 column tiles
    ("bf16", "same", 64, 16, 71, 1, "auto"),                # 71: 36 + 35 in 3 tiles
    ("bf16", "same", 128, 16, 10, 2, "valu"),               # 5 (vector kernel)
    ("f16", "same", 64, 8, 24, 1, "valu"),                  # 24: 3 x 8
    ("bf16", "fp8_e4m3", 128, 16, 10, 2, "auto"),           # 5, 8-bit cache
    ("f16", "fp8_e4m3", 128, 32, 40, 1, "auto"),            # 40: 2 x 20 in 2 tiles, 8-bit cache
    ("bf16", "fp8_e4m3", 64, 16, 3, 1, "valu"),             # 3, 8-bit cache
    ("f16", "same", 64, 32, 64, 1, "auto"),                 # 64: 4 column tiles
    ("f16", "same", 64, 16, 128, 1, "auto"),                # 128: 2 x 64
    ("bf16", "fp8_e4m3", 64, 16, 48, 1, "auto"),            # 48: 3 tiles, 8-bit cache
    ("bf16", "same", 64, 8, 40, 2, "auto"),                 # 20, 8-token blocks: 2 x 10, one tile
    ("bf16", "same", 128, 64, 24, 1, "mfma"),               # 24, 64-token blocks: 2 x 12
]


def _layout(q_dtype, kv_format, D, B, Hq, Hkv, window, seed):
    lens = [1, B - 1, B + 1, 77, 300, 1000, 2049]
    fp8 = kv_format == "fp8_e4m3"
    cfg = DecodeConfig(f"groups_{q_dtype}_G{Hq // Hkv}", num_seqs=len(lens), num_q_heads=Hq,
                       num_kv_heads=Hkv, head_dim=D, dtype=q_dtype, block_size=B, lengths="fixed",
                       fixed_lengths=(1,), pool_factor=1.5, sliding_window=window,
                       kv_format=kv_format if fp8 else "same",
                       k_scale=1.0 / 16 if fp8 else 1.0, v_scale=1.0 / 8 if fp8 else 1.0)
    return cfg, make_layout(cfg, seed, lengths=lens)


@pytest.mark.parametrize("q_dtype,kv_format,D,B,Hq,Hkv,kernel", GROUP_CASES)
@pytest.mark.parametrize("window", [0, 300])
def test_any_group_every_row(q_dtype, kv_format, D, B, Hq, Hkv, kernel, window):
    cfg, lay = _layout(q_dtype, kv_format, D, B, Hq, Hkv, window, seed=Hq * 7 + Hkv + window)
    host = host_values(lay)
    step = DeviceStep.from_host(lay, host)
    step.scatter()
    want, kc, _ = oracle_step(lay, host)
    assert to_storage_np(step.k_cache, cfg.kv_dtype).tobytes() == kc.tobytes()
    for part in (0, 64):
        label = f"G{Hq // Hkv} {q_dtype}/{kv_format} D{D} B{B} Hkv{Hkv} {kernel} w{window} p{part}"
        say(label)
        out = step.attend(partition_size=part, kernel=kernel)
        torch.cuda.synchronize()
        assert_rows_close(widen(out), want, q_dtype, label)


@pytest.mark.parametrize("Hq,Hkv,kernel", [(71, 1, "auto"), (24, 1, "valu"), (10, 2, "auto")])
def test_chunked_groups_through_decode_step(Hq, Hkv, kernel):
    """decode_step (new tokens stored by the plan launch) with head chunks,
    against the oracle and bit for bit against scatter + attend."""
    cfg, lay = _layout("bf16", "same", 64, 16, Hq, Hkv, 0, seed=5 + Hq)
    host = host_values(lay)
    a = DeviceStep.from_host(lay, host)
    a.scatter()
    ref = a.attend(partition_size=64, kernel=kernel)
    b = DeviceStep.from_host(lay, host)
    say(f"decode_step G{Hq // Hkv} {kernel}")
    out = torch.empty_like(b.q)
    pkv.decode_step(out, b.q, b.k_new, b.v_new, b.k_cache, b.v_cache, b.slots, b.tables, b.lens, cfg.scale,
                    cfg.block_size, cfg.num_kv_heads, max(1, lay.max_context_len), partition_size=64,
                    kernel=kernel)
    torch.cuda.synchronize()
    assert torch.equal(a.k_cache.view(torch.int16), b.k_cache.view(torch.int16))
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    want, _, _ = oracle_step(lay, host)
    assert_rows_close(widen(out), want, "bf16", f"decode_step G{Hq // Hkv}")
