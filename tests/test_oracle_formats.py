"""Exhaustive pin of the oracle's format decoders against torch's conversions."""
import numpy as np
import torch

from oracle.formats import decode


def _same(a, b):
    return np.array_equal(a, b, equal_nan=True)


def test_bf16_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = decode(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(ours, ref)


def test_f16_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = decode(bits.view(np.float16), "f16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.float16).to(torch.float64).numpy()
    assert _same(ours, ref)


def test_f32_sampled_patterns():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    ours = decode(bits.view(np.float32), "f32")
    ref = torch.from_numpy(bits.view(np.int32)).view(torch.float32).to(torch.float64).numpy()
    assert _same(ours, ref)
