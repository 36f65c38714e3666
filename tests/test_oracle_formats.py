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


# ---------------------------------------------------------------------------
# 8-bit E4M3 (OCP "fn") codes of the quantized cache: pinned to torch's own
# float8_e4m3fn conversions and to the format's closed forms.
# ---------------------------------------------------------------------------
from oracle.formats import E4M3_MAX, decode_e4m3, quantize_e4m3  # noqa: E402


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(decode_e4m3(codes), ref)
    assert decode_e4m3(np.array([0x7E]))[0] == E4M3_MAX == 448.0
    assert decode_e4m3(np.array([0x01]))[0] == 2.0 ** -9          # smallest subnormal
    assert decode_e4m3(np.array([0x08]))[0] == 2.0 ** -6          # smallest normal
    assert np.isnan(decode_e4m3(np.array([0x7F, 0xFF]))).all()


def test_e4m3_quantize_matches_torch_in_range_including_every_tie():
    v = decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    mids = ((v[1:] + v[:-1]) / 2).astype(np.float32)             # exact ties
    rng = np.random.default_rng(3)
    xs = np.concatenate([v.astype(np.float32), mids, -mids, -v.astype(np.float32),
                         rng.uniform(-E4M3_MAX, E4M3_MAX, 200000).astype(np.float32),
                         (rng.standard_normal(100000) * 0.01).astype(np.float32)])
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(quantize_e4m3(xs), ref)


def test_e4m3_quantize_closed_forms():
    q = lambda x: int(quantize_e4m3(np.array([x], dtype=np.float32))[0])
    assert q(464.0) == q(480.0) == q(1e30) == q(np.inf) == 0x7E        # saturation at 448
    assert q(-1e30) == q(-np.inf) == 0xFE
    assert q(np.nan) == 0x7F
    assert q(-0.0) == 0x80 and q(0.0) == 0x00
    assert q(2.0 ** -10) == 0x00                                      # tie between 0 and 2^-9: even code
    assert q(3 * 2.0 ** -10) == 0x02                                  # tie between 2^-9 and 2^-8: even code
    assert q(1.0625) == 0x38 and q(1.1875) == 0x3A                    # ties to even mantissa
    assert q(17.0) == 0x58                                            # 16 (even) rather than 18
