"""GPU parity of decode attention with shared prefixes: each group's shared
prompt blocks are read once for all its samples (the members become the
query heads of one grouped-query pass), each sample's own tokens in a second
pass, and the two parts are merged through their softmax denominators.

The output must match the oracle's plain attention (the same softmax over
every token of each sequence) within the per-row tolerance, and the plain
decode call on the library within the same tolerance."""
import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_339_amd as pkv
from paged_kv_cache_339_amd._lib import AttnOptions
from synthetic import CONFIGS, host_values, make_layout, shared_prefix_groups
from tests.gpu_util import DeviceStep, assert_rows_close, ints, oracle_step, say, widen

pytestmark = pytest.mark.gpu

SHARED = CONFIGS[5]


def run_shared(step, members, prefix, partition_size=0, kernel="auto", max_prefix=None, out=None,
               cache_policy="stream"):
    cfg, lay = step.layout.cfg, step.layout
    if out is None:
        out = torch.empty_like(step.q)
    mp = int(prefix.max()) if max_prefix is None else max_prefix
    pkv.paged_attention_decode_shared_prefix(
        out, step.q, step.k_cache, step.v_cache, step.tables, step.lens, ints(prefix), ints(members), mp,
        cfg.scale, cfg.block_size, cfg.num_kv_heads, max(1, lay.max_context_len), partition_size=partition_size,
        kernel=kernel, kv_format=cfg.kv_format, k_scale=cfg.k_scale, v_scale=cfg.v_scale,
        cache_policy=cache_policy)
    torch.cuda.synchronize()
    return out


def scaled(dtype="bf16", Hq=8, Hkv=8, prompts=3, samples=4, prompt_len=200, tail=90, B=16, **kw):
    return SHARED.scaled(num_seqs=prompts * samples, num_q_heads=Hq, num_kv_heads=Hkv, dtype=dtype,
                         samples_per_prompt=samples, prompt_len=prompt_len, len_hi=tail, block_size=B,
                         partition_size=0, cache_policy="stream", **kw)


@pytest.mark.parametrize("dtype,Hq,Hkv,B", [
    ("bf16", 8, 8, 16), ("f16", 8, 8, 16), ("f32", 4, 4, 16), ("bf16", 16, 4, 16), ("f16", 12, 4, 32),
    ("bf16", 8, 1, 16), ("bf16", 8, 8, 8), ("f16", 4, 4, 64), ("bf16", 64, 8, 32)])
def test_shared_prefix_every_row(dtype, Hq, Hkv, B):
    cfg = scaled(dtype, Hq, Hkv, B=B, prompt_len=200 if B != 64 else 300)
    lay = make_layout(cfg, seed=51)
    host = host_values(lay)
    members, prefix = shared_prefix_groups(lay)
    say(f"shared prefix {dtype} Hq={Hq} Hkv={Hkv} B={B}: {len(lay.context_lens)} seqs, prefix {prefix[0]}")
    step = DeviceStep.from_host(lay, host)
    step.scatter()
    got = widen(run_shared(step, members, prefix))
    want, _, _ = oracle_step(lay, host)
    assert_rows_close(got, want, dtype, "shared-prefix decode vs oracle")
    plain = widen(step.attend(partition_size=0))
    assert_rows_close(got, plain, dtype, "shared-prefix decode vs plain decode")


@pytest.mark.parametrize("partition_size", [16, 32, 64, 512])
def test_shared_prefix_with_split_partitions(partition_size):
    cfg = scaled("bf16", 8, 8, prompt_len=700, tail=300)
    lay = make_layout(cfg, seed=52)
    host = host_values(lay)
    members, prefix = shared_prefix_groups(lay)
    say(f"shared prefix, partitions of {partition_size}")
    step = DeviceStep.from_host(lay, host)
    step.scatter()
    got = widen(run_shared(step, members, prefix, partition_size=partition_size))
    want, _, _ = oracle_step(lay, host)
    assert_rows_close(got, want, "bf16", f"shared-prefix decode, partition {partition_size}")


def test_irregular_groups():
    """Groups with unused slots, a group of one, a group with no shared
    tokens, and sequences in no group."""
    cfg = scaled("bf16", 8, 4, prompts=4, samples=4, prompt_len=120)
    lay = make_layout(cfg, seed=53)
    host = host_values(lay)
    members, prefix = shared_prefix_groups(lay)
    P = int(prefix[0])
    m = np.full((4, 5), -1, dtype=np.int32)
    m[0, :4] = members[0]                     # a whole prompt
    m[1, [0, 2, 4]] = members[1][[0, 1, 3]]   # three samples, two unused slots
    m[2, 3] = members[2][2]                   # a group of one
    m[3, :2] = members[3][:2]                 # two samples with nothing shared
    pre = np.zeros_like(prefix)
    for row, p in ((0, P), (1, P), (2, P), (3, 0)):
        for s in m[row]:
            if s >= 0:
                pre[s] = p
    say(f"irregular groups, prefix {P}")
    step = DeviceStep.from_host(lay, host)
    step.scatter()
    got = widen(run_shared(step, m, pre, max_prefix=P + 16))
    want, _, _ = oracle_step(lay, host)
    assert_rows_close(got, want, "bf16", "irregular groups")


def test_prefix_covering_the_whole_sequence():
    """A sample whose every token is in the shared prefix (an empty own part)."""
    cfg = scaled("f16", 8, 8, prompts=2, samples=4, prompt_len=64)
    lay0 = make_layout(cfg, seed=54)
    lens = lay0.context_lens.copy()
    lens[1] = 64
    lens[6] = 64
    lay = make_layout(cfg, seed=54, lengths=lens)
    host = host_values(lay)
    members, prefix = shared_prefix_groups(lay)
    assert prefix[1] == 64 and lay.context_lens[1] == 64
    say("prefix = whole sequence")
    step = DeviceStep.from_host(lay, host)
    step.scatter()
    got = widen(run_shared(step, members, prefix))
    want, _, _ = oracle_step(lay, host)
    assert_rows_close(got, want, "f16", "prefix covering a whole sequence")


def test_no_groups_is_the_plain_decode_bitwise():
    cfg = scaled("bf16", 8, 8)
    lay = make_layout(cfg, seed=55)
    host = host_values(lay)
    say("no groups")
    step = DeviceStep.from_host(lay, host)
    step.scatter()
    out = torch.empty_like(step.q)
    pkv.paged_attention_decode_shared_prefix(
        out, step.q, step.k_cache, step.v_cache, step.tables, step.lens,
        ints(np.zeros(len(lay.context_lens))), ints(np.zeros((0, 1))), 0, cfg.scale, cfg.block_size,
        cfg.num_kv_heads, lay.max_context_len)
    torch.cuda.synchronize()
    plain = step.attend(partition_size=0)
    assert torch.equal(out.view(torch.int16), plain.view(torch.int16))


def test_fp8_cache_with_shared_prefix():
    cfg = scaled("bf16", 16, 4, kv_format="fp8_e4m3", k_scale=1 / 32, v_scale=1 / 32)
    lay = make_layout(cfg, seed=56)
    host = host_values(lay)
    members, prefix = shared_prefix_groups(lay)
    say("shared prefix, 8-bit cache")
    step = DeviceStep.from_host(lay, host)
    step.scatter()
    got = widen(run_shared(step, members, prefix))
    want, _, _ = oracle_step(lay, host)
    assert_rows_close(got, want, "bf16", "shared prefix with an 8-bit cache")


def test_data_error_in_a_shared_block_stays_in_its_group():
    cfg = scaled("bf16", 8, 8)
    lay = make_layout(cfg, seed=57)
    host = host_values(lay)
    members, prefix = shared_prefix_groups(lay)
    tables = lay.block_tables.copy()
    tables[members[1][0], 2] = lay.num_blocks + 5      # first member's table: read for the whole group
    say("data error in a shared block")
    step = DeviceStep.from_host(lay, host)
    step.tables = ints(tables)
    step.scatter()
    got = widen(run_shared(step, members, prefix))
    bad = set(members[1].tolist())
    for s in range(len(lay.context_lens)):
        rows_nan = np.isnan(got[s]).all(axis=-1)
        assert rows_nan.all() == (s in bad), f"sequence {s}"
    want, _, _ = oracle_step(lay, host)
    keep = [s for s in range(len(lay.context_lens)) if s not in bad]
    assert_rows_close(got[keep], want[keep], "bf16", "rows outside the bad group")


def test_rejects_bad_arguments():
    cfg = scaled("bf16", 8, 8)
    lay = make_layout(cfg, seed=58)
    host = host_values(lay)
    members, prefix = shared_prefix_groups(lay)
    step = DeviceStep.from_host(lay, host)
    out = torch.empty_like(step.q)
    say("argument checks")
    # A sliding window is not supported with shared prefixes (the wrapper has
    # no window argument: call the C function with a window in the options).
    opts = AttnOptions(0, 0, None, None, 256, 0, 1.0, 1.0, 0, 0)
    vp = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    pre, mem = ints(prefix), ints(members)
    st = pkv.lib.pkv_paged_attention_decode_shared_prefix(
        vp(out), vp(step.q), vp(step.k_cache), vp(step.v_cache), vp(step.tables), vp(step.lens), vp(pre), vp(mem),
        members.shape[0], members.shape[1], int(prefix.max()), cfg.scale, cfg.block_size, cfg.num_kv_heads,
        len(lay.context_lens), cfg.num_q_heads, cfg.head_dim, lay.block_tables.shape[1], lay.max_context_len,
        lay.num_blocks, 2, None, 0, ctypes.byref(opts), None)
    assert st == -4
    with pytest.raises(pkv.PkvError):          # prefix bound above max_context_len
        run_shared(step, members, prefix, max_prefix=lay.max_context_len + 1)
