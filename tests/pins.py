"""Checks that pin a paged-attention implementation to facts other than its
own formula.  Each check takes an implementation with the signature of
oracle.paged_attention_decode and raises AssertionError when it is wrong.

They are run on the oracle (all must pass) and on planted-mistake variants of
the oracle (each mistake must be caught by at least one check).

Inputs here are built "logical first": every sequence's keys and values are
drawn as contiguous [L, Hkv, D] arrays and then written token by token into a
poisoned pool at a random placement, by code local to this file.
"""
from __future__ import annotations

import numpy as np
import scipy.special
import torch

from synthetic import POISON_BITS, to_storage


def widen(raw, dtype):
    """fp64 copy of stored values, through torch (independent of the oracle)."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(raw))
    return t.to(torch.float64).numpy()


class Paged:
    """A batch of sequences written into a block pool at a chosen placement."""

    def __init__(self, K, V, q, block_size, dtype, placement_seed, spare_blocks=3, share=None):
        self.K, self.V, self.q = K, V, q
        self.B, self.dtype = block_size, dtype
        S = len(K)
        Hkv, D = K[0].shape[1], K[0].shape[2]
        lens = [k.shape[0] for k in K]
        nb = [-(-L // block_size) for L in lens]
        rng = np.random.default_rng(placement_seed)
        need = sum(nb)
        N = need + spare_blocks
        perm = rng.permutation(N)
        table = np.full((S, max(1, max(nb))), -1, dtype=np.int32)
        storage = K[0].dtype
        width = {"f32": np.uint32, "fp8": np.uint8}.get(dtype, np.uint16)
        poison = 0xFF if dtype == "fp8" else POISON_BITS[dtype]
        kp = np.full((N, Hkv, block_size, D), poison, dtype=width).view(storage)
        vp = np.full((N, Hkv, block_size, D), poison, dtype=width).view(storage)
        pos = 0
        for s in range(S):
            if share is not None and share.get(s) is not None:
                src, nshared = share[s]
                table[s, :nshared] = table[src, :nshared]
                own = perm[pos:pos + nb[s] - nshared]
                pos += nb[s] - nshared
                table[s, nshared:nb[s]] = own
            else:
                table[s, :nb[s]] = perm[pos:pos + nb[s]]
                pos += nb[s]
            for t in range(lens[s]):
                blk = table[s, t // block_size]
                kp[blk, :, t % block_size, :] = K[s][t]
                vp[blk, :, t % block_size, :] = V[s][t]
        self.k_cache, self.v_cache, self.table = kp, vp, table
        self.lens = np.array(lens, dtype=np.int32)

    def run(self, attn, scale, num_kv_heads, rows=None, window=0):
        return attn(self.q, self.k_cache, self.v_cache, self.table, self.lens, scale,
                    self.B, num_kv_heads, self.dtype, rows=rows, sliding_window=window)

    def free_before_window(self, window):
        """Copy whose table entries for blocks wholly before each sequence's
        window are -1 and whose blocks there are poisoned (freed blocks)."""
        import copy
        other = copy.copy(self)
        other.table = self.table.copy()
        other.k_cache = self.k_cache.copy()
        other.v_cache = self.v_cache.copy()
        width = np.uint32 if self.dtype == "f32" else np.uint16
        for s, L in enumerate(self.lens.tolist()):
            for b in range(max(0, L - window) // self.B):
                blk = other.table[s, b]
                other.k_cache.view(width)[blk] = POISON_BITS[self.dtype]
                other.v_cache.view(width)[blk] = POISON_BITS[self.dtype]
                other.table[s, b] = -1
        return other


def draw(rng, lens, Hq, Hkv, D, dtype):
    K = [to_storage(rng.standard_normal((L, Hkv, D)), dtype) for L in lens]
    V = [to_storage(rng.standard_normal((L, Hkv, D)), dtype) for L in lens]
    q = to_storage(rng.standard_normal((len(lens), Hq, D)), dtype)
    return K, V, q


def sdpa_reference(K, V, q, scale, dtype, values_are_fp64=False):
    """torch's scaled-dot-product attention, fp64, on the contiguous sequences
    (K, V in storage format `dtype`, or already fp64 with values_are_fp64)."""
    S, Hq, D = q.shape
    out = np.zeros((S, Hq, D))
    for s in range(S):
        kk = K[s] if values_are_fp64 else widen(K[s], dtype)
        vv = V[s] if values_are_fp64 else widen(V[s], dtype)
        k = torch.from_numpy(np.ascontiguousarray(kk)).permute(1, 0, 2)    # [Hkv, L, D]
        v = torch.from_numpy(np.ascontiguousarray(vv)).permute(1, 0, 2)
        g = Hq // k.shape[0]
        k = k.repeat_interleave(g, dim=0).contiguous()
        v = v.repeat_interleave(g, dim=0).contiguous()
        qq = torch.from_numpy(widen(q[s], dtype))[:, None, :]            # [Hq, 1, D]
        o = torch.nn.functional.scaled_dot_product_attention(qq, k, v, scale=float(np.float32(scale)))
        out[s] = o[:, 0, :].numpy()
    return out


# ----------------------------------------------------------------------------
# The checks.
# ----------------------------------------------------------------------------

def check_against_sdpa(attn):
    """Paged through a random placement == torch SDPA on the contiguous data."""
    cases = [
        (dict(lens=[5, 17, 33, 64], Hq=2, Hkv=2, D=64, dtype="f32", B=16), 11),
        (dict(lens=[1, 15, 16, 17, 40], Hq=4, Hkv=4, D=32, dtype="f16", B=8), 12),
        (dict(lens=[3, 31, 32, 33, 70], Hq=8, Hkv=2, D=16, dtype="bf16", B=32), 13),
        (dict(lens=[100, 7], Hq=6, Hkv=3, D=8, dtype="f16", B=16), 14),
    ]
    for c, seed in cases:
        rng = np.random.default_rng(seed)
        K, V, q = draw(rng, c["lens"], c["Hq"], c["Hkv"], c["D"], c["dtype"])
        scale = 1.0 / np.sqrt(c["D"]) * 1.37
        paged = Paged(K, V, q, c["B"], c["dtype"], placement_seed=seed + 100)
        got = paged.run(attn, scale, c["Hkv"])
        want = sdpa_reference(K, V, q, scale, c["dtype"])
        err = np.max(np.abs(got - want))
        assert err <= 1e-12, f"paged vs SDPA max |err| {err} in case {c}"


def check_closed_forms(attn):
    rng = np.random.default_rng(21)
    D, B = 16, 8
    # One token: the output is that token's value row, exactly.
    K, V, q = draw(rng, [1, 1], 2, 2, D, "f32")
    out = Paged(K, V, q, B, "f32", 1).run(attn, 0.25, 2)
    for s in range(2):
        assert np.array_equal(out[s], widen(V[s][0], "f32")), "L=1 must return v_0"
    # Equal value rows: the output is that row whatever the weights.
    L = 37
    K, V, q = draw(rng, [L], 2, 2, D, "f32")
    V[0][:] = V[0][5]
    out = Paged(K, V, q, B, "f32", 2).run(attn, 0.5, 2)
    assert np.max(np.abs(out[0] - widen(V[0][5], "f32"))) <= 1e-13, "constant V rows"
    # Zero query: uniform weights, the mean of the value rows.
    K, V, q = draw(rng, [L], 2, 2, D, "f32")
    q[:] = 0
    out = Paged(K, V, q, B, "f32", 3).run(attn, 0.5, 2)
    want = widen(V[0], "f32").mean(axis=0)
    assert np.max(np.abs(out[0] - want)) <= 1e-13, "q = 0 gives the mean of V"
    # One key far ahead of the rest: the output is that key's value row.
    K, V, q = draw(rng, [L], 1, 1, D, "f32")
    K[0][:] = to_storage(rng.standard_normal((L, 1, D)) * 0.01, "f32")
    K[0][9, 0] = q[0, 0] * np.float32(40.0)
    out = Paged(K, V, q, B, "f32", 4).run(attn, 1.0, 1)
    assert np.max(np.abs(out[0, 0] - widen(V[0][9, 0], "f32"))) <= 1e-12, "dominant key"
    # Two tokens: weights are the logistic function of the score difference.
    K, V, q = draw(rng, [2], 1, 1, D, "f32")
    k0, k1 = widen(K[0][0, 0], "f32"), widen(K[0][1, 0], "f32")
    qq = widen(q[0, 0], "f32")
    scale = 0.3
    d = float(np.float32(scale)) * (float(np.dot(qq, k0)) - float(np.dot(qq, k1)))
    w0 = scipy.special.expit(d)
    want = w0 * widen(V[0][0, 0], "f32") + (1 - w0) * widen(V[0][1, 0], "f32")
    out = Paged(K, V, q, B, "f32", 5).run(attn, scale, 1)
    assert np.max(np.abs(out[0, 0] - want)) <= 1e-14, "two-token logistic form"


def check_invariances(attn):
    """Exact invariance under placement, block size, batch order, sharing,
    and GQA vs replicated KV heads; poisoned slots never reach the output."""
    rng = np.random.default_rng(31)
    lens = [1, 7, 8, 9, 16, 17, 50]
    Hq, Hkv, D = 4, 2, 16
    K, V, q = draw(rng, lens, Hq, Hkv, D, "bf16")
    base = Paged(K, V, q, 8, "bf16", 1).run(attn, 0.25, Hkv)
    assert np.all(np.isfinite(base)), "poisoned slots leaked into the output"
    other = Paged(K, V, q, 8, "bf16", 2, spare_blocks=9).run(attn, 0.25, Hkv)
    assert np.array_equal(base, other), "output depends on physical placement"
    for B in (16, 32, 64):
        out = Paged(K, V, q, B, "bf16", 3).run(attn, 0.25, Hkv)
        assert np.array_equal(base, out), f"output depends on block size {B}"
    perm = np.random.default_rng(5).permutation(len(lens))
    outp = Paged([K[i] for i in perm], [V[i] for i in perm], q[perm], 8, "bf16", 4).run(attn, 0.25, Hkv)
    assert np.array_equal(outp, base[perm]), "batch order changes results"
    # Replicate each KV head over its query group: MHA gives the GQA result.
    g = Hq // Hkv
    Kr = [np.repeat(k, g, axis=1) for k in K]
    Vr = [np.repeat(v, g, axis=1) for v in V]
    mha = Paged(Kr, Vr, q, 8, "bf16", 6).run(attn, 0.25, Hq)
    assert np.array_equal(mha, base), "GQA head mapping disagrees with replicated MHA"
    # Shared prefix blocks vs private copies of the same rows.
    P = 24
    Kp = rng.standard_normal((P, Hkv, D))
    Ks, Vs = [], []
    for _ in range(3):
        tail = rng.integers(1, 20)
        Ks.append(to_storage(np.concatenate([Kp, rng.standard_normal((tail, Hkv, D))]), "bf16"))
        Vs.append(to_storage(np.concatenate([Kp[::-1] * 0.5, rng.standard_normal((tail, Hkv, D))]), "bf16"))
    qs = to_storage(rng.standard_normal((3, Hq, D)), "bf16")
    copied = Paged(Ks, Vs, qs, 8, "bf16", 7).run(attn, 0.25, Hkv)
    shared = Paged(Ks, Vs, qs, 8, "bf16", 7, share={1: (0, 3), 2: (0, 3)}).run(attn, 0.25, Hkv)
    assert np.array_equal(copied, shared), "shared prefix blocks change results"


def check_rows_subset(attn):
    """Asking for a subset of (sequence, head) rows returns those rows."""
    rng = np.random.default_rng(41)
    K, V, q = draw(rng, [9, 30, 2], 4, 2, 8, "f16")
    p = Paged(K, V, q, 8, "f16", 1)
    full = p.run(attn, 0.3, 2)
    rows = [(2, 3), (0, 0), (1, 2), (1, 1)]
    sub = p.run(attn, 0.3, 2, rows=rows)
    assert np.array_equal(sub, np.stack([full[s, j] for s, j in rows]))


def check_sliding_window(attn):
    """Sliding window: SDPA over the contiguous last-W slice; W >= L is no
    window; W = 1 returns the last value row; blocks wholly before the window
    can be freed (table entry -1, contents poisoned) without any effect;
    the block size does not matter."""
    rng = np.random.default_rng(51)
    lens = [1, 7, 16, 17, 40, 70, 129]
    Hq, Hkv, D = 4, 2, 16
    K, V, q = draw(rng, lens, Hq, Hkv, D, "f16")
    scale = 0.31
    paged = Paged(K, V, q, 8, "f16", 3, spare_blocks=5)
    for W in (1, 5, 8, 9, 33, 64):
        got = paged.run(attn, scale, Hkv, window=W)
        want = sdpa_reference([k[-W:] for k in K], [v[-W:] for v in V], q, scale, "f16")
        err = np.max(np.abs(got - want))
        assert err <= 1e-12, f"window {W}: paged vs SDPA on the last W tokens, max |err| {err}"
        freed = paged.free_before_window(W).run(attn, scale, Hkv, window=W)
        assert np.array_equal(freed, got), f"window {W}: freed blocks before the window changed results"
        for B in (16, 32):
            other = Paged(K, V, q, B, "f16", 4).run(attn, scale, Hkv, window=W)
            assert np.array_equal(other, got), f"window {W}: block size {B} changed results"
    full = paged.run(attn, scale, Hkv)
    assert np.array_equal(paged.run(attn, scale, Hkv, window=max(lens)), full), "W >= L must be no window"
    one = paged.run(attn, scale, Hkv, window=1)
    g = Hq // Hkv
    for s in range(len(lens)):
        for j in range(Hq):
            assert np.array_equal(one[s, j], widen(V[s][-1, j // g], "f16")), "W = 1 returns the last value"


def fp8_paged(rng, lens, Hq, Hkv, D, B, placement_seed, q_dtype="f16"):
    """A batch whose cache holds random finite E4M3 codes (placed like Paged)."""
    K = [rng.integers(0, 0x7F, size=(L, Hkv, D)).astype(np.uint8) | (rng.integers(0, 2, size=(L, Hkv, D)) * 0x80).astype(np.uint8)
         for L in lens]
    V = [rng.integers(0, 0x7F, size=(L, Hkv, D)).astype(np.uint8) | (rng.integers(0, 2, size=(L, Hkv, D)) * 0x80).astype(np.uint8)
         for L in lens]
    # keep magnitudes moderate: codes of exponent field <= 9 (|value| < 8)
    K = [np.where(((k >> 3) & 15) > 9, k & 0x87, k).astype(np.uint8) for k in K]
    V = [np.where(((v >> 3) & 15) > 9, v & 0x87, v).astype(np.uint8) for v in V]
    q = to_storage(rng.standard_normal((len(lens), Hq, D)), q_dtype)
    p = Paged(K, V, q, B, "fp8", placement_seed)
    return p, K, V, q


def torch_e4m3(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def check_fp8_kv(attn):
    """8-bit cache: SDPA on torch's decoding of the codes times the scales;
    scaling v_scale by 2 doubles the output exactly; placement and block
    size change nothing."""
    rng = np.random.default_rng(61)
    lens = [1, 9, 16, 33, 70]
    Hq, Hkv, D = 4, 2, 16
    p, K, V, q = fp8_paged(rng, lens, Hq, Hkv, D, 8, 1)
    ks, vs, scale = 0.375, 0.0625, 0.25

    def run(paged, **kw):
        return attn(paged.q, paged.k_cache, paged.v_cache, paged.table, paged.lens, scale, paged.B, Hkv, "f16",
                    kv_format="fp8_e4m3", **kw)

    got = run(p, k_scale=ks, v_scale=vs)
    Kf = [torch_e4m3(k) * ks for k in K]
    Vf = [torch_e4m3(v) * vs for v in V]
    want = sdpa_reference(Kf, Vf, q, scale, "f16", values_are_fp64=True)
    err = np.max(np.abs(got - want))
    assert err <= 1e-12, f"fp8 cache vs SDPA on dequantized values: {err}"
    assert np.array_equal(run(p, k_scale=ks, v_scale=2 * vs), 2 * got), "v_scale must scale the output"
    other = Paged(K, V, q, 16, "fp8", 9, spare_blocks=7)
    assert np.array_equal(run(other, k_scale=ks, v_scale=vs), got), "placement / block size changed results"


ALL_CHECKS = [check_against_sdpa, check_closed_forms, check_invariances, check_rows_subset,
              check_sliding_window, check_fp8_kv]
