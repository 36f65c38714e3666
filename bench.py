#!/usr/bin/env python3
"""Benchmark of the paged-attention decode step on one MI355X.

A step is the decode hot path for one batch: pkv_decode_step, which stores
the token each sequence appends (reshape_and_cache) in the launch that
builds the attention work list, then runs paged decode attention over all
cached tokens (main kernel, plus the split-K reduce when partitions split a
sequence).  On the shared-prefix workload the step is reshape_and_cache and
pkv_paged_attention_decode_shared_prefix, which reads each prompt's shared
blocks once for all its samples (--per-sample-prefix: the plain decode step
instead); that batch is built the way a server builds it (block manager,
stores, and the copy-on-write copies made by copy_blocks at the divergence
step), and the divergence step's copy_blocks is timed on its own.  Inputs
are synthetic, seeded, N(0, 1), and resident in HBM before timing starts.

Default run: the headline workload is the largest one that fits one GPU, a
70B-style grouped-query layer (batch 256, 64 query / 8 KV heads, head_dim
128, bf16, 32-token blocks, context lengths uniform in [1024, 32768], split-K
partitions of 512 tokens + the reduce kernel); the same JSON line carries
`per_config` with the tiny fp32 step, the Llama-2-7B and -13B layers and the
shared-prefix sampling batch at the same --steps and --warmup.

Prints ONE JSON line:
  value        KV GB/s read per step (sum(L) * Hkv * D * 2 * bytes / step time),
               from K steps timed between two HIP events
  roofline     the main attention kernel: algorithmic bytes per launch / its
               average duration vs 8 TB/s HBM.  The duration comes from a
               second pass on the kernel's stream: K launches of the main
               kernel alone, back to back between two HIP events (the work
               list of the first pass reused), or, when a split-K reduce
               follows it (and on the shared-prefix call, for its pass over
               each sequence's own tokens), events right before and after it
               in K steps
  cpu_baseline the fp64 CPU oracle on a bounded sample of the same workload,
               on this host's cores (a reported baseline, not the target)
  per_config   (default run) the other workloads' step time, GB/s, % of peak,
               seq*heads/s and main-kernel roofline fraction

    python bench.py [--steps K] [--warmup W] [--config N] [--gpus 1]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from synthetic import (BEAM_CONFIGS, CONFIGS, DTYPE_BYTES, beam_parents, host_values, kv_bytes,  # noqa: E402
                       make_layout)

METRIC = "paged decode attn: KV GB/s read (% of HBM peak) + seq·heads/sec, 1 GPU"
HBM_PEAK_GBPS = 8000.0
LENGTH_DESC = {
    1: "fixed {5,17,33,64}",
    2: "uniform [128, 2048]",
    3: "lognormal median 400 sigma 1.0, clipped [1, 4096]",
    4: "uniform [1024, 32768]",
    5: "1000-token shared prompt + uniform [1, 512] per-sample tail",
    6: "uniform [1024, 16384], attention over the last 4096",
    8: "uniform [128, 2048]",
    9: "uniform [1024, 32768]",
    10: "uniform [1024, 8192]",
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, run before the GPU is touched (the worker pool
# forks), over a bounded sample of sequences of the same workload.
# ---------------------------------------------------------------------------
_CPU = {}


def _oracle_rows(s):
    import oracle
    c = _CPU
    cfg = c["cfg"]
    oracle.paged_attention_decode(c["q"][s:s + 1], c["k"], c["v"], c["tables"][s:s + 1], c["lens"][s:s + 1],
                                  cfg.scale, cfg.block_size, cfg.num_kv_heads, cfg.dtype,
                                  sliding_window=cfg.sliding_window, kv_format=cfg.kv_format,
                                  k_scale=cfg.k_scale, v_scale=cfg.v_scale)
    return s


def _one_blas_thread():
    """Each worker process runs single-threaded BLAS (one worker per core)."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass


def cpu_baseline(cfg, layout, cpu_seconds: float):
    import multiprocessing as mp

    workers = max(1, min(len(os.sched_getaffinity(0)), 16))
    spp = cfg.samples_per_prompt or 1
    # Enough sequences to keep every worker busy, but a pool small enough to
    # draw on the host in seconds (about 2.5e8 cached values).
    attended = layout.context_lens.astype(np.int64)
    if cfg.sliding_window > 0:
        attended = np.minimum(attended, cfg.sliding_window)
    per_seq = attended * cfg.num_kv_heads * cfg.head_dim * 2
    k, acc = 0, 0
    while k < len(per_seq) and (k < workers or acc < 2.5e8):
        acc += int(per_seq[k])
        k += 1
        if acc >= 2.5e8 and k >= spp:
            break
    k = min(len(per_seq), -(-k // spp) * spp)
    workers = min(workers, k)
    lens = layout.context_lens[:k]
    sub = make_layout(cfg.scaled(num_seqs=k), seed=1000 + k, lengths=lens)
    host = host_values(sub)
    _CPU.update(cfg=cfg, q=host.q, k=host.k_cache, v=host.v_cache, tables=sub.block_tables,
                lens=sub.context_lens)
    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_one_blas_thread) as pool:
        pool.map(_oracle_rows, range(k), chunksize=1)          # warm the workers
        reps, t0 = 0, time.perf_counter()
        while True:
            pool.map(_oracle_rows, range(k), chunksize=1)
            reps += 1
            elapsed = time.perf_counter() - t0
            if elapsed >= cpu_seconds:
                break
    nbytes = kv_bytes(lens, cfg.num_kv_heads, cfg.head_dim, cfg.kv_dtype, cfg.sliding_window) * reps
    return {
        "value": round(nbytes / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": workers,
        "kind": "oracle",
        "sample": (f"first {k} of {len(layout.context_lens)} sequences (all {cfg.num_q_heads} heads, "
                   f"their real lengths, sum {int(lens.sum())} tokens) x {reps} passes, fp64 numpy, "
                   f"{workers} worker processes, {elapsed:.2f} s wall"),
        "seq_heads_per_s": round(k * reps * cfg.num_q_heads / elapsed, 2),
    }


# ---------------------------------------------------------------------------
# HIP events on the launch stream (ctypes on the HIP runtime).
# ---------------------------------------------------------------------------
def loaded_hip_runtime() -> str:
    """Path of the HIP runtime already mapped into this process (torch's own
    copy), so events live in the same runtime as torch's streams."""
    for line in open("/proc/self/maps"):
        path = line.split()[-1]
        if "libamdhip64.so" in path:
            return path
    raise RuntimeError("no HIP runtime loaded")


class HipEvents:
    def __init__(self):
        self.hip = ctypes.CDLL(loaded_hip_runtime())
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []

    def create(self):
        ev = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
        self.events.append(ev)
        return ev

    def record(self, ev, stream):
        assert self.hip.hipEventRecord(ev, ctypes.c_void_p(stream)) == 0

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.hip.hipEventSynchronize(b) == 0
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
        return float(out.value)

    def close(self):
        for ev in self.events:
            self.hip.hipEventDestroy(ev)
        self.events = []


PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "paged_kv_cache_339_amd", "csrc")


def library_source_digest() -> str:
    """sha256 over the library's sources (file names and contents, sorted)."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    counter summary (FETCH_SIZE and WRITE_SIZE, calibrated on copy_blocks),
    or None when there is none or the library changed since it was taken."""
    path = os.path.join(PROFILES, f"{kernel}__{workload}__hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("library_source_sha256") != library_source_digest():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def profiled_duration_us(kernel: str, workload: str):
    """Average duration of `kernel` in the committed rocprofv3 kernel
    statistics of `workload`, or None when there are none for the current
    library sources."""
    path = os.path.join(PROFILES, f"{kernel}__{workload}__kernel_stats.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read().splitlines()
    digest = [l.split(":", 1)[1].strip() for l in text if l.startswith("library_source_sha256:")]
    if not digest or digest[0] != library_source_digest():
        return None
    for line in text:
        if line.startswith(f"pkv::{kernel}"):
            args = line[line.index("<") + 1:line.index(">")].split(", ") if "<" in line else []
            if kernel == "attn_valu_kernel" and len(args) == 9 and args[8] == "true":
                continue      # the one-launch decode-step instance; the roofline times the plain one
            try:
                return float(line.split()[-3])
            except (IndexError, ValueError):
                return None
    return None


def calibrate_copy(launches: int):
    """copy_blocks of 2048 distinct blocks of 128 KiB in each of two caches:
    exactly 512 MiB read and 512 MiB written per launch."""
    import torch
    import paged_kv_cache_339_amd as pkv

    dev = torch.device("cuda:0")
    N, Hkv, B, D = 4096, 32, 16, 128
    kc = torch.zeros((N, Hkv, B, D), dtype=torch.float16, device=dev)
    vc = torch.zeros_like(kc)
    perm = torch.randperm(N, generator=torch.Generator().manual_seed(0))
    pairs = torch.stack([perm[:N // 2], perm[N // 2:]], dim=1).to(torch.int32).to(dev)
    for _ in range(max(1, launches)):
        pkv.copy_blocks(kc, vc, pairs)
    torch.cuda.synchronize()
    per = (N // 2) * Hkv * B * D * 2 * 2
    print(json.dumps({"calibration": "copy_blocks", "launches": launches, "read_bytes_per_launch": per,
                      "write_bytes_per_launch": per}), flush=True)


def beam_cpu_baseline(cfg, cpu_seconds: float):
    """The oracle (block-manager twin, bitwise copy and scatter, fp64
    attention) running the same beam search on host arrays, one core, for a
    bounded number of steps of a 2-request slice of the workload."""
    import oracle
    from synthetic import POISON_BITS, prompt_values, step_values

    sub = cfg.scaled(num_requests=2)
    R, W, B, Hkv, D = sub.num_requests, sub.beam_width, sub.block_size, sub.num_kv_heads, sub.head_dim
    N = sub.pool_blocks()
    width = np.uint32 if sub.dtype == "f32" else np.uint16
    storage = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[sub.dtype]
    kc = np.full((N, Hkv, B, D), POISON_BITS[sub.dtype], dtype=width).view(storage)
    vc = kc.copy()
    bm = oracle.BlockManager(N, B, np.random.default_rng(0).permutation(N))
    pk, pv = prompt_values(sub, 0)
    for r in range(R):
        bm.add_seq(r * W)
        slots = [bm.append(r * W)[0] for _ in range(sub.prompt_len)]
        oracle.reshape_and_cache(pk[r], pv[r], kc, vc, np.array(slots), B)
    parents = beam_parents(sub, 0)
    bank, nbytes, steps, t0 = 0, 0, 0, time.perf_counter()
    while steps < sub.steps and time.perf_counter() - t0 < cpu_seconds:
        old = list(range(bank * R * W, (bank + 1) * R * W))
        new = list(range((1 - bank) * R * W, (2 - bank) * R * W))
        for r in range(R):
            for b in range(W):
                bm.fork(old[r * W + (0 if steps == 0 else int(parents[steps, r, b]))], new[r * W + b])
        for r in range(R):
            for b in range(W):
                if steps > 0 or b == 0:
                    bm.free_seq(old[r * W + b])
        bank = 1 - bank
        slots, pairs = [], []
        for sq in new:
            slot, cow = bm.append(sq)
            slots.append(slot)
            if cow is not None:
                pairs.append(cow)
        if pairs:
            oracle.copy_blocks(kc, vc, pairs)
        q, kn, vn = step_values(sub, 0, steps)
        oracle.reshape_and_cache(kn, vn, kc, vc, np.array(slots), B)
        M = max(len(bm.block_table(sq)) for sq in new)
        tables = np.full((len(new), M), -1, dtype=np.int32)
        for i, sq in enumerate(new):
            tables[i, :len(bm.block_table(sq))] = bm.block_table(sq)
        lens = np.array([bm.seq_len(sq) for sq in new])
        oracle.paged_attention_decode(q, kc, vc, tables, lens, sub.scale, B, Hkv, sub.dtype)
        nbytes += kv_bytes(lens, Hkv, D, sub.dtype)
        steps += 1
    elapsed = time.perf_counter() - t0
    return {"value": round(nbytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": (f"{R} of {cfg.num_requests} requests x {W} beams, {steps} search steps "
                       f"(block manager twin, copy, scatter, fp64 attention), one process, {elapsed:.2f} s")}


def beam_bench(args):
    """Beam search over the paged cache: each timed step is the host control
    plane (fork the chosen parents, free the old beams, reserve slots and
    copy-on-write pairs), the copies of tables / slots / pairs to the GPU,
    pkv_copy_blocks, pkv_reshape_and_cache and
    pkv_paged_attention_decode_shared_prefix (each request's whole prompt
    blocks read once for its beams; --per-sample-prefix: pkv_decode_step),
    then a stream synchronisation (a real search reads the step's scores
    before choosing parents)."""
    import torch
    import paged_kv_cache_339_amd as pkv
    from paged_kv_cache_339_amd._lib import CACHE_POLICIES, AttnOptions, lib
    from paged_kv_cache_339_amd.ops import dtype_code

    K, W = args.steps, args.warmup
    base = BEAM_CONFIGS[args.config]
    policy = args.cache_policy or base.cache_policy
    cfg = base.scaled(steps=max(base.steps, K + W))
    seed = args.config if args.seed is None else args.seed
    R, Wb, B, Hq, Hkv, D = cfg.num_requests, cfg.beam_width, cfg.block_size, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    S, N = cfg.num_seqs, cfg.pool_blocks()
    es = DTYPE_BYTES[cfg.dtype]
    log(f"beam workload {cfg.name}: {R} requests x {Wb} beams, prompt {cfg.prompt_len}, pool {N} blocks")
    cpu = None if args.no_cpu_baseline else beam_cpu_baseline(base, args.cpu_seconds)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[cfg.dtype]
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    kc = torch.randn((N, Hkv, B, D), generator=g, device=dev, dtype=torch.float32).to(tdt)
    vc = torch.randn((N, Hkv, B, D), generator=g, device=dev, dtype=torch.float32).to(tdt)
    total = K + W
    qs = torch.randn((total, S, Hq, D), generator=g, device=dev, dtype=torch.float32).to(tdt)
    ks = torch.randn((total, S, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(tdt)
    vs = torch.randn((total, S, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(tdt)
    parents = beam_parents(cfg, seed)
    cache = pkv.BeamSearchCache(R, Wb, N, B, np.random.default_rng(seed).permutation(N))
    prompt_slots = cache.prefill(cfg.prompt_len)
    for r in range(R):
        pk = torch.randn((cfg.prompt_len, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(tdt)
        pv = torch.randn((cfg.prompt_len, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(tdt)
        pkv.reshape_and_cache(pk, pv, kc, vc, torch.from_numpy(prompt_slots[r]).to(dev))
    M = -(-(cfg.prompt_len + cfg.steps + 1) // B)
    max_ctx = cfg.prompt_len + cfg.steps + 1
    code = dtype_code(kc)
    grouped = not args.per_sample_prefix
    members_np, prefix_np = cache.shared_prefix()
    members = torch.from_numpy(members_np).to(dev)
    prefix_lens = torch.from_numpy(prefix_np).to(dev)
    max_prefix = int(prefix_np.max())
    ws_need = (pkv.shared_prefix_workspace_bytes(S, Hq, Hkv, D, B, max_ctx, R, Wb, max_prefix, code,
                                                 cache_policy=policy) if grouped
               else pkv.workspace_bytes(S, Hq, Hkv, D, B, max_ctx, code))
    ws = torch.empty(max(256, ws_need), dtype=torch.uint8, device=dev)
    out = torch.empty((S, Hq, D), dtype=tdt, device=dev)
    # The step's tables, lengths, slots and copy pairs travel in one pinned
    # buffer and one copy (each piece starting on 16 bytes).
    shapes = dict(tables=(S, M), lens=(S,), slots=(S,), pairs=(S, 2))
    offs, total_ints = {}, 0
    for k, shp in shapes.items():
        offs[k] = total_ints
        total_ints += -(-int(np.prod(shp)) // 4) * 4
    host_flat = torch.empty(total_ints, dtype=torch.int32).pin_memory()
    dev_flat = torch.empty(total_ints, dtype=torch.int32, device=dev)

    def views(flat):
        return {k: flat[offs[k]:offs[k] + int(np.prod(shp))].view(shp) for k, shp in shapes.items()}

    pin, dbuf = views(host_flat), views(dev_flat)
    stream = torch.cuda.current_stream()
    ev = HipEvents()
    vp = ctypes.c_void_p
    begins = [ev.create() for _ in range(total)]
    ends = [ev.create() for _ in range(total)]
    step_start = [ev.create() for _ in range(total)]
    step_end = [ev.create() for _ in range(total)]
    kv_step = []
    own_step = []       # bytes the timed kernel reads per step: K/V of its tokens and table entries
    host_s = []

    def step(t):
        h0 = time.perf_counter()
        _, slots, pairs = cache.step(parents[t])
        tables, lens = cache.tables(M)
        host_s.append(time.perf_counter() - h0)
        pin["tables"].numpy()[:] = tables
        pin["lens"].numpy()[:] = lens
        pin["slots"].numpy()[:] = slots
        n_pairs = len(pairs)
        if n_pairs:
            pin["pairs"].numpy()[:n_pairs] = pairs
        ev.record(step_start[t], stream.cuda_stream)
        dev_flat.copy_(host_flat, non_blocking=True)
        if n_pairs:
            st = lib.pkv_copy_blocks(vp(kc.data_ptr()), vp(vc.data_ptr()), vp(dbuf["pairs"].data_ptr()), n_pairs,
                                     Hkv, B, D, N, code, vp(stream.cuda_stream))
            assert st == 0, st
        opts = AttnOptions(0, 0, begins[t], ends[t], 0, 0, 1.0, 1.0, 0, CACHE_POLICIES[policy])
        if grouped:
            st = lib.pkv_reshape_and_cache(vp(ks[t].data_ptr()), vp(vs[t].data_ptr()), vp(kc.data_ptr()),
                                           vp(vc.data_ptr()), vp(dbuf["slots"].data_ptr()), S, Hkv, D, B, N, code,
                                           vp(stream.cuda_stream))
            assert st == 0, st
            st = lib.pkv_paged_attention_decode_shared_prefix(
                vp(out.data_ptr()), vp(qs[t].data_ptr()), vp(kc.data_ptr()), vp(vc.data_ptr()),
                vp(dbuf["tables"].data_ptr()), vp(dbuf["lens"].data_ptr()), vp(prefix_lens.data_ptr()),
                vp(members.data_ptr()), R, Wb, max_prefix, cfg.scale, B, Hkv, S, Hq, D, M, max_ctx, N, code,
                vp(ws.data_ptr()), ws.numel(), ctypes.byref(opts), vp(stream.cuda_stream))
            assert st == 0, st
        else:
            st = lib.pkv_decode_step(vp(out.data_ptr()), vp(qs[t].data_ptr()), vp(ks[t].data_ptr()),
                                     vp(vs[t].data_ptr()), vp(kc.data_ptr()), vp(vc.data_ptr()),
                                     vp(dbuf["slots"].data_ptr()), vp(dbuf["tables"].data_ptr()),
                                     vp(dbuf["lens"].data_ptr()), cfg.scale, B, Hkv, S, Hq, D, M, max_ctx, N, code,
                                     vp(ws.data_ptr()), ws.numel(), ctypes.byref(opts), vp(stream.cuda_stream))
            assert st == 0, st
        ev.record(step_end[t], stream.cuda_stream)
        stream.synchronize()
        kv_step.append(kv_bytes(lens, Hkv, D, cfg.dtype))
        l64 = lens.astype(np.int64)
        own = l64 - (prefix_np if grouped else 0)
        own_blk = -(-l64 // B) - ((prefix_np // B) if grouped else 0)
        own_step.append(int(own.sum()) * Hkv * D * 2 * es + int(own_blk.sum()) * 4 * Hkv)

    for t in range(W):
        step(t)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for t in range(W, total):
        step(t)
    wall = time.perf_counter() - wall0
    gpu_ms = [ev.ms(step_start[t], step_end[t]) for t in range(W, total)]
    main_ms = [ev.ms(begins[t], ends[t]) for t in range(W, total)]
    ev.close()
    cache.close()
    assert torch.isfinite(out.float()).all().item(), "non-finite attention output"
    kv = float(np.mean(kv_step[W:]))
    step_s = wall / K
    main_s = float(np.mean(main_ms)) / 1e3
    alg = float(np.mean(own_step[W:])) + 2 * S * Hq * D * es + S * (8 if grouped else 4)
    tag = cfg.name + ("" if policy == base.cache_policy else f"_{policy}") + ("" if grouped else "_persample")
    print(json.dumps({
        "metric": METRIC, "value": round(kv / step_s / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(step_s * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": tag,
                   "cache_policy": policy, "requests": R, "beam_width": Wb, "prompt_len": cfg.prompt_len,
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "block_size": B, "kv_dtype": cfg.dtype,
                   "pool_blocks": N, "kv_bytes_per_step": int(kv),
                   "step": "host fork/free/append + H2D tables + copy_blocks + " + (
                       "reshape_and_cache + decode_shared_prefix (each request's prompt blocks read once) + sync"
                       if grouped else "decode_step + sync")},
        "pct_hbm_peak": round(100 * kv / step_s / 1e9 / HBM_PEAK_GBPS, 2),
        "seq_heads_per_s": round(S * Hq / step_s, 1),
        "host_ms_per_step": round(1e3 * float(np.mean(host_s[W:])), 4),
        "gpu_ms_per_step": round(float(np.mean(gpu_ms)), 4),
        "roofline": {"bound": "hbm", "achieved": round(alg / main_s / 1e9, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(alg / main_s / 1e9 / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "attn_valu_kernel", "bytes_per_launch": int(alg),
                     "note": ("the pass over each beam's own tokens (the prompt's whole blocks are read by the "
                              "grouped pass)") if grouped else
                             "logical bytes: the beams of a request share their prompt blocks, served from cache"},
        "cpu_baseline": cpu,
    }), flush=True)


def swap_bench(args):
    """Swapping for preemption: a quarter of the workload's live blocks go
    to a pinned host pool (swap out) and come back (swap in), each direction
    one pkv_swap_blocks launch, timed with HIP events."""
    import torch
    import paged_kv_cache_339_amd as pkv
    from synthetic import device_values

    cfg = CONFIGS[args.config]
    layout = make_layout(cfg, seed=args.config)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, kc, vc, _, _ = device_values(layout, device=dev)
    used = layout.pool_order[:layout.used_blocks]
    n = max(1, len(used) // 4)
    host_k = torch.empty((n,) + tuple(kc.shape[1:]), dtype=kc.dtype, pin_memory=True)
    host_v = torch.empty_like(host_k, pin_memory=True)
    out_pairs = torch.from_numpy(np.stack([used[:n], np.arange(n)], axis=1).astype(np.int32)).to(dev)
    in_pairs = torch.from_numpy(np.stack([np.arange(n), used[:n]], axis=1).astype(np.int32)).to(dev)
    block_bytes = kc[0].numel() * kc.element_size()
    ev = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    for name, fn in (("out", lambda: pkv.swap_blocks(host_k, host_v, kc, vc, out_pairs)),
                     ("in", lambda: pkv.swap_blocks(kc, vc, host_k, host_v, in_pairs))):
        for _ in range(args.warmup):
            fn()
        a, b = ev.create(), ev.create()
        ev.record(a, stream)
        for _ in range(args.steps):
            fn()
        ev.record(b, stream)
        ms = ev.ms(a, b) / args.steps
        res[name] = {"ms": round(ms, 4), "GBps": round(2 * n * block_bytes / ms / 1e6, 2)}
    ev.close()
    print(json.dumps({"metric": "swap_blocks GB/s between HBM and pinned host memory, 1 GPU",
                      "value": round((res["out"]["GBps"] + res["in"]["GBps"]) / 2, 2), "unit": "GB/s",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
                      "data": "synthetic", "config": {"workload": cfg.name, "blocks": int(n),
                                                      "bytes_per_direction": int(2 * n * block_bytes)},
                      "swap_out": res["out"], "swap_in": res["in"]}), flush=True)


W_COPY = 3          # untimed copy_blocks launches before the timed ones


def shared_prefix_state(cfg, layout, dev, seed: int) -> dict:
    """The shared-prefix sampling batch built the way a server builds it.

    The host block manager (pkv_bm_*, the C++ control plane) prefills each
    prompt, forks it for the samples, and appends their tokens one decode
    step at a time (every sample one token per step).  The library stores
    every token (pkv_reshape_and_cache) and, at the divergence step, makes the
    copy-on-write copies of each prompt's partial last block (pkv_copy_blocks)
    before any sample token lands in them.  The pool size and the context
    lengths are the workload's (`layout`); values are N(0, 1) drawn on the GPU.
    The last token of each sequence is left for the timed step to store."""
    import torch
    import paged_kv_cache_339_amd as pkv

    S, spp, P, B = len(layout.context_lens), cfg.samples_per_prompt, cfg.prompt_len, cfg.block_size
    Hq, Hkv, D, N = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, layout.num_blocks
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[cfg.dtype]
    g = torch.Generator(device=dev)
    g.manual_seed(seed * 64 + 9)

    def randn(*shape):
        return torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(tdt)

    def ints(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    # Slots that hold no token stay all-ones bits (NaN in every format).
    kc = torch.full((N, Hkv, B, D), -1, dtype=torch.int16 if tdt != torch.float32 else torch.int32,
                    device=dev).view(tdt)
    vc = kc.clone()
    bm = pkv.BlockManager(N, B, S, free_order=layout.pool_order)
    prompt_slots = []
    for p in range(S // spp):
        bm.add_seq(p * spp)
        sl, pr = bm.append_batch([p * spp] * P)
        assert len(pr) == 0
        prompt_slots.append(sl)
    prompt_slots = np.concatenate(prompt_slots)
    pkv.reshape_and_cache(randn(len(prompt_slots), Hkv, D), randn(len(prompt_slots), Hkv, D), kc, vc,
                          ints(prompt_slots))
    for p in range(S // spp):
        for k in range(1, spp):
            bm.fork(p * spp, p * spp + k)
    tails = layout.context_lens.astype(np.int64) - P
    assert tails.min() >= 1
    stored, last = [], np.full(S, -1, dtype=np.int32)
    div_pairs = None
    for t in range(int(tails.max())):
        seqs = np.nonzero(tails > t)[0].astype(np.int32)
        sl, pr = bm.append_batch(seqs)
        if t == 0:
            div_pairs = pr
            if len(pr):
                pkv.copy_blocks(kc, vc, ints(pr))          # before any sample token is stored
        else:
            assert len(pr) == 0
        fin = tails[seqs] == t + 1
        last[seqs[fin]] = sl[fin]
        stored.append(sl[~fin])
    stored = np.concatenate(stored)
    pkv.reshape_and_cache(randn(len(stored), Hkv, D), randn(len(stored), Hkv, D), kc, vc, ints(stored))
    M = layout.block_tables.shape[1]
    tables, lens = bm.export(np.arange(S), M)
    bm.close()
    assert np.array_equal(lens, layout.context_lens) and (last >= 0).all()
    torch.cuda.synchronize()
    return {"q": randn(S, Hq, D), "k_cache": kc, "v_cache": vc, "k_new": randn(S, Hkv, D),
            "v_new": randn(S, Hkv, D), "tables": tables, "lens": lens, "slots": last,
            "pairs": div_pairs}


def launch_floor(steps: int) -> dict:
    """The shortest back-to-back library launch on this GPU: K launches of a
    one-token pkv_reshape_and_cache (head_dim 64, two heads, fp32) through
    the C ABI with prepared arguments, as the timed steps are issued, between
    two events.  The latency floor a tiny decode step sits on."""
    import torch
    from paged_kv_cache_339_amd._lib import lib
    dev = torch.device("cuda:0")
    k = torch.zeros((1, 2, 64), dtype=torch.float32, device=dev)
    kc = torch.zeros((4, 2, 16, 64), dtype=torch.float32, device=dev)
    vc = torch.zeros_like(kc)
    slot = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    vp = ctypes.c_void_p
    a_ = (vp(k.data_ptr()), vp(k.data_ptr()), vp(kc.data_ptr()), vp(vc.data_ptr()), vp(slot.data_ptr()),
          1, 2, 64, 16, 4, 0, vp(stream))
    for _ in range(5):
        assert lib.pkv_reshape_and_cache(*a_) == 0
    torch.cuda.synchronize()
    ev = HipEvents()
    a, b = ev.create(), ev.create()
    ev.record(a, stream)
    for _ in range(steps):
        lib.pkv_reshape_and_cache(*a_)
    ev.record(b, stream)
    us = ev.ms(a, b) * 1e3 / steps
    ev.close()
    return {"us": round(us, 2),
            "what": "one-token reshape_and_cache through the C ABI, K back-to-back launches between two events"}


def per_config_entry(r: dict) -> dict:
    """The per-workload summary carried beside the headline."""
    keys = ("ms_per_step", "value", "unit", "pct_hbm_peak", "seq_heads_per_s", "attention_main_us")
    e = {k: r[k] for k in keys}
    e["config"] = {k: r["config"][k] for k in ("batch", "q_heads", "kv_heads", "head_dim", "block_size",
                                               "kv_dtype", "partition_tokens", "partitions_per_seq", "kernel",
                                               "step")}
    rf = r["roofline"]
    e["main_kernel"] = {k: rf[k] for k in ("kernel", "achieved", "frac", "bytes_per_launch", "timing",
                                           "rocprof_avg_us", "traffic")}
    for k in ("grouped_prefix", "copy_blocks", "launch_floor"):
        if k in r:
            e[k] = r[k]
    return e


def run_child(args, idx: int, extra=()) -> dict:
    """One workload in a process of its own (fresh device memory, as a
    server allocates its pool once at start-up); its JSON line is returned
    and its progress lines pass through to stderr."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--config", str(idx), "--steps", str(args.steps),
           "--warmup", str(args.warmup), "--no-cpu-baseline", *extra]
    if args.seed is not None:
        cmd += ["--seed", str(args.seed)]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
    if res.returncode != 0:
        sys.exit(f"workload {idx} failed (exit {res.returncode})")
    return json.loads([line for line in res.stdout.splitlines() if line.startswith("{")][-1])


def suite(args):
    """The default run: the headline workload (the largest single-GPU one,
    the 70B-style GQA layer at its stated 512-token split-K with the reduce
    kernel) with its roofline and CPU baseline, and in the same JSON line the
    other workloads (tiny fp32, Llama-2-7B and -13B layers, shared-prefix
    sampling) at the same steps and warmup.  This process never touches the
    GPU: the oracle baseline runs here first (its worker pool forks), then
    each workload runs in a child process of its own, one after the other.
    (In one process, a workload allocated after another's buffers had been
    freed measured 2-4% slower.)"""
    cpu = None
    if not args.no_cpu_baseline:
        cfg = CONFIGS[4]
        layout = make_layout(cfg, seed=4 if args.seed is None else args.seed)
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(cfg, layout, args.cpu_seconds)
        log(f"cpu baseline: {cpu['value']} GB/s on {cpu['cores']} cores")
    head = run_child(args, 4)
    head["cpu_baseline"] = cpu
    per = {}
    for idx in (1, 2, 3, 5):
        r = run_child(args, idx, ["--launch-floor"] if idx == 1 else [])
        per[r["config"]["workload"]] = per_config_entry(r)
    head["per_config"] = per
    head["process_per_workload"] = True
    return head


def decode_workload(args, idx: int, with_cpu: bool, cpu=None) -> dict:
    """One decode workload: K timed steps, the main kernel's duration, and
    (with_cpu) the oracle's CPU baseline, or `cpu` when it was measured
    before.  Returns the result record."""
    cfg = CONFIGS[idx]
    part = cfg.partition_size if args.partition_size < 0 else args.partition_size
    # The workload's name, tagged with every change from its stated form.
    tag = cfg.name
    if args.tp_share > 1:
        if cfg.num_kv_heads % args.tp_share:
            sys.exit(f"--tp-share {args.tp_share} does not divide {cfg.num_kv_heads} KV heads")
        cfg = cfg.scaled(num_q_heads=cfg.num_q_heads // args.tp_share,
                         num_kv_heads=cfg.num_kv_heads // args.tp_share)
        tag += f"_tp{args.tp_share}share"
    if args.block_size:
        cfg = cfg.scaled(block_size=args.block_size)
        tag += f"_b{args.block_size}"
    if args.placement:
        cfg = cfg.scaled(placement=args.placement)
        tag += "" if args.placement == "shuffled" else f"_{args.placement}"
    if args.cache_policy and args.cache_policy != cfg.cache_policy:
        cfg = cfg.scaled(cache_policy=args.cache_policy)
        tag += f"_{args.cache_policy}"
    if args.per_sample_prefix and cfg.lengths != "shared_prefix":
        sys.exit("--per-sample-prefix needs a shared-prefix workload")
    grouped = cfg.lengths == "shared_prefix" and not args.per_sample_prefix
    if args.per_sample_prefix:
        tag += "_persample"
    if grouped:
        # The prefix is read once per group: no partition at the prompt's end
        # and no cache-resident re-reads are needed.
        if args.partition_size < 0:
            part = 0
        if not args.cache_policy:
            cfg = cfg.scaled(cache_policy="stream")
        cfg = cfg.scaled(partition_size=part)
    if part != cfg.partition_size:
        tag += f"_partition{part or 'auto'}"
    if args.kernel != "auto":
        tag += f"_{args.kernel}"
    seed = idx if args.seed is None else args.seed
    layout = make_layout(cfg, seed=seed)
    S, Hq, Hkv, D, B = len(layout.context_lens), cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    es = DTYPE_BYTES[cfg.dtype]
    step_kv = kv_bytes(layout.context_lens, Hkv, D, cfg.kv_dtype, cfg.sliding_window)
    log(f"workload {cfg.name}: S={S} Hq={Hq} Hkv={Hkv} D={D} B={B} {cfg.dtype} sum(L)={int(layout.context_lens.sum())} "
        f"pool={layout.num_blocks} blocks KV/step={step_kv / 1e9:.3f} GB")

    if with_cpu and cpu is None:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(cfg, layout, args.cpu_seconds)
        log(f"cpu baseline: {cpu['value']} GB/s on {cpu['cores']} cores")

    import torch
    import paged_kv_cache_339_amd as pkv
    from paged_kv_cache_339_amd._lib import CACHE_POLICIES, KERNELS, KV_FORMATS, AttnOptions, lib
    from paged_kv_cache_339_amd.ops import dtype_code
    from synthetic import device_values

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def ints(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    extra = {}
    cow = None
    if cfg.lengths == "shared_prefix":
        # Built as a server builds it: block manager, stores, and the
        # copy-on-write copies made by copy_blocks at the divergence step.
        st = shared_prefix_state(cfg, layout, dev, seed)
        q, kc, vc, kn, vn = st["q"], st["k_cache"], st["v_cache"], st["k_new"], st["v_new"]
        layout.block_tables, layout.context_lens, layout.new_slots = st["tables"], st["lens"], st["slots"]
        cow = st["pairs"]
    else:
        q, kc, vc, kn, vn = device_values(layout, device=dev)
    tables, lens, slots = ints(layout.block_tables), ints(layout.context_lens), ints(layout.new_slots)
    out = torch.empty_like(q)
    code = dtype_code(q)
    max_ctx = layout.max_context_len
    ws_bytes = pkv.workspace_bytes(S, Hq, Hkv, D, B, max_ctx, code, part, args.kernel, cfg.sliding_window,
                                   cfg.kv_format, cfg.k_scale, cfg.v_scale)
    if grouped:
        from synthetic import shared_prefix_groups
        members_np, prefix_np = shared_prefix_groups(layout)
        members, prefix_lens = ints(members_np), ints(prefix_np)
        Gn, Gs, max_prefix = members_np.shape[0], members_np.shape[1], int(prefix_np.max())
        ws_bytes = pkv.shared_prefix_workspace_bytes(S, Hq, Hkv, D, B, max_ctx, Gn, Gs, max_prefix, code, part,
                                                     args.kernel, cfg.kv_format, cfg.k_scale, cfg.v_scale,
                                                     cfg.cache_policy)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()

    ev = HipEvents()
    vp = ctypes.c_void_p
    if cow is not None:
        # The divergence step's copies, timed on their own: the same sources
        # copied into blocks no table names (the real copies were made once,
        # in setup, before the samples' tokens landed in them).
        used = set(np.unique(layout.block_tables[layout.block_tables >= 0]).tolist())
        free = np.array([b for b in range(layout.num_blocks) if b not in used][:len(cow)], dtype=np.int64)
        assert len(free) == len(cow), "pool has no room for a second set of copy destinations"
        cpairs = ints(np.stack([cow[:, 0], free], axis=1))
        cargs = (vp(kc.data_ptr()), vp(vc.data_ptr()), vp(cpairs.data_ptr()), len(cow), Hkv, B, D,
                 layout.num_blocks, dtype_code(kc), vp(stream))
        for _ in range(W_COPY):
            assert lib.pkv_copy_blocks(*cargs) == 0
        c0, c1 = ev.create(), ev.create()
        ev.record(c0, stream)
        for _ in range(args.steps):
            assert lib.pkv_copy_blocks(*cargs) == 0
        ev.record(c1, stream)
        copy_us = ev.ms(c0, c1) * 1e3 / args.steps
        moved = 2 * 2 * len(cow) * Hkv * B * D * DTYPE_BYTES[cfg.kv_dtype]      # read + written, K and V
        extra["copy_blocks"] = {"pairs": int(len(cow)), "us": round(copy_us, 2),
                                "bytes_moved": int(moved), "GBps": round(moved / copy_us / 1e3, 1),
                                "timing": "K back-to-back launches between two events",
                                "note": "64 sources copied 7 times each: repeated source reads come from cache"}

    def step_args(opts):
        """pkv_decode_step: store each sequence's new token and attend."""
        return (vp(out.data_ptr()), vp(q.data_ptr()), vp(kn.data_ptr()), vp(vn.data_ptr()), vp(kc.data_ptr()),
                vp(vc.data_ptr()), vp(slots.data_ptr()), vp(tables.data_ptr()), vp(lens.data_ptr()), cfg.scale,
                B, Hkv, S, Hq, D, layout.block_tables.shape[1], max_ctx, layout.num_blocks, code,
                vp(ws.data_ptr()), ws.numel(), ctypes.byref(opts), vp(stream))

    def decode_args(opts):
        """pkv_paged_attention_decode over the caches as the steps left them."""
        return (vp(out.data_ptr()), vp(q.data_ptr()), vp(kc.data_ptr()), vp(vc.data_ptr()), vp(tables.data_ptr()),
                vp(lens.data_ptr()), cfg.scale, B, Hkv, S, Hq, D, layout.block_tables.shape[1], max_ctx,
                layout.num_blocks, code, vp(ws.data_ptr()), ws.numel(), ctypes.byref(opts), vp(stream))

    def grouped_args(opts):
        """pkv_paged_attention_decode_shared_prefix over the caches as the steps left them."""
        return (vp(out.data_ptr()), vp(q.data_ptr()), vp(kc.data_ptr()), vp(vc.data_ptr()), vp(tables.data_ptr()),
                vp(lens.data_ptr()), vp(prefix_lens.data_ptr()), vp(members.data_ptr()), Gn, Gs, max_prefix,
                cfg.scale, B, Hkv, S, Hq, D, layout.block_tables.shape[1], max_ctx, layout.num_blocks, code,
                vp(ws.data_ptr()), ws.numel(), ctypes.byref(opts), vp(stream))

    if grouped:
        step_args = grouped_args      # noqa: F811  (the step's attention call)

    scatter_args = (vp(kn.data_ptr()), vp(vn.data_ptr()), vp(kc.data_ptr()), vp(vc.data_ptr()), vp(slots.data_ptr()),
                    S, Hkv, D, B, layout.num_blocks, code, vp(stream))

    K, W = args.steps, args.warmup
    win = cfg.sliding_window
    kvf = KV_FORMATS[cfg.kv_format]
    chosen_part, parts_per_seq, kernel_used = pkv.plan_info(S, Hq, Hkv, D, B, max_ctx, code, part, args.kernel, win,
                                                            cfg.kv_format, cfg.k_scale, cfg.v_scale)
    cp = CACHE_POLICIES[cfg.cache_policy]
    plain = AttnOptions(part, KERNELS[args.kernel], None, None, win, kvf, cfg.k_scale, cfg.v_scale, 0, cp)
    warm_args = step_args(plain)

    def step(a):
        if grouped:
            # The new tokens' store, then attention with each prompt's shared
            # blocks read once for its samples.
            st = lib.pkv_reshape_and_cache(*scatter_args)
            assert st == 0, st
            st = lib.pkv_paged_attention_decode_shared_prefix(*a)
        else:
            st = lib.pkv_decode_step(*a)
        assert st == 0, st

    for _ in range(W):
        step(warm_args)
    torch.cuda.synchronize()

    # Pass 1: the K timed steps, bracketed by two events only (an event
    # recorded between two kernels delays the second by several us).
    t_start, t_stop = ev.create(), ev.create()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev.record(t_start, stream)
    for i in range(K):
        step(warm_args)
    ev.record(t_stop, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = ev.ms(t_start, t_stop)
    # Pass 2: the main attention kernel's duration.  Without a split-K reduce
    # it runs K times back to back on the work list pass 1 left in the
    # workspace (reuse_plan), between two events; with one, events go right
    # before and after the main kernel inside each of K more steps.
    if parts_per_seq == 1 and not grouped:
        reuse = AttnOptions(part, KERNELS[args.kernel], None, None, win, kvf, cfg.k_scale, cfg.v_scale, 1, cp)
        dec = decode_args(reuse)
        m0, m1 = ev.create(), ev.create()
        ev.record(m0, stream)
        for i in range(K):
            st = lib.pkv_paged_attention_decode(*dec)
            assert st == 0, st
        ev.record(m1, stream)
        torch.cuda.synchronize()
        main_ms = [ev.ms(m0, m1) / K]
        main_timing = "K back-to-back launches of the main kernel between two events"
    else:
        begins = [ev.create() for _ in range(K)]
        ends = [ev.create() for _ in range(K)]
        for i in range(K):
            step(step_args(AttnOptions(part, KERNELS[args.kernel], begins[i], ends[i], win, kvf, cfg.k_scale,
                                       cfg.v_scale, 0, cp)))
        torch.cuda.synchronize()
        main_ms = [ev.ms(begins[i], ends[i]) for i in range(K)]
        main_timing = "events right before and after the main kernel in each of K steps"
        if grouped:
            main_timing += " (the pass over each sequence's own tokens)"
    ev.close()
    assert torch.isfinite(out.float()).all().item(), "non-finite attention output"

    step_s = total_ms / 1e3 / K
    main_s = float(np.mean(main_ms)) / 1e3
    lens64 = layout.context_lens.astype(np.int64)
    first = np.maximum(0, lens64 - win) // B if win > 0 else np.zeros_like(lens64)
    nblk = -(-lens64 // B) - first                    # table entries read per (sequence, KV head)
    alg_bytes = step_kv + 2 * S * Hq * D * es + int(nblk.sum()) * 4 * Hkv + S * 4   # es: q / out format
    if grouped:
        # The timed kernel is the pass over each sequence's own tokens
        # [P_s, L_s); the shared prefixes are read by the grouped pass.
        kvs = DTYPE_BYTES[cfg.kv_dtype]
        own = lens64 - prefix_np
        own_blk = -(-lens64 // B) - prefix_np // B
        alg_bytes = int(own.sum()) * Hkv * D * 2 * kvs + 2 * S * Hq * D * es + int(own_blk.sum()) * 4 * Hkv + S * 8
        pre_tokens = int(prefix_np[members_np[:, 0]].sum())
        extra["grouped_prefix"] = {
            "groups": Gn, "members": Gs, "prefix_tokens": int(prefix_np[0]),
            "unique_kv_bytes_per_step": (pre_tokens + int(own.sum())) * Hkv * D * 2 * kvs,
            "prefix_pass_kv_bytes": pre_tokens * Hkv * D * 2 * kvs,
            "own_pass_kv_bytes": int(own.sum()) * Hkv * D * 2 * kvs}
    achieved = alg_bytes / main_s / 1e9
    kv_gbps = step_kv / step_s / 1e9
    result = {
        "metric": METRIC,
        "value": round(kv_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(total_ms / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # The workload's query / output format (caches: config.kv_dtype); the
        # arithmetic is in "compute".
        "dtype": cfg.dtype,
        "compute": ("fp32 on the vector ALUs" if kernel_used == "valu" else
                    f"{cfg.dtype} operands (8-bit codes widened to them) on the matrix cores, fp32 accumulation"),
        "data": "synthetic",
        "config": {
            "workload": tag,
            "batch": S, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "block_size": B,
            "kv_dtype": cfg.kv_dtype, "context_lens": LENGTH_DESC[idx],
            "sum_context_tokens": int(layout.context_lens.sum()), "pool_blocks": layout.num_blocks,
            "kv_bytes_per_step": step_kv, "partition_size": part, "partition_tokens": chosen_part,
            "partitions_per_seq": parts_per_seq, "kernel": kernel_used,
            "sliding_window": win, "kv_format": cfg.kv_format, "cache_policy": cfg.cache_policy,
            "step": ("reshape_and_cache + decode_shared_prefix (grouped prefix pass, own-token pass, merge)"
                     if grouped else "decode_step (new-token store + plan, attention)"),
        },
        **extra,
        "pct_hbm_peak": round(100 * kv_gbps / HBM_PEAK_GBPS, 2),
        "seq_heads_per_s": round(S * Hq / step_s, 1),
        "attention_main_us": round(main_s * 1e6, 2),
        "wall_ms_per_step": round(wall * 1e3 / K, 5),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(f"attn_{kernel_used}_kernel", tag),
            "kernel": f"attn_{kernel_used}_kernel",
            "bytes_per_launch": int(alg_bytes),
            "timing": main_timing,
            "rocprof_avg_us": profiled_duration_us(f"attn_{kernel_used}_kernel", tag),
        },
        "cpu_baseline": cpu,
    }
    return result


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=None, choices=sorted(CONFIGS) + sorted(BEAM_CONFIGS),
                    help="one workload; default: the headline (workload 4) with workloads 1, 2, 3 and 5 "
                         "in per_config")
    ap.add_argument("--partition-size", type=int, default=-1,
                    help="split-K partition in tokens (0 = library default; -1 = the workload's own)")
    ap.add_argument("--kernel", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--placement", default=None, choices=["shuffled", "contiguous"],
                    help="contiguous: each sequence's blocks adjacent and in order (the cost of paging)")
    ap.add_argument("--block-size", type=int, default=0, help="override the workload's block size")
    ap.add_argument("--tp-share", type=int, default=1,
                    help="N > 1: one GPU's share of N-way tensor parallelism (heads / N)")
    ap.add_argument("--cache-policy", default=None, choices=["stream", "keep"],
                    help="override the workload's key/value load policy")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU work budget of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--launch-floor", action="store_true",
                    help="also time the shortest back-to-back library launch (a one-token reshape_and_cache)")
    ap.add_argument("--per-sample-prefix", action="store_true",
                    help="shared-prefix workloads: read the shared prompt blocks once per sample (plain decode "
                         "step, cache-resident re-reads) instead of once per prompt for all its samples "
                         "(pkv_paged_attention_decode_shared_prefix, the default)")
    ap.add_argument("--swap", action="store_true",
                    help="instead of the decode step, time pkv_swap_blocks of a quarter of the workload's "
                         "blocks to a pinned host pool and back (PCIe-bound)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="instead of the decode step, run copy_blocks over a known number of bytes "
                         "(the reference reading for the HBM traffic counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        log("bench.py measures one GPU only: the library has no multi-GPU path "
            "(the decode step shards by KV head or by sequence with no exchange); run with --gpus 1")
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.steps)
        return
    if args.config in BEAM_CONFIGS:
        beam_bench(args)
        return
    if args.swap:
        if args.config is None:
            sys.exit("--swap needs --config")
        swap_bench(args)
        return

    if args.config is None:
        result = suite(args)
    else:
        result = decode_workload(args, args.config, not args.no_cpu_baseline)
        if args.launch_floor:
            result["launch_floor"] = launch_floor(args.steps)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
