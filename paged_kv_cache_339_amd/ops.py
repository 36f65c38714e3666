"""Argument marshalling from torch tensors / numpy arrays to the C ABI.

Device tensors must be contiguous and on the GPU; the stream defaults to
torch's current stream.  Nothing here computes: each call is one library
call (plus, at most, a workspace allocation when the caller passes none,
marked as used by the call's stream).
"""
from __future__ import annotations

import ctypes

import numpy as np

from ._lib import CACHE_POLICIES, KERNELS, KV_FORMATS, AttnOptions, PkvError, c_i32p, check, lib


def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    """Element format of a tensor: 8-bit caches are uint8 (or float8_e4m3fn) tensors of E4M3 codes."""
    torch = _torch()
    codes = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.uint8: 3, torch.float8_e4m3fn: 3}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _stream(stream):
    torch = _torch()
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dev(t, name, dtype=None, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _options(partition_size, kernel, main_events, sliding_window=0, kv_format="same", k_scale=1.0, v_scale=1.0,
             reuse_plan=False, cache_policy="stream"):
    ev0, ev1 = (None, None) if main_events is None else main_events
    return AttnOptions(int(partition_size), KERNELS[kernel],
                       None if ev0 is None else ctypes.c_void_p(int(ev0)),
                       None if ev1 is None else ctypes.c_void_p(int(ev1)), int(sliding_window),
                       KV_FORMATS[kv_format], float(k_scale), float(v_scale), int(bool(reuse_plan)),
                       CACHE_POLICIES[cache_policy])


def plan_info(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len, dtype_code_,
              partition_size=0, kernel="auto", sliding_window=0, kv_format="same", k_scale=1.0, v_scale=1.0):
    """(partition_size, max_parts, kernel name) a decode call with these arguments launches."""
    opts = _options(partition_size, kernel, None, sliding_window, kv_format, k_scale, v_scale)
    part, parts, kern = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    st = lib.pkv_paged_attention_plan_info(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                           max_context_len, dtype_code_, ctypes.byref(opts), ctypes.byref(part),
                                           ctypes.byref(parts), ctypes.byref(kern))
    check(st, "plan_info")
    names = {v: k for k, v in KERNELS.items()}
    return part.value, parts.value, names[kern.value]


def workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len,
                    dtype_code_, partition_size=0, kernel="auto", sliding_window=0, kv_format="same",
                    k_scale=1.0, v_scale=1.0) -> int:
    opts = _options(partition_size, kernel, None, sliding_window, kv_format, k_scale, v_scale)
    return int(lib.pkv_paged_attention_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                       block_size, max_context_len, dtype_code_,
                                                       ctypes.byref(opts)))


def _check_attention_shapes(out, q, k_cache, v_cache, block_tables, context_lens, block_size, num_kv_heads,
                            kv_format="same"):
    S, Hq, D = q.shape
    N, Hkv, B, D2 = k_cache.shape
    if tuple(out.shape) != (S, Hq, D) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must match each other")
    if kv_format == "same" and k_cache.dtype != q.dtype:
        raise ValueError("the caches must have q's dtype")
    if kv_format == "fp8_e4m3" and dtype_code(k_cache) != 3:
        raise ValueError("8-bit caches must be uint8 (or float8_e4m3fn) tensors of E4M3 codes")
    if D2 != D or B != block_size or Hkv != num_kv_heads:
        raise ValueError("cache shape disagrees with head_dim / block_size / num_kv_heads")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [S, M] and context_lens [S]")


def _torch_stream(stream):
    """torch stream object for a `stream` argument (None: None)."""
    torch = _torch()
    if stream is None:
        return None
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _temp_workspace(need, device, stream):
    """A workspace the wrapper allocates for one call.  torch's caching
    allocator ties the block to the current stream, but the library's kernels
    run on `stream`: the block is marked as used there too, so the allocator
    does not hand its bytes to another allocation before that stream's work
    (the plan, main and reduce kernels) is done."""
    torch = _torch()
    workspace = torch.empty(need, dtype=torch.uint8, device=device)
    ts = _torch_stream(stream)
    if ts is not None:
        workspace.record_stream(ts)
    return workspace


def _workspace(workspace, S, Hq, Hkv, D, B, max_context_len, code, partition_size, kernel, device,
               sliding_window=0, kv_format="same", k_scale=1.0, v_scale=1.0, stream=None):
    need = workspace_bytes(S, Hq, Hkv, D, B, max_context_len, code, partition_size, kernel, sliding_window,
                           kv_format, k_scale, v_scale)
    if need and workspace is None:
        workspace = _temp_workspace(need, device, stream)
    return workspace


def _ws_args(workspace):
    if workspace is None:
        return None, 0
    return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


def paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                           num_kv_heads, max_context_len, partition_size=0, kernel="auto",
                           workspace=None, stream=None, main_events=None, sliding_window=0, kv_format="same",
                           k_scale=1.0, v_scale=1.0, reuse_plan=False, cache_policy="stream"):
    """out[s, j] = softmax(scale * q[s, j] K_s^T) V_s through the block tables.

    q, out: [S, Hq, D]; k_cache, v_cache: [N, Hkv, B, D]; block_tables int32
    [S, M]; context_lens int32 [S] (device); max_context_len: host int >=
    every context length.  `workspace`: optional uint8 device tensor of at
    least workspace_bytes(...) bytes.  reuse_plan: the workspace holds the
    work list of an earlier call with the same batch (see pkv.h).
    cache_policy: "stream" (nontemporal loads) or "keep" (plain loads, for
    batches whose sequences share blocks)."""
    if reuse_plan and workspace is None:
        raise ValueError("reuse_plan needs the workspace of the call that built the work list")
    torch = _torch()
    S, Hq, D = q.shape
    N, Hkv, B, D2 = k_cache.shape
    _check_attention_shapes(out, q, k_cache, v_cache, block_tables, context_lens, block_size, num_kv_heads,
                            kv_format)
    code = dtype_code(q)
    workspace = _workspace(workspace, S, Hq, Hkv, D, B, max_context_len, code, partition_size, kernel, q.device,
                           sliding_window, kv_format, k_scale, v_scale, stream)
    opts = _options(partition_size, kernel, main_events, sliding_window, kv_format, k_scale, v_scale, reuse_plan,
                    cache_policy)
    st = lib.pkv_paged_attention_decode(
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32),
        float(scale), B, Hkv, S, Hq, D, block_tables.shape[1], int(max_context_len), N, code,
        *_ws_args(workspace), ctypes.byref(opts), _stream(stream))
    check(st, "paged_attention_decode")
    return out


def paged_attention_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                                   num_kv_heads, max_context_len, partition_size=0, kernel="auto", stream=None,
                                   main_events=None, sliding_window=0, kv_format="same", k_scale=1.0, v_scale=1.0,
                                   reuse_plan=False, cache_policy="stream"):
    """paged_attention_decode with no workspace: the work list and split-K
    partials live in the library's fixed device scratch (NOALLOC_SCRATCH_BYTES
    per GPU, shared by every call on that GPU: calls that overlap in time
    race).  Nothing is allocated.  Raises PkvError (status -11) when the call
    needs more than the scratch holds."""
    torch = _torch()
    S, Hq, D = q.shape
    N, Hkv, B, D2 = k_cache.shape
    _check_attention_shapes(out, q, k_cache, v_cache, block_tables, context_lens, block_size, num_kv_heads,
                            kv_format)
    opts = _options(partition_size, kernel, main_events, sliding_window, kv_format, k_scale, v_scale, reuse_plan,
                    cache_policy)
    st = lib.pkv_paged_attention_decode_noalloc(
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32),
        float(scale), B, Hkv, S, Hq, D, block_tables.shape[1], int(max_context_len), N, dtype_code(q),
        ctypes.byref(opts), _stream(stream))
    check(st, "paged_attention_decode_noalloc")
    return out


def shared_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len,
                                  num_groups, group_size, max_prefix_len, dtype_code_, partition_size=0,
                                  kernel="auto", kv_format="same", k_scale=1.0, v_scale=1.0, cache_policy="stream"):
    opts = _options(partition_size, kernel, None, 0, kv_format, k_scale, v_scale, False, cache_policy)
    return int(lib.pkv_paged_attention_shared_prefix_workspace_bytes(
        num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len, num_groups, group_size,
        max_prefix_len, dtype_code_, ctypes.byref(opts)))


def paged_attention_decode_shared_prefix(out, q, k_cache, v_cache, block_tables, context_lens, prefix_lens,
                                         group_members, max_prefix_len, scale, block_size, num_kv_heads,
                                         max_context_len, partition_size=0, kernel="auto", workspace=None,
                                         stream=None, main_events=None, kv_format="same", k_scale=1.0,
                                         v_scale=1.0, reuse_plan=False, cache_policy="stream"):
    """paged_attention_decode for groups of sequences whose first
    prefix_lens[s] tokens are the same blocks (parallel samples of a prompt,
    beams): each group's shared prefix is read once for all its members.

    group_members: int32 [num_groups, group_size] sequence indices (-1 =
    unused slot); prefix_lens: int32 [S], equal within a group, 0 outside any
    group, <= the sequence's length; max_prefix_len: host int >= every
    prefix_lens[s].  Other arguments as paged_attention_decode."""
    if reuse_plan and workspace is None:
        raise ValueError("reuse_plan needs the workspace of the call that built the work lists")
    torch = _torch()
    S, Hq, D = q.shape
    N, Hkv, B, D2 = k_cache.shape
    _check_attention_shapes(out, q, k_cache, v_cache, block_tables, context_lens, block_size, num_kv_heads,
                            kv_format)
    if group_members.dim() != 2:
        raise ValueError("group_members must be [num_groups, group_size]")
    if prefix_lens.shape != (S,):
        raise ValueError("prefix_lens must be [num_seqs]")
    Gn, Gs = group_members.shape
    code = dtype_code(q)
    if workspace is None:
        need = shared_prefix_workspace_bytes(S, Hq, Hkv, D, B, max_context_len, Gn, Gs, max_prefix_len, code,
                                             partition_size, kernel, kv_format, k_scale, v_scale, cache_policy)
        if need:
            workspace = _temp_workspace(need, q.device, stream)
    opts = _options(partition_size, kernel, main_events, 0, kv_format, k_scale, v_scale, reuse_plan, cache_policy)
    st = lib.pkv_paged_attention_decode_shared_prefix(
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32),
        _dev(prefix_lens, "prefix_lens", torch.int32), _dev(group_members, "group_members", torch.int32),
        Gn, Gs, int(max_prefix_len), float(scale), B, Hkv, S, Hq, D, block_tables.shape[1],
        int(max_context_len), N, code, *_ws_args(workspace), ctypes.byref(opts), _stream(stream))
    check(st, "paged_attention_decode_shared_prefix")
    return out


def decode_step(out, q, k_new, v_new, k_cache, v_cache, slot_mapping, block_tables, context_lens, scale,
                block_size, num_kv_heads, max_context_len, partition_size=0, kernel="auto", workspace=None,
                stream=None, main_events=None, sliding_window=0, kv_format="same", k_scale=1.0, v_scale=1.0,
                reuse_plan=False, cache_policy="stream"):
    """reshape_and_cache(k_new, v_new, ..., slot_mapping) followed by
    paged_attention_decode(...), with the token store and the attention work
    list in one launch.  k_new, v_new: [S, Hkv, D]; slot_mapping int32 [S]."""
    if reuse_plan and workspace is None:
        raise ValueError("reuse_plan needs the workspace of the call that built the work list")
    torch = _torch()
    S, Hq, D = q.shape
    N, Hkv, B, D2 = k_cache.shape
    _check_attention_shapes(out, q, k_cache, v_cache, block_tables, context_lens, block_size, num_kv_heads,
                            kv_format)
    if tuple(k_new.shape) != (S, Hkv, D) or tuple(v_new.shape) != (S, Hkv, D):
        raise ValueError("k_new and v_new must be [num_seqs, num_kv_heads, head_dim]")
    if k_new.dtype != q.dtype or v_new.dtype != q.dtype:
        raise TypeError("dtype mismatch")
    if slot_mapping.shape != (S,):
        raise ValueError("slot_mapping must be [num_seqs]")
    code = dtype_code(q)
    workspace = _workspace(workspace, S, Hq, Hkv, D, B, max_context_len, code, partition_size, kernel, q.device,
                           sliding_window, kv_format, k_scale, v_scale, stream)
    opts = _options(partition_size, kernel, main_events, sliding_window, kv_format, k_scale, v_scale, reuse_plan,
                    cache_policy)
    st = lib.pkv_decode_step(
        _dev(out, "out"), _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(slot_mapping, "slot_mapping", torch.int32),
        _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32),
        float(scale), B, Hkv, S, Hq, D, block_tables.shape[1], int(max_context_len), N, code,
        *_ws_args(workspace), ctypes.byref(opts), _stream(stream))
    check(st, "decode_step")
    return out


def reshape_and_cache_fp8(k, v, k_cache, v_cache, slot_mapping, k_scale, v_scale, stream=None):
    """k_cache[slot // B, :, slot % B] = E4M3 code of k[i] / k_scale (and v), for every slot >= 0.
    k, v: f32/f16/bf16 [T, Hkv, D]; caches uint8 [N, Hkv, B, D]."""
    torch = _torch()
    T, Hkv, D = k.shape
    N, Hkv2, B, D2 = k_cache.shape
    if tuple(v.shape) != (T, Hkv, D) or (Hkv2, D2) != (Hkv, D) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("shape mismatch between new tokens and caches")
    if dtype_code(k_cache) != 3 or dtype_code(v_cache) != 3 or k.dtype != v.dtype:
        raise TypeError("caches must hold E4M3 codes and k, v share a dtype")
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [num_tokens]")
    st = lib.pkv_reshape_and_cache_fp8(_dev(k, "k"), _dev(v, "v"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                       _dev(slot_mapping, "slot_mapping", torch.int32), T, Hkv, D, B, N,
                                       dtype_code(k), float(k_scale), float(v_scale), _stream(stream))
    check(st, "reshape_and_cache_fp8")


def reshape_and_cache(k, v, k_cache, v_cache, slot_mapping, stream=None):
    """k_cache[slot // B, :, slot % B] = k[i] (and v) for every slot >= 0."""
    torch = _torch()
    T, Hkv, D = k.shape
    N, Hkv2, B, D2 = k_cache.shape
    if tuple(v.shape) != (T, Hkv, D) or (Hkv2, D2) != (Hkv, D) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("shape mismatch between new tokens and caches")
    if not (k.dtype == v.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("dtype mismatch")
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [num_tokens]")
    st = lib.pkv_reshape_and_cache(_dev(k, "k"), _dev(v, "v"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                   _dev(slot_mapping, "slot_mapping", torch.int32), T, Hkv, D, B, N,
                                   dtype_code(k), _stream(stream))
    check(st, "reshape_and_cache")


def copy_blocks(k_cache, v_cache, src_dst_pairs, stream=None):
    """Block dst of both caches becomes a copy of block src, for each pair."""
    torch = _torch()
    N, Hkv, B, D = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape) or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache must match")
    if src_dst_pairs.dim() != 2 or src_dst_pairs.shape[1] != 2:
        raise ValueError("src_dst_pairs must be [num_pairs, 2]")
    n = src_dst_pairs.shape[0]
    st = lib.pkv_copy_blocks(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                             _dev(src_dst_pairs, "src_dst_pairs", torch.int32) if n else None,
                             n, Hkv, B, D, N, dtype_code(k_cache), _stream(stream))
    check(st, "copy_blocks")


def swap_blocks(dst_k, dst_v, src_k, src_v, src_dst_pairs, stream=None):
    """Block dst of (dst_k, dst_v) becomes a copy of block src of (src_k,
    src_v) for each pair.  Pools [N, Hkv, B, D] on the GPU or in pinned host
    memory (pin_memory=True); pairs: int32 GPU tensor [P, 2]."""
    torch = _torch()
    Ns, Hkv, B, D = src_k.shape
    Nd = dst_k.shape[0]
    if tuple(dst_k.shape[1:]) != (Hkv, B, D) or dst_v.shape != dst_k.shape or src_v.shape != src_k.shape:
        raise ValueError("pools must share [Hkv, B, D]")
    if not (src_k.dtype == src_v.dtype == dst_k.dtype == dst_v.dtype):
        raise TypeError("pools must share a dtype")
    for t, name in ((dst_k, "dst_k"), (dst_v, "dst_v"), (src_k, "src_k"), (src_v, "src_v")):
        if not t.is_contiguous() or not (t.is_cuda or t.is_pinned()):
            raise ValueError(f"{name} must be a contiguous GPU or pinned host tensor")
    n = src_dst_pairs.shape[0]
    st = lib.pkv_swap_blocks(ctypes.c_void_p(dst_k.data_ptr()), ctypes.c_void_p(dst_v.data_ptr()),
                             ctypes.c_void_p(src_k.data_ptr()), ctypes.c_void_p(src_v.data_ptr()),
                             _dev(src_dst_pairs, "src_dst_pairs", torch.int32) if n else None, n, Ns, Nd,
                             Hkv, B, D, dtype_code(src_k), _stream(stream))
    check(st, "swap_blocks")


def gather_kv(cache, block_tables, context_lens, kv_head, max_context_len, out=None, stream=None):
    """Contiguous [S, max_context_len, D] copy of one KV head through the tables
    (rows past a sequence's length keep out's previous contents; zeros if out is None)."""
    torch = _torch()
    N, Hkv, B, D = cache.shape
    S, M = block_tables.shape
    if out is None:
        out = torch.zeros((S, max_context_len, D), dtype=cache.dtype, device=cache.device)
    st = lib.pkv_gather_kv(_dev(out, "out"), _dev(cache, "cache"), _dev(block_tables, "block_tables", torch.int32),
                           _dev(context_lens, "context_lens", torch.int32), S, M, int(max_context_len),
                           int(kv_head), Hkv, D, B, N, dtype_code(cache), _stream(stream))
    check(st, "gather_kv")
    return out


def _i32(a):
    arr = np.ascontiguousarray(a, dtype=np.int32)
    return arr, arr.ctypes.data_as(c_i32p)


class BlockManager:
    """Host block manager of libpkv (free list, refcounts, tables, CoW)."""

    def __init__(self, num_blocks: int, block_size: int, max_seqs: int, free_order=None):
        self.block_size = block_size
        self.num_blocks = num_blocks
        keep = None
        ptr = None
        if free_order is not None:
            keep, ptr = _i32(free_order)
            if keep.shape != (num_blocks,):
                raise ValueError("free_order must list every block once")
        self._h = lib.pkv_bm_create(num_blocks, block_size, max_seqs, ptr)
        if not self._h:
            raise ValueError("pkv_bm_create rejected its arguments")

    def close(self):
        if getattr(self, "_h", None):
            lib.pkv_bm_destroy(self._h)
            self._h = None

    __del__ = close

    def add_seq(self, seq):
        check(lib.pkv_bm_add_seq(self._h, seq), "bm_add_seq")

    def fork(self, parent, child):
        check(lib.pkv_bm_fork(self._h, parent, child), "bm_fork")

    def fork_batch(self, parents, children):
        pa, pp = _i32(parents)
        ca, cp = _i32(children)
        if pa.shape != ca.shape:
            raise ValueError("parents and children must have the same length")
        done = ctypes.c_int32()
        st = lib.pkv_bm_fork_batch(self._h, pp, cp, len(pa), ctypes.byref(done))
        if st != 0:
            err = PkvError(st, "bm_fork_batch")
            err.num_done = done.value
            raise err

    def free_batch(self, seqs):
        sa, sp = _i32(seqs)
        done = ctypes.c_int32()
        st = lib.pkv_bm_free_batch(self._h, sp, len(sa), ctypes.byref(done))
        if st != 0:
            err = PkvError(st, "bm_free_batch")
            err.num_done = done.value
            raise err

    def append(self, seq):
        slot, src, dst = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        check(lib.pkv_bm_append(self._h, seq, ctypes.byref(slot), ctypes.byref(src), ctypes.byref(dst)),
              "bm_append")
        return slot.value, (None if src.value < 0 else (src.value, dst.value))

    def append_batch(self, seqs):
        seqs_a, seqs_p = _i32(seqs)
        n = len(seqs_a)
        slots, slots_p = _i32(np.zeros(n))
        pairs, pairs_p = _i32(np.zeros(2 * max(1, n)))
        npairs, done = ctypes.c_int32(), ctypes.c_int32()
        st = lib.pkv_bm_append_batch(self._h, seqs_p, n, slots_p, pairs_p, n, ctypes.byref(npairs),
                                     ctypes.byref(done))
        if st != 0:
            err = PkvError(st, "bm_append_batch")
            err.num_done = done.value
            raise err
        return slots, pairs[: 2 * npairs.value].reshape(-1, 2).copy()

    def free_seq(self, seq):
        check(lib.pkv_bm_free_seq(self._h, seq), "bm_free_seq")

    def move_seq(self, other: "BlockManager", seq):
        """Move `seq` to `other` (swap out / in); returns the (block here,
        block there) pairs to copy with swap_blocks, int32 [P, 2]."""
        cap = max(1, -(-self.seq_len(seq) // self.block_size))
        buf, ptr = _i32(np.zeros(2 * cap))
        n = ctypes.c_int32()
        check(lib.pkv_bm_move_seq(self._h, other._h, seq, ptr, cap, ctypes.byref(n)), "bm_move_seq")
        return buf[: 2 * n.value].reshape(-1, 2).copy()

    def slide_window(self, seq, window):
        n = lib.pkv_bm_slide_window(self._h, seq, window)
        if n < 0:
            raise PkvError(n, "bm_slide_window")
        return n

    def seq_len(self, seq):
        n = lib.pkv_bm_seq_len(self._h, seq)
        if n < 0:
            raise PkvError(n, "bm_seq_len")
        return n

    def block_table(self, seq):
        cap = max(1, -(-self.seq_len(seq) // self.block_size))
        buf, ptr = _i32(np.zeros(cap))
        n = lib.pkv_bm_block_table(self._h, seq, ptr, cap)
        if n < 0:
            raise PkvError(n, "bm_block_table")
        return buf[:n].tolist()

    def export(self, seqs, max_blocks):
        seqs_a, seqs_p = _i32(seqs)
        n = len(seqs_a)
        tables, tp = _i32(np.zeros((n, max_blocks)))
        lens, lp = _i32(np.zeros(n))
        check(lib.pkv_bm_export(self._h, seqs_p, n, tp, max_blocks, lp), "bm_export")
        return tables, lens

    def refcount(self, block):
        n = lib.pkv_bm_refcount(self._h, block)
        if n < 0:
            raise PkvError(n, "bm_refcount")
        return n

    def num_free(self):
        return lib.pkv_bm_num_free(self._h)

    def free_list(self):
        buf, ptr = _i32(np.zeros(max(1, self.num_blocks)))
        n = lib.pkv_bm_free_list(self._h, ptr, max(1, self.num_blocks))
        return buf[:n].tolist()
