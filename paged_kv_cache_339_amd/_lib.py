"""Loading of libpkv.so and ctypes prototypes of its C ABI (include/pkv.h)."""
from __future__ import annotations

import ctypes
import os

# PKV_LIBRARY names another build of the same library (the host-sanitizer
# build the CPU tests load); by default the in-tree libpkv.so.
LIB_PATH = os.environ.get("PKV_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

PKV_F32, PKV_F16, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2, 3
KV_FORMATS = {"same": 0, "fp8_e4m3": 1}
KERNELS = {"auto": 0, "valu": 1, "mfma": 2}
CACHE_POLICIES = {"stream": 0, "keep": 1}
# Bytes of the fixed device scratch pkv_paged_attention_decode_noalloc uses
# (PKV_NOALLOC_SCRATCH_BYTES in pkv.h).
NOALLOC_SCRATCH_BYTES = 64 << 20

c_i32, c_f32, c_size, c_vp = ctypes.c_int32, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
c_i32p = ctypes.POINTER(ctypes.c_int32)


class AttnOptions(ctypes.Structure):
    _fields_ = [("partition_size", c_i32), ("kernel", c_i32),
                ("main_begin_event", c_vp), ("main_end_event", c_vp), ("sliding_window", c_i32),
                ("kv_format", c_i32), ("k_scale", c_f32), ("v_scale", c_f32), ("reuse_plan", c_i32),
                ("cache_policy", c_i32)]


class PkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = lib.pkv_last_error().decode() if status == -7 else ""
        super().__init__(f"{where}: {lib.pkv_status_str(status).decode()} (status {status})"
                         + (f": {detail}" if detail else ""))


def load(path: str = LIB_PATH):
    """ctypes handle of a libpkv build with every prototype set."""
    # torch ships its own HIP runtime (same soname as ROCm's).  Load it first
    # so libpkv binds to the runtime that owns torch's memory and streams;
    # loading libpkv first would put a second HIP runtime in the process.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python paged_kv_cache_339_amd/build.py` "
            "(hipcc, gfx950). There is no fallback implementation.")
    L = ctypes.CDLL(path)
    sig = {
        "pkv_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "pkv_last_error": (ctypes.c_char_p, []),
        "pkv_paged_attention_workspace_bytes": (c_size, [c_i32] * 6 + [ctypes.c_int, ctypes.POINTER(AttnOptions)]),
        "pkv_paged_attention_plan_info": (ctypes.c_int, [c_i32] * 6 + [ctypes.c_int, ctypes.POINTER(AttnOptions),
                                                                      c_i32p, c_i32p, c_i32p]),
        "pkv_paged_attention_decode": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_f32, c_i32, c_i32,
                                                      c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, ctypes.c_int,
                                                      c_vp, c_size, ctypes.POINTER(AttnOptions), c_vp]),
        "pkv_paged_attention_decode_noalloc": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_f32, c_i32,
                                                              c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                                              ctypes.c_int, ctypes.POINTER(AttnOptions), c_vp]),
        "pkv_paged_attention_shared_prefix_workspace_bytes": (
            c_size, [c_i32] * 9 + [ctypes.c_int, ctypes.POINTER(AttnOptions)]),
        "pkv_paged_attention_decode_shared_prefix": (
            ctypes.c_int, [c_vp] * 8 + [c_i32, c_i32, c_i32, c_f32] + [c_i32] * 8 + [ctypes.c_int, c_vp, c_size,
                                                                             ctypes.POINTER(AttnOptions), c_vp]),
        "pkv_decode_step": (ctypes.c_int, [c_vp] * 9 + [c_f32] + [c_i32] * 8 + [ctypes.c_int, c_vp, c_size,
                                                                              ctypes.POINTER(AttnOptions), c_vp]),
        "pkv_reshape_and_cache": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                                                 c_i32, ctypes.c_int, c_vp]),
        "pkv_reshape_and_cache_fp8": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                                                     c_i32, ctypes.c_int, c_f32, c_f32, c_vp]),
        "pkv_copy_blocks": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, ctypes.c_int,
                                           c_vp]),
        "pkv_swap_blocks": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                           ctypes.c_int, c_vp]),
        "pkv_bm_move_seq": (ctypes.c_int, [c_vp, c_vp, c_i32, c_i32p, c_i32, c_i32p]),
        "pkv_gather_kv": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                         c_i32, c_i32, ctypes.c_int, c_vp]),
        "pkv_bm_create": (c_vp, [c_i32, c_i32, c_i32, c_i32p]),
        "pkv_bm_destroy": (None, [c_vp]),
        "pkv_bm_add_seq": (ctypes.c_int, [c_vp, c_i32]),
        "pkv_bm_fork": (ctypes.c_int, [c_vp, c_i32, c_i32]),
        "pkv_bm_append": (ctypes.c_int, [c_vp, c_i32, c_i32p, c_i32p, c_i32p]),
        "pkv_bm_append_batch": (ctypes.c_int, [c_vp, c_i32p, c_i32, c_i32p, c_i32p, c_i32, c_i32p, c_i32p]),
        "pkv_bm_free_seq": (ctypes.c_int, [c_vp, c_i32]),
        "pkv_bm_fork_batch": (ctypes.c_int, [c_vp, c_i32p, c_i32p, c_i32, c_i32p]),
        "pkv_bm_free_batch": (ctypes.c_int, [c_vp, c_i32p, c_i32, c_i32p]),
        "pkv_bm_slide_window": (ctypes.c_int, [c_vp, c_i32, c_i32]),
        "pkv_bm_seq_len": (ctypes.c_int, [c_vp, c_i32]),
        "pkv_bm_block_table": (ctypes.c_int, [c_vp, c_i32, c_i32p, c_i32]),
        "pkv_bm_export": (ctypes.c_int, [c_vp, c_i32p, c_i32, c_i32p, c_i32, c_i32p]),
        "pkv_bm_refcount": (ctypes.c_int, [c_vp, c_i32]),
        "pkv_bm_num_free": (ctypes.c_int, [c_vp]),
        "pkv_bm_free_list": (ctypes.c_int, [c_vp, c_i32p, c_i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


lib = load()


def check(status: int, where: str) -> None:
    if status != 0:
        raise PkvError(status, where)
