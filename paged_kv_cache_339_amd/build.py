"""Build libpkv.so for gfx950 in-tree with hipcc.

    python paged_kv_cache_339_amd/build.py [--jobs N]

Each HIP/C++ source is compiled to an object under _build/ (in parallel),
then linked into paged_kv_cache_339_amd/libpkv.so.  Every call compiles
everything again.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpkv.so")
ARCH = "gfx950"

# Packed fp32 arithmetic stays off: the compiler may otherwise fuse pairs of
# fp32 operations into v_pk_* instructions.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                # torch's bundled HIP runtime may predate code object v6
                "-mcode-object-version=5"]
COMMON = ["-O3", "-fPIC", "-std=c++17", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall",
          "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpkv)")


def sources():
    out = []
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".cpp")):
            out.append(os.path.join(CSRC, name))
    return out


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, *extra, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc(), *COMMON, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(line for line in (res.stdout + res.stderr).splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(jobs: int | None = None, verbose: bool = True, out: str = LIB, build_dir: str = BUILD,
          defines=()) -> str:
    """Compile every source and link `out`.  `defines` are extra -D options
    (tuning constants of the kernels)."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    extra = [f"-D{d}" for d in defines]
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), srcs))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-mcode-object-version=5", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


# Host-code sanitizer build (CPU tests only): the C ABI's argument checks and
# split-K planning (api.cpp, noalloc.hip) and the host block manager
# (block_manager.cpp) compiled with AddressSanitizer and
# UndefinedBehaviorSanitizer, linked with the regular objects of the kernel
# sources (whose host code only launches).
# The sanitizer flags apply to host code only (-Xarch_host); no GPU code is
# instrumented.  A process loading the result needs the ASan runtime first
# (LD_PRELOAD=sanitizer_runtime()).
SANITIZED_SOURCES = ("api.cpp", "block_manager.cpp", "noalloc.hip")
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
SANITIZED_LIB = os.path.join(BUILD, "libpkv_sanitized.so")


def sanitizer_runtime() -> str:
    """Path of the clang AddressSanitizer runtime of the ROCm toolchain."""
    out = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True).stdout.strip()
    if out and os.path.isabs(out) and os.path.exists(out):
        return out
    import glob
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("clang AddressSanitizer runtime not found")
    return found[-1]


def build_sanitized(jobs: int | None = None, out: str = SANITIZED_LIB, build_dir: str = BUILD) -> str:
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    plain = [s for s in srcs if os.path.basename(s) not in SANITIZED_SOURCES]
    san = [s for s in srcs if os.path.basename(s) in SANITIZED_SOURCES]
    missing = [s for s in plain if not os.path.exists(os.path.join(build_dir, os.path.basename(s) + ".o"))]
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    san_dir = os.path.join(build_dir, "sanitized")
    os.makedirs(san_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda src: _compile(src, build_dir), missing))
        san_objs = list(ex.map(lambda src: _compile(src, san_dir, SANITIZE_FLAGS), san))
    objs = [os.path.join(build_dir, os.path.basename(s) + ".o") for s in plain] + san_objs
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-mcode-object-version=5", "-shared", "-fPIC",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--sanitize", action="store_true",
                    help="build _build/libpkv_sanitized.so: host code under ASan and UBSan (CPU tests)")
    a = ap.parse_args()
    if a.sanitize:
        print(build_sanitized(a.jobs))
    else:
        build(a.jobs)
