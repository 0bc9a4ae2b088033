"""Build libfp4rl.so (the C-ABI library with the gfx950 kernels) in-tree.

    python -m fp4_quantized_rl_amd.build        # or: from ... import build; build()

Every source under csrc/ is compiled by hipcc for gfx950 only, then linked
into fp4_quantized_rl_amd/libfp4rl.so. Floating point is IEEE: no fast-math,
fp32 denormals kept, correctly rounded fp32 division and sqrt (the quantiser's
scale recipe and the RMSNorm depend on them). Packed-fp32 instructions are
disabled for the device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libfp4rl.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libfp4rl")
    return path


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the same
# sources (the argument validation, workspace layout and launch set-up of the
# C ABI); each -fsanitize= applies to the host pass only, the gfx950 code is
# built as usual. The library leaves the sanitizer runtime unresolved: load it
# into a process that preloads the ASan runtime (sanitizer_runtime()).
SANITIZE_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                  "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer").split()
SANITIZED_DIR = os.path.join(BUILD_DIR, "sanitized")
SANITIZED_LIB = os.path.join(SANITIZED_DIR, "libfp4rl_sanitized.so")


def _compile(src: str, extra=(), out_dir: str = BUILD_DIR) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def _build_into(lib_path: str, out_dir: str, extra=()) -> str:
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as pool:
        objs = list(pool.map(lambda s: _compile(s, extra, out_dir), srcs))
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip for gfx950 and link libfp4rl.so; returns its path."""
    _build_into(LIB_PATH, BUILD_DIR)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


def build_sanitized() -> str:
    """The host-sanitized library (under _build/, not the package); returns its path."""
    return _build_into(SANITIZED_LIB, SANITIZED_DIR, SANITIZE_FLAGS)


def sanitizer_runtime() -> str:
    """Path of the compiler's shared ASan runtime (it also carries the UBSan handlers)."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the ASan runtime of hipcc's clang was not found")
    return path


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
