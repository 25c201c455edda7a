"""Build libsnapkv.so (the C-ABI library and its gfx950 kernels) in-tree.

    python -m long_context_kv_snapkv_amd.build [--verbose]

Compiles every source under csrc/ with hipcc for gfx950 and links the shared
library to long_context_kv_snapkv_amd/_lib/libsnapkv.so. Objects go to
_build/ at the repository root.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(HERE, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "libsnapkv.so")
OBJ_DIR = os.path.join(ROOT, "_build", "obj")
ARCH = "gfx950"

# Packed fp32 VALU forms are kept out of the generated code on purpose.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build libsnapkv)")
    return path


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; harmless
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    return obj


SAN_DIR = os.path.join(ROOT, "_build", "sanitize")
SAN_LIB = os.path.join(SAN_DIR, "libsnapkv_san.so")
# AddressSanitizer and UndefinedBehaviorSanitizer on the host code only (each
# -fsanitize= right after -Xarch_host; the device code is built as usual)
SAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host",
                  "-fno-sanitize-recover=undefined"]


def asan_runtime() -> str:
    """The AddressSanitizer runtime of ROCm's clang (to preload into a
    process that loads the sanitized library)."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang's AddressSanitizer runtime was not found under /opt/rocm/llvm")
    return hits[-1]


def build_sanitized(verbose: bool = False) -> str:
    """libsnapkv_san.so under _build/sanitize: the host source (argument
    validation, planning, launches) compiled with ASan and UBSan, linked with
    the kernels' objects. Returns its path. For host-side tests only: the
    process must preload asan_runtime()."""
    os.makedirs(SAN_DIR, exist_ok=True)
    objs = []
    for src in sources():
        if src.endswith(".cpp"):
            obj = os.path.join(SAN_DIR, os.path.basename(src) + ".o")
            cmd = [hipcc(), *HIPCC_FLAGS, *SAN_HOST_FLAGS, "-c", src, "-o", obj]
        else:
            obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
            if os.path.exists(obj):
                objs.append(obj)
                continue
            os.makedirs(OBJ_DIR, exist_ok=True)
            cmd = [hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n" + res.stdout + res.stderr)
        objs.append(obj)
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host",
           "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", *objs,
           "-o", SAN_LIB]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("sanitized link failed:\n" + res.stdout + res.stderr)
    return SAN_LIB


def build(verbose: bool = False) -> str:
    """Compile and link; returns the library path. Always recompiles."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
