"""Build libdflash.so (the HIP library behind include/dflash.h) for gfx950, in-tree.

    python -m block_diffusion_drafter_tap_amd.build

Each .hip source is compiled in parallel with hipcc, then linked into a shared
library next to this file. Packed-fp32 VALU instructions are disabled for the
device code (the flag is a device-only target feature; the host pass warns that
it does not know it, which is harmless).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libdflash.so")
SOURCES = ["api.hip", "gemm.hip", "gateup.hip", "finish.hip", "lmhead.hip", "attention.hip", "small.hip",
           "prefill.hip", "tree.hip", "sampling.hip", "blaslt.hip"]
ARCH = os.environ.get("DFLASH_OFFLOAD_ARCH", "gfx950")

DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# hipBLASLt (the staging stage's plain fc product), found at run time next to the HIP runtime
ROCM_LIB = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
LINK_FLAGS = ["-lhipblaslt", "-Wl,-rpath," + ROCM_LIB]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-c",
           *DEVICE_FLAGS, "-I", INCLUDE, os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, *LINK_FLAGS, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The compiler's shared AddressSanitizer runtime (preloaded into the host
    process that loads a sanitized library)."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the AddressSanitizer runtime of hipcc's clang was not found")
    return path


def build_host_sanitized(verbose: bool = False) -> str:
    """A copy of the library whose host code (api.hip: argument validation,
    config guards, state / workspace layouts, the block policy) is built with
    AddressSanitizer and UndefinedBehaviorSanitizer; device code is unchanged.
    For CPU-only checks of the host paths; it lands in _build/, never next to
    the package."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    headers = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")] + \
        [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h")]
    newest_header = max(os.path.getmtime(h) for h in headers)

    def stale(src: str) -> bool:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        return not os.path.exists(obj) or os.path.getmtime(obj) < max(newest_header,
                                                                      os.path.getmtime(os.path.join(CSRC, src)))
    todo = [s for s in SOURCES if s != "api.hip" and stale(s)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, len(todo))) as ex:
        list(ex.map(lambda s: _compile(s, verbose), todo))
    out_dir = os.path.join(BUILD_DIR, "host_sanitized")
    os.makedirs(out_dir, exist_ok=True)
    obj = os.path.join(out_dir, "api.o")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-c", *DEVICE_FLAGS, *HOST_SANITIZE,
           "-I", INCLUDE, os.path.join(CSRC, "api.hip"), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on the sanitized api.hip:\n{r.stderr}")
    objs = [obj] + [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "api.hip"]
    lib = os.path.join(out_dir, "libdflash.so")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-shared-libsan", *HOST_SANITIZE,
           *objs, *LINK_FLAGS, "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of the sanitized library failed:\n{r.stderr}")
    return lib


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        print(build_host_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
