"""Build liblk.so (the gfx950 HIP library behind include/lk.h) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "liblk.so")
SOURCES = ["quantize.hip", "score.hip", "topk.hip", "mla.hip", "probe.hip", "lk_api.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled for all device code.
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


# Per-file flags.  The score kernels see only finite values (a documented input
# contract), so ReLU may compile to a single v_max without IEEE NaN canonicalization;
# their MFMA accumulators stay in VGPRs, which the epilogue reads directly.
FILE_FLAGS = {"score.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
              "probe.hip": ["-fno-honor-nans"],
              "mla.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, out_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    # the host pass does not know the packed-fp32 feature and says so; keep other warnings
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if warn:
        print(warn, file=sys.stderr)
    return obj


def build(out_dir: str = BUILD_DIR, lib_path: str = LIB_PATH, extra=()) -> str:
    os.makedirs(out_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, out_dir, extra), SOURCES))
    tmp = lib_path + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


# Debug build: every kernel fills its shared memory with 0xFF bytes (NaN as float32, f16
# and e4m3fn) before first use, so a read of LDS that no thread wrote shows up in the
# GPU tests that compare this build's outputs with the library's, bit for bit.
POISON_BUILD_DIR = os.path.join(PKG, "_build_lds_poison")
POISON_LIB_PATH = os.path.join(PKG, "liblk_lds_poison.so")


def build_lds_poison() -> str:
    return build(POISON_BUILD_DIR, POISON_LIB_PATH, ["-DLK_POISON_LDS"])


# Host-side AddressSanitizer / UndefinedBehaviorSanitizer build (device code as
# usual): every sanitizer flag applies to the host pass only.  Used by the CPU tests of
# the argument validation; loading it needs clang's ASan runtime preloaded.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_host_sanitized(out_dir: str) -> str:
    """liblk.so with the host code instrumented, built into out_dir; returns its path."""
    os.makedirs(out_dir, exist_ok=True)

    def one(src: str) -> str:
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), *HOST_SANITIZE, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(one, SOURCES))
    out = os.path.join(out_dir, "liblk.so")
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *HOST_SANITIZE, "-shared-libsan",
                        *objs, "-o", out], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return out


if __name__ == "__main__":
    print(build())
