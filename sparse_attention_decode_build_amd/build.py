"""Build libsad.so (HIP, gfx950) in-tree with hipcc."""

from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsad.so")
SOURCES = ("abi.hip", "build_indices.hip", "indexer.hip", "indexer_q.hip", "gather.hip", "attention.hip",
           "attention_dsplit.hip", "out_quant.hip", "cache_write.hip")
ARCH = "gfx950"

# hipcc flags: gfx950 only; packed-FP32 VALU ops disabled (hipcc's host pass warns
# that it does not know the feature, which is harmless).
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]
# Per-file extra flags.  The indexer's MFMA results feed VALU work right away, so its
# MFMAs write VGPRs.  The dim-split attention kernel runs two waves per SIMD (256
# registers each): its PV waves' 144 accumulators and its QK waves' Q^T fragments only
# fit one register split between the two roles when every MFMA operand is a VGPR (the
# other attention kernel keeps its accumulators in AGPRs).
EXTRA_FLAGS = {"indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
               "attention_dsplit.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libsad.so")
    return exe


# Host-code sanitizers (the device code is built as usual): AddressSanitizer and
# UndefinedBehaviorSanitizer on the ABI's argument checks, workspace sizing and launch
# set-up.  The library needs the clang ASan runtime loaded first (LD_PRELOAD of
# libclang_rt.asan-x86_64.so, ASAN_OPTIONS=detect_leaks=0 under Python).
HOST_SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                       "-Xarch_host", "-fno-omit-frame-pointer"]
HOST_SANITIZED_LIB = os.path.join(PKG, "libsad_hostsan.so")


def build(verbose: bool = False, host_sanitize: bool = False) -> str:
    """Compile every source for gfx950 and link libsad.so (or, with host_sanitize, the
    host-sanitized libsad_hostsan.so); returns its path."""
    hipcc = _hipcc()
    obj_dir = os.path.join(ROOT, "_build_hostsan" if host_sanitize else "_build")
    os.makedirs(obj_dir, exist_ok=True)
    san = HOST_SANITIZE_FLAGS if host_sanitize else []
    lib = HOST_SANITIZED_LIB if host_sanitize else LIB

    def compile_one(src: str) -> str:
        obj = os.path.join(obj_dir, src.replace(".hip", ".o"))
        cmd = [hipcc, *FLAGS, *san, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
        if verbose and res.stderr.strip():
            print(res.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = lib + ".tmp"
    link_san = [*HOST_SANITIZE_FLAGS, "-shared-libasan"] if host_sanitize else []
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_san, *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(lib)} failed:\n{res.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    import sys

    print(build(verbose=True, host_sanitize="--host-sanitize" in sys.argv[1:]))
