"""Build the HIP library (gfx950) in-tree: rank_sgmv_bgmv_amd/_build/liblora_hip.so.

    python -m rank_sgmv_bgmv_amd.build [--verbose] [--asan]

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled.  The result is a plain C-ABI shared library (include/lora.h).

--asan builds _build/liblora_hip_asan.so instead: the host code (argument
checks, workspace layout, launch configuration) instrumented with
AddressSanitizer, the device code as usual.  It is for CPU-side tests of the
C ABI's validation path: load it into a process started with the sanitizer
runtime preloaded (asan_runtime() gives its path).
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "liblora_hip.so")
SOURCES = ["lora_api.hip", "lora_plan.hip", "lora_valu.hip", "lora_mfma.hip", "lora_merge.hip", "lora_calib.hip"]
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.exists(c) or c == "hipcc":
            return c
    raise RuntimeError("hipcc not found")


ASAN_LIB = os.path.join(OUT_DIR, "liblora_hip_asan.so")
# host-only sanitizer flags: every -fsanitize applies to the host pass alone
ASAN_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """Path of the AddressSanitizer runtime of the compiler hipcc drives."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    res = subprocess.run([clang, "--print-resource-dir"], capture_output=True, text=True, check=True).stdout.strip()
    return os.path.join(res, "lib", "linux", "libclang_rt.asan-x86_64.so")


def build(verbose: bool = False, extra=(), asan: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    lib_path = ASAN_LIB if asan else LIB
    if asan:
        extra = [*extra, *ASAN_FLAGS]
    objs = []
    with tempfile.TemporaryDirectory(dir=OUT_DIR) as tmp:
        procs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        failed = []
        for src, p in procs:
            log, _ = p.communicate()
            if log and (verbose or p.returncode):
                print(log, file=sys.stderr)
            if p.returncode:
                failed.append(src)
        if failed:
            raise RuntimeError(f"hipcc failed for {failed}")
        tmp_lib = lib_path + f".tmp{os.getpid()}"
        link_extra = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-shared-libsan"] if asan else []
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp_lib]
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv, asan="--asan" in sys.argv))
