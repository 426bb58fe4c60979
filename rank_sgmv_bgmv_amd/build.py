"""Build the HIP library (gfx950) in-tree: rank_sgmv_bgmv_amd/_build/liblora_hip.so.

    python -m rank_sgmv_bgmv_amd.build [--verbose]

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled.  The result is a plain C-ABI shared library (include/lora.h).
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
SOURCES = ["lora_api.hip", "lora_plan.hip", "lora_valu.hip", "lora_mfma.hip", "lora_merge.hip"]
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


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
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
            out, _ = p.communicate()
            if out and (verbose or p.returncode):
                print(out, file=sys.stderr)
            if p.returncode:
                failed.append(src)
        if failed:
            raise RuntimeError(f"hipcc failed for {failed}")
        tmp_lib = LIB + f".tmp{os.getpid()}"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv)
    print(LIB)
