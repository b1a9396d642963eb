"""Builds libhmoe.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m weight_only_quantized_moe_amd.build [-v]

Every source is compiled with hipcc for gfx950 only; packed FP32 instructions
are disabled for the device code (-packed-fp32-ops).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libhmoe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["host.cpp", "route.hip", "align.hip", "decode.hip", "prefill.hip", "dequant.hip",
           "repack.hip", "noalloc.hip", "w4a4.hip"]
# the streaming kernels must keep every value in registers: private-memory (scratch)
# traffic shares the vector memory counter with the prefetched loads and drains them
NO_SCRATCH = {"decode.hip", "prefill.hip", "w4a4.hip"}

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function",
]


def _compile(src: str, obj_dir: str, verbose: bool) -> str:
    obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    check = ["-Rpass-analysis=kernel-resource-usage"] if src in NO_SCRATCH else []
    cmd = [HIPCC, *COMMON, *lang, *check, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    lines = (r.stdout + r.stderr).splitlines()
    msgs = "\n".join(l for l in lines
                     if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if check:
        kernel, spills = None, []
        for l in lines:
            if "Function Name:" in l:
                kernel = l.split("Function Name:")[1].split("[")[0].strip()
            elif "ScratchSize [bytes/lane]:" in l:
                n = int(l.split("ScratchSize [bytes/lane]:")[1].split("[")[0])
                if n:
                    spills.append(f"{kernel}: {n} bytes/lane")
        if spills:
            raise RuntimeError(f"{src}: kernels use private memory:\n" + "\n".join(spills))
    if verbose and msgs.strip():
        print(msgs)
    return obj


def build(verbose: bool = False) -> str:
    obj_dir = os.path.join(PKG, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    jobs = int(os.environ.get("MAX_JOBS", "8"))
    with ThreadPoolExecutor(max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
