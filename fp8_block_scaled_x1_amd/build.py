"""Build libfp8bs.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run as ``python -m fp8_block_scaled_x1_amd.build``; the library is written
next to this file. Every build compiles from source (no caching).
"""

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfp8bs.so")
SOURCES = ["api.hip", "quant.hip", "gemm.hip", "moe.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # packed FP32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfp8bs)")


def build(verbose=False, jobs=None):
    """Compile every source and link libfp8bs.so; returns the library path."""
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="fp8bs_build_")
    try:
        objs = []
        procs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [cc, *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
        for src, p in procs:
            out, _ = p.communicate()
            text = out.decode(errors="replace")
            if p.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{text}")
            if verbose and text.strip():
                print(text, flush=True)
        out_tmp = LIB + f".tmp{os.getpid()}"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + res.stdout.decode(errors="replace"))
        os.replace(out_tmp, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
