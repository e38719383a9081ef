"""Build ``libq1.so`` (the C-ABI library) in-tree with hipcc for gfx950.

Usage: ``python -m gemm_decode_q1_amd.build`` or ``build()`` from Python.
"""
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libq1.so")
SOURCES = ([os.path.join(PKG, "csrc", "q1_api.cpp"), os.path.join(PKG, "csrc", "q1_kernels.hip"),
            os.path.join(PKG, "csrc", "q1_mma.hip"), os.path.join(PKG, "csrc", "q1_ffn.hip"),
            os.path.join(PKG, "csrc", "q1_wide.hip"),
            os.path.join(PKG, "csrc", "q1_meta.hip"), os.path.join(PKG, "csrc", "q1_scratch.hip"),
            os.path.join(PKG, "csrc", "q1_gemv.hip")])
# Packed-FP32 instructions are disabled for all device code (see the design
# notes): hipcc otherwise forms v_pk_*_f32 from plain float code.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def build(verbose: bool = False) -> str:
    """Compile every source into ``libq1.so`` (always recompiles)."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    inc = ["-I", os.path.join(ROOT, "include")]
    objs = []
    procs = []
    t0 = time.time()
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    for src in SOURCES:
        while sum(p.poll() is None for p, _ in procs) >= jobs:
            time.sleep(0.2)
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [cc, *HIP_FLAGS, *inc, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True), src))
        objs.append(obj)
    for p, src in procs:
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines() if "not a recognized feature" not in l)
        if p.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{out}")
        if verbose and out.strip():
            print(out)
    tmp = LIB + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
