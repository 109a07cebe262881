"""Build libssmscan.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Flags: -O3, --offload-arch=gfx950, -ffp-contract=off (only explicit fmaf
fuses, which fixes the association/rounding of every kernel), packed-FP32
VALU instructions disabled, IEEE float32 denormals (hipcc's default).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libssmscan.so")
SOURCES = ["ssm_fwd.hip", "ssm_bwd.hip", "ssm_step.hip", "ssm_proj.hip", "affine_scan.hip", "noalloc.hip",
           "ssm_lpar.hip",
           "capi.cpp"]
FLAGS = ["-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-command-line-argument"]


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source to an object in parallel, then link the .so."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc, *FLAGS, *inc, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        text = "\n".join(l for l in text.splitlines() if "is not a recognized feature for this target" not in l)
        if p.returncode != 0:
            failed.append((src, text))
        elif verbose and text.strip():
            print(text)
    if failed:
        for src, text in failed:
            print(f"--- {src}\n{text}", file=sys.stderr)
        raise RuntimeError("hipcc failed for " + ", ".join(s for s, _ in failed))
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
