"""Build the gfx950 attention library in-tree with hipcc.

    python -m attention_forward_attn_amd.build [--verbose]

Produces ``attention_forward_attn_amd/libattn_fwd.so`` (HIP kernels + C ABI) and
``libattn_ceiling.so`` (the benchmark's measured-ceiling diagnostics, not part of
the attention boundary).
Whole-program compilation (no -fgpu-rdc), so the compiler sees every kernel
in one translation unit and nothing spills to scratch because of separate
device linking.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn_fwd.so")
CEILING_LIB = os.path.join(HERE, "libattn_ceiling.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
    f"--offload-arch={ARCH}",
    # never let the backend form packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return [os.path.join(CSRC, "attn_kernels.hip"), os.path.join(CSRC, "attn_bwd.hip"),
            os.path.join(CSRC, "attn_qkv.hip"), os.path.join(CSRC, "api.cpp")]


def build(verbose: bool = False, resource_report: bool = False, defines=(), out: str = LIB) -> str:
    objs = []
    os.makedirs(os.path.join(ROOT, "_build"), exist_ok=True)
    for src in sources():
        tag = str(abs(hash(tuple(defines)))) if defines else ""
        obj = os.path.join(ROOT, "_build", os.path.basename(src) + tag + ".o")
        cmd = [HIPCC] + COMMON + [f"-D{d}" for d in defines] + ["-c", src, "-o", obj]
        if src.endswith(".cpp"):
            cmd = [HIPCC] + COMMON + [f"-D{d}" for d in defines] + ["-x", "hip", "-c", src, "-o", obj]
        if resource_report and src.endswith(".hip"):
            cmd += ["-Rpass-analysis=kernel-resource-usage"]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        text = (r.stdout or "") + (r.stderr or "")
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
        if r.returncode != 0:
            sys.stderr.write("\n".join(lines) + "\n")
            raise RuntimeError(f"hipcc failed on {src}")
        if verbose or resource_report:
            print("\n".join(lines))
        objs.append(obj)
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    if out == LIB:
        build_ceiling(verbose)
    return out


def build_ceiling(verbose: bool = False) -> str:
    """The MFMA-loop and copy diagnostics bench.py measures ceilings with."""
    src = os.path.join(CSRC, "ceiling.hip")
    tmp = CEILING_LIB + ".tmp"
    cmd = [HIPCC] + COMMON + ["-shared", src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    os.replace(tmp, CEILING_LIB)
    return CEILING_LIB


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv, resource_report="--resources" in sys.argv)
    print(LIB)
