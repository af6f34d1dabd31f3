"""Build libattn_mi355x.so in-tree for gfx950 with hipcc.

    python -m attention_forward_online_attn_amd.build

Compiles every time it is called: each csrc/*.hip translation unit (the host
code and one file per kernel family) to an object, in parallel, then one link.
Flags: -O3, gfx950 only, packed fp32 vector instructions disabled
(-packed-fp32-ops), hidden visibility with the C ABI of include/attn.h
exported.
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CSRC = os.path.join(PKG, "csrc")
# host code (attn_abi.hip) and one translation unit per kernel family (inst_*.hip)
SOURCES = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
OUTPUT = os.path.join(PKG, "libattn_mi355x.so")

COMPILE_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# one-step build of a single source (used by tools that compile one file)
FLAGS = [*COMPILE_FLAGS, "-shared"]
# Per-file additions.  The backward units hold the one-wave dK/dV kernel
# (D = 128), whose accumulators, K and V fragments fill both halves of the
# register file: by default the compiler puts every MFMA result of such a
# kernel in AGPRs, and the scores and dP that the vector ALU reads next are
# then copied to VGPRs element by element (64 to 192 moves per step).  The
# VGPR form keeps MFMA results in VGPRs, while the K and V fragments are
# pinned to AGPRs in the kernel itself (MFMA B operands may be AGPRs).
FILE_FLAGS = {
    "inst_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "inst_bwd_bias.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def compile_flags(src: str) -> list[str]:
    """hipcc flags for one translation unit."""
    return [*COMPILE_FLAGS, *FILE_FLAGS.get(os.path.basename(src), [])]


def _noise(stderr: str):
    # hipcc's host pass does not know the packed-fp32 feature; drop that warning only
    return [ln for ln in stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()
            and not ln.startswith("1 warning generated") and not ln.endswith("warnings generated.")]


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every csrc/*.hip to an object in parallel, then link the
    shared library (replaced atomically)."""
    jobs = jobs or max(1, min(len(SOURCES), os.cpu_count() or 1))
    with tempfile.TemporaryDirectory(prefix="attn_build_") as tmpdir:
        def compile_one(src):
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cmd = [HIPCC, *compile_flags(src), "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            return obj, subprocess.run(cmd, capture_output=True, text=True)

        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(compile_one, SOURCES))
        for (obj, res), src in zip(results, SOURCES):
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n" + res.stderr)
            if verbose and _noise(res.stderr):
                print("\n".join(_noise(res.stderr)), file=sys.stderr)
        tmp = OUTPUT + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-fvisibility=hidden",
               *[obj for obj, _ in results], "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + res.stderr)
    os.replace(tmp, OUTPUT)
    return OUTPUT


if __name__ == "__main__":
    print(build(verbose=True))
