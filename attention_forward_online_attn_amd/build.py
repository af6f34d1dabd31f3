"""Build libattn_mi355x.so in-tree for gfx950 with hipcc.

    python -m attention_forward_online_attn_amd.build

Compiles every time it is called.  Flags: -O3, gfx950 only, packed fp32 vector
instructions disabled (-packed-fp32-ops), hidden visibility with the C ABI of
include/attn.h exported.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = [os.path.join(PKG, "csrc", "attn_abi.hip")]
OUTPUT = os.path.join(PKG, "libattn_mi355x.so")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    tmp = OUTPUT + ".tmp"
    cmd = [HIPCC, *FLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; drop that warning only
    noise = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()
             and not ln.startswith("1 warning generated") and not ln.endswith("warnings generated.")]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stderr)
    if noise and verbose:
        print("\n".join(noise), file=sys.stderr)
    os.replace(tmp, OUTPUT)
    return OUTPUT


if __name__ == "__main__":
    print(build(verbose=True))
