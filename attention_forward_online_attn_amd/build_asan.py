"""CPU-only AddressSanitizer build of the C ABI's host code.

    python -m attention_forward_online_attn_amd.build_asan

Builds _build/asan/libattn_mi355x_asan.so: csrc/attn_abi.hip -- argument
validation, size and grid checks, workspace sizing, status strings -- at
-O0 -g with AddressSanitizer on the host pass only (device code is never
sanitized), linked with the kernel translation units built as in build.py.
`run_abi_tests()` then runs tests/test_abi.py, which calls only host paths
(no device is touched), against that library in a child Python with the
clang ASan runtime preloaded; any sanitizer report fails the run.
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

from . import build as _build

OUT_DIR = os.path.join(_build.ROOT, "_build", "asan")
OUTPUT = os.path.join(OUT_DIR, "libattn_mi355x_asan.so")
HOST_SRC = os.path.join(_build.CSRC, "attn_abi.hip")
# the host pass only: each sanitizer flag directly after -Xarch_host
ASAN_HOST = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()


def _flags(src):
    flags = _build.compile_flags(src)
    if src == HOST_SRC:
        flags = [f for f in flags if f != "-O3"] + ["-O0", "-g", *ASAN_HOST]
    return flags


def asan_runtime() -> str:
    """Path of the clang ASan runtime that matches hipcc's host compiler."""
    clang = os.path.join(os.path.dirname(os.path.realpath(_build.HIPCC)), "..", "llvm", "bin", "clang")
    res = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError(f"clang ASan runtime not found ({res.stderr.strip() or path})")
    return path


def build(jobs: int | None = None) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    jobs = jobs or max(1, min(len(_build.SOURCES), os.cpu_count() or 1))
    with tempfile.TemporaryDirectory(prefix="attn_asan_") as tmpdir:
        def compile_one(src):
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cmd = [_build.HIPCC, *_flags(src), "-c", src, "-o", obj]
            return obj, subprocess.run(cmd, capture_output=True, text=True)

        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(compile_one, _build.SOURCES))
        for (obj, res), src in zip(results, _build.SOURCES):
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n" + res.stderr)
        tmp = OUTPUT + ".tmp"
        cmd = [_build.HIPCC, f"--offload-arch={_build.ARCH}", "-shared", "-fPIC", "-fvisibility=hidden",
               *ASAN_HOST, *[obj for obj, _ in results], "-o", tmp]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + res.stderr)
    os.replace(tmp, OUTPUT)
    return OUTPUT


def run_abi_tests(lib: str = OUTPUT) -> subprocess.CompletedProcess:
    """tests/test_abi.py against `lib` under the ASan runtime (leak checks
    off: the interpreter itself is not instrumented)."""
    env = dict(os.environ)
    env["ATTN_LIBRARY"] = lib
    preload = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = asan_runtime() + (":" + preload if preload else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86"
    cmd = [sys.executable, "-m", "pytest", os.path.join(_build.ROOT, "tests", "test_abi.py"),
           "-q", "-m", "not gpu", "-p", "no:cacheprovider"]
    return subprocess.run(cmd, capture_output=True, text=True, env=env, cwd=_build.ROOT)


if __name__ == "__main__":
    print(build())
    r = run_abi_tests()
    print(r.stdout[-2000:], r.stderr[-4000:], sep="\n")
    sys.exit(r.returncode)
