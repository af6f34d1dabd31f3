"""The C ABI's host code under AddressSanitizer (CPU only, no device).

attn_abi.hip (argument validation, overflow and grid-size checks, workspace
sizing, status strings) is rebuilt at -O0 -g with ASan on its host pass, and
tests/test_abi.py runs against that library in a child interpreter with the
ASan runtime preloaded: every validation path it takes must pass with no
sanitizer report.  The build takes about a minute.
"""

import pytest

from attention_forward_online_attn_amd import build_asan


def test_abi_checks_clean_under_asan():
    try:
        build_asan.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = build_asan.build()
    r = build_asan.run_abi_tests(lib)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]
