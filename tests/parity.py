"""Comparison helpers for the GPU parity tests (HIP path vs the fp64 oracle)."""

import numpy as np
import torch

# Max-abs bounds.  bf16 inputs with fp32 accumulation: O 1e-2, LSE 1e-3,
# tO 3e-2 relative to max|tO|; fp32 inputs: 1e-4 for each.
TOL = {
    torch.bfloat16: dict(o=1e-2, lse=1e-3, to=3e-2),
    # fp16 inputs: the tutorial page's fp16 test allows 1e-2 on O; held here
    # to a tighter bound from fp16's 11-bit significand -- O stored in fp16
    # (half an ulp, <= 9.8e-4 for |O| < 4) plus P rounded to fp16 (<= 2^-11
    # max|v|, about 2.2e-3) -> 5e-3; the LSE is fp32 as for bf16; tO 1e-2
    # relative to max|tO|.
    torch.float16: dict(o=5e-3, lse=1e-3, to=1e-2),
    torch.float32: dict(o=1e-4, lse=1e-4, to=1e-4),
}


def host64(t):
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.numpy().astype(np.float64)


def lse_err(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    ninf_ref, ninf_got = np.isneginf(ref), np.isneginf(got)
    if np.any(ninf_ref != ninf_got):
        return np.inf
    fin = ~ninf_ref
    return float(np.max(np.abs(got[fin] - ref[fin]), initial=0.0))


def max_err(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    if got.size == 0:
        return 0.0
    if not np.all(np.isfinite(got)):
        return np.inf
    return float(np.max(np.abs(got - ref)))


def storage_floor(ref, dtype=torch.bfloat16):
    """max |round(x) - x| over the exact result x stored in `dtype`: what
    storing the exact result alone costs."""
    r = torch.from_numpy(np.ascontiguousarray(ref))
    return float((r.float().to(dtype).double() - r).abs().max()) if r.numel() else 0.0


def bf16_floor(ref):
    """max |bf16(x) - x|: what storing the exact result in bf16 alone costs."""
    return storage_floor(ref, torch.bfloat16)


# Margin over the storage floor for a 16-bit O: the kernel's own error beyond
# rounding the exact result (P's 16-bit rounding, fp32 sums).
FLOOR_MARGIN = 2e-3


def assert_close(dtype, o, lse, o_ref, lse_ref, to=None, to_ref=None, label="", v_std=1.0):
    """The bounds above for N(0, 1) values; with values of spread v_std, O
    and its absolute error scale by v_std, and so does the O bound.  A 16-bit
    O whose exact value cannot be stored within that bound (|O| >= 4 in bf16:
    half an ulp is 0.0156) is held to its storage floor plus FLOOR_MARGIN
    instead, the kernel's own share of the error."""
    tol = dict(TOL[dtype])
    tol["o"] *= v_std
    if dtype in (torch.bfloat16, torch.float16):
        tol["o"] = max(tol["o"], storage_floor(o_ref, dtype) + FLOOR_MARGIN * v_std)
    eo = max_err(o, o_ref)
    el = lse_err(lse, lse_ref)
    msg = f"{label}: max|dO|={eo:.3e} (tol {tol['o']:.2e}), max|dLSE|={el:.3e} (tol {tol['lse']:.0e})"
    if dtype == torch.bfloat16:
        msg += f", bf16 floor of O={bf16_floor(o_ref):.3e}"
    ok = eo <= tol["o"] and el <= tol["lse"]
    if to is not None:
        scale = max(float(np.max(np.abs(to_ref), initial=0.0)), 1e-30)
        et = max_err(to, to_ref) / scale
        msg += f", max|dtO|/max|tO|={et:.3e} (tol {tol['to']:.0e})"
        ok = ok and et <= tol["to"]
    print(msg, flush=True)
    assert ok, msg


# Peaked rows (one key carries most of a row's weight): O tracks single
# values of V, so storing O in bf16 alone costs up to half an ulp of |O|
# (7.8e-3 for |O| in [2, 4)).  Beyond that storage floor the kernel's own
# error comes from P's 16-bit rounding; with the dominant term taken at the
# exact running max (p = 1, no rounding) it stays far below this margin.
PEAKED_MARGIN = FLOOR_MARGIN


def assert_within_floor(o, o_ref, label="", margin=PEAKED_MARGIN):
    """max|O - O_ref| <= (bf16 storage floor of O_ref) + margin."""
    eo, fl = max_err(o, o_ref), bf16_floor(o_ref)
    msg = f"{label}: max|dO|={eo:.3e}, bf16 floor={fl:.3e}, excess={eo - fl:.2e} (margin {margin:.0e})"
    print(msg, flush=True)
    assert eo <= fl + margin, msg
