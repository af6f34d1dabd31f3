"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/attn.h declares, and rejects bad arguments on the host before
anything is enqueued (status codes as documented in the header)."""

import ctypes
import os
import re

import pytest

import attention_forward_online_attn_amd as attn
from attention_forward_online_attn_amd.binding import Strides3, Strides4

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "attn.h")

OK, INVALID, UNSUPPORTED, CAUSAL, WORKSPACE = 0, -1, -2, -3, -4
BF16, FP32, FP16 = 0, 1, 2
P = 1 << 20  # a 16-byte aligned fake device address: validation fails before any use


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(attn.library_path()):
        pytest.fail("libattn_mi355x.so is not built (run __graft_entry__.build())")
    return attn.load_library()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"ATTN_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_symbols() == sorted(
        ["attn_fwd", "attn_fwd_bias", "attn_fwd_dv", "attn_fwd_jvp", "jagged_attn_workspace_bytes", "jagged_attn_fwd",
         "attn_bwd_workspace_bytes", "attn_bwd", "attn_bwd_bias", "jagged_attn_bwd_workspace_bytes", "jagged_attn_bwd",
         "attn_status_string", "jagged_attn_fwd_noalloc"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
    # and nothing of the implementation leaks (hidden visibility)
    out = os.popen(f"nm -D --defined-only {attn.library_path()}").read()
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert exported == set(declared_symbols()), exported


def dense_strides(B, H, N, D):
    return Strides4(H * N * D, N * D, D, 1)


def call_fwd(lib, dtype=BF16, B=1, H=2, Nq=128, Nkv=128, D=64, scale=0.125, causal=0,
             q=P, k=P, v=P, o=P, lse=P, sq=None, so=None):
    sq = sq or dense_strides(B, H, Nq, D)
    sk = dense_strides(B, H, Nkv, D)
    so = so or dense_strides(B, H, Nq, D)
    return lib.attn_fwd(dtype, q, sq, k, sk, v, sk, o, so, lse, B, H, Nq, Nkv, D, scale, causal, None)


def test_oversized_extents_are_rejected(lib):
    """Extents whose products would overflow 64-bit integers, or whose
    (batch, head) count exceeds the 32-bit device indices, are rejected on
    the host before any product is formed; the workspace sizes report 0."""
    huge = 1 << 40
    assert call_fwd(lib, B=huge, H=huge) == INVALID
    assert call_fwd(lib, B=(1 << 31) - 1, H=2) == INVALID
    assert call_fwd(lib, Nq=1 << 31, Nkv=1 << 31) == INVALID
    st = dense_strides(1, 2, 128, 64)
    assert lib.attn_bwd(BF16, P, st, P, st, P, st, P, st, P, st, P, P, st, P, st, P, st,
                        huge, huge, 128, 128, 64, 0.125, 0, P, 1 << 20, None) == INVALID
    assert lib.attn_bwd_workspace_bytes(huge, huge, huge) == 0
    assert lib.attn_bwd_workspace_bytes(1 << 20, 1 << 20, 2) == 0
    assert lib.attn_bwd_workspace_bytes(1 << 10, 1 << 10, 1 << 10) == 8 << 30
    assert lib.jagged_attn_bwd_workspace_bytes(4, (1 << 31) - 1, (1 << 31) - 1) == 0


def test_status_strings(lib):
    assert lib.attn_status_string(0) == b"ok"
    for rc in (INVALID, UNSUPPORTED, CAUSAL, WORKSPACE, -5):
        assert lib.attn_status_string(rc) not in (b"ok", b"unknown status")
    assert lib.attn_status_string(7) == b"unknown status"


def test_dense_validation(lib):
    assert call_fwd(lib, D=96) == UNSUPPORTED
    assert call_fwd(lib, D=0) == INVALID
    assert call_fwd(lib, dtype=5) == UNSUPPORTED
    assert call_fwd(lib, dtype=FP16, D=96) == UNSUPPORTED
    assert call_fwd(lib, dtype=FP16, B=0) == OK
    assert call_fwd(lib, causal=1, Nkv=64) == CAUSAL
    assert call_fwd(lib, scale=-0.5) == INVALID
    assert call_fwd(lib, scale=float("nan")) == INVALID
    assert call_fwd(lib, scale=float("inf")) == INVALID
    assert call_fwd(lib, Nq=-1) == INVALID
    assert call_fwd(lib, q=0) == INVALID
    assert call_fwd(lib, lse=0) == INVALID
    assert call_fwd(lib, k=0) == INVALID
    assert call_fwd(lib, q=P + 2) == UNSUPPORTED                      # misaligned base
    assert call_fwd(lib, sq=Strides4(2 * 128 * 64, 128 * 64, 64, 2)) == INVALID  # head dim not unit stride
    assert call_fwd(lib, sq=Strides4(2 * 128 * 64, 128 * 64, 65, 1)) == UNSUPPORTED  # row stride not 16 B
    big = Strides4(0, 0, (1 << 22) + 8, 1)                                # K row stride beyond the 32-bit lane offsets
    assert lib.attn_fwd(BF16, P, dense_strides(1, 2, 128, 64), P, big, P, dense_strides(1, 2, 128, 64), P,
                        dense_strides(1, 2, 128, 64), P, 1, 2, 128, 128, 64, 0.125, 0, None) == UNSUPPORTED
    # no work: nothing is enqueued, null data pointers are fine
    assert call_fwd(lib, B=0, q=0, k=0, v=0, o=0, lse=0) == OK
    assert call_fwd(lib, Nq=0, q=0, k=0, v=0, o=0, lse=0) == OK


def test_bias_validation(lib):
    B, H, N, D = 1, 2, 128, 64
    st = dense_strides(B, H, N, D)
    full = Strides4(H * N * N, N * N, N, 1)
    ADD, MASK = 1, 2

    def call(kind=ADD, bias=P, bs=full, dtype=BF16, Nkv=N, B=B, D=D):
        sk = dense_strides(B, H, Nkv, D)
        return lib.attn_fwd_bias(dtype, P, st, P, sk, P, sk, P, st, P, bias, kind, bs, B, H, N, Nkv, D,
                                 0.125, 0, None)
    assert call(kind=0) == UNSUPPORTED
    assert call(kind=3) == UNSUPPORTED
    assert call(bias=0) == INVALID                                        # no bias with keys to bias
    assert call(bs=Strides4(H * N * N, N * N, N, 2)) == INVALID           # key stride must be 1
    assert call(bs=Strides4(-1, N * N, N, 1)) == INVALID
    assert call(bias=P + 2) == UNSUPPORTED                                # bf16 bias base not 16-byte aligned
    assert call(bs=Strides4(H * N * N, N * N, N + 4, 1)) == UNSUPPORTED  # row stride of 8 bytes (bf16)
    assert call(kind=MASK, bias=P + 8, bs=Strides4(0, 0, N + 4, 1)) == UNSUPPORTED  # mask rows: 8-byte multiples
    assert call(kind=MASK, bias=P + 4) == UNSUPPORTED
    assert call(dtype=FP32, bs=Strides4(0, 0, N + 2, 1)) == UNSUPPORTED  # fp32 bias rows: 16-byte multiples
    assert call(D=96) == UNSUPPORTED
    # no work: nothing is enqueued
    assert call(B=0) == OK
    assert call(B=0, bias=0) == OK


def test_jvp_validation(lib):
    s = dense_strides(1, 1, 64, 64)
    args = lambda tq=P, to=P, D=64: lib.attn_fwd_jvp(BF16, P, P, P, tq, P, P, s, s, s, P, to, s, P, None,
                                                     1, 1, 64, 64, D, 0.125, 0, None)
    assert args(tq=0) == INVALID
    assert args(to=0) == INVALID
    assert args(D=48) == UNSUPPORTED


def test_jagged_validation(lib):
    H, T, D, S = 2, 100, 64, 3
    st = Strides3(T * D, D, 1)
    need = lib.jagged_attn_workspace_bytes(S, T)
    assert need >= 16 + 8 * ((T + S * 63) // 64)
    assert lib.jagged_attn_workspace_bytes(-1, T) == 0

    def call(ws=P, ws_bytes=need, msl=64, D=64, offsets=P):
        return lib.jagged_attn_fwd(BF16, P, st, P, st, P, st, P, st, P, offsets, S, H, T, D, msl,
                                   0.125, 0, ws, ws_bytes, None)
    assert call(ws=0) == WORKSPACE
    assert call(ws_bytes=16) == WORKSPACE
    assert call(ws=P + 8) == WORKSPACE
    assert call(msl=0) == INVALID
    assert call(offsets=0) == INVALID
    assert call(D=48) == UNSUPPORTED
    assert lib.jagged_attn_fwd(BF16, 0, st, 0, st, 0, st, 0, st, 0, 0, 0, H, 0, D, 64,
                               0.125, 0, 0, 0, None) == OK


def test_jagged_noalloc_validation(lib):
    """The argument checks of jagged_attn_fwd, and the plan's bound: it must
    fit the 2^20-byte static scratch (16 + 8 x query tiles), checked on the
    host before any device call."""
    H, D = 2, 64

    def call(S, T, offsets=P, msl=64, D=D, q=P):
        st = Strides3(T * D, D, 1)
        return lib.jagged_attn_fwd_noalloc(BF16, q, st, P, st, P, st, P, st, P, offsets, S, H, T, D, msl, 0.125, 0, None)
    assert call(3, 100, offsets=0) == INVALID
    assert call(3, 100, msl=0) == INVALID
    assert call(3, 100, q=0) == INVALID
    assert call(3, 100, D=48) == UNSUPPORTED
    assert call(0, 100) == OK and call(3, 0) == OK
    # 131071 one-row sequences: 131071 tiles of 128 rows -> 16 + 8 * 131071 bytes, one tile too many
    assert call(131071, 131071) == WORKSPACE
    # one long sequence: (T + 127) / 128 tiles
    assert call(1, 131071 * 128) == WORKSPACE
    assert b"static scratch" in lib.attn_status_string(WORKSPACE)


def test_binding_rejects_host_tensors(lib):
    import torch
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(attn.AttnError):
        attn.fwd(x, x, x)
    with pytest.raises(attn.AttnError):
        attn.fwd(x.float(), x, x)


def test_bwd_validation(lib):
    B, H, N, D = 1, 2, 128, 64
    st = dense_strides(B, H, N, D)
    need = lib.attn_bwd_workspace_bytes(B, H, N)
    assert need == 8 * B * H * N
    assert lib.attn_bwd_workspace_bytes(-1, H, N) == 0

    def call(dtype=BF16, D=64, causal=0, Nkv=N, ws=P, ws_bytes=need, q=P, dq=P, lse=P, scale=0.125, sq=st):
        sk = dense_strides(B, H, Nkv, D)
        return lib.attn_bwd(dtype, q, sq, P, sk, P, sk, P, st, P, st, lse, dq, st, P, sk, P, sk,
                            B, H, N, Nkv, D, scale, causal, ws, ws_bytes, None)
    assert call(dtype=FP32) == UNSUPPORTED
    assert call(D=96) == UNSUPPORTED
    assert call(causal=1, Nkv=64) == CAUSAL
    assert call(ws=0) == WORKSPACE
    assert call(ws_bytes=need - 4) == WORKSPACE
    assert call(ws=P + 4) == WORKSPACE
    assert call(q=0) == INVALID
    assert call(dq=0) == INVALID
    assert call(lse=0) == INVALID
    assert call(scale=-1.0) == INVALID
    assert call(q=P + 2) == UNSUPPORTED
    assert call(sq=Strides4(H * N * D, N * D, D, 2)) == INVALID
    zero = lib.attn_bwd(BF16, 0, st, 0, st, 0, st, 0, st, 0, st, 0, 0, st, 0, st, 0, st,
                        0, H, N, N, D, 0.125, 0, 0, 0, None)
    assert zero == OK


def test_bwd_grid_bounds(lib):
    """The backward's prep kernel takes 8 rows per block at head dim 256: B H
    Nq = 2^34 rows would need 2^31 blocks, one past an int grid.  Rejected
    on the host, before anything is enqueued (the pointers are never used)."""
    B, H, N, D = 1, 1 << 20, 1 << 14, 256
    st = dense_strides(B, H, N, D)
    need = lib.attn_bwd_workspace_bytes(B, H, N)
    assert lib.attn_bwd(BF16, P, st, P, st, P, st, P, st, P, st, P, P, st, P, st, P, st,
                        B, H, N, N, D, 0.0625, 0, P, need, None) == INVALID
    sj = Strides3(N * D, D, 1)
    assert lib.jagged_attn_bwd(BF16, P, sj, P, sj, P, sj, P, sj, P, sj, P, P, sj, P, sj, P, sj,
                               P, 1, H, N, D, N, 0.0625, 0, P, 1 << 40, None) == INVALID


def test_jagged_bwd_validation(lib):
    H, T, D, S = 2, 100, 64, 3
    st = Strides3(T * D, D, 1)
    need = lib.jagged_attn_bwd_workspace_bytes(S, H, T)
    assert need >= 16 + 8 * ((T + S * 127) // 128) + 8 * H * T and need % 16 == 0
    assert lib.jagged_attn_bwd_workspace_bytes(-1, H, T) == 0

    def call(dtype=BF16, ws=P, ws_bytes=need, msl=64, D=64, offsets=P, lse=P, dq=P, H=H):
        return lib.jagged_attn_bwd(dtype, P, st, P, st, P, st, P, st, P, st, lse, dq, st, P, st, P, st,
                                   offsets, S, H, T, D, msl, 0.125, 0, ws, ws_bytes, None)
    assert call(dtype=FP32) == UNSUPPORTED
    assert call(D=48) == UNSUPPORTED
    assert call(ws=0) == WORKSPACE
    assert call(ws_bytes=need - 1) == WORKSPACE
    assert call(ws=P + 8) == WORKSPACE
    assert call(msl=0) == INVALID
    assert call(offsets=0) == INVALID
    assert call(lse=0) == INVALID
    assert call(dq=0) == INVALID
    assert call(H=0) == OK


def test_dv_validation(lib):
    B, H, N = 1, 2, 128
    sq = dense_strides(B, H, N, 64)
    sv = dense_strides(B, H, N, 128)

    def call(Dqk=64, Dv=128, tq=0, tk=0, tv=0, to=0, tlse=0, B=B):
        return lib.attn_fwd_dv(BF16, P, P, P, tq, tk, tv, sq, sq, sv, P, to, sv, P, tlse,
                               B, H, N, N, Dqk, Dv, 0.125, 0, None)
    assert call(Dv=96) == UNSUPPORTED
    assert call(Dv=0) == INVALID
    assert call(Dqk=48) == UNSUPPORTED
    assert call(Dqk=16, Dv=16, B=0) == OK
    assert call(Dqk=16, Dv=32, B=0) == OK
    assert call(Dqk=128, Dv=16, tq=P, tk=P, tv=P, to=P, B=0) == OK  # the 128-wide JVP with 16-wide values
    assert call(tk=P) == INVALID          # tangents without tq: not a JVP call
    assert call(to=P) == INVALID
    assert call(tq=P, tk=P, tv=P) == INVALID  # JVP without to
    assert call(B=0) == OK


def test_bwd_bias_validation(lib):
    B, H, N, D = 1, 2, 128, 64
    st = dense_strides(B, H, N, D)
    full = Strides4(H * N * N, N * N, N, 1)
    need = lib.attn_bwd_workspace_bytes(B, H, N)
    ADD, MASK = 1, 2

    def call(kind=ADD, bias=P, bs=full, dbias=0, dbs=full, dtype=BF16, B=B):
        return lib.attn_bwd_bias(dtype, P, st, P, st, P, st, P, st, P, st, P, bias, kind, bs, dbias, dbs,
                                 P, st, P, st, P, st, B, H, N, N, D, 0.125, 0, P, need, None)
    assert call(kind=0) == UNSUPPORTED
    assert call(dtype=FP32) == UNSUPPORTED
    assert call(bias=0) == INVALID
    assert call(bs=Strides4(0, 0, N, 2)) == INVALID                      # key stride must be 1
    assert call(bias=P + 2) == UNSUPPORTED
    assert call(kind=MASK, dbias=P) == INVALID                           # a mask has no gradient
    assert call(dbias=P, dbs=Strides4(H * N * N, 0, N, 1)) == INVALID    # heads would share (race)
    assert call(dbias=P, dbs=Strides4(H * N * N, N * N, 0, 1)) == INVALID
    assert call(dbias=P + 8) == UNSUPPORTED
    assert call(B=0) == OK


def test_d256_paths(lib):
    """Head dim 256 runs the forward (biased or not), the JVP (bf16, fp16
    and fp32) and the backward."""
    B, H, N, D = 0, 2, 128, 256  # B = 0: nothing is enqueued when the call is accepted
    st = dense_strides(1, H, N, D)
    assert call_fwd(lib, D=256, B=0) == OK
    for dt in (BF16, FP16, FP32):
        assert lib.attn_fwd_jvp(dt, P, P, P, P, P, P, st, st, st, P, P, st, P, None, 0, H, N, N, D, 0.1, 0, None) == OK
    full = Strides4(H * N * N, N * N, N, 1)
    assert lib.attn_fwd_bias(BF16, P, st, P, st, P, st, P, st, P, P, 1, full, 0, H, N, N, D, 0.1, 0, None) == OK
    need = lib.attn_bwd_workspace_bytes(1, H, N)
    assert lib.attn_bwd(BF16, P, st, P, st, P, st, P, st, P, st, P, P, st, P, st, P, st, 0, H, N, N, D, 0.1, 0,
                        P, need, None) == OK
    assert lib.attn_bwd(BF16, P, st, P, st, P, st, P, st, P, st, P, P, st, P, st, P, st, 1, H, N, N, 512, 0.1, 0,
                        P, need, None) == UNSUPPORTED
    assert lib.attn_fwd_dv(BF16, P, P, P, 0, 0, 0, st, st, st, P, 0, st, P, 0, 0, H, N, N, 256, 128, 0.1, 0, None) == OK


def test_value_head_dims(lib):
    """Every pair of query/key and value head dims in {16, 32, 64, 128, 256}
    is accepted, plain and JVP, in every dtype (B = 0: nothing enqueued);
    other value widths are not head dims."""
    H, N = 2, 64
    dims = (16, 32, 64, 128, 256)
    for dt in (BF16, FP16, FP32):
        for dq in dims:
            for dv in dims:
                sq, sv = dense_strides(1, H, N, dq), dense_strides(1, H, N, dv)
                for jvp in (0, 1):
                    t = P if jvp else 0
                    rc = lib.attn_fwd_dv(dt, P, P, P, t, t, t, sq, sq, sv, P, t, sv, P, 0, 0, H, N, N, dq, dv, 0.1, 0,
                                         None)
                    assert rc == OK, (dt, dq, dv, jvp, rc)
    sq, sv = dense_strides(1, H, N, 64), dense_strides(1, H, N, 48)
    assert lib.attn_fwd_dv(BF16, P, P, P, 0, 0, 0, sq, sq, sv, P, 0, sv, P, 0, 0, H, N, N, 64, 48, 0.1, 0, None) \
        == UNSUPPORTED
    assert lib.attn_fwd_dv(BF16, P, P, P, 0, 0, 0, sq, sq, sv, P, 0, sv, P, 0, 0, H, N, N, 512, 64, 0.1, 0, None) \
        == UNSUPPORTED


def test_d16_paths(lib):
    """Head dim 16 runs the forward (biased or not), the JVP and the
    backward; other widths below 32 are not head dims."""
    H, N = 2, 128
    st = dense_strides(1, H, N, 16)
    assert call_fwd(lib, D=16, B=0) == OK
    full = Strides4(H * N * N, N * N, N, 1)
    assert lib.attn_fwd_bias(BF16, P, st, P, st, P, st, P, st, P, P, 1, full, 0, H, N, N, 16, 0.1, 0, None) == OK
    need = lib.attn_bwd_workspace_bytes(1, H, N)
    # B = 0: the head dim passes validation and nothing is launched
    assert lib.attn_bwd(BF16, P, st, P, st, P, st, P, st, P, st, P, P, st, P, st, P, st, 0, H, N, N, 16, 0.1, 0,
                        P, need, None) == OK
    assert lib.attn_bwd(BF16, P, st, P, st, P, st, P, st, P, st, P, P, st, P, st, P, st, 1, H, N, N, 24, 0.1, 0,
                        P, need, None) == UNSUPPORTED
