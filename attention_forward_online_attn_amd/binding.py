"""ctypes binding of libattn_mi355x.so (declarations in include/attn.h).

Argument marshalling only: tensors become device pointers and element strides,
outputs are allocated with torch.empty, the stream is torch's current HIP
stream.  A missing library or a non-zero status raises AttnError; there is no
fallback of any kind.
"""

from __future__ import annotations

import ctypes
import os

import torch

_LIB_NAME = "libattn_mi355x.so"
_lib = None

ATTN_BF16 = 0
ATTN_FP32 = 1
ATTN_FP16 = 2
ATTN_BIAS_ADD = 1
ATTN_BIAS_MASK = 2


class AttnError(RuntimeError):
    """A failed library call; ``status`` holds the C status code."""

    def __init__(self, msg, status=None):
        super().__init__(msg)
        self.status = status


class Strides4(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64),
                ("n", ctypes.c_int64), ("d", ctypes.c_int64)]


class Strides3(ctypes.Structure):
    _fields_ = [("h", ctypes.c_int64), ("t", ctypes.c_int64), ("d", ctypes.c_int64)]


def library_path() -> str:
    """The in-tree libattn_mi355x.so, or the build that ATTN_LIBRARY names
    (another build of the same C ABI, such as the host-sanitizer build)."""
    override = os.environ.get("ATTN_LIBRARY")
    if override:
        return override
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), _LIB_NAME)


def load_library():
    """Load libattn_mi355x.so and declare its entry points (once)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise AttnError(f"{path} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    vp, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    S4, S3 = Strides4, Strides3
    lib.attn_fwd.argtypes = [i32, vp, S4, vp, S4, vp, S4, vp, S4, vp,
                             i64, i64, i64, i64, i64, f32, i32, vp]
    lib.attn_fwd.restype = i32
    lib.attn_fwd_bias.argtypes = [i32, vp, S4, vp, S4, vp, S4, vp, S4, vp, vp, i32, S4,
                                  i64, i64, i64, i64, i64, f32, i32, vp]
    lib.attn_fwd_bias.restype = i32
    lib.attn_fwd_dv.argtypes = [i32, vp, vp, vp, vp, vp, vp, S4, S4, S4, vp, vp, S4, vp, vp,
                                i64, i64, i64, i64, i64, i64, f32, i32, vp]
    lib.attn_fwd_dv.restype = i32
    lib.attn_fwd_jvp.argtypes = [i32, vp, vp, vp, vp, vp, vp, S4, S4, S4, vp, vp, S4, vp, vp,
                                 i64, i64, i64, i64, i64, f32, i32, vp]
    lib.attn_fwd_jvp.restype = i32
    lib.jagged_attn_workspace_bytes.argtypes = [i64, i64]
    lib.jagged_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.jagged_attn_fwd.argtypes = [i32, vp, S3, vp, S3, vp, S3, vp, S3, vp, vp,
                                    i64, i64, i64, i64, i64, f32, i32, vp, ctypes.c_size_t, vp]
    lib.jagged_attn_fwd.restype = i32
    lib.jagged_attn_fwd_noalloc.argtypes = [i32, vp, S3, vp, S3, vp, S3, vp, S3, vp, vp,
                                            i64, i64, i64, i64, i64, f32, i32, vp]
    lib.jagged_attn_fwd_noalloc.restype = i32
    lib.attn_bwd_workspace_bytes.argtypes = [i64, i64, i64]
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_bwd.argtypes = [i32, vp, S4, vp, S4, vp, S4, vp, S4, vp, S4, vp, vp, S4, vp, S4, vp, S4,
                             i64, i64, i64, i64, i64, f32, i32, vp, ctypes.c_size_t, vp]
    lib.attn_bwd.restype = i32
    lib.jagged_attn_bwd_workspace_bytes.argtypes = [i64, i64, i64]
    lib.jagged_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.jagged_attn_bwd.argtypes = [i32, vp, S3, vp, S3, vp, S3, vp, S3, vp, S3, vp, vp, S3, vp, S3, vp, S3,
                                    vp, i64, i64, i64, i64, i64, f32, i32, vp, ctypes.c_size_t, vp]
    lib.jagged_attn_bwd.restype = i32
    lib.attn_bwd_bias.argtypes = [i32, vp, S4, vp, S4, vp, S4, vp, S4, vp, S4, vp, vp, i32, S4, vp, S4,
                                  vp, S4, vp, S4, vp, S4, i64, i64, i64, i64, i64, f32, i32, vp, ctypes.c_size_t, vp]
    lib.attn_bwd_bias.restype = i32
    lib.attn_status_string.argtypes = [i32]
    lib.attn_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc):
    if rc != 0:
        msg = load_library().attn_status_string(rc).decode()
        raise AttnError(f"attention library call failed: {msg} (status {rc})", rc)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_FP32
    if t.dtype == torch.float16:
        return ATTN_FP16
    raise AttnError(f"unsupported dtype {t.dtype}; expected bfloat16, float16 or float32")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _s4(t):
    return Strides4(*t.stride())


def _s3(t):
    return Strides3(*t.stride())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _same(ref, *ts):
    for t in ts:
        if t.dtype != ref.dtype or t.device != ref.device:
            raise AttnError("all tensors must share dtype and device")
        if not t.is_cuda:
            raise AttnError("tensors must be on a HIP device")


def fwd(q, k, v, causal=False, sm_scale=None):
    """Dense forward.  q [B,H,Nq,D], k [B,H,Nkv,D], v [B,H,Nkv,Dv] ->
    (o [B,H,Nq,Dv], lse fp32 [B,H,Nq]); Dv != D goes through attn_fwd_dv."""
    lib = load_library()
    _same(q, k, v)
    B, H, Nq, D = q.shape
    Nkv, Dv = k.shape[2], v.shape[3]
    if sm_scale is None:
        sm_scale = D ** -0.5
    o = torch.empty((B, H, Nq, Dv), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if Dv != D:
        none = ctypes.c_void_p(0)
        _check(lib.attn_fwd_dv(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), none, none, none, _s4(q), _s4(k), _s4(v),
                               _ptr(o), none, _s4(o), _ptr(lse), none, B, H, Nq, Nkv, D, Dv,
                               float(sm_scale), int(bool(causal)), _stream(q)))
        return o, lse
    _check(lib.attn_fwd(_dtype_code(q), _ptr(q), _s4(q), _ptr(k), _s4(k), _ptr(v), _s4(v),
                        _ptr(o), _s4(o), _ptr(lse), B, H, Nq, Nkv, D,
                        float(sm_scale), int(bool(causal)), _stream(q)))
    return o, lse


def fwd_bias(q, k, v, bias=None, mask=None, causal=False, sm_scale=None):
    """Dense forward with an additive bias (dtype of q) or a boolean mask
    (torch.bool or uint8; False / 0 removes the key), either broadcastable to
    [B,H,Nq,Nkv] with the key dimension contiguous; broadcast dimensions are
    passed as stride 0, never materialised.  -> (o, lse) as fwd."""
    lib = load_library()
    _same(q, k, v)
    if (bias is None) == (mask is None):
        raise AttnError("pass exactly one of bias and mask")
    B, H, Nq, D = q.shape
    Nkv = k.shape[2]
    if sm_scale is None:
        sm_scale = D ** -0.5
    if bias is not None:
        if bias.dtype != q.dtype or bias.device != q.device:
            raise AttnError("bias must have the dtype and device of q")
        op, kind = bias.expand(B, H, Nq, Nkv), ATTN_BIAS_ADD
    else:
        if mask.dtype not in (torch.bool, torch.uint8) or mask.device != q.device:
            raise AttnError("mask must be a bool or uint8 tensor on the device of q")
        op, kind = mask.expand(B, H, Nq, Nkv), ATTN_BIAS_MASK
    o = torch.empty((B, H, Nq, D), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check(lib.attn_fwd_bias(_dtype_code(q), _ptr(q), _s4(q), _ptr(k), _s4(k), _ptr(v), _s4(v),
                             _ptr(o), _s4(o), _ptr(lse), _ptr(op), kind, _s4(op), B, H, Nq, Nkv, D,
                             float(sm_scale), int(bool(causal)), _stream(q)))
    return o, lse


def fwd_jvp(q, k, v, tq, tk, tv, causal=False, sm_scale=None, return_tlse=False):
    """Dense forward fused with the JVP -> (o, to, lse), or (o, to, lse, tlse)
    with return_tlse (tlse fp32 [B,H,Nq], the tangent of lse).  Tangents must
    have the strides of their primals."""
    lib = load_library()
    _same(q, k, v, tq, tk, tv)
    for t, p in ((tq, q), (tk, k), (tv, v)):
        if t.shape != p.shape or t.stride() != p.stride():
            raise AttnError("tangents must match their primals in shape and strides")
    B, H, Nq, D = q.shape
    Nkv, Dv = k.shape[2], v.shape[3]
    if sm_scale is None:
        sm_scale = D ** -0.5
    o = torch.empty((B, H, Nq, Dv), dtype=q.dtype, device=q.device)
    to = torch.empty_like(o)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    tlse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if return_tlse else None
    if Dv != D:
        _check(lib.attn_fwd_dv(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(tq), _ptr(tk), _ptr(tv),
                               _s4(q), _s4(k), _s4(v), _ptr(o), _ptr(to), _s4(o), _ptr(lse), _ptr(tlse),
                               B, H, Nq, Nkv, D, Dv, float(sm_scale), int(bool(causal)), _stream(q)))
    else:
        _check(lib.attn_fwd_jvp(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(tq), _ptr(tk), _ptr(tv),
                                _s4(q), _s4(k), _s4(v), _ptr(o), _ptr(to), _s4(o), _ptr(lse), _ptr(tlse),
                                B, H, Nq, Nkv, D, float(sm_scale), int(bool(causal)), _stream(q)))
    return (o, to, lse, tlse) if return_tlse else (o, to, lse)


def jagged_workspace_bytes(num_seqs, total_len) -> int:
    return int(load_library().jagged_attn_workspace_bytes(int(num_seqs), int(total_len)))


def jagged_fwd(q, k, v, offsets, max_seq_len, causal=False, sm_scale=None, workspace=None):
    """Jagged forward.  q/k/v [H, total_len, D], offsets int64 [num_seqs+1] on
    the device -> (o [H, total_len, D], lse fp32 [H, total_len])."""
    lib = load_library()
    _same(q, k, v)
    if offsets.dtype != torch.int64 or offsets.device != q.device or offsets.dim() != 1:
        raise AttnError("offsets must be a 1-D int64 tensor on the same device")
    offsets = offsets.contiguous()
    H, T, D = q.shape
    S = offsets.numel() - 1
    if sm_scale is None:
        sm_scale = D ** -0.5
    need = jagged_workspace_bytes(S, T)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    o = torch.empty((H, T, D), dtype=q.dtype, device=q.device)
    lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    _check(lib.jagged_attn_fwd(_dtype_code(q), _ptr(q), _s3(q), _ptr(k), _s3(k), _ptr(v), _s3(v),
                               _ptr(o), _s3(o), _ptr(lse), _ptr(offsets), S, H, T, D,
                               int(max_seq_len), float(sm_scale), int(bool(causal)),
                               _ptr(workspace), workspace.numel(), _stream(q)))
    return o, lse


def jagged_fwd_noalloc(q, k, v, offsets, max_seq_len, causal=False, sm_scale=None, out=None):
    """jagged_fwd without a workspace: the library keeps the tile plan in a
    static device array (calls on one GPU must not overlap).  With
    out=(o, lse) -- [H, total_len, D] of q's dtype and contiguous fp32
    [H, total_len] -- nothing at all is allocated."""
    lib = load_library()
    _same(q, k, v)
    if offsets.dtype != torch.int64 or offsets.device != q.device or offsets.dim() != 1 or not offsets.is_contiguous():
        raise AttnError("offsets must be a contiguous 1-D int64 tensor on the same device")
    H, T, D = q.shape
    S = offsets.numel() - 1
    if sm_scale is None:
        sm_scale = D ** -0.5
    if out is None:
        o = torch.empty((H, T, D), dtype=q.dtype, device=q.device)
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _same(q, o)
        if o.shape != (H, T, D) or lse.shape != (H, T) or lse.dtype != torch.float32 or not lse.is_contiguous() \
                or lse.device != q.device:
            raise AttnError("out must be (o [H, total_len, D], lse contiguous fp32 [H, total_len])")
    _check(lib.jagged_attn_fwd_noalloc(_dtype_code(q), _ptr(q), _s3(q), _ptr(k), _s3(k), _ptr(v), _s3(v),
                                       _ptr(o), _s3(o), _ptr(lse), _ptr(offsets), S, H, T, D,
                                       int(max_seq_len), float(sm_scale), int(bool(causal)), _stream(q)))
    return o, lse


def bwd_workspace_bytes(B, H, Nq) -> int:
    return int(load_library().attn_bwd_workspace_bytes(int(B), int(H), int(Nq)))


def bwd(q, k, v, o, do, lse, causal=False, sm_scale=None, workspace=None):
    """Dense backward (bf16 or fp16).  q/o/do [B,H,Nq,D], k/v [B,H,Nkv,D], lse fp32
    [B,H,Nq] from fwd with the same q, k, v -> (dq, dk, dv) shaped like q, k, v."""
    lib = load_library()
    _same(q, k, v, o, do)
    if lse.dtype != torch.float32 or lse.device != q.device:
        raise AttnError("lse must be a float32 tensor on the same device")
    B, H, Nq, D = q.shape
    Nkv = k.shape[2]
    if lse.shape != (B, H, Nq) or not lse.is_contiguous():
        raise AttnError("lse must be a contiguous [B, H, Nq] tensor")
    if sm_scale is None:
        sm_scale = D ** -0.5
    need = bwd_workspace_bytes(B, H, Nq)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    dq = torch.empty_like(q, memory_format=torch.contiguous_format)
    dk = torch.empty_like(k, memory_format=torch.contiguous_format)
    dv = torch.empty_like(v, memory_format=torch.contiguous_format)
    _check(lib.attn_bwd(_dtype_code(q), _ptr(q), _s4(q), _ptr(k), _s4(k), _ptr(v), _s4(v), _ptr(o), _s4(o),
                        _ptr(do), _s4(do), _ptr(lse), _ptr(dq), _s4(dq), _ptr(dk), _s4(dk), _ptr(dv), _s4(dv),
                        B, H, Nq, Nkv, D, float(sm_scale), int(bool(causal)),
                        _ptr(workspace), workspace.numel(), _stream(q)))
    return dq, dk, dv


def jagged_bwd_workspace_bytes(num_seqs, H, total_len) -> int:
    return int(load_library().jagged_attn_bwd_workspace_bytes(int(num_seqs), int(H), int(total_len)))


def jagged_bwd(q, k, v, o, do, lse, offsets, max_seq_len, causal=False, sm_scale=None, workspace=None):
    """Jagged backward (bf16 or fp16).  q/k/v/o/do [H, total_len, D], lse fp32
    [H, total_len] from jagged_fwd with the same inputs, offsets int64
    [num_seqs+1] on the device -> (dq, dk, dv) shaped like q, k, v."""
    lib = load_library()
    _same(q, k, v, o, do)
    if offsets.dtype != torch.int64 or offsets.device != q.device or offsets.dim() != 1:
        raise AttnError("offsets must be a 1-D int64 tensor on the same device")
    H, T, D = q.shape
    if lse.dtype != torch.float32 or lse.device != q.device or lse.shape != (H, T) or not lse.is_contiguous():
        raise AttnError("lse must be a contiguous float32 [H, total_len] tensor on the same device")
    offsets = offsets.contiguous()
    S = offsets.numel() - 1
    if sm_scale is None:
        sm_scale = D ** -0.5
    need = jagged_bwd_workspace_bytes(S, H, T)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _check(lib.jagged_attn_bwd(_dtype_code(q), _ptr(q), _s3(q), _ptr(k), _s3(k), _ptr(v), _s3(v), _ptr(o), _s3(o),
                               _ptr(do), _s3(do), _ptr(lse), _ptr(dq), _s3(dq), _ptr(dk), _s3(dk), _ptr(dv), _s3(dv),
                               _ptr(offsets), S, H, T, D, int(max_seq_len), float(sm_scale), int(bool(causal)),
                               _ptr(workspace), workspace.numel(), _stream(q)))
    return dq, dk, dv


def bwd_bias(q, k, v, o, do, lse, bias=None, mask=None, causal=False, sm_scale=None, workspace=None,
             return_dbias=False):
    """Dense backward with the score operand of fwd_bias (pass the same bias
    or mask, and the lse fwd_bias returned) -> (dq, dk, dv), or
    (dq, dk, dv, dbias) with return_dbias (additive bias only; dbias is the
    full [B,H,Nq,Nkv] dS, a view of rows padded to 16 bytes: sum it over the
    dimensions the bias broadcasts)."""
    lib = load_library()
    _same(q, k, v, o, do)
    if (bias is None) == (mask is None):
        raise AttnError("pass exactly one of bias and mask")
    B, H, Nq, D = q.shape
    Nkv = k.shape[2]
    if lse.dtype != torch.float32 or lse.shape != (B, H, Nq) or not lse.is_contiguous():
        raise AttnError("lse must be a contiguous float32 [B, H, Nq] tensor")
    if sm_scale is None:
        sm_scale = D ** -0.5
    if bias is not None:
        if bias.dtype != q.dtype or bias.device != q.device:
            raise AttnError("bias must have the dtype and device of q")
        op, kind = bias.expand(B, H, Nq, Nkv), ATTN_BIAS_ADD
    else:
        if mask.dtype not in (torch.bool, torch.uint8) or mask.device != q.device:
            raise AttnError("mask must be a bool or uint8 tensor on the device of q")
        if return_dbias:
            raise AttnError("a mask has no gradient")
        op, kind = mask.expand(B, H, Nq, Nkv), ATTN_BIAS_MASK
    if workspace is None:
        workspace = torch.empty(max(bwd_workspace_bytes(B, H, Nq), 16), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dbias = None
    if return_dbias:  # rows padded to a multiple of 8 elements (16 bytes), returned as the [.., :Nkv] view
        dbias = torch.empty((B, H, Nq, (Nkv + 7) // 8 * 8), dtype=q.dtype, device=q.device)[..., :Nkv]
    db_strides = _s4(dbias) if dbias is not None else Strides4(0, 0, 0, 1)
    _check(lib.attn_bwd_bias(_dtype_code(q), _ptr(q), _s4(q), _ptr(k), _s4(k), _ptr(v), _s4(v), _ptr(o), _s4(o),
                             _ptr(do), _s4(do), _ptr(lse), _ptr(op), kind, _s4(op), _ptr(dbias), db_strides,
                             _ptr(dq), _s4(dq), _ptr(dk), _s4(dk), _ptr(dv), _s4(dv), B, H, Nq, Nkv, D,
                             float(sm_scale), int(bool(causal)), _ptr(workspace), workspace.numel(), _stream(q)))
    return (dq, dk, dv, dbias) if return_dbias else (dq, dk, dv)
