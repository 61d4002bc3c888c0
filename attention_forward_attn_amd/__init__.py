"""Python binding of the gfx950 fused attention forward (C ABI in include/attn_fwd.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libattn_fwd.so``. PyTorch supplies device memory and the stream.
There is no CPU fallback; if the library is missing, importing the binding's
entry points raises.

    out, lse = dense(q, k, v, causal=True, scale=None, sinks=None)
    out, lse = sparse_topk(q, kv, idx, d_v=512, scale=None, sinks=None)
    dq, dk, dv, dsinks = dense_backward(q, k, v, out, dout, lse, causal=True, sinks=None)
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn_fwd.so")

ATTN_OK, ATTN_INVALID_ARGUMENT, ATTN_UNSUPPORTED, ATTN_ABI_MISMATCH, ATTN_HIP_ERROR = range(5)
ATTN_BF16, ATTN_F32 = 0, 1
ABI_VERSION = 13
NOALLOC_SCRATCH_BYTES = 64 << 20  # the library's per-device scratch array (ATTN_NOALLOC_SCRATCH_BYTES)


class AttnDenseArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Tq", ctypes.c_int32), ("Tk", ctypes.c_int32),
        ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("q_sb", ctypes.c_int64), ("q_sh", ctypes.c_int64), ("q_st", ctypes.c_int64),
        ("k", ctypes.c_void_p), ("k_sb", ctypes.c_int64), ("k_sh", ctypes.c_int64), ("k_st", ctypes.c_int64),
        ("v", ctypes.c_void_p), ("v_sb", ctypes.c_int64), ("v_sh", ctypes.c_int64), ("v_st", ctypes.c_int64),
        ("out", ctypes.c_void_p), ("o_sb", ctypes.c_int64), ("o_sh", ctypes.c_int64), ("o_st", ctypes.c_int64),
        ("lse", ctypes.c_void_p),
        ("sinks", ctypes.c_void_p),
        ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32),
        ("q_rope", ctypes.c_void_p), ("qr_sb", ctypes.c_int64), ("qr_sh", ctypes.c_int64), ("qr_st", ctypes.c_int64),
        ("k_rope", ctypes.c_void_p), ("kr_sb", ctypes.c_int64), ("kr_sh", ctypes.c_int64), ("kr_st", ctypes.c_int64),
        ("keep", ctypes.c_void_p), ("m_sb", ctypes.c_int64), ("m_sh", ctypes.c_int64), ("m_st", ctypes.c_int64),
        ("p_drop", ctypes.c_float),
    ]


class AttnSparseArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("Sq", ctypes.c_int32), ("Hq", ctypes.c_int32), ("N", ctypes.c_int32),
        ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32), ("topk", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("q_ss", ctypes.c_int64), ("q_sh", ctypes.c_int64),
        ("kv", ctypes.c_void_p), ("kv_sn", ctypes.c_int64),
        ("indices", ctypes.c_void_p), ("idx_ss", ctypes.c_int64),
        ("out", ctypes.c_void_p), ("o_ss", ctypes.c_int64), ("o_sh", ctypes.c_int64),
        ("lse", ctypes.c_void_p),
        ("sinks", ctypes.c_void_p),
    ]


class AttnPlan(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("path", ctypes.c_char * 64),
        ("block_rows", ctypes.c_int32), ("block_keys", ctypes.c_int32), ("waves", ctypes.c_int32),
        ("grid", ctypes.c_int32), ("lds_bytes", ctypes.c_int32), ("fold_g", ctypes.c_int32),
        ("folded_rows", ctypes.c_int64),
        ("hbm_score_bytes", ctypes.c_int64),
        ("budget_bytes", ctypes.c_int64),
        ("score_elt_bytes", ctypes.c_int32),
        ("budget_tile_rows", ctypes.c_int64),
        ("budget_tiles", ctypes.c_int64),
    ]


class AttnDenseBwdArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Tq", ctypes.c_int32), ("Tk", ctypes.c_int32), ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("q_sb", ctypes.c_int64), ("q_sh", ctypes.c_int64), ("q_st", ctypes.c_int64),
        ("k", ctypes.c_void_p), ("k_sb", ctypes.c_int64), ("k_sh", ctypes.c_int64), ("k_st", ctypes.c_int64),
        ("v", ctypes.c_void_p), ("v_sb", ctypes.c_int64), ("v_sh", ctypes.c_int64), ("v_st", ctypes.c_int64),
        ("out", ctypes.c_void_p), ("o_sb", ctypes.c_int64), ("o_sh", ctypes.c_int64), ("o_st", ctypes.c_int64),
        ("dout", ctypes.c_void_p), ("do_sb", ctypes.c_int64), ("do_sh", ctypes.c_int64), ("do_st", ctypes.c_int64),
        ("lse", ctypes.c_void_p),
        ("sinks", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dq_sb", ctypes.c_int64), ("dq_sh", ctypes.c_int64), ("dq_st", ctypes.c_int64),
        ("dk", ctypes.c_void_p), ("dk_sb", ctypes.c_int64), ("dk_sh", ctypes.c_int64), ("dk_st", ctypes.c_int64),
        ("dv", ctypes.c_void_p), ("dv_sb", ctypes.c_int64), ("dv_sh", ctypes.c_int64), ("dv_st", ctypes.c_int64),
        ("dsinks", ctypes.c_void_p),
        ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
        ("keep", ctypes.c_void_p), ("m_sb", ctypes.c_int64), ("m_sh", ctypes.c_int64), ("m_st", ctypes.c_int64),
        ("p_drop", ctypes.c_float),
    ]


class AttnSparseBwdArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("Sq", ctypes.c_int32), ("Hq", ctypes.c_int32), ("N", ctypes.c_int32),
        ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32), ("topk", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("q_ss", ctypes.c_int64), ("q_sh", ctypes.c_int64),
        ("kv", ctypes.c_void_p), ("kv_sn", ctypes.c_int64),
        ("indices", ctypes.c_void_p), ("idx_ss", ctypes.c_int64),
        ("out", ctypes.c_void_p), ("o_ss", ctypes.c_int64), ("o_sh", ctypes.c_int64),
        ("dout", ctypes.c_void_p), ("do_ss", ctypes.c_int64), ("do_sh", ctypes.c_int64),
        ("lse", ctypes.c_void_p),
        ("sinks", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dq_ss", ctypes.c_int64), ("dq_sh", ctypes.c_int64),
        ("dkv", ctypes.c_void_p), ("dkv_sn", ctypes.c_int64),
        ("dsinks", ctypes.c_void_p),
    ]


class AttnSparseFp8Args(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("Sq", ctypes.c_int32), ("Hq", ctypes.c_int32), ("N", ctypes.c_int32), ("d", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("q_ss", ctypes.c_int64), ("q_sh", ctypes.c_int64),
        ("codes", ctypes.c_void_p), ("c_sn", ctypes.c_int64),
        ("scales", ctypes.c_void_p), ("s_sn", ctypes.c_int64),
        ("indices", ctypes.c_void_p), ("idx_ss", ctypes.c_int64),
        ("out", ctypes.c_void_p), ("o_ss", ctypes.c_int64), ("o_sh", ctypes.c_int64),
        ("lse", ctypes.c_void_p),
        ("sinks", ctypes.c_void_p),
    ]


EXPORTS = (
    "attn_abi_version", "attn_fwd_dense", "attn_fwd_sparse_topk", "attn_plan_dense",
    "attn_plan_sparse_topk", "attn_status_string", "attn_last_error", "attn_dispatch_count",
    "attn_reset_dispatch_counts", "attn_budget_tile_rows", "attn_fwd_dense_splitkv",
    "attn_splitkv_workspace_bytes", "attn_splitkv_choose", "attn_bwd_dense", "attn_bwd_dense_workspace_bytes",
    "attn_fwd_dense_qkv", "attn_qkv_workspace_bytes", "attn_fwd_varlen", "attn_bwd_sparse_topk",
    "attn_bwd_sparse_workspace_bytes", "attn_fwd_dense_extras", "attn_fwd_sparse_fp8",
    "attn_sparse_fp8_workspace_bytes", "attn_fwd_dense_splitkv_noalloc",
)
ATTN_KV_Q4_0, ATTN_KV_Q8_0 = 2, 8
KV_FORMATS = {"q8_0": ATTN_KV_Q8_0, "q4_0": ATTN_KV_Q4_0}


class AttnVarlenArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("max_seqlen_q", ctypes.c_int32),
        ("total_q", ctypes.c_int32), ("total_k", ctypes.c_int32), ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("q_st", ctypes.c_int64), ("q_sh", ctypes.c_int64),
        ("k", ctypes.c_void_p), ("k_st", ctypes.c_int64), ("k_sh", ctypes.c_int64),
        ("v", ctypes.c_void_p), ("v_st", ctypes.c_int64), ("v_sh", ctypes.c_int64),
        ("out", ctypes.c_void_p), ("o_st", ctypes.c_int64), ("o_sh", ctypes.c_int64),
        ("lse", ctypes.c_void_p),
        ("sinks", ctypes.c_void_p),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("cu_seqlens_k", ctypes.c_void_p),
        ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
    ]


class AttnQkvArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("kv_format", ctypes.c_int32),
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Tq", ctypes.c_int32), ("Tk", ctypes.c_int32), ("d", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("q_sb", ctypes.c_int64), ("q_sh", ctypes.c_int64), ("q_st", ctypes.c_int64),
        ("k", ctypes.c_void_p), ("k_sb", ctypes.c_int64), ("k_sh", ctypes.c_int64), ("k_st", ctypes.c_int64),
        ("v", ctypes.c_void_p), ("v_sb", ctypes.c_int64), ("v_sh", ctypes.c_int64), ("v_st", ctypes.c_int64),
        ("out", ctypes.c_void_p), ("o_sb", ctypes.c_int64), ("o_sh", ctypes.c_int64), ("o_st", ctypes.c_int64),
        ("lse", ctypes.c_void_p),
        ("sinks", ctypes.c_void_p),
    ]

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libattn_fwd.so (built by attention_forward_attn_amd.build). Raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m attention_forward_attn_amd.build` "
            "(there is no fallback path)")
    lib = ctypes.CDLL(path)
    lib.attn_abi_version.restype = ctypes.c_int
    lib.attn_fwd_dense.argtypes = [ctypes.POINTER(AttnDenseArgs), ctypes.c_void_p]
    lib.attn_fwd_dense.restype = ctypes.c_int
    lib.attn_fwd_sparse_topk.argtypes = [ctypes.POINTER(AttnSparseArgs), ctypes.c_void_p]
    lib.attn_fwd_sparse_topk.restype = ctypes.c_int
    lib.attn_plan_dense.argtypes = [ctypes.POINTER(AttnDenseArgs), ctypes.POINTER(AttnPlan)]
    lib.attn_plan_dense.restype = ctypes.c_int
    lib.attn_plan_sparse_topk.argtypes = [ctypes.POINTER(AttnSparseArgs), ctypes.POINTER(AttnPlan)]
    lib.attn_plan_sparse_topk.restype = ctypes.c_int
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_dispatch_count.argtypes = [ctypes.c_char_p]
    lib.attn_dispatch_count.restype = ctypes.c_uint64
    lib.attn_reset_dispatch_counts.restype = None
    lib.attn_budget_tile_rows.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
    lib.attn_budget_tile_rows.restype = ctypes.c_int64
    lib.attn_fwd_dense_splitkv.argtypes = [ctypes.POINTER(AttnDenseArgs), ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.c_int64, ctypes.c_void_p]
    lib.attn_fwd_dense_splitkv.restype = ctypes.c_int
    lib.attn_fwd_dense_splitkv_noalloc.argtypes = [ctypes.POINTER(AttnDenseArgs), ctypes.c_int32, ctypes.c_void_p]
    lib.attn_fwd_dense_splitkv_noalloc.restype = ctypes.c_int
    lib.attn_splitkv_workspace_bytes.argtypes = [ctypes.POINTER(AttnDenseArgs), ctypes.c_int32]
    lib.attn_splitkv_workspace_bytes.restype = ctypes.c_int64
    lib.attn_splitkv_choose.argtypes = [ctypes.POINTER(AttnDenseArgs)]
    lib.attn_splitkv_choose.restype = ctypes.c_int32
    lib.attn_bwd_dense.argtypes = [ctypes.POINTER(AttnDenseBwdArgs), ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.attn_bwd_dense.restype = ctypes.c_int
    lib.attn_bwd_dense_workspace_bytes.argtypes = [ctypes.POINTER(AttnDenseBwdArgs)]
    lib.attn_bwd_dense_workspace_bytes.restype = ctypes.c_int64
    lib.attn_fwd_dense_qkv.argtypes = [ctypes.POINTER(AttnQkvArgs), ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_void_p]
    lib.attn_fwd_dense_qkv.restype = ctypes.c_int
    lib.attn_qkv_workspace_bytes.argtypes = [ctypes.POINTER(AttnQkvArgs), ctypes.c_int32]
    lib.attn_qkv_workspace_bytes.restype = ctypes.c_int64
    lib.attn_fwd_varlen.argtypes = [ctypes.POINTER(AttnVarlenArgs), ctypes.c_void_p]
    lib.attn_fwd_varlen.restype = ctypes.c_int
    lib.attn_bwd_sparse_topk.argtypes = [ctypes.POINTER(AttnSparseBwdArgs), ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_void_p]
    lib.attn_bwd_sparse_topk.restype = ctypes.c_int
    lib.attn_bwd_sparse_workspace_bytes.argtypes = [ctypes.POINTER(AttnSparseBwdArgs)]
    lib.attn_bwd_sparse_workspace_bytes.restype = ctypes.c_int64
    lib.attn_fwd_dense_extras.argtypes = [ctypes.POINTER(AttnDenseArgs), ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.attn_fwd_dense_extras.restype = ctypes.c_int
    lib.attn_fwd_sparse_fp8.argtypes = [ctypes.POINTER(AttnSparseFp8Args), ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_void_p]
    lib.attn_fwd_sparse_fp8.restype = ctypes.c_int
    lib.attn_sparse_fp8_workspace_bytes.argtypes = [ctypes.POINTER(AttnSparseFp8Args), ctypes.c_int32]
    lib.attn_sparse_fp8_workspace_bytes.restype = ctypes.c_int64
    v = lib.attn_abi_version()
    if v != ABI_VERSION:
        raise RuntimeError(f"libattn_fwd.so ABI version {v}, binding expects {ABI_VERSION}")
    _lib = lib
    return lib


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class AttnInvalidArgument(AttnError, ValueError):
    pass


class AttnUnsupported(AttnError, NotImplementedError):
    pass


def _check(status: int):
    if status == ATTN_OK:
        return
    lib = load_library()
    msg = f"{lib.attn_status_string(status).decode()}: {lib.attn_last_error().decode()}"
    if status == ATTN_INVALID_ARGUMENT:
        raise AttnInvalidArgument(status, msg)
    if status == ATTN_UNSUPPORTED:
        raise AttnUnsupported(status, msg)
    raise AttnError(status, msg)


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise AttnUnsupported(ATTN_UNSUPPORTED, f"unsupported dtype {t.dtype}")


def _stream_handle(stream) -> int:
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _bad(msg: str):
    raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT, msg)


def _expect(t, name: str, shape=None, dtype=None, contiguous: bool = False):
    """A tensor argument: its shape (None entries are free), dtype and layout.
    The C library sees only pointers and sizes, so a tensor that does not match
    the sizes taken from the others would be read or written out of bounds."""
    if t is None:
        _bad(f"{name} is required")
    if shape is not None:
        if t.dim() != len(shape) or any(s is not None and int(t.shape[i]) != int(s) for i, s in enumerate(shape)):
            want = "[" + ", ".join("*" if s is None else str(int(s)) for s in shape) + "]"
            _bad(f"{name} must have shape {want}, got {list(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        _bad(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        _bad(f"{name} must be contiguous")
    if t.dim() > 0 and t.numel() > 0 and t.stride(-1) != 1:
        _bad(f"{name}: last dimension must be contiguous")


def _on_device(**tensors):
    """Every given tensor lives on one GPU (a host tensor would hand the kernels a
    host pointer)."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            _bad(f"{name} must be a GPU tensor, got one on {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            _bad(f"{name} is on {t.device}, the other tensors on {dev}")


def _check_dense(q, k, v, out, lse, sinks, q_rope=None, k_rope=None, device=True):
    """Shapes, dtypes and devices of a dense call: q [B,H,Tq,d], k [B,Hkv,Tk,d],
    v [B,Hkv,Tk,d_v], out [B,H,Tq,d_v] in q's dtype, lse fp32 [B,H,Tq] contiguous,
    sinks fp32 [H] contiguous."""
    import torch

    _expect(q, "q", (None, None, None, None))
    B, H, Tq, dqk = q.shape
    _expect(k, "k", (B, None, None, dqk), q.dtype)
    Hkv, Tk = k.shape[1], k.shape[2]
    _expect(v, "v", (B, Hkv, Tk, None), q.dtype)
    _expect(out, "out", (B, H, Tq, v.shape[-1]), q.dtype)
    _expect(lse, "lse", (B, H, Tq), torch.float32, contiguous=True)
    if sinks is not None:
        _expect(sinks, "sinks", (H,), torch.float32, contiguous=True)
    if device:
        _on_device(q=q, k=k, v=v, out=out, lse=lse, sinks=sinks, q_rope=q_rope, k_rope=k_rope)


def _set_keep(a, keep, p_drop: float, B: int, H: int, Tq: int, Tk: int):
    """Dropout fields: ``keep`` int32 [B,H,Tq,ceil(Tk/32)] bit-packed keep mask (bit i
    of word w = key 32 w + i, as ``synth.pack_keep`` writes), or None."""
    if keep is None:
        return
    import torch

    if keep.dtype != torch.int32 or keep.dim() != 4 or tuple(keep.shape[:3]) != (B, H, Tq) or keep.stride(-1) != 1 \
            or keep.shape[3] < (Tk + 31) // 32:
        raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT, "keep must be int32 [B, H, Tq, ceil(Tk/32)] (bit-packed)")
    _on_device(keep=keep)
    a.keep, (a.m_sb, a.m_sh, a.m_st) = keep.data_ptr(), keep.stride()[:3]
    a.p_drop = float(p_drop)


def dense_args(q, k, v, out, lse, *, causal: bool, scale: float, sinks=None,
               window: Tuple[int, int] = (-1, -1), q_rope=None, k_rope=None, keep=None,
               p_drop: float = 0.0) -> AttnDenseArgs:
    """Fill the C argument struct from tensors (BHSD or any strided view with unit last stride).

    With ``q_rope`` [B,H,Tq,r] and ``k_rope`` [B,Hkv,Tk,r] the query and key rows are
    [q || q_rope] and [k || k_rope] (d_qk = q's width + r), read in place; a rope key
    shared by the kv heads is passed as an expanded view (head stride 0)."""
    _check_dense(q, k, v, out, lse, sinks, q_rope, k_rope)
    B, H, Tq, dqk = q.shape
    _, Hkv, Tk, _ = k.shape
    dv = v.shape[-1]
    rope = 0
    if q_rope is not None or k_rope is not None:
        if q_rope is None or k_rope is None:
            raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT, "q_rope and k_rope go together")
        rope = q_rope.shape[-1]
        if (tuple(q_rope.shape) != (B, H, Tq, rope) or tuple(k_rope.shape) != (B, Hkv, Tk, rope)
                or k.shape[-1] != dqk or q_rope.stride(-1) != 1 or k_rope.stride(-1) != 1
                or q_rope.dtype != q.dtype or k_rope.dtype != q.dtype):
            raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT,
                                      "q_rope [B,H,Tq,r] and k_rope [B,Hkv,Tk,r] with unit last stride, q's dtype")
        dqk += rope
    a = AttnDenseArgs()
    a.struct_size = ctypes.sizeof(AttnDenseArgs)
    a.dtype = _dtype_code(q)
    a.B, a.H, a.Hkv, a.Tq, a.Tk, a.d_qk, a.d_v = B, H, Hkv, Tq, Tk, dqk, dv
    a.causal = 1 if causal else 0
    a.scale = float(scale)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.stride(-1) != 1:
            raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT, f"{name}: last dimension must be contiguous")
    a.q, (a.q_sb, a.q_sh, a.q_st) = q.data_ptr(), q.stride()[:3]
    a.k, (a.k_sb, a.k_sh, a.k_st) = k.data_ptr(), k.stride()[:3]
    a.v, (a.v_sb, a.v_sh, a.v_st) = v.data_ptr(), v.stride()[:3]
    a.out, (a.o_sb, a.o_sh, a.o_st) = out.data_ptr(), out.stride()[:3]
    a.lse = lse.data_ptr()
    a.sinks = sinks.data_ptr() if sinks is not None else None
    a.window_left, a.window_right = int(window[0]), int(window[1])
    _set_keep(a, keep, p_drop, B, H, Tq, Tk)
    a.rope_dim = rope
    if rope:
        a.q_rope, (a.qr_sb, a.qr_sh, a.qr_st) = q_rope.data_ptr(), q_rope.stride()[:3]
        a.k_rope, (a.kr_sb, a.kr_sh, a.kr_st) = k_rope.data_ptr(), k_rope.stride()[:3]
    return a


def dense(q, k, v, *, causal: bool = True, scale: Optional[float] = None, sinks=None,
          out=None, lse=None, stream=None, window: Tuple[int, int] = (-1, -1), q_rope=None,
          k_rope=None, keep=None, p_drop: float = 0.0) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """Fused dense attention forward on the GPU.

    q [B,H,Tq,d_qk], k [B,Hkv,Tk,d_qk], v [B,Hkv,Tk,d_v] (bf16, or fp32 for the
    split-bf16 path), sinks [H] fp32 or None. ``window`` = (left, right) keys
    around each row's diagonal position t + Tk - Tq (-1: unbounded; bf16 only;
    it never widens the causal mask). ``q_rope``/``k_rope``: MLA's rope parts
    read in place (see :func:`dense_args`). ``keep``/``p_drop``: attention dropout with
    the caller's bit-packed keep mask (pass the same mask to :func:`dense_backward`).
    Returns (out [B,H,Tq,d_v] in the input
    dtype, lse [B,H,Tq] fp32). Launches on ``stream`` (default: torch's current
    stream) and does not synchronise.
    """
    import torch

    lib = load_library()
    _expect(q, "q", (None, None, None, None))
    _expect(v, "v", (None, None, None, None))
    B, H, Tq, dqk = q.shape
    dv = v.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(dqk + (q_rope.shape[-1] if q_rope is not None else 0))
    if out is None:
        out = torch.empty((B, H, Tq, dv), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Tq), dtype=torch.float32, device=q.device)
    a = dense_args(q, k, v, out, lse, causal=causal, scale=scale, sinks=sinks, window=window, q_rope=q_rope,
                   k_rope=k_rope, keep=keep, p_drop=p_drop)
    _check(lib.attn_fwd_dense(ctypes.byref(a), ctypes.c_void_p(_stream_handle(stream))))
    return out, lse


def dense_extras(q, k, v, out, lse, *, causal: bool = True, scale: Optional[float] = None, sinks=None,
                 window: Tuple[int, int] = (-1, -1), want_p: bool = True, want_row_max: bool = True, p=None,
                 row_max=None, stream=None):
    """The forward's extra returns after :func:`dense` on the same arguments (``lse``
    is the forward's, read): (p [B,H,Tq,Tk] fp32 or None, row_max [B,H,Tq] fp32 or
    None). p = exp(scale q.k - lse) on visible keys, 0 elsewhere; row_max = the
    largest visible scaled score (-inf without keys)."""
    import torch

    lib = load_library()
    _expect(q, "q", (None, None, None, None))
    _expect(v, "v", (None, None, None, None))
    B, H, Tq, dqk = q.shape
    Tk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if want_p and p is None:
        p = torch.empty((B, H, Tq, Tk), dtype=torch.float32, device=q.device)
    if want_row_max and row_max is None:
        row_max = torch.empty((B, H, Tq), dtype=torch.float32, device=q.device)
    if p is not None and (p.dtype != torch.float32 or tuple(p.shape) != (B, H, Tq, Tk) or p.stride(-1) != 1):
        raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT, "p must be fp32 [B, H, Tq, Tk] with a contiguous last dim")
    if row_max is not None and (row_max.dtype != torch.float32 or tuple(row_max.shape) != (B, H, Tq)
                                or not row_max.is_contiguous()):
        raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT, "row_max must be contiguous fp32 [B, H, Tq]")
    a = dense_args(q, k, v, out, lse, causal=causal, scale=scale, sinks=sinks, window=window)
    ps = p.stride()[:3] if p is not None else (0, 0, 0)
    _check(lib.attn_fwd_dense_extras(ctypes.byref(a), ctypes.c_void_p(p.data_ptr() if p is not None else None),
                                     ps[0], ps[1], ps[2],
                                     ctypes.c_void_p(row_max.data_ptr() if row_max is not None else None),
                                     ctypes.c_void_p(_stream_handle(stream))))
    return p, row_max


def dense_splitkv(q, k, v, *, causal: bool = True, scale: Optional[float] = None, sinks=None,
                  n_splits: int = 0, out=None, lse=None, workspace=None, stream=None,
                  window: Tuple[int, int] = (-1, -1), q_rope=None, k_rope=None):
    """Split-KV dense forward (decode and other few-row shapes): same inputs
    and results as :func:`dense`. The keys are cut into ``n_splits`` ranges
    (0: the library's choice); the fp32 partials go to ``workspace``, a uint8
    device tensor of at least :func:`splitkv_workspace_bytes` bytes (allocated
    here when None). Launches on ``stream`` and does not synchronise.
    """
    import torch

    lib = load_library()
    _expect(q, "q", (None, None, None, None))
    _expect(v, "v", (None, None, None, None))
    B, H, Tq, dqk = q.shape
    dv = v.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(dqk + (q_rope.shape[-1] if q_rope is not None else 0))
    if out is None:
        out = torch.empty((B, H, Tq, dv), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Tq), dtype=torch.float32, device=q.device)
    a = dense_args(q, k, v, out, lse, causal=causal, scale=scale, sinks=sinks, window=window, q_rope=q_rope,
                   k_rope=k_rope)
    need = int(lib.attn_splitkv_workspace_bytes(ctypes.byref(a), int(n_splits)))
    if need < 0:
        _check(ATTN_INVALID_ARGUMENT)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.attn_fwd_dense_splitkv(ctypes.byref(a), int(n_splits), ctypes.c_void_p(ws_ptr), ws_bytes,
                                      ctypes.c_void_p(_stream_handle(stream))))
    return out, lse


def dense_splitkv_noalloc(q, k, v, out, lse, *, causal: bool = True, scale: Optional[float] = None, sinks=None,
                          n_splits: int = 0, stream=None, window: Tuple[int, int] = (-1, -1)):
    """:func:`dense_splitkv` for callers that cannot allocate: ``out`` [B,H,Tq,d_v] and
    ``lse`` [B,H,Tq] fp32 are the caller's, and the partials go to the library's
    per-device scratch array (``NOALLOC_SCRATCH_BYTES``) instead of a workspace.
    Neither this function nor the library allocates. Calls that overlap on one
    device share that array and must be ordered by the caller. A plan whose
    partials exceed the array raises AttnInvalidArgument (ask for fewer ranges)."""
    lib = load_library()
    _expect(q, "q", (None, None, None, None))
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    a = dense_args(q, k, v, out, lse, causal=causal, scale=scale, sinks=sinks, window=window)
    _check(lib.attn_fwd_dense_splitkv_noalloc(ctypes.byref(a), int(n_splits), ctypes.c_void_p(_stream_handle(stream))))
    return out, lse


def _shape_args(B, H, Hkv, Tq, Tk, d_qk, d_v, dtype, causal, sinks, scale) -> AttnDenseArgs:
    a = AttnDenseArgs()
    a.struct_size = ctypes.sizeof(AttnDenseArgs)
    a.dtype = ATTN_BF16 if dtype == "bf16" else ATTN_F32
    a.B, a.H, a.Hkv, a.Tq, a.Tk, a.d_qk, a.d_v = B, H, Hkv, Tq, Tk, d_qk, d_v
    a.causal = 1 if causal else 0
    a.scale = float(scale if scale is not None else 1.0 / math.sqrt(d_qk))
    a.q, a.q_sb, a.q_sh, a.q_st = _FAKE_PTR, H * Tq * d_qk, Tq * d_qk, d_qk
    a.k, a.k_sb, a.k_sh, a.k_st = _FAKE_PTR, Hkv * Tk * d_qk, Tk * d_qk, d_qk
    a.v, a.v_sb, a.v_sh, a.v_st = _FAKE_PTR, Hkv * Tk * d_v, Tk * d_v, d_v
    a.out, a.o_sb, a.o_sh, a.o_st = _FAKE_PTR, H * Tq * d_v, Tq * d_v, d_v
    a.lse = _FAKE_PTR
    a.sinks = _FAKE_PTR if sinks else None
    a.window_left = a.window_right = -1
    return a


def splitkv_workspace_bytes(B, H, Hkv, Tq, Tk, d_qk, d_v, *, n_splits: int = 0, dtype: str = "bf16",
                            causal: bool = True, sinks: bool = False, scale: Optional[float] = None) -> int:
    """Workspace bytes of a contiguous BHSD split-KV call (host only); 0 when one range suffices."""
    a = _shape_args(B, H, Hkv, Tq, Tk, d_qk, d_v, dtype, causal, sinks, scale)
    n = int(load_library().attn_splitkv_workspace_bytes(ctypes.byref(a), int(n_splits)))
    if n < 0:
        _check(ATTN_INVALID_ARGUMENT)
    return n


def splitkv_choose(B, H, Hkv, Tq, Tk, d_qk, d_v, *, dtype: str = "bf16", causal: bool = True,
                   sinks: bool = False, scale: Optional[float] = None) -> int:
    """Key ranges the library picks for this shape on the current device (host only)."""
    a = _shape_args(B, H, Hkv, Tq, Tk, d_qk, d_v, dtype, causal, sinks, scale)
    n = int(load_library().attn_splitkv_choose(ctypes.byref(a)))
    if n < 0:
        _check(ATTN_INVALID_ARGUMENT)
    return n


def _check_sparse(q, kv, idx, out, lse, sinks, d_v: int, device=True):
    """q [Sq,Hq,d_qk], kv [N,>=d_qk] in q's dtype, idx int32 [Sq,topk],
    out [Sq,Hq,d_v], lse fp32 [Sq,Hq] contiguous, sinks fp32 [Hq] contiguous."""
    import torch

    _expect(q, "q", (None, None, None))
    Sq, Hq, dqk = q.shape
    _expect(kv, "kv", (None, None), q.dtype)
    if kv.shape[1] < dqk:
        _bad(f"kv rows hold {kv.shape[1]} values, q rows {dqk}")
    _expect(idx, "indices", (Sq, None), torch.int32)
    _expect(out, "out", (Sq, Hq, d_v), q.dtype)
    _expect(lse, "lse", (Sq, Hq), torch.float32, contiguous=True)
    if sinks is not None:
        _expect(sinks, "sinks", (Hq,), torch.float32, contiguous=True)
    if device:
        _on_device(q=q, kv=kv, indices=idx, out=out, lse=lse, sinks=sinks)


def sparse_args(q, kv, idx, out, lse, *, d_v: int, scale: float, sinks=None) -> AttnSparseArgs:
    _check_sparse(q, kv, idx, out, lse, sinks, d_v)
    Sq, Hq, dqk = q.shape
    N = kv.shape[0]
    a = AttnSparseArgs()
    a.struct_size = ctypes.sizeof(AttnSparseArgs)
    a.dtype = _dtype_code(q)
    a.Sq, a.Hq, a.N, a.d_qk, a.d_v, a.topk = Sq, Hq, N, dqk, d_v, idx.shape[1]
    a.scale = float(scale)
    for name, t in (("q", q), ("kv", kv), ("indices", idx), ("out", out)):
        if t.stride(-1) != 1:
            raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT, f"{name}: last dimension must be contiguous")
    a.q, (a.q_ss, a.q_sh) = q.data_ptr(), q.stride()[:2]
    a.kv, a.kv_sn = kv.data_ptr(), kv.stride(0)
    a.indices, a.idx_ss = idx.data_ptr(), idx.stride(0)
    a.out, (a.o_ss, a.o_sh) = out.data_ptr(), out.stride()[:2]
    a.lse = lse.data_ptr()
    a.sinks = sinks.data_ptr() if sinks is not None else None
    return a


def sparse_topk(q, kv, idx, *, d_v: Optional[int] = None, scale: Optional[float] = None, sinks=None,
                out=None, lse=None, stream=None):
    """Sparse top-k attention forward on the GPU.

    q [Sq,Hq,d_qk] bf16, kv [N,d_qk] bf16 (one pool; values = kv[:, :d_v]),
    idx [Sq,topk] int32 (entries outside [0, N) skipped). Returns
    (out [Sq,Hq,d_v] bf16, lse [Sq,Hq] fp32).
    """
    import torch

    lib = load_library()
    Sq, Hq, dqk = q.shape
    d_v = dqk if d_v is None else d_v
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if idx.dtype != torch.int32:
        raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT, "indices must be int32")
    if out is None:
        out = torch.empty((Sq, Hq, d_v), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((Sq, Hq), dtype=torch.float32, device=q.device)
    a = sparse_args(q, kv, idx, out, lse, d_v=d_v, scale=scale, sinks=sinks)
    _check(lib.attn_fwd_sparse_topk(ctypes.byref(a), ctypes.c_void_p(_stream_handle(stream))))
    return out, lse


def sparse_backward(q, kv, idx, out, dout, lse, *, d_v: Optional[int] = None, scale: Optional[float] = None,
                    sinks=None, dq=None, dkv=None, dsinks=None, workspace=None, stream=None):
    """Sparse top-k backward: q [Sq,Hq,d], kv [N,d], idx [Sq,topk] int32 as in
    :func:`sparse_topk`, the forward's out and lse, dout = dL/dO. Returns
    (dq [Sq,Hq,d] bf16, dkv [N,d] fp32 -- the pool's gradient, key and value
    roles summed, overwritten --, dsinks [Hq] fp32 or None). ``workspace``: a
    uint8 device tensor of at least the library's workspace size (allocated here
    when None). Launches on ``stream`` and does not synchronise."""
    import torch

    lib = load_library()
    Sq, Hq, dqk = q.shape
    N = kv.shape[0]
    d_v = dqk if d_v is None else d_v
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if idx.dtype != torch.int32:
        raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT, "indices must be int32")
    if dq is None:
        dq = torch.empty_like(q)
    if dkv is None:
        dkv = torch.empty((N, dqk), dtype=torch.float32, device=q.device)
    if sinks is not None and dsinks is None:
        dsinks = torch.empty_like(sinks)
    _check_sparse(q, kv, idx, out, lse, sinks, d_v, device=False)
    _expect(dout, "dout", tuple(out.shape), out.dtype)
    _expect(dq, "dq", tuple(q.shape), q.dtype)
    _expect(dkv, "dkv", (N, dqk), torch.float32)
    if dsinks is not None:
        _expect(dsinks, "dsinks", (Hq,), torch.float32, contiguous=True)
    _on_device(q=q, kv=kv, indices=idx, out=out, lse=lse, sinks=sinks, dout=dout, dq=dq, dkv=dkv, dsinks=dsinks)
    a = AttnSparseBwdArgs()
    a.struct_size = ctypes.sizeof(AttnSparseBwdArgs)
    a.dtype = _dtype_code(q)
    a.Sq, a.Hq, a.N, a.d_qk, a.d_v, a.topk = Sq, Hq, N, dqk, d_v, idx.shape[1]
    a.scale = float(scale)
    a.q, (a.q_ss, a.q_sh) = q.data_ptr(), q.stride()[:2]
    a.kv, a.kv_sn = kv.data_ptr(), kv.stride(0)
    a.indices, a.idx_ss = idx.data_ptr(), idx.stride(0)
    a.out, (a.o_ss, a.o_sh) = out.data_ptr(), out.stride()[:2]
    a.dout, (a.do_ss, a.do_sh) = dout.data_ptr(), dout.stride()[:2]
    a.lse = lse.data_ptr()
    a.sinks = sinks.data_ptr() if sinks is not None else None
    a.dq, (a.dq_ss, a.dq_sh) = dq.data_ptr(), dq.stride()[:2]
    a.dkv, a.dkv_sn = dkv.data_ptr(), dkv.stride(0)
    a.dsinks = dsinks.data_ptr() if dsinks is not None else None
    need = int(lib.attn_bwd_sparse_workspace_bytes(ctypes.byref(a)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.attn_bwd_sparse_topk(ctypes.byref(a), ctypes.c_void_p(ws_ptr), ws_bytes,
                                    ctypes.c_void_p(_stream_handle(stream))))
    return dq, dkv, dsinks


def sparse_fp8(q, codes, scales, idx, *, scale: Optional[float] = None, sinks=None, n_splits: int = 0, out=None,
               lse=None, workspace=None, stream=None):
    """Sparse top-k decode over an fp8 pool: q [Sq,Hq,512] bf16, codes [N,512] uint8
    (OCP E4M3), scales [N,4] fp32 (one per 128 columns), idx [Sq,topk] int32. Returns
    (out [Sq,Hq,512] bf16, lse [Sq,Hq] fp32), the sparse forward over the decoded pool."""
    import torch

    lib = load_library()
    Sq, Hq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if idx.dtype != torch.int32 or codes.dtype != torch.uint8 or scales.dtype != torch.float32:
        raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT, "idx int32, codes uint8, scales fp32")
    if out is None:
        out = torch.empty((Sq, Hq, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((Sq, Hq), dtype=torch.float32, device=q.device)
    _expect(q, "q", (Sq, Hq, d), torch.bfloat16)
    _expect(codes, "codes", (None, d))
    N = codes.shape[0]
    _expect(scales, "scales", (N, d // 128))
    _expect(idx, "indices", (Sq, None))
    _expect(out, "out", (Sq, Hq, d), torch.bfloat16)
    _expect(lse, "lse", (Sq, Hq), torch.float32, contiguous=True)
    if sinks is not None:
        _expect(sinks, "sinks", (Hq,), torch.float32, contiguous=True)
    _on_device(q=q, codes=codes, scales=scales, indices=idx, out=out, lse=lse, sinks=sinks)
    a = AttnSparseFp8Args()
    a.struct_size = ctypes.sizeof(AttnSparseFp8Args)
    a.Sq, a.Hq, a.N, a.d, a.topk = Sq, Hq, codes.shape[0], d, idx.shape[1]
    a.scale = float(scale)
    a.q, (a.q_ss, a.q_sh) = q.data_ptr(), q.stride()[:2]
    a.codes, a.c_sn = codes.data_ptr(), codes.stride(0)
    a.scales, a.s_sn = scales.data_ptr(), scales.stride(0)
    a.indices, a.idx_ss = idx.data_ptr(), idx.stride(0)
    a.out, (a.o_ss, a.o_sh) = out.data_ptr(), out.stride()[:2]
    a.lse = lse.data_ptr()
    a.sinks = sinks.data_ptr() if sinks is not None else None
    need = int(lib.attn_sparse_fp8_workspace_bytes(ctypes.byref(a), int(n_splits)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.attn_fwd_sparse_fp8(ctypes.byref(a), int(n_splits), ctypes.c_void_p(ws_ptr), ws_bytes,
                                   ctypes.c_void_p(_stream_handle(stream))))
    return out, lse


def sparse_fp8_workspace_bytes(Sq: int, Hq: int, N: int, d: int, topk: int, n_splits: int = 0) -> int:
    """Workspace bytes of :func:`sparse_fp8` for these sizes (host only)."""
    a = AttnSparseFp8Args()
    a.struct_size = ctypes.sizeof(AttnSparseFp8Args)
    a.Sq, a.Hq, a.N, a.d, a.topk = Sq, Hq, N, d, topk
    a.scale = 1.0 / math.sqrt(d)
    n = int(load_library().attn_sparse_fp8_workspace_bytes(ctypes.byref(a), int(n_splits)))
    if n < 0:
        _check(ATTN_INVALID_ARGUMENT)
    return n


_FAKE_PTR = 1 << 12  # never dereferenced: plans are computed on the host only


def _plan_to_dict(p: AttnPlan) -> dict:
    return {f: (getattr(p, f).decode() if f == "path" else getattr(p, f)) for f, _ in AttnPlan._fields_
            if f != "struct_size"}


def plan_dense(B, H, Hkv, Tq, Tk, d_qk, d_v, *, dtype: str = "bf16", causal: bool = True,
               sinks: bool = False, scale: Optional[float] = None) -> dict:
    """The launch plan for a contiguous BHSD problem of this shape (host only)."""
    lib = load_library()
    a = _shape_args(B, H, Hkv, Tq, Tk, d_qk, d_v, dtype, causal, sinks, scale)
    p = AttnPlan()
    p.struct_size = ctypes.sizeof(AttnPlan)
    _check(lib.attn_plan_dense(ctypes.byref(a), ctypes.byref(p)))
    return _plan_to_dict(p)


def plan_sparse_topk(Sq, Hq, N, d_qk, d_v, topk, *, scale: Optional[float] = None) -> dict:
    lib = load_library()
    a = AttnSparseArgs()
    a.struct_size = ctypes.sizeof(AttnSparseArgs)
    a.dtype = ATTN_BF16
    a.Sq, a.Hq, a.N, a.d_qk, a.d_v, a.topk = Sq, Hq, N, d_qk, d_v, topk
    a.scale = float(scale if scale is not None else 1.0 / math.sqrt(d_qk))
    a.q, a.q_ss, a.q_sh = _FAKE_PTR, Hq * d_qk, d_qk
    a.kv, a.kv_sn = _FAKE_PTR, d_qk
    a.indices, a.idx_ss = _FAKE_PTR, topk
    a.out, a.o_ss, a.o_sh = _FAKE_PTR, Hq * d_v, d_v
    a.lse = _FAKE_PTR
    p = AttnPlan()
    p.struct_size = ctypes.sizeof(AttnPlan)
    _check(lib.attn_plan_sparse_topk(ctypes.byref(a), ctypes.byref(p)))
    return _plan_to_dict(p)


def dispatch_count(path: str) -> int:
    return int(load_library().attn_dispatch_count(path.encode()))


def reset_dispatch_counts() -> None:
    load_library().attn_reset_dispatch_counts()


def budget_tile_rows(budget_bytes: int, Tk: int, elt_bytes: int) -> int:
    return int(load_library().attn_budget_tile_rows(budget_bytes, Tk, elt_bytes))


def abi_version() -> int:
    return int(load_library().attn_abi_version())


def dense_bwd_args(q, k, v, out, dout, lse, dq, dk, dv, *, causal: bool, scale: float, sinks=None,
                   dsinks=None, window: Tuple[int, int] = (-1, -1), keep=None, p_drop: float = 0.0) -> AttnDenseBwdArgs:
    """Fill the backward's C argument struct from tensors (unit last stride)."""
    import torch

    _check_dense(q, k, v, out, lse, sinks, device=False)
    _expect(dout, "dout", tuple(out.shape), q.dtype)
    _expect(dq, "dq", tuple(q.shape), q.dtype)
    _expect(dk, "dk", tuple(k.shape), q.dtype)
    _expect(dv, "dv", tuple(v.shape), q.dtype)
    if dsinks is not None:
        _expect(dsinks, "dsinks", (q.shape[1],), torch.float32, contiguous=True)
    _on_device(q=q, k=k, v=v, out=out, lse=lse, sinks=sinks, dout=dout, dq=dq, dk=dk, dv=dv, dsinks=dsinks)
    B, H, Tq, dqk = q.shape
    _, Hkv, Tk, _ = k.shape
    a = AttnDenseBwdArgs()
    a.struct_size = ctypes.sizeof(AttnDenseBwdArgs)
    a.dtype = _dtype_code(q)
    a.B, a.H, a.Hkv, a.Tq, a.Tk, a.d_qk, a.d_v = B, H, Hkv, Tq, Tk, dqk, v.shape[-1]
    a.causal = 1 if causal else 0
    a.scale = float(scale)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        if t.stride(-1) != 1:
            raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT, f"{name}: last dimension must be contiguous")
    a.q, (a.q_sb, a.q_sh, a.q_st) = q.data_ptr(), q.stride()[:3]
    a.k, (a.k_sb, a.k_sh, a.k_st) = k.data_ptr(), k.stride()[:3]
    a.v, (a.v_sb, a.v_sh, a.v_st) = v.data_ptr(), v.stride()[:3]
    a.out, (a.o_sb, a.o_sh, a.o_st) = out.data_ptr(), out.stride()[:3]
    a.dout, (a.do_sb, a.do_sh, a.do_st) = dout.data_ptr(), dout.stride()[:3]
    a.dq, (a.dq_sb, a.dq_sh, a.dq_st) = dq.data_ptr(), dq.stride()[:3]
    a.dk, (a.dk_sb, a.dk_sh, a.dk_st) = dk.data_ptr(), dk.stride()[:3]
    a.dv, (a.dv_sb, a.dv_sh, a.dv_st) = dv.data_ptr(), dv.stride()[:3]
    a.lse = lse.data_ptr()
    a.sinks = sinks.data_ptr() if sinks is not None else None
    a.dsinks = dsinks.data_ptr() if dsinks is not None else None
    a.window_left, a.window_right = int(window[0]), int(window[1])
    _set_keep(a, keep, p_drop, B, H, Tq, Tk)
    return a


def dense_backward(q, k, v, out, dout, lse, *, causal: bool = True, scale: Optional[float] = None, sinks=None,
                   dq=None, dk=None, dv=None, dsinks=None, workspace=None, stream=None,
                   window: Tuple[int, int] = (-1, -1), keep=None, p_drop: float = 0.0):
    """Dense attention backward on the GPU (bf16): returns (dq, dk, dv, dsinks).

    ``out`` and ``lse`` are the forward's results for (q, k, v, sinks); ``dout``
    is dL/dout. dk and dv are summed over the query heads that share each kv
    head. dsinks (fp32 [H]) is computed when ``sinks`` is given, else None.
    ``workspace`` is a uint8 device tensor of at least
    :func:`bwd_workspace_bytes` bytes (allocated here when None). Launches on
    ``stream`` and does not synchronise.
    """
    import torch

    lib = load_library()
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    if dq is None:
        dq = torch.empty_like(q)
    if dk is None:
        dk = torch.empty_like(k)
    if dv is None:
        dv = torch.empty_like(v)
    if sinks is not None:
        if sinks.dtype != torch.float32 or not sinks.is_contiguous():
            raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT, "sinks must be contiguous fp32 [H]")
        if dsinks is None:
            dsinks = torch.empty_like(sinks)
    if not lse.is_contiguous() or lse.dtype != torch.float32:
        raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT, "lse must be contiguous fp32 [B, H, Tq]")
    a = dense_bwd_args(q, k, v, out, dout, lse, dq, dk, dv, causal=causal, scale=scale, sinks=sinks,
                       dsinks=dsinks, window=window, keep=keep, p_drop=p_drop)
    # a negative size means invalid sizes or head dims: the call below then
    # reports the library's own status before launching anything
    need = int(lib.attn_bwd_dense_workspace_bytes(ctypes.byref(a)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.attn_bwd_dense(ctypes.byref(a), ctypes.c_void_p(ws_ptr), ws_bytes,
                              ctypes.c_void_p(_stream_handle(stream))))
    return dq, dk, dv, dsinks


def bwd_workspace_bytes(B, H, Hkv, Tq, Tk, d_qk, d_v) -> int:
    """Workspace bytes of the dense backward for these sizes (host only)."""
    a = AttnDenseBwdArgs()
    a.struct_size = ctypes.sizeof(AttnDenseBwdArgs)
    a.dtype = ATTN_BF16
    a.B, a.H, a.Hkv, a.Tq, a.Tk, a.d_qk, a.d_v = B, H, Hkv, Tq, Tk, d_qk, d_v
    a.causal, a.scale = 1, 1.0 / math.sqrt(d_qk)
    a.window_left = a.window_right = -1
    n = int(load_library().attn_bwd_dense_workspace_bytes(ctypes.byref(a)))
    if n < 0:
        _check(ATTN_INVALID_ARGUMENT)
    return n


def qkv_args(q, k, v, out, lse, *, fmt: str, causal: bool, scale: float, sinks=None) -> AttnQkvArgs:
    """Fill the quantized-cache call's struct: q/out bf16 [B,H,T,d]; k, v uint8
    [B,Hkv,Tk,row bytes] in llama.cpp's ``fmt`` ("q8_0" or "q4_0") blocks."""
    import torch

    _expect(q, "q", (None, None, None, None), torch.bfloat16)
    B, H, Tq, d = q.shape
    _expect(k, "k", (B, None, None, None))
    _, Hkv, Tk, _ = k.shape
    if k.dtype != torch.uint8 or v.dtype != torch.uint8:
        raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT, "k, v must be uint8 block data")
    _expect(v, "v", (B, Hkv, Tk, None))
    _expect(out, "out", (B, H, Tq, d), torch.bfloat16)
    _expect(lse, "lse", (B, H, Tq), torch.float32, contiguous=True)
    if sinks is not None:
        _expect(sinks, "sinks", (H,), torch.float32, contiguous=True)
    if fmt not in KV_FORMATS:
        raise AttnUnsupported(ATTN_UNSUPPORTED, f"kv format {fmt!r}")
    row_bytes = d // 32 * (34 if fmt == "q8_0" else 18)
    if d % 32 != 0 or k.shape[-1] != row_bytes or v.shape[-1] != row_bytes:
        raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT, f"k, v rows must hold {row_bytes} bytes ({fmt}, d={d})")
    _on_device(q=q, k=k, v=v, out=out, lse=lse, sinks=sinks)
    a = AttnQkvArgs()
    a.struct_size = ctypes.sizeof(AttnQkvArgs)
    a.kv_format = KV_FORMATS[fmt]
    a.B, a.H, a.Hkv, a.Tq, a.Tk, a.d = B, H, Hkv, Tq, Tk, d
    a.causal = 1 if causal else 0
    a.scale = float(scale)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.stride(-1) != 1:
            raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT, f"{name}: last dimension must be contiguous")
    a.q, (a.q_sb, a.q_sh, a.q_st) = q.data_ptr(), q.stride()[:3]
    a.k, (a.k_sb, a.k_sh, a.k_st) = k.data_ptr(), k.stride()[:3]
    a.v, (a.v_sb, a.v_sh, a.v_st) = v.data_ptr(), v.stride()[:3]
    a.out, (a.o_sb, a.o_sh, a.o_st) = out.data_ptr(), out.stride()[:3]
    a.lse = lse.data_ptr()
    a.sinks = sinks.data_ptr() if sinks is not None else None
    return a


def dense_qkv(q, k, v, *, fmt: str, causal: bool = True, scale: Optional[float] = None, sinks=None,
              n_splits: int = 0, out=None, lse=None, workspace=None, stream=None):
    """Decode forward over a quantized K/V cache (q8_0 / q4_0 blocks, dequantized
    tile by tile inside the kernel). Same results as :func:`dense` on the
    decoded cache; returns (out bf16 [B,H,Tq,d], lse fp32 [B,H,Tq])."""
    import torch

    lib = load_library()
    B, H, Tq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, Tq, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Tq), dtype=torch.float32, device=q.device)
    if not lse.is_contiguous():
        raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT, "lse must be contiguous")
    a = qkv_args(q, k, v, out, lse, fmt=fmt, causal=causal, scale=scale, sinks=sinks)
    need = int(lib.attn_qkv_workspace_bytes(ctypes.byref(a), int(n_splits)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.attn_fwd_dense_qkv(ctypes.byref(a), int(n_splits), ctypes.c_void_p(ws_ptr), ws_bytes,
                                  ctypes.c_void_p(_stream_handle(stream))))
    return out, lse


def dense_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, *, causal: bool = True,
                 scale: Optional[float] = None, sinks=None, window: Tuple[int, int] = (-1, -1), out=None, lse=None,
                 stream=None):
    """Packed variable-length forward (bf16): q [total_q, H, d_qk], k, v [total_k, Hkv, d],
    cu_seqlens_* int32 device tensors [B + 1]. Returns (out [total_q, H, d_v], lse [H, total_q])."""
    import torch

    lib = load_library()
    total_q, H, dqk = q.shape
    total_k, Hkv, _ = k.shape
    dv = v.shape[-1]
    B = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != B + 1:
        raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT, "cu_seqlens_q and cu_seqlens_k must have the same length")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT, f"{name} must be a contiguous int32 tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if out is None:
        out = torch.empty((total_q, H, dv), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.stride(-1) != 1:
            raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT, f"{name}: last dimension must be contiguous")
    if v.shape[:2] != k.shape[:2] or tuple(out.shape) != (total_q, H, dv) or out.dtype != q.dtype:
        raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT, "v must be [total_k, Hkv, d_v] and out [total_q, H, d_v]")
    if tuple(lse.shape) != (H, total_q) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise AttnInvalidArgument(ATTN_INVALID_ARGUMENT, "lse must be a contiguous fp32 [H, total_q] tensor")
    _expect(k, "k", (None, None, dqk), q.dtype)
    _expect(v, "v", (total_k, Hkv, None), q.dtype)
    if sinks is not None:
        _expect(sinks, "sinks", (H,), torch.float32, contiguous=True)
    _on_device(q=q, k=k, v=v, out=out, lse=lse, sinks=sinks, cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k)
    a = AttnVarlenArgs()
    a.struct_size = ctypes.sizeof(AttnVarlenArgs)
    a.dtype = _dtype_code(q)
    a.B, a.H, a.Hkv, a.max_seqlen_q, a.total_q, a.total_k, a.d_qk, a.d_v = (B, H, Hkv, int(max_seqlen_q), total_q,
                                                                           total_k, dqk, dv)
    a.causal = 1 if causal else 0
    a.scale = float(scale)
    a.q, (a.q_st, a.q_sh) = q.data_ptr(), q.stride()[:2]
    a.k, (a.k_st, a.k_sh) = k.data_ptr(), k.stride()[:2]
    a.v, (a.v_st, a.v_sh) = v.data_ptr(), v.stride()[:2]
    a.out, (a.o_st, a.o_sh) = out.data_ptr(), out.stride()[:2]
    a.lse = lse.data_ptr()
    a.sinks = sinks.data_ptr() if sinks is not None else None
    a.cu_seqlens_q, a.cu_seqlens_k = cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr()
    a.window_left, a.window_right = int(window[0]), int(window[1])
    _check(lib.attn_fwd_varlen(ctypes.byref(a), ctypes.c_void_p(_stream_handle(stream))))
    return out, lse
