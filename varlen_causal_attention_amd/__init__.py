"""Python binding of ``libvlca.so`` (gfx950 varlen causal attention forward).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (``include/varlen_causal_attn.h``).  torch supplies
device memory and the current stream.  There is no fallback: if the library is
not built, or a tensor is not on a ROCm device, the call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

__all__ = [
    "VlcaError", "library", "library_path", "fwd", "build_worklist", "fwd_with_worklist",
    "worklist_capacity", "single_kernel", "tile_rows", "strerror", "call_module", "EXPORTED_SYMBOLS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libvlca.so")
_lib = None
_call = None  # the CPython trampoline for fwd / fwd_worklist (ctypes when it is not built)

EXPORTED_SYMBOLS = (
    "varlen_causal_attn_fwd",
    "varlen_causal_attn_worklist_capacity",
    "varlen_causal_attn_build_worklist",
    "varlen_causal_attn_fwd_worklist",
    "varlen_causal_attn_single_kernel",
    "varlen_causal_attn_tile_rows",
    "varlen_causal_attn_strerror",
)


class VlcaError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: error {code}: {strerror(code)}")
        self.code = code


def library_path() -> str:
    return _LIB_PATH


def library():
    """Load ``libvlca.so`` (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m varlen_causal_attention_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32p, i64p = ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64)
    c_int, c_float = ctypes.c_int, ctypes.c_float
    lib.varlen_causal_attn_fwd.argtypes = [vp, i32p, c_int, c_int, c_int, c_int, c_float, vp, vp]
    lib.varlen_causal_attn_fwd.restype = c_int
    lib.varlen_causal_attn_worklist_capacity.argtypes = [c_int, c_int, i64p]
    lib.varlen_causal_attn_worklist_capacity.restype = c_int
    lib.varlen_causal_attn_build_worklist.argtypes = [i32p, c_int, c_int, i32p, ctypes.c_int64, i32p, vp]
    lib.varlen_causal_attn_build_worklist.restype = c_int
    lib.varlen_causal_attn_fwd_worklist.argtypes = [vp, i32p, c_int, c_int, c_int, c_int, c_float, i32p,
                                                    ctypes.c_int64, i32p, vp, vp]
    lib.varlen_causal_attn_fwd_worklist.restype = c_int
    lib.varlen_causal_attn_single_kernel.argtypes = [c_int, c_int, c_int, ctypes.POINTER(ctypes.c_int)]
    lib.varlen_causal_attn_single_kernel.restype = c_int
    lib.varlen_causal_attn_tile_rows.argtypes = []
    lib.varlen_causal_attn_tile_rows.restype = c_int
    lib.varlen_causal_attn_strerror.argtypes = [c_int]
    lib.varlen_causal_attn_strerror.restype = ctypes.c_char_p
    global _call
    try:
        from . import _vlca_call
    except ImportError:
        _vlca_call = None
    if _vlca_call is not None:
        _vlca_call.set_entries(ctypes.cast(lib.varlen_causal_attn_fwd, vp).value,
                               ctypes.cast(lib.varlen_causal_attn_fwd_worklist, vp).value)
        _call = _vlca_call
    _lib = lib
    return lib


def call_module():
    """The CPython call trampoline in use for fwd / fwd_worklist, or None (ctypes)."""
    library()
    return _call


def strerror(code: int) -> str:
    return library().varlen_causal_attn_strerror(int(code)).decode()


def tile_rows() -> int:
    return int(library().varlen_causal_attn_tile_rows())


def single_kernel(num_users: int, max_seqlen: int, n_heads: int = 8) -> bool:
    """True when :func:`fwd` runs as one kernel (no worklist buffer) for these sizes on this device."""
    flag = ctypes.c_int(0)
    rc = library().varlen_causal_attn_single_kernel(int(num_users), int(max_seqlen), int(n_heads), ctypes.byref(flag))
    if rc != 0:
        raise VlcaError(rc, "varlen_causal_attn_single_kernel")
    return bool(flag.value)


def worklist_capacity(num_users: int, max_seqlen: int) -> int:
    cap = ctypes.c_int64(0)
    rc = library().varlen_causal_attn_worklist_capacity(int(num_users), int(max_seqlen), ctypes.byref(cap))
    if rc != 0:
        raise VlcaError(rc, "varlen_causal_attn_worklist_capacity")
    return int(cap.value)


_torch = None


def _torch_mod():
    global _torch
    if _torch is None:
        import torch

        _torch = torch
    return _torch


def _stream_handle(device) -> int:
    """Raw handle of torch's current stream on ``device`` (no Stream object is built)."""
    torch = _torch_mod()
    idx = device.index if device.index is not None else torch.cuda.current_device()
    return torch._C._cuda_getCurrentRawStream(idx)


def _check_cu(cu_seqlens):
    torch = _torch_mod()
    if not cu_seqlens.is_cuda or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a 1-D device tensor")
    if cu_seqlens.dtype == torch.int64:
        cu_seqlens = cu_seqlens.to(torch.int32)  # device-side conversion, no host sync
    if cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32 or int64")
    return cu_seqlens.contiguous()


def _check_qkv(qkv, n_heads, head_dim):
    torch = _torch_mod()
    if not qkv.is_cuda or qkv.dtype != torch.bfloat16 or qkv.dim() != 2:
        raise ValueError("qkv must be a 2-D bfloat16 device tensor")
    if qkv.shape[1] != 3 * n_heads * head_dim:
        raise ValueError(f"qkv has {qkv.shape[1]} columns, expected 3*{n_heads}*{head_dim}")
    if not qkv.is_contiguous():
        raise ValueError("qkv must be contiguous")
    if qkv.shape[0] >= 2**31:
        raise ValueError("total tokens must be < 2^31")


def _out_tensor(qkv, n_heads, head_dim, out):
    torch = _torch_mod()
    shape = (qkv.shape[0], n_heads * head_dim)
    if out is None:
        return torch.empty(shape, dtype=torch.bfloat16, device=qkv.device)
    if (tuple(out.shape) != shape or out.dtype != torch.bfloat16 or not out.is_contiguous()
            or not out.is_cuda or out.get_device() != qkv.get_device()):
        raise ValueError(f"out must be a contiguous bfloat16 tensor of shape {shape} on {qkv.device}")
    return out


def fwd(qkv, cu_seqlens, max_seqlen: int, n_heads: int = 8, head_dim: int = 64,
        scale: Optional[float] = None, out=None):
    """Block-diagonal causal attention over packed users; returns ``out`` [T, n_heads*head_dim] bf16.

    ``max_seqlen`` is an upper bound on every user's length (a bucket constant is
    fine).  The call is asynchronous on torch's current stream.
    """
    _check_qkv(qkv, n_heads, head_dim)
    cu = _check_cu(cu_seqlens)
    out = _out_tensor(qkv, n_heads, head_dim, out)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    lib = library()
    args = (qkv.data_ptr(), cu.data_ptr(), cu.shape[0] - 1, int(max_seqlen), int(n_heads), int(head_dim),
            float(scale), out.data_ptr(), _stream_handle(qkv.device))
    rc = _call.fwd(*args) if _call is not None else lib.varlen_causal_attn_fwd(*args)
    if rc != 0:
        raise VlcaError(rc, "varlen_causal_attn_fwd")
    return out


def build_worklist(cu_seqlens, max_seqlen: int) -> Tuple["object", "object"]:
    """Run the segment scheduler alone; returns (items int32 [capacity, 4], count int32 [1]) on the device.

    Rows ``items[:count]`` are (user, q_tile, row_start, length) in the scheduler's order;
    later rows are unspecified.
    """
    torch = _torch_mod()
    cu = _check_cu(cu_seqlens)
    cap = worklist_capacity(cu.shape[0] - 1, max_seqlen)
    items = torch.empty((cap, 4), dtype=torch.int32, device=cu.device)
    count = torch.empty((1,), dtype=torch.int32, device=cu.device)
    rc = library().varlen_causal_attn_build_worklist(cu.data_ptr(), cu.shape[0] - 1, int(max_seqlen),
                                                     items.data_ptr(), cap, count.data_ptr(),
                                                     _stream_handle(cu.device))
    if rc != 0:
        raise VlcaError(rc, "varlen_causal_attn_build_worklist")
    return items, count


def fwd_with_worklist(qkv, cu_seqlens, max_seqlen: int, items, count, n_heads: int = 8, head_dim: int = 64,
                      scale: Optional[float] = None, out=None):
    """Attention kernel alone over a worklist from :func:`build_worklist` (same cu_seqlens/max_seqlen)."""
    torch = _torch_mod()
    _check_qkv(qkv, n_heads, head_dim)
    cu = _check_cu(cu_seqlens)
    if items.dtype != torch.int32 or items.dim() != 2 or items.shape[1] != 4 or not items.is_contiguous():
        raise ValueError("items must be a contiguous int32 [capacity, 4] tensor")
    if count.dtype != torch.int32 or count.numel() != 1 or not count.is_cuda:
        raise ValueError("count must be a device int32 tensor with one element")
    out = _out_tensor(qkv, n_heads, head_dim, out)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    lib = library()
    args = (qkv.data_ptr(), cu.data_ptr(), cu.shape[0] - 1, int(max_seqlen), int(n_heads), int(head_dim),
            float(scale), items.data_ptr(), items.shape[0], count.data_ptr(), out.data_ptr(),
            _stream_handle(qkv.device))
    rc = _call.fwd_worklist(*args) if _call is not None else lib.varlen_causal_attn_fwd_worklist(*args)
    if rc != 0:
        raise VlcaError(rc, "varlen_causal_attn_fwd_worklist")
    return out
