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
    "VlcaError", "library", "library_path", "fwd", "fwd_masked", "fwd_noalloc", "fwd_lse", "bwd", "attention",
    "ln_qkv", "out_residual", "attention_block",
    "build_worklist", "fwd_with_worklist",
    "worklist_capacity", "single_kernel", "tile_rows", "strerror", "call_module", "EXPORTED_SYMBOLS",
    "GraphRunner", "PAGES_BUCKETS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libvlca.so")
_lib = None
_call = None  # the CPython trampoline for fwd / fwd_worklist (ctypes when it is not built)

EXPORTED_SYMBOLS = (
    "varlen_causal_attn_fwd",
    "varlen_causal_attn_fwd_lse",
    "varlen_causal_attn_fwd_masked",
    "varlen_causal_attn_bwd",
    "varlen_causal_attn_ln_qkv",
    "varlen_causal_attn_out_residual",
    "varlen_causal_attn_fwd_noalloc",
    "varlen_causal_attn_worklist_capacity",
    "varlen_causal_attn_build_worklist",
    "varlen_causal_attn_fwd_worklist",
    "varlen_causal_attn_single_kernel",
    "varlen_causal_attn_runner_create",
    "varlen_causal_attn_runner_run",
    "varlen_causal_attn_runner_bucket",
    "varlen_causal_attn_runner_captured",
    "varlen_causal_attn_runner_destroy",
    "varlen_causal_attn_tile_rows",
    "varlen_causal_attn_strerror",
)


class _Mask(ctypes.Structure):
    """Mirror of ``vlca_mask`` (include/varlen_causal_attn.h)."""
    _fields_ = [("num_contexts", ctypes.c_void_p), ("num_targets", ctypes.c_void_p),
                ("target_group_size", ctypes.c_int), ("window_left", ctypes.c_int), ("window_right", ctypes.c_int)]


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
    lib.varlen_causal_attn_fwd_lse.argtypes = [vp, i32p, c_int, c_int, c_int, c_int, c_float, vp, vp, vp]
    lib.varlen_causal_attn_fwd_lse.restype = c_int
    lib.varlen_causal_attn_fwd_masked.argtypes = [vp, i32p, c_int, c_int, c_int, c_int, c_float,
                                                  ctypes.POINTER(_Mask), vp, vp]
    lib.varlen_causal_attn_fwd_masked.restype = c_int
    lib.varlen_causal_attn_ln_qkv.argtypes = [vp, vp, vp, c_float, vp, vp, c_int, c_int, c_int, vp, vp]
    lib.varlen_causal_attn_ln_qkv.restype = c_int
    lib.varlen_causal_attn_out_residual.argtypes = [vp, vp, vp, vp, c_int, c_int, c_int, vp, vp]
    lib.varlen_causal_attn_out_residual.restype = c_int
    lib.varlen_causal_attn_bwd.argtypes = [vp, vp, vp, vp, i32p, c_int, c_int, c_int, c_int, c_float, vp, vp]
    lib.varlen_causal_attn_bwd.restype = c_int
    lib.varlen_causal_attn_fwd_noalloc.argtypes = [vp, i32p, c_int, c_int, c_int, c_int, c_float, vp, vp]
    lib.varlen_causal_attn_fwd_noalloc.restype = c_int
    lib.varlen_causal_attn_worklist_capacity.argtypes = [c_int, c_int, i64p]
    lib.varlen_causal_attn_worklist_capacity.restype = c_int
    lib.varlen_causal_attn_build_worklist.argtypes = [i32p, c_int, c_int, i32p, ctypes.c_int64, i32p, vp]
    lib.varlen_causal_attn_build_worklist.restype = c_int
    lib.varlen_causal_attn_fwd_worklist.argtypes = [vp, i32p, c_int, c_int, c_int, c_int, c_float, i32p,
                                                    ctypes.c_int64, i32p, vp, vp]
    lib.varlen_causal_attn_fwd_worklist.restype = c_int
    lib.varlen_causal_attn_single_kernel.argtypes = [c_int, c_int, c_int, ctypes.POINTER(ctypes.c_int)]
    lib.varlen_causal_attn_single_kernel.restype = c_int
    ip = ctypes.POINTER(ctypes.c_int)
    lib.varlen_causal_attn_runner_create.argtypes = [ctypes.POINTER(ctypes.c_int32), c_int, c_int, c_int, c_float,
                                                     vp, vp, c_int, ctypes.POINTER(vp)]
    lib.varlen_causal_attn_runner_create.restype = c_int
    lib.varlen_causal_attn_runner_run.argtypes = [vp, vp, i32p, c_int, c_int, c_int, vp, vp, ip]
    lib.varlen_causal_attn_runner_run.restype = c_int
    lib.varlen_causal_attn_runner_bucket.argtypes = [vp, c_int, c_int, ip]
    lib.varlen_causal_attn_runner_bucket.restype = c_int
    lib.varlen_causal_attn_runner_captured.argtypes = [vp, ip]
    lib.varlen_causal_attn_runner_captured.restype = c_int
    lib.varlen_causal_attn_runner_destroy.argtypes = [vp]
    lib.varlen_causal_attn_runner_destroy.restype = c_int
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


def fwd_masked(qkv, cu_seqlens, max_seqlen: int, num_contexts=None, num_targets=None, target_group_size: int = 1,
               window=(-1, 0), n_heads: int = 8, head_dim: int = 64, scale: Optional[float] = None, out=None):
    """Forward with the HSTU-style mask variants (``vlca_mask``): per-user context and
    candidate counts (int32 device tensors [num_users] or None), the candidates'
    group size, and ``window = (left, right)`` (-1: unbounded; right 0: causal)."""
    torch = _torch_mod()
    _check_qkv(qkv, n_heads, head_dim)
    cu = _check_cu(cu_seqlens)
    users = cu.shape[0] - 1
    ptrs = []
    for name, t in (("num_contexts", num_contexts), ("num_targets", num_targets)):
        if t is None:
            ptrs.append(None)
            continue
        if (t.dtype != torch.int32 or not t.is_cuda or t.dim() != 1 or t.shape[0] != users
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int32 device tensor of {users} entries")
        ptrs.append(t.data_ptr())
    out = _out_tensor(qkv, n_heads, head_dim, out)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    m = _Mask(ptrs[0], ptrs[1], int(target_group_size), int(window[0]), int(window[1]))
    rc = library().varlen_causal_attn_fwd_masked(qkv.data_ptr(), cu.data_ptr(), users, int(max_seqlen), int(n_heads),
                                                 int(head_dim), float(scale), ctypes.byref(m), out.data_ptr(),
                                                 _stream_handle(qkv.device))
    if rc != 0:
        raise VlcaError(rc, "varlen_causal_attn_fwd_masked")
    return out


def _check_bf16(name, t, shape, device):
    torch = _torch_mod()
    if (tuple(t.shape) != tuple(shape) or t.dtype != torch.bfloat16 or not t.is_contiguous() or not t.is_cuda
            or (device.index is not None and t.get_device() != device.index)):
        raise ValueError(f"{name} must be a contiguous bfloat16 device tensor of shape {tuple(shape)}")


def ln_qkv(x, gamma, beta, w_qkv, b_qkv, eps: float = 1e-5, out=None):
    """qkv = LayerNorm(x) w_qkv^T + b_qkv (x bf16 [T, 512]; w_qkv [n_out, 512] as nn.Linear stores it)."""
    torch = _torch_mod()
    T, d = x.shape
    n_out = w_qkv.shape[0]
    for name, t, shape in (("x", x, (T, d)), ("gamma", gamma, (d,)), ("beta", beta, (d,)),
                           ("w_qkv", w_qkv, (n_out, d)), ("b_qkv", b_qkv, (n_out,))):
        _check_bf16(name, t, shape, x.device)
    if out is None:
        out = torch.empty((T, n_out), dtype=torch.bfloat16, device=x.device)
    _check_bf16("out", out, (T, n_out), x.device)
    rc = library().varlen_causal_attn_ln_qkv(x.data_ptr(), gamma.data_ptr(), beta.data_ptr(), float(eps),
                                             w_qkv.data_ptr(), b_qkv.data_ptr(), T, d, n_out, out.data_ptr(),
                                             _stream_handle(x.device))
    if rc != 0:
        raise VlcaError(rc, "varlen_causal_attn_ln_qkv")
    return out


def out_residual(attn, w_out, b_out, residual, out=None):
    """y = residual + attn w_out^T + b_out (attn bf16 [T, 512]; w_out [n_out, 512])."""
    torch = _torch_mod()
    T, d = attn.shape
    n_out = w_out.shape[0]
    for name, t, shape in (("attn", attn, (T, d)), ("w_out", w_out, (n_out, d)), ("b_out", b_out, (n_out,)),
                           ("residual", residual, (T, n_out))):
        _check_bf16(name, t, shape, attn.device)
    if out is None:
        out = torch.empty((T, n_out), dtype=torch.bfloat16, device=attn.device)
    _check_bf16("out", out, (T, n_out), attn.device)
    rc = library().varlen_causal_attn_out_residual(attn.data_ptr(), w_out.data_ptr(), b_out.data_ptr(),
                                                   residual.data_ptr(), T, d, n_out, out.data_ptr(),
                                                   _stream_handle(attn.device))
    if rc != 0:
        raise VlcaError(rc, "varlen_causal_attn_out_residual")
    return out


def attention_block(x, cu_seqlens, max_seqlen: int, gamma, beta, w_qkv, b_qkv, w_out, b_out, eps: float = 1e-5,
                    n_heads: int = 8, scale: Optional[float] = None):
    """The layer's attention sub-block: x + Linear_out(attention(Linear_qkv(LayerNorm(x)))),
    three library calls (LayerNorm fused into the qkv product, bias and residual into
    the output product)."""
    qkv = ln_qkv(x, gamma, beta, w_qkv, b_qkv, eps)
    attn = fwd(qkv, cu_seqlens, max_seqlen, n_heads=n_heads, scale=scale)
    return out_residual(attn, w_out, b_out, x)


def fwd_lse(qkv, cu_seqlens, max_seqlen: int, n_heads: int = 8, head_dim: int = 64,
            scale: Optional[float] = None, out=None, lse=None):
    """:func:`fwd` that also returns the rows' log-sum-exp: ``(out, lse)``, lse fp32 [T, n_heads]."""
    torch = _torch_mod()
    _check_qkv(qkv, n_heads, head_dim)
    cu = _check_cu(cu_seqlens)
    out = _out_tensor(qkv, n_heads, head_dim, out)
    if lse is None:
        lse = torch.empty((qkv.shape[0], n_heads), dtype=torch.float32, device=qkv.device)
    elif (tuple(lse.shape) != (qkv.shape[0], n_heads) or lse.dtype != torch.float32 or not lse.is_contiguous()
          or lse.get_device() != qkv.get_device()):
        raise ValueError("lse must be a contiguous float32 [T, n_heads] tensor on the qkv device")
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    rc = library().varlen_causal_attn_fwd_lse(qkv.data_ptr(), cu.data_ptr(), cu.shape[0] - 1, int(max_seqlen),
                                              int(n_heads), int(head_dim), float(scale), out.data_ptr(),
                                              lse.data_ptr(), _stream_handle(qkv.device))
    if rc != 0:
        raise VlcaError(rc, "varlen_causal_attn_fwd_lse")
    return out, lse


def bwd(qkv, out, dout, lse, cu_seqlens, max_seqlen: int, n_heads: int = 8, head_dim: int = 64,
        scale: Optional[float] = None, dqkv=None):
    """Gradient of the forward w.r.t. qkv given ``dout``; returns dqkv bf16 [T, 3*n_heads*head_dim]."""
    torch = _torch_mod()
    _check_qkv(qkv, n_heads, head_dim)
    cu = _check_cu(cu_seqlens)
    shape_o = (qkv.shape[0], n_heads * head_dim)
    for name, t in (("out", out), ("dout", dout)):
        if (tuple(t.shape) != shape_o or t.dtype != torch.bfloat16 or not t.is_contiguous()
                or t.get_device() != qkv.get_device()):
            raise ValueError(f"{name} must be a contiguous bfloat16 {shape_o} tensor on the qkv device")
    if (tuple(lse.shape) != (qkv.shape[0], n_heads) or lse.dtype != torch.float32 or not lse.is_contiguous()
            or lse.get_device() != qkv.get_device()):
        raise ValueError("lse must be a contiguous float32 [T, n_heads] tensor on the qkv device")
    if dqkv is None:
        dqkv = torch.empty_like(qkv)
    elif (dqkv.shape != qkv.shape or dqkv.dtype != torch.bfloat16 or not dqkv.is_contiguous()
          or dqkv.get_device() != qkv.get_device()):
        raise ValueError("dqkv must be a contiguous bfloat16 tensor shaped like qkv")
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    rc = library().varlen_causal_attn_bwd(qkv.data_ptr(), out.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                                          cu.data_ptr(), cu.shape[0] - 1, int(max_seqlen), int(n_heads),
                                          int(head_dim), float(scale), dqkv.data_ptr(), _stream_handle(qkv.device))
    if rc != 0:
        raise VlcaError(rc, "varlen_causal_attn_bwd")
    return dqkv


_autograd_fn = None


def _attention_function():
    """A torch.autograd.Function whose forward and backward are the two library calls."""
    global _autograd_fn
    if _autograd_fn is None:
        torch = _torch_mod()

        class VarlenCausalAttention(torch.autograd.Function):
            @staticmethod
            def forward(ctx, qkv, cu_seqlens, max_seqlen, n_heads, head_dim, scale):
                out, lse = fwd_lse(qkv, cu_seqlens, max_seqlen, n_heads, head_dim, scale)
                ctx.save_for_backward(qkv, cu_seqlens, out, lse)
                ctx.args = (max_seqlen, n_heads, head_dim, scale)
                return out

            @staticmethod
            def backward(ctx, dout):
                qkv, cu, out, lse = ctx.saved_tensors
                max_seqlen, n_heads, head_dim, scale = ctx.args
                dqkv = bwd(qkv, out, dout.contiguous(), lse, cu, max_seqlen, n_heads, head_dim, scale)
                return dqkv, None, None, None, None, None

        _autograd_fn = VarlenCausalAttention
    return _autograd_fn


def attention(qkv, cu_seqlens, max_seqlen: int, n_heads: int = 8, head_dim: int = 64,
              scale: Optional[float] = None):
    """Differentiable forward (autograd runs :func:`bwd`); same output as :func:`fwd`."""
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return _attention_function().apply(qkv, cu_seqlens, int(max_seqlen), int(n_heads), int(head_dim), float(scale))


def fwd_noalloc(qkv, cu_seqlens, max_seqlen: int, out, n_heads: int = 8, head_dim: int = 64,
                scale: Optional[float] = None):
    """:func:`fwd` through ``varlen_causal_attn_fwd_noalloc``: same bits, no allocation in the library.

    ``out`` must be given (this call allocates nothing, torch included) and
    ``cu_seqlens`` must already be an int32 device tensor.  Calls that overlap
    on one device race on the library's fixed scratch array.
    """
    torch = _torch_mod()
    _check_qkv(qkv, n_heads, head_dim)
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or cu_seqlens.dim() != 1 \
            or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 device tensor")
    if out is None:
        raise ValueError("fwd_noalloc needs a preallocated out tensor")
    out = _out_tensor(qkv, n_heads, head_dim, out)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    rc = library().varlen_causal_attn_fwd_noalloc(qkv.data_ptr(), cu_seqlens.data_ptr(), cu_seqlens.shape[0] - 1,
                                                  int(max_seqlen), int(n_heads), int(head_dim), float(scale),
                                                  out.data_ptr(), _stream_handle(qkv.device))
    if rc != 0:
        raise VlcaError(rc, "varlen_causal_attn_fwd_noalloc")
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


# The pages' token buckets: ten buckets from 2560 to 7168 in steps of 512
# (cti2026 README, CUDA Graph section, bucketed padding).
PAGES_BUCKETS = tuple(range(2560, 7168 + 1, 512))


class GraphRunner:
    """Bucketed graph runner over ``varlen_causal_attn_runner_*`` (argument marshalling only).

    ``qkv_static`` / ``out_static`` are allocated here with torch (top-bucket rows)
    and handed to the library, which captures one HIP graph per bucket over them.
    ``run`` replays the bucket of a batch (or runs the eager forward above the top
    bucket) and returns ``(out, bucket)``; with ``qkv`` the static buffer itself
    (filled by the caller, e.g. ``runner.qkv_static[:T] = ...``) nothing is copied in.
    """

    def __init__(self, buckets=PAGES_BUCKETS, max_users: int = 20, n_heads: int = 8, head_dim: int = 64,
                 scale: Optional[float] = None, precapture: bool = True, device="cuda"):
        torch = _torch_mod()
        self.buckets = tuple(int(b) for b in buckets)
        self.max_users, self.n_heads, self.head_dim = int(max_users), int(n_heads), int(head_dim)
        if head_dim != 64:
            raise ValueError("head_dim must be 64")
        self.scale = 1.0 / math.sqrt(head_dim) if scale is None else float(scale)
        top = max(self.buckets) if self.buckets else 0
        self.qkv_static = torch.zeros((top, 3 * n_heads * head_dim), dtype=torch.bfloat16, device=device)
        self.out_static = torch.zeros((top, n_heads * head_dim), dtype=torch.bfloat16, device=device)
        self._handle = ctypes.c_void_p(None)
        arr = (ctypes.c_int32 * max(1, len(self.buckets)))(*self.buckets)
        with torch.cuda.device(self.qkv_static.device):
            rc = library().varlen_causal_attn_runner_create(arr, len(self.buckets), self.max_users, self.n_heads,
                                                            self.scale, self.qkv_static.data_ptr(),
                                                            self.out_static.data_ptr(), 1 if precapture else 0,
                                                            ctypes.byref(self._handle))
        if rc != 0:
            raise VlcaError(rc, "varlen_causal_attn_runner_create")

    def bucket(self, num_users: int, total_tokens: int) -> int:
        b = ctypes.c_int(-1)
        rc = library().varlen_causal_attn_runner_bucket(self._handle, int(num_users), int(total_tokens),
                                                        ctypes.byref(b))
        if rc != 0:
            raise VlcaError(rc, "varlen_causal_attn_runner_bucket")
        return b.value

    def captured(self) -> int:
        n = ctypes.c_int(0)
        rc = library().varlen_causal_attn_runner_captured(self._handle, ctypes.byref(n))
        if rc != 0:
            raise VlcaError(rc, "varlen_causal_attn_runner_captured")
        return n.value

    def run(self, qkv, cu_seqlens, total_tokens: int, max_seqlen: int, out=None):
        """One batch; ``total_tokens`` = cu_seqlens[-1] as a host int (picks the bucket)."""
        torch = _torch_mod()
        _check_qkv(qkv, self.n_heads, self.head_dim)
        if qkv.data_ptr() != self.qkv_static.data_ptr() and qkv.shape[0] != total_tokens:
            raise ValueError("qkv must have total_tokens rows (or be the runner's static buffer)")
        if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or cu_seqlens.dim() != 1 \
                or not cu_seqlens.is_contiguous():
            raise ValueError("cu_seqlens must be a contiguous 1-D int32 device tensor")
        if out is None:
            out = torch.empty((total_tokens, self.n_heads * self.head_dim), dtype=torch.bfloat16, device=qkv.device)
        b = ctypes.c_int(-1)
        rc = library().varlen_causal_attn_runner_run(self._handle, qkv.data_ptr(), cu_seqlens.data_ptr(),
                                                     cu_seqlens.shape[0] - 1, int(total_tokens), int(max_seqlen),
                                                     out.data_ptr(), _stream_handle(qkv.device), ctypes.byref(b))
        if rc != 0:
            raise VlcaError(rc, "varlen_causal_attn_runner_run")
        return out, b.value

    def close(self):
        if self._handle:
            rc = library().varlen_causal_attn_runner_destroy(self._handle)
            self._handle = ctypes.c_void_p(None)
            if rc != 0:
                raise VlcaError(rc, "varlen_causal_attn_runner_destroy")

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover - interpreter shutdown
            pass
