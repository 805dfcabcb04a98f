"""Python face of the fused attention forward library (``libfa.so``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/fa.h``. PyTorch supplies device memory
and the current stream. There is no fallback: if the library is missing,
importing works but every call raises.

    o, lse = forward(q, k, v, causal=True)              # f32 / f16 / bf16
    o, lse = forward_fp8(q8, k8, v8, qd, kd, vd)         # e4m3fn + descales
    dq, dk, dv = backward(q, k, v, o, lse, do, causal=True)   # f16 / bf16
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

# fa_dtype (include/fa.h)
FA_F32, FA_F16, FA_BF16, FA_FP8_E4M3 = 0, 1, 2, 3
_DTYPE_CODE = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16,
               torch.float8_e4m3fn: FA_FP8_E4M3}
_OUT_DTYPE = {torch.float32: torch.float32, torch.float16: torch.float16,
              torch.bfloat16: torch.bfloat16, torch.float8_e4m3fn: torch.bfloat16}

# fa_status (include/fa.h)
STATUS = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_DTYPE",
          4: "FA_ERR_UNSUPPORTED", 5: "FA_ERR_ALIGN", 6: "FA_ERR_SCALE", 7: "FA_ERR_ALIAS",
          8: "FA_ERR_OVERFLOW", 9: "FA_ERR_HIP", 10: "FA_ERR_SCRATCH"}

EXPORTS = ("fa_forward", "fa_forward_fp8", "fa_forward_strided", "fa_forward_varlen",
           "fa_forward_splitkv", "fa_splitkv_workspace_size", "fa_splitkv_splits",
           "fa_forward_splitkv_noalloc", "fa_noalloc_scratch_bytes",
           "fa_backward", "fa_backward_workspace_size", "fa_backward_varlen", "fa_forward_unfused",
           "fa_unfused_workspace_size", "fa_status_string", "fa_last_hip_error",
           "fa_abi_version")

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa.so (once) and declare its signatures. Raises if missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() "
                           "(the HIP library is required, there is no fallback)")
    lib = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.fa_forward.restype = i
    lib.fa_forward_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, f, f, f, vp]
    lib.fa_forward_fp8.restype = i
    sz = ctypes.c_size_t
    lib.fa_forward_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i, vp, sz, vp]
    lib.fa_forward_splitkv.restype = i
    lib.fa_forward_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i, vp]
    lib.fa_forward_splitkv_noalloc.restype = i
    lib.fa_noalloc_scratch_bytes.argtypes = []
    lib.fa_noalloc_scratch_bytes.restype = sz
    lib.fa_splitkv_workspace_size.argtypes = [i, i, i, i, i]
    lib.fa_splitkv_workspace_size.restype = sz
    lib.fa_splitkv_splits.argtypes = [i, i, i, i, i]
    lib.fa_splitkv_splits.restype = i
    lib.fa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp, sz, vp]
    lib.fa_backward.restype = i
    lib.fa_backward_workspace_size.argtypes = [i, i, i]
    lib.fa_backward_workspace_size.restype = sz
    lib.fa_backward_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i,
                                       vp, sz, vp]
    lib.fa_backward_varlen.restype = i
    lib.fa_forward_unfused.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp, sz, vp]
    lib.fa_forward_unfused.restype = i
    lib.fa_unfused_workspace_size.argtypes = [i, i, i]
    lib.fa_unfused_workspace_size.restype = sz
    lib.fa_forward_strided.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, vp, f, i, i, vp]
    lib.fa_forward_strided.restype = i
    lib.fa_forward_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    lib.fa_forward_varlen.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_last_hip_error.argtypes = []
    lib.fa_last_hip_error.restype = i
    lib.fa_abi_version.argtypes = []
    lib.fa_abi_version.restype = i
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def _check(status: int):
    if status != 0:
        lib = load_library()
        msg = lib.fa_status_string(status).decode()
        if status == 9:
            msg += f" (hipError_t {lib.fa_last_hip_error()})"
        raise FAError(status, msg)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _require(name: str, t: torch.Tensor, shape, dtype, device=None):
    """A caller-supplied output or workspace tensor must be exactly what the
    C ABI writes: the library sizes every write from q's shape, so a smaller
    or differently typed buffer would be written past its end."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, not {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, not {t.device}")


def _require_workspace(t: torch.Tensor, need: int, device):
    _require("workspace", t, None, None, device)
    if t.numel() * t.element_size() < need:
        raise ValueError(f"workspace holds {t.numel() * t.element_size()} bytes; {need} needed")


def _prepare(q, k, v, out, lse):
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [batch, heads, n, d_k] shape")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    if q.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    b, h, n, d = q.shape
    if out is not None:
        _require("out", out, (b, h, n, d), _OUT_DTYPE[q.dtype])
    if lse is not None:
        _require("lse", lse, (b, h, n), torch.float32)
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous device tensors")
        if t.device != q.device:
            raise ValueError("q, k, v must be on one device")
    for name, t in (("out", out), ("lse", lse)):
        if t is not None and t.device != q.device:
            raise ValueError(f"{name} must be on {q.device}, not {t.device}")
    if out is None:
        out = torch.empty((b, h, n, d), dtype=_OUT_DTYPE[q.dtype], device=q.device)
    if lse is None:
        lse = torch.empty((b, h, n), dtype=torch.float32, device=q.device)
    return out, lse


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
            scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, want_lse: bool = True
            ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """O and LSE of softmax(scale * q k^T + mask) v via ``fa_forward``.

    q, k, v: contiguous [batch, heads, n, d_k] device tensors (f32, f16 or
    bf16; e4m3fn means all descales are 1). scale defaults to 1/sqrt(d_k).
    Enqueued on torch's current stream; returns immediately.
    """
    lib = load_library()
    out, lse = _prepare(q, k, v, out, lse if want_lse else None)
    if not want_lse:
        lse = None
    b, h, n, d = q.shape
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib.fa_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), b, h, n, d, s,
                        1 if causal else 0, _DTYPE_CODE[q.dtype], _stream(q.device))
    _check(st)
    return out, lse


def forward_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_descale: float,
                k_descale: float, v_descale: float, causal: bool = False,
                scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """``fa_forward_fp8``: e4m3fn q, k, v with per-tensor fp32 descales; bf16 O."""
    lib = load_library()
    if q.dtype != torch.float8_e4m3fn:
        raise ValueError("forward_fp8 takes float8_e4m3fn tensors")
    out, lse = _prepare(q, k, v, out, lse)
    b, h, n, d = q.shape
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib.fa_forward_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), b, h, n, d, s,
                            1 if causal else 0, float(q_descale), float(k_descale),
                            float(v_descale), _stream(q.device))
    _check(st)
    return out, lse


def splitkv_workspace_size(batch: int, heads: int, n: int, d_k: int, splits: int) -> int:
    """Bytes of workspace ``forward_splitkv`` needs (0: the keys are not split)."""
    return int(load_library().fa_splitkv_workspace_size(batch, heads, n, d_k, splits))


def splitkv_splits(batch: int, heads: int, n: int, causal: bool, compute_units: int = 0) -> int:
    """``fa_splitkv_splits``: the library's key-block count for these sizes
    (compute_units <= 0: the current device's)."""
    return int(load_library().fa_splitkv_splits(batch, heads, n, 1 if causal else 0, int(compute_units)))


def forward_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, splits: Optional[int] = None,
                    causal: bool = False, scale: Optional[float] = None,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None):
    """``fa_forward_splitkv``: keys cut into ``splits`` blocks (None: the count
    ``fa_splitkv_splits`` gives), partial results merged by their log-sum-exp.
    Returns (O, LSE, workspace); the workspace (uint8 device tensor, allocated
    here unless given) holds the per-block partials after the call."""
    lib = load_library()
    out, lse = _prepare(q, k, v, out, lse)
    b, h, n, d = q.shape
    if splits is None:
        splits = splitkv_splits(b, h, n, causal)
    need = splitkv_workspace_size(b, h, n, d, splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    else:
        _require_workspace(workspace, need, q.device)
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib.fa_forward_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), b, h, n, d, s,
                                1 if causal else 0, _DTYPE_CODE[q.dtype], int(splits),
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(q.device))
    _check(st)
    return out, lse, workspace



def forward_splitkv_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, splits: Optional[int] = None,
                            causal: bool = False, scale: Optional[float] = None,
                            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """``fa_forward_splitkv_noalloc``: ``forward_splitkv`` with the per-block
    partials in the library's fixed per-GPU scratch instead of a workspace
    (for callers that cannot allocate; pass ``out`` and ``lse`` to allocate
    nothing here either). Returns (O, LSE)."""
    lib = load_library()
    out, lse = _prepare(q, k, v, out, lse)
    b, h, n, d = q.shape
    if splits is None:
        splits = splitkv_splits(b, h, n, causal)
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib.fa_forward_splitkv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), b, h, n, d, s,
                                        1 if causal else 0, _DTYPE_CODE[q.dtype], int(splits),
                                        _stream(q.device))
    _check(st)
    return out, lse


def noalloc_scratch_bytes() -> int:
    """Bytes of the fixed per-GPU scratch of ``forward_splitkv_noalloc``."""
    return int(load_library().fa_noalloc_scratch_bytes())


def backward_workspace_size(batch: int, heads: int, n: int) -> int:
    """Bytes of workspace ``backward`` needs."""
    return int(load_library().fa_backward_workspace_size(batch, heads, n))


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
             dout: torch.Tensor, causal: bool = False, scale: Optional[float] = None,
             dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
             dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """``fa_backward``: (dQ, dK, dV) of the attention ``forward`` computed, given
    its O and LSE and the output gradient dO. f16 or bf16, contiguous
    [batch, heads, n, d_k] device tensors; LSE fp32 [batch, heads, n]."""
    lib = load_library()
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("backward takes float16 or bfloat16 tensors")
    for t in (k, v, o, dout):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v, o and dout must share one shape and dtype")
    for t in (q, k, v, o, dout, lse):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous device tensors")
    if q.dim() != 4:
        raise ValueError("tensors are [batch, heads, n, d_k]")
    b, h, n, d = q.shape
    if lse.dtype != torch.float32 or tuple(lse.shape) != (b, h, n):
        raise ValueError("lse must be float32 [batch, heads, n]")
    for t in (k, v, o, dout, lse):
        if t.device != q.device:
            raise ValueError("all tensors must be on one device")
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is not None:
            _require(name, t, q.shape, q.dtype, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    need = backward_workspace_size(b, h, n)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    else:
        _require_workspace(workspace, need, q.device)
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib.fa_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                         _ptr(dk), _ptr(dv), b, h, n, d, s, 1 if causal else 0, _DTYPE_CODE[q.dtype],
                         _ptr(workspace), workspace.numel() * workspace.element_size(),
                         _stream(q.device))
    _check(st)
    return dq, dk, dv


def unfused_workspace_size(batch: int, heads: int, n: int) -> int:
    """Bytes of workspace ``forward_unfused`` needs (S fp32 plus P, n x n per head)."""
    return int(load_library().fa_unfused_workspace_size(batch, heads, n))


def forward_unfused(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                    scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """``fa_forward_unfused``: O and LSE computed with S and P materialised.
    Returns (O, LSE, workspace); the workspace holds S (fp32) and P after the call."""
    lib = load_library()
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("forward_unfused takes float16 or bfloat16 tensors")
    out, lse = _prepare(q, k, v, out, lse)
    b, h, n, d = q.shape
    need = unfused_workspace_size(b, h, n)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    else:
        _require_workspace(workspace, need, q.device)
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib.fa_forward_unfused(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), b, h, n, d, s,
                                1 if causal else 0, _DTYPE_CODE[q.dtype], _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(st)
    return out, lse, workspace


def _head_strides(t: torch.Tensor, layout: str):
    """(batch, head, row) element strides of a 4-D tensor in layout "bhsd" or "bshd"."""
    if t.stride(-1) != 1:
        raise ValueError("the last (d_k) dimension must be contiguous")
    s = t.stride()
    return (s[0], s[1], s[2]) if layout == "bhsd" else (s[0], s[2], s[1])


def forward_strided(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, layout: str = "bshd",
                    causal: bool = False, scale: Optional[float] = None,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    out_layout: Optional[str] = None):
    """``fa_forward_strided``: q, k, v are 4-D device tensors (any strides, d_k
    contiguous) indexed [batch, heads, n, d_k] ("bhsd") or [batch, n, heads,
    d_k] ("bshd"). O is allocated in ``out_layout`` (default: ``layout``) unless
    given. Returns (O, LSE [batch, heads, n])."""
    lib = load_library()
    if layout not in ("bhsd", "bshd"):
        raise ValueError("layout is 'bhsd' or 'bshd'")
    out_layout = out_layout or layout
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one 4-D shape and dtype")
    if q.dtype not in _DTYPE_CODE or not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors of a supported dtype")
    if out_layout not in ("bhsd", "bshd"):
        raise ValueError("out_layout is 'bhsd' or 'bshd'")
    if layout == "bhsd":
        b, h, n, d = q.shape
    else:
        b, n, h, d = q.shape
    shape = (b, h, n, d) if out_layout == "bhsd" else (b, n, h, d)
    for t in (k, v):
        if t.device != q.device:
            raise ValueError("q, k, v must be on one device")
    if out is None:
        out = torch.empty(shape, dtype=_OUT_DTYPE[q.dtype], device=q.device)
    else:
        # any strides with d_k contiguous (the C ABI checks that rows do not overlap),
        # but the extents and type the kernel writes
        if tuple(out.shape) != shape or out.dtype != _OUT_DTYPE[q.dtype] or out.device != q.device:
            raise ValueError(f"out must be a {_OUT_DTYPE[q.dtype]} tensor of shape {shape} on {q.device}")
    if lse is None:
        lse = torch.empty((b, h, n), dtype=torch.float32, device=q.device)
    else:
        _require("lse", lse, (b, h, n), torch.float32, q.device)
    st = [*_head_strides(q, layout), *_head_strides(k, layout), *_head_strides(v, layout),
          *_head_strides(out, out_layout)]
    arr = (ctypes.c_int64 * 12)(*st)
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    r = lib.fa_forward_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), b, h, n, d,
                               ctypes.cast(arr, ctypes.c_void_p), s, 1 if causal else 0,
                               _DTYPE_CODE[q.dtype], _stream(q.device))
    _check(r)
    return out, lse


def forward_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                   max_seqlen: int, causal: bool = False, scale: Optional[float] = None,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """``fa_forward_varlen``: q, k, v [total, heads, d_k] contiguous device tensors
    holding packed sequences; cu_seqlens an int32 device tensor of batch + 1
    offsets. Returns (O [total, heads, d_k], LSE [heads, total])."""
    lib = load_library()
    if q.dim() != 3 or k.shape != q.shape or v.shape != q.shape or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one [total, heads, d_k] shape and dtype")
    for t in (q, k, v, cu_seqlens):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous device tensors")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor")
    total, h, d = q.shape
    batch = cu_seqlens.numel() - 1
    for t in (k, v, cu_seqlens):
        if t.device != q.device:
            raise ValueError("all tensors must be on one device")
    if out is None:
        out = torch.empty((total, h, d), dtype=_OUT_DTYPE[q.dtype], device=q.device)
    else:
        _require("out", out, (total, h, d), _OUT_DTYPE[q.dtype], q.device)
    if lse is None:
        lse = torch.empty((h, total), dtype=torch.float32, device=q.device)
    else:
        _require("lse", lse, (h, total), torch.float32, q.device)
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    r = lib.fa_forward_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens),
                              batch, total, int(max_seqlen), h, d, s, 1 if causal else 0,
                              _DTYPE_CODE[q.dtype], _stream(q.device))
    _check(r)
    return out, lse


def backward_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                    lse: torch.Tensor, dout: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
                    causal: bool = False, scale: Optional[float] = None,
                    workspace: Optional[torch.Tensor] = None):
    """``fa_backward_varlen``: (dQ, dK, dV) [total, heads, d_k] of ``forward_varlen``,
    given its O [total, heads, d_k] and LSE [heads, total] and dO."""
    lib = load_library()
    if q.dtype not in (torch.float16, torch.bfloat16) or q.dim() != 3:
        raise ValueError("backward_varlen takes [total, heads, d_k] float16 / bfloat16 tensors")
    for t in (k, v, o, dout):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v, o and dout must share one shape and dtype")
    for t in (q, k, v, o, dout, lse, cu_seqlens):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous device tensors")
    total, h, d = q.shape
    if lse.dtype != torch.float32 or tuple(lse.shape) != (h, total):
        raise ValueError("lse must be float32 [heads, total]")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor")
    for t in (k, v, o, dout, lse, cu_seqlens):
        if t.device != q.device:
            raise ValueError("all tensors must be on one device")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    need = backward_workspace_size(1, h, max(total, 1))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    else:
        _require_workspace(workspace, need, q.device)
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib.fa_backward_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                                _ptr(dk), _ptr(dv), _ptr(cu_seqlens), cu_seqlens.numel() - 1, total,
                                int(max_seqlen), h, d, s, 1 if causal else 0, _DTYPE_CODE[q.dtype],
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(q.device))
    _check(st)
    return dq, dk, dv
