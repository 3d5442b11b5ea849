"""Python binding of the C ABI in ``include/vx.h`` (ctypes).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libvx.so``.  torch is used for device memory and streams; the
functions accept torch tensors (device pointers are taken with
``data_ptr()``) and the current torch stream unless one is given.  There is
no CPU fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

from . import build as _build

VX_F32, VX_BF16 = 0, 1
STATUS = {0: "VX_OK", 1: "VX_ERR_NULL", 2: "VX_ERR_INVALID", 3: "VX_ERR_UNSUPPORTED",
          4: "VX_ERR_ALIGN", 5: "VX_ERR_HIP"}
EXPORTS = ("vx_adaln_modulate", "vx_adaln_modulate_ex", "vx_rope3d_apply", "vx_flash_attn_fwd",
           "vx_flash_attn_fwd_kv", "vx_flash_attn_fwd_masked", "vx_attn_merge2", "vx_last_error",
           "vx_version")


class VxError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class RopeDesc(ctypes.Structure):
    """vx_rope3d_desc."""
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32),
                ("n_prefix", ctypes.c_int32), ("d_t", ctypes.c_int32), ("d_h", ctypes.c_int32),
                ("d_w", ctypes.c_int32), ("theta", ctypes.c_float), ("pairing", ctypes.c_int32)]

    @classmethod
    def of(cls, grid, split, theta=10000.0, n_prefix=0, pairing=0):
        return cls(int(grid[0]), int(grid[1]), int(grid[2]), int(n_prefix), int(split[0]),
                   int(split[1]), int(split[2]), float(theta), int(pairing))


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the in-tree libvx.so; build it first only if it does not exist."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or _build.LIB
    if not os.path.exists(path):
        _build.build()
    lib = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.vx_adaln_modulate.argtypes = [vp, vp, vp, vp, i64, i64, ctypes.c_float, ctypes.c_int, vp]
    lib.vx_adaln_modulate.restype = ctypes.c_int
    lib.vx_adaln_modulate_ex.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    lib.vx_adaln_modulate_ex.restype = ctypes.c_int
    lib.vx_rope3d_apply.argtypes = [vp, vp, i64, i64, i64, i64, ctypes.POINTER(RopeDesc),
                                    ctypes.c_int, vp]
    lib.vx_rope3d_apply.restype = ctypes.c_int
    lib.vx_flash_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float,
                                      ctypes.POINTER(RopeDesc), ctypes.c_int, vp]
    lib.vx_flash_attn_fwd.restype = ctypes.c_int
    lib.vx_flash_attn_fwd_kv.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                         ctypes.c_float, ctypes.POINTER(RopeDesc), ctypes.c_int, vp]
    lib.vx_flash_attn_fwd_kv.restype = ctypes.c_int
    lib.vx_flash_attn_fwd_masked.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                             ctypes.c_float, ctypes.POINTER(RopeDesc), vp,
                                             ctypes.c_int, vp]
    lib.vx_flash_attn_fwd_masked.restype = ctypes.c_int
    lib.vx_attn_merge2.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, vp]
    lib.vx_attn_merge2.restype = ctypes.c_int
    lib.vx_last_error.argtypes = []
    lib.vx_last_error.restype = ctypes.c_char_p
    lib.vx_version.argtypes = []
    lib.vx_version.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise VxError(status, load().vx_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return VX_BF16
    if t.dtype == torch.float32:
        return VX_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _same(ref, *others, names=()):
    """Every tensor: on a GPU, contiguous, same shape and dtype as ref."""
    for i, t in enumerate((ref,) + others):
        if t is None:
            continue
        name = names[i] if i < len(names) else f"arg{i}"
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError(f"{name} is {tuple(t.shape)} {t.dtype}, expected "
                             f"{tuple(ref.shape)} {ref.dtype}")


def adaln_modulate(x, shift, scale, y, eps: float = 1e-6, stream=None):
    """y = LN(x) * (1 + scale) + shift, rows of x's last dimension."""
    _same(x, shift, scale, y, names=("x", "shift", "scale", "y"))
    hidden = x.shape[-1]
    rows = x.numel() // hidden if hidden else 0
    _check(load().vx_adaln_modulate(_ptr(x), _ptr(shift), _ptr(scale), _ptr(y), rows, hidden,
                                    eps, _dtype_code(x), _stream(stream)))
    return y


def adaln_modulate_ex(x, shift, scale, y, eps: float = 1e-6, stream=None):
    """y = LN(x) * (1 + scale) + shift with x, y [B, N, D] and tables [B, N, D]
    (per token) or [B, 1, D] (per sample); each tensor bf16 or float32."""
    if x.dim() != 3:
        raise ValueError(f"x must be [batch, tokens, hidden], got {tuple(x.shape)}")
    b, n, d = x.shape
    for name, t in (("x", x), ("shift", shift), ("scale", scale), ("y", y)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if tuple(y.shape) != (b, n, d):
        raise ValueError(f"y is {tuple(y.shape)}, expected {(b, n, d)}")
    if shift.shape != scale.shape or shift.dtype != scale.dtype:
        raise ValueError("shift and scale must have the same shape and dtype")
    if shift.dim() != 3 or shift.shape[0] != b or shift.shape[2] != d or shift.shape[1] not in (1, n):
        raise ValueError(f"tables are {tuple(shift.shape)}, expected {(b, n, d)} or {(b, 1, d)}")
    _check(load().vx_adaln_modulate_ex(_ptr(x), _ptr(shift), _ptr(scale), _ptr(y), b, n, d,
                                       shift.shape[1], eps, _dtype_code(x), _dtype_code(shift),
                                       _dtype_code(y), _stream(stream)))
    return y


def rope3d_apply(q, k, rope: RopeDesc, stream=None):
    """Rotate q and/or k ([B, N, H, d]) in place."""
    ref = q if q is not None else k
    if ref is None:
        raise ValueError("q and k are both None")
    _same(ref, k if q is not None else None, names=("q", "k"))
    b, n, h, d = ref.shape
    _check(load().vx_rope3d_apply(_ptr(q), _ptr(k), b, n, h, d, ctypes.byref(rope),
                                  _dtype_code(ref), _stream(stream)))


def _check_lse(lse, b, h, n, name="lse"):
    if lse is None:
        return
    import torch
    if (not lse.is_cuda or not lse.is_contiguous() or lse.dtype != torch.float32
            or tuple(lse.shape) != (b, h, n)):
        raise ValueError(f"{name} must be a contiguous float32 GPU tensor of shape {(b, h, n)}")


def flash_attn_fwd(q, k, v, o, lse=None, softmax_scale: float = 0.0,
                   rope_q: RopeDesc | None = None, stream=None):
    """o = softmax(scale q k^T) v for [B, N, H, d] tensors; optional lse [B, H, N]."""
    _same(q, k, v, o, names=("q", "k", "v", "o"))
    b, n, h, d = q.shape
    _check_lse(lse, b, h, n)
    _check(load().vx_flash_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), b, n, h, d,
                                    softmax_scale,
                                    ctypes.byref(rope_q) if rope_q is not None else None,
                                    _dtype_code(q), _stream(stream)))
    return o


def flash_attn_fwd_kv(q, k, v, o, lse=None, softmax_scale: float = 0.0,
                      rope_q: RopeDesc | None = None, stream=None):
    """Attention of q, o [B, Nq, H, d] over k, v [B, Nkv, H, d]; optional lse [B, H, Nq]."""
    _same(q, o, names=("q", "o"))
    _same(k, v, names=("k", "v"))
    b, nq, h, d = q.shape
    if k.dtype != q.dtype or k.shape[0] != b or tuple(k.shape[2:]) != (h, d):
        raise ValueError(f"k is {tuple(k.shape)} {k.dtype}, q is {tuple(q.shape)} {q.dtype}")
    nk = k.shape[1]
    _check_lse(lse, b, h, nq)
    _check(load().vx_flash_attn_fwd_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), b, nq, nk,
                                       h, d, softmax_scale,
                                       ctypes.byref(rope_q) if rope_q is not None else None,
                                       _dtype_code(q), _stream(stream)))
    return o


def flash_attn_fwd_masked(q, k, v, o, key_pad, lse=None, softmax_scale: float = 0.0,
                          rope_q: RopeDesc | None = None, stream=None):
    """As flash_attn_fwd_kv; keys lo <= j < hi of sample b (key_pad[b] = (lo, hi)) take no weight."""
    _same(q, o, names=("q", "o"))
    _same(k, v, names=("k", "v"))
    b, nq, h, d = q.shape
    if k.dtype != q.dtype or k.shape[0] != b or tuple(k.shape[2:]) != (h, d):
        raise ValueError(f"k is {tuple(k.shape)} {k.dtype}, q is {tuple(q.shape)} {q.dtype}")
    pads = [(int(lo), int(hi)) for lo, hi in key_pad]
    if len(pads) != b:
        raise ValueError(f"key_pad has {len(pads)} entries, batch is {b}")
    arr = (ctypes.c_int32 * (2 * b))(*[x for p in pads for x in p])
    _check_lse(lse, b, h, nq)
    _check(load().vx_flash_attn_fwd_masked(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), b, nq,
                                           k.shape[1], h, d, softmax_scale,
                                           ctypes.byref(rope_q) if rope_q is not None else None,
                                           ctypes.cast(arr, ctypes.c_void_p), _dtype_code(q),
                                           _stream(stream)))
    return o


def attn_merge2(o_a, lse_a, o_b, lse_b, o, lse=None, stream=None):
    """Merge two partial attention results ([B, N, H, d] + lse [B, H, N]) by their LSEs."""
    _same(o_a, o_b, o, names=("o_a", "o_b", "o"))
    b, n, h, d = o_a.shape
    for name, t in (("lse_a", lse_a), ("lse_b", lse_b)):
        if t is None:
            raise ValueError(f"{name} is required")
        _check_lse(t, b, h, n, name)
    _check_lse(lse, b, h, n)
    _check(load().vx_attn_merge2(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o),
                                 _ptr(lse), b, n, h, d, _dtype_code(o_a), _stream(stream)))
    return o
