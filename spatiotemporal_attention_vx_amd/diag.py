"""Measurement aid (not the hot path): time the bf16 MFMA ceiling on given data.

Loads ``libvx_diag.so`` (``diag/mfma_ceiling.hip``) and times its pure
``v_mfma_f32_32x32x16_bf16`` loop with HIP events on the launch stream.  The
chip lowers its clock under dense MFMA work to stay within its power limit,
and the limit depends on how many operand bits toggle, so the rate this loop
reaches on N(0,1) bf16 operands is the ceiling the attention kernel's own
data allows, beside the nominal 2.5 PFLOP/s.
"""
from __future__ import annotations

import ctypes
import os

from . import build as _build

_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    path = path or _build.DIAG_LIB
    if not os.path.exists(path):
        _build.build_diag()
    lib = ctypes.CDLL(path)
    lib.vx_diag_mfma_bf16_loop.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_void_p]
    lib.vx_diag_mfma_bf16_loop.restype = ctypes.c_int
    lib.vx_diag_mfma_bf16_loop_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.vx_diag_mfma_bf16_loop_flops.restype = ctypes.c_double
    _lib = lib
    return lib


OPERAND_BYTES_PER_WORKGROUP = 8 * 16 * 64 * 16   # 8 waves x 16 fragments x 64 lanes x 16 B


def mfma_loop(operands, out, workgroups: int, iters: int, stream=None) -> None:
    """One launch; operands: bf16 GPU tensor of workgroups * 65,536 elements,
    out: float32 GPU tensor of workgroups * 512 elements."""
    import torch
    if operands.dtype != torch.bfloat16 or not operands.is_cuda or not operands.is_contiguous():
        raise ValueError("operands must be a contiguous bf16 GPU tensor")
    if operands.numel() * 2 < workgroups * OPERAND_BYTES_PER_WORKGROUP:
        raise ValueError("operands too small for this many workgroups")
    if out.dtype != torch.float32 or not out.is_cuda or out.numel() < workgroups * 512:
        raise ValueError("out must be a float32 GPU tensor of workgroups * 512 elements")
    st = (stream or torch.cuda.current_stream()).cuda_stream
    rc = load().vx_diag_mfma_bf16_loop(operands.data_ptr(), out.data_ptr(), workgroups, iters, st)
    if rc != 0:
        raise RuntimeError(f"vx_diag_mfma_bf16_loop returned {rc}")


def ceiling(kind: str = "normal", workgroups: int = 1024, iters: int = 64000, reps: int = 3,
            warmup: int = 2, seed: int = 0) -> dict:
    """Median TFLOP/s of the loop over `reps` launches after `warmup`, on N(0,1)
    bf16 operands (kind 'normal') or zeros."""
    import torch
    dev = torch.device("cuda:0")
    n = workgroups * OPERAND_BYTES_PER_WORKGROUP // 2
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    ops = (torch.randn(n, device=dev, generator=g).to(torch.bfloat16) if kind == "normal"
           else torch.zeros(n, device=dev, dtype=torch.bfloat16))
    out = torch.empty(workgroups * 512, device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        mfma_loop(ops, out, workgroups, iters, stream)
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        mfma_loop(ops, out, workgroups, iters, stream)
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = sorted(times)[len(times) // 2]
    flops = load().vx_diag_mfma_bf16_loop_flops(workgroups, iters)
    return {"tflops": flops / (ms * 1e-3) / 1e12, "ms": ms, "operands": kind,
            "launch": f"{workgroups} workgroups x 8 waves x {8 * iters} MFMAs"}
