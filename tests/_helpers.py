"""Helpers shared by the GPU parity tests: host<->device moves and the
tolerance check.  Tolerances: fp32 outputs within 1e-5 max abs of the fp64
oracle; bf16 outputs within 2e-2 max abs and 1e-2 relative L2.
"""
import sys

import numpy as np

from spatiotemporal_attention_vx_amd import inputs

F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 1e-2


def say(*a):
    """Name the case before a GPU step, flushed, so a failure names it."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    """Host storage array (float32, or bf16 bits as uint16) -> GPU tensor."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a.astype(np.float32, copy=False)).cuda()


def host(t):
    """GPU tensor -> float32 numpy values (bf16 widened exactly)."""
    import torch
    if t.dtype == torch.bfloat16:
        return inputs.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.float().cpu().numpy()


def bits(t):
    """GPU tensor -> raw bits as a numpy array (for bit-exact comparisons)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.view(torch.int32).cpu().numpy()


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got - ref
    max_abs = float(np.abs(d).max()) if d.size else 0.0
    denom = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(d) / denom) if denom > 0 else float(np.linalg.norm(d))
    return max_abs, rel


def check(got, ref, dtype, what=""):
    """Assert the stated tolerance; return (max_abs, rel_l2)."""
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    max_abs, rel = errors(got, ref)
    say(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    if dtype == "f32":
        assert max_abs <= F32_MAX_ABS, f"{what}: max abs {max_abs:.3e} > {F32_MAX_ABS}"
    else:
        assert max_abs <= BF16_MAX_ABS, f"{what}: max abs {max_abs:.3e} > {BF16_MAX_ABS}"
        assert rel <= BF16_REL_L2, f"{what}: rel L2 {rel:.3e} > {BF16_REL_L2}"
    return max_abs, rel


class ChunkCheck:
    """The tolerance check over a tensor compared chunk by chunk: max abs over
    all chunks, relative L2 from the summed squares of every chunk."""

    def __init__(self, dtype, what):
        self.dtype, self.what = dtype, what
        self.max_abs, self.d2, self.r2, self.n = 0.0, 0.0, 0.0, 0

    def add(self, got, ref):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        assert np.all(np.isfinite(got)), f"{self.what}: non-finite output"
        d = got - ref
        if d.size:
            self.max_abs = max(self.max_abs, float(np.abs(d).max()))
        self.d2 += float(np.sum(d * d))
        self.r2 += float(np.sum(ref * ref))
        self.n += d.size

    def done(self):
        rel = float(np.sqrt(self.d2 / self.r2)) if self.r2 > 0 else float(np.sqrt(self.d2))
        say(f"  {self.what}: {self.n} values, max_abs={self.max_abs:.3e} rel_l2={rel:.3e}")
        if self.dtype == "f32":
            assert self.max_abs <= F32_MAX_ABS, f"{self.what}: max abs {self.max_abs:.3e}"
        else:
            assert self.max_abs <= BF16_MAX_ABS, f"{self.what}: max abs {self.max_abs:.3e}"
            assert rel <= BF16_REL_L2, f"{self.what}: rel L2 {rel:.3e}"
        return self.max_abs, rel
