"""MI355X (gfx950) video-DiT block hot path: per-token AdaLN, 3D RoPE and
flash attention as HIP kernels behind a C ABI (``include/vx.h``).

The Python side only marshals arguments (``binding``), describes the
workloads (``configs``) and draws seeded synthetic inputs (``inputs``).
"""
from . import configs, inputs
from .binding import (RopeDesc, VxError, adaln_modulate, flash_attn_fwd, load,
                      rope3d_apply)

__all__ = ["configs", "inputs", "RopeDesc", "VxError", "adaln_modulate", "flash_attn_fwd",
           "load", "rope3d_apply"]
