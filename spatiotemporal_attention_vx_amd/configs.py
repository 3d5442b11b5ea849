"""The five token-grid workloads of the video-DiT block hot path.

Each workload is one attention layer of a video diffusion transformer at a
given latent grid: full non-causal attention over every patchified token,
3D RoPE on Q and K, and per-token AdaLN modulation of an activation row of
width ``heads * head_dim``.  Grid shapes mirror the latent grids of the
models benchmarked in the vidax paper (arXiv 2609.18077, §4, Table 2):
the 21x30x52 grid is Wan2.2 A14B at 832x480/81 frames, 21x45x80 is Wan2.1
14B at 1280x720/81, and 226 text tokens + 21x48x85 is a CogVideoX1.5-style
joint text+video sequence (§3.1, "CogVideoX").  The strides that map pixels
to tokens are not given on the pages; the grids are taken as given.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    config_id: int          # enters the input seed (see inputs.py)
    grid: tuple             # latent token grid (T, H, W); time outermost
    n_prefix: int           # leading unrotated (text) tokens
    heads: int
    head_dim: int
    dtype: str              # "f32" or "bf16": storage and I/O type
    split: tuple            # RoPE band widths (d_t, d_h, d_w), sum == head_dim
    theta: float = 10000.0  # RoPE base
    eps: float = 1e-6       # LayerNorm epsilon
    batch: int = 1
    oracle_rows: int = 0    # 0: the oracle checks every row; else a sample

    @property
    def n_video(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def n_tokens(self) -> int:
        return self.n_prefix + self.n_video

    @property
    def hidden(self) -> int:
        return self.heads * self.head_dim

    def attn_flops(self) -> float:
        """Two GEMMs (QK^T and PV) at 2 flop per MAC: 4 N^2 d H per batch."""
        n = self.n_tokens
        return 4.0 * n * n * self.head_dim * self.heads * self.batch

    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def adaln_bytes(self) -> float:
        """x, shift, scale read once and y written once."""
        return 4.0 * self.n_tokens * self.hidden * self.elem_bytes() * self.batch

    def rope_bytes(self) -> float:
        """Rotated rows of Q and K read and written once."""
        return 4.0 * self.n_video * self.hidden * self.elem_bytes() * self.batch


WORKLOADS = {
    "tiny": Workload("tiny", 0, (3, 4, 4), 0, 2, 64, "f32", (16, 24, 24)),
    "small": Workload("small", 1, (4, 32, 32), 0, 8, 128, "bf16", (44, 42, 42)),
    "mid": Workload("mid", 2, (21, 30, 52), 0, 40, 128, "bf16", (44, 42, 42),
                    oracle_rows=256),
    "large": Workload("large", 3, (21, 45, 80), 0, 40, 128, "bf16", (44, 42, 42),
                      oracle_rows=256),
    "mixed": Workload("mixed", 4, (21, 48, 85), 226, 48, 64, "bf16", (16, 24, 24),
                      oracle_rows=256),
}

# The measured workload: 75,600 tokens, 40 heads x 128.
BENCH_WORKLOAD = "large"
