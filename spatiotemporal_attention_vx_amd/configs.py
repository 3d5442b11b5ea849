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
    sp: int = 1             # sequence-parallel degree this is one GPU's share of
    pairing: int = 0        # RoPE pairs: 0 adjacent, 1 halves of the head, 2 halves of each band

    @property
    def adaln_rows(self) -> int:
        """Tokens one GPU modulates: its token shard, the largest of an even split."""
        return -(-self.n_tokens // self.sp)

    @property
    def adaln_hidden(self) -> int:
        """AdaLN row width: the model width, all heads (sp * heads * head_dim)."""
        return self.sp * self.heads * self.head_dim

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
        return 4.0 * self.adaln_rows * self.adaln_hidden * self.elem_bytes() * self.batch

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

# One GPU's share of a workload under Ulysses sequence parallelism over P
# GPUs (vidax paper §2 "Spatiotemporal tensor and sequence sharding": tokens
# are sharded for the per-token work, an all-to-all regathers the sequence
# and shards the heads for attention; §4, Table 2 runs Wan2.2 A14B with
# SP 2 and CogVideoX1.5 with SP 4).  A GPU then attends over all N tokens
# with H/P heads (RoPE is applied in that layout too, where every token's
# grid position is global) and modulates ceil(N/P) tokens at the full model
# width.  The all-to-alls themselves need more than one GPU and are not
# part of these shapes.
SP_WORKLOADS = {
    "mid_sp2": Workload("mid_sp2", 5, (21, 30, 52), 0, 20, 128, "bf16", (44, 42, 42),
                        oracle_rows=256, sp=2),
    "large_sp2": Workload("large_sp2", 6, (21, 45, 80), 0, 20, 128, "bf16", (44, 42, 42),
                          oracle_rows=256, sp=2),
    "large_sp8": Workload("large_sp8", 7, (21, 45, 80), 0, 5, 128, "bf16", (44, 42, 42),
                          oracle_rows=256, sp=8),
    "mixed_sp2": Workload("mixed_sp2", 8, (21, 48, 85), 226, 24, 64, "bf16", (16, 24, 24),
                          oracle_rows=256, sp=2),
    "mixed_sp4": Workload("mixed_sp4", 9, (21, 48, 85), 226, 12, 64, "bf16", (16, 24, 24),
                          oracle_rows=256, sp=4),
}


# Model-family shapes beyond the five grids.  CogVideoX1.5 patches two
# latent frames into one token (temporal patch 2), so its 1360x768 / 81-frame
# video is an 11 x 48 x 85 token grid; with its 226 text tokens that is
# 45,106 tokens, the "about 45k" joint-attention length the vidax paper
# reports for it (§4, Table 3, and the agihunt.info summary).  48 heads x
# 64, RoPE bands 16/24/24 as for the mixed workload.
FAMILY_WORKLOADS = {
    "cogvx15": Workload("cogvx15", 10, (11, 48, 85), 226, 48, 64, "bf16", (16, 24, 24),
                        oracle_rows=256),
}


def get(name: str) -> Workload:
    """A workload by name: one of WORKLOADS, SP_WORKLOADS or FAMILY_WORKLOADS."""
    for table in (WORKLOADS, SP_WORKLOADS, FAMILY_WORKLOADS):
        if name in table:
            return table[name]
    known = sorted(WORKLOADS) + sorted(SP_WORKLOADS) + sorted(FAMILY_WORKLOADS)
    raise KeyError(f"unknown workload {name!r}; known: {known}")


# The measured workload: 75,600 tokens, 40 heads x 128.
BENCH_WORKLOAD = "large"
