"""Per-token AdaLN modulation, fp64 (oracle; test infrastructure only).

Source: the vidax paper (arXiv 2609.18077), §2 "Spatiotemporal tensor and
sequence sharding" and §3.1 (Table 1, Wan2.2 "per-token AdaLN"), and the
agihunt.info summary of the same paper: Wan2.2 applies a LayerNorm and then
a scale and shift that differ for every token, which is why activations, not
weights, bound its memory.  The vidax blog post "Weight offloading: trading
bandwidth for memory", section "A14B (Wan2.2)", adds that this per-token
modulation tensor alone is several GB at high resolution.

Wan2.1 (same paper, §3.1 and Table 1) instead modulates every token of a
sample with one scale and shift row; ``adaln_modulate_per_sample`` writes
that form out.  Which dtype each tensor is stored in (bf16 or fp32: §3.2
"Weight import, precision, and verification" keeps Wan2.1's residual stream
and LTX-2.5's AdaLN tables in fp32) changes only the input values the
oracle is handed, never its fp64 arithmetic.

Readings where the pages are silent:
* modulation form ``LN(x) * (1 + scale) + shift`` (so zero modulation is a
  plain LayerNorm);
* LayerNorm without a learnable affine, biased variance (divide by D),
  epsilon inside the square root;
* statistics over the hidden axis of each token separately.
"""
from __future__ import annotations

import numpy as np


def layer_norm(x, eps: float) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) over the last axis; two passes over x."""
    x = np.asarray(x, dtype=np.float64)
    mean = x.mean(axis=-1, keepdims=True)
    var = np.square(x - mean).mean(axis=-1, keepdims=True)
    return (x - mean) / np.sqrt(var + eps)


def adaln_modulate(x, shift, scale, eps: float = 1e-6) -> np.ndarray:
    """y[n, :] = LN(x[n, :]) * (1 + scale[n, :]) + shift[n, :], in float64.

    ``x``, ``shift`` and ``scale`` share the shape [..., D]; the result has
    that shape and dtype float64.
    """
    shift = np.asarray(shift, dtype=np.float64)
    scale = np.asarray(scale, dtype=np.float64)
    return layer_norm(x, eps) * (1.0 + scale) + shift


def adaln_modulate_per_sample(x, shift, scale, eps: float = 1e-6) -> np.ndarray:
    """y[b, n, :] = LN(x[b, n, :]) * (1 + scale[b, :]) + shift[b, :], in float64.

    ``x`` is [B, N, D]; ``shift`` and ``scale`` are [B, D], one row per
    sample, the same for all N tokens of that sample.
    """
    ln = layer_norm(x, eps)                                 # [B, N, D]
    shift = np.asarray(shift, dtype=np.float64)[:, None, :]
    scale = np.asarray(scale, dtype=np.float64)[:, None, :]
    return ln * (1.0 + scale) + shift
