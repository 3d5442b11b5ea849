"""Per-token AdaLN modulation, fp64 (oracle; test infrastructure only).

Source: the vidax paper (arXiv 2609.18077), §2 "Spatiotemporal tensor and
sequence sharding" and §3.1 (Table 1, Wan2.2 "per-token AdaLN"), and the
agihunt.info summary of the same paper: Wan2.2 applies a LayerNorm and then
a scale and shift that differ for every token, which is why activations, not
weights, bound its memory.  The vidax blog post "Weight offloading: trading
bandwidth for memory", section "A14B (Wan2.2)", adds that this per-token
modulation tensor alone is several GB at high resolution.

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
