"""Full non-causal attention, fp64 (oracle; test infrastructure only).

Source: the vidax paper (arXiv 2609.18077), §1 "Spatiotemporal constraints
in video generation" (full self-attention over all patch tokens of a
multi-frame latent) and §2 "3D RoPE, 3D VAEs, and flash attention"
(unmasked attention goes to flash-attention kernels, Dao et al. 2022, which
give the exact softmax attention without storing the whole score matrix).
The agihunt.info summary states the same.  The oracle computes the plain
definition, materialising each score row in full:

    s_j = (q . k_j) * scale            over all N keys
    p_j = exp(s_j - max s) / sum_j exp(s_j - max s)
    o   = sum_j p_j v_j
    lse = max s + ln sum_j exp(s_j - max s)

No mask, no causality, no dropout.  scale defaults to 1 / sqrt(head_dim).
The queries and the keys may be different token sets (q has its own row
count), which is attention over one part of a key-split sequence.

``attention_masked`` leaves a range of keys out of the softmax (key
padding, e.g. the padded tail of a joint sequence's text prefix).

``merge_lse`` combines two such partial results over disjoint key sets.
From the definition, exp(lse) is a row's softmax denominator Z and o its
Z-weighted mean of values, so over the union
    Z = Z_a + Z_b,   o = (Z_a o_a + Z_b o_b) / Z,   lse = ln Z.
This is the step that puts a key-sharded attention back together (the
vidax paper §2 "Spatiotemporal tensor and sequence sharding" shards the
token axis across devices).
"""
from __future__ import annotations

import numpy as np

from .rope3d import rope3d_apply


def attention(q, k, v, scale: float = 0.0, rows=None, row_block: int = 512):
    """Attention outputs for the query rows ``rows`` (default: all).

    q: [N, H, d] (only the rows selected are read), k, v: [N, H, d].
    Returns (o [R, H, d] float64, lse [H, R] float64), R = len(rows).
    """
    n, heads, d = k.shape
    if scale <= 0.0:
        scale = 1.0 / np.sqrt(d)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.empty((rows.size, heads, d), dtype=np.float64)
    lse = np.empty((heads, rows.size), dtype=np.float64)
    for h in range(heads):
        kh = np.asarray(k[:, h, :], dtype=np.float64)
        vh = np.asarray(v[:, h, :], dtype=np.float64)
        for r0 in range(0, rows.size, row_block):
            sel = rows[r0:r0 + row_block]
            qh = np.asarray(q[sel, h, :], dtype=np.float64)
            s = (qh @ kh.T) * scale                           # [r, N]
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            total = e.sum(axis=1, keepdims=True)
            o[r0:r0 + sel.size, h, :] = (e @ vh) / total
            lse[h, r0:r0 + sel.size] = m[:, 0] + np.log(total[:, 0])
    return o, lse


def attention_masked(q, k, v, lo: int, hi: int, scale: float = 0.0, rows=None):
    """Attention in which keys lo <= j < hi take no weight (key padding).

    The plain definition: the softmax runs over the remaining keys only,
    so this is ``attention`` over K and V with those rows removed.  At
    least one key must remain.  Returns (o [R, H, d], lse [H, R]).
    """
    keep = np.ones(k.shape[0], dtype=bool)
    keep[lo:hi] = False
    if not keep.any():
        raise ValueError("every key is masked")
    return attention(q, k[keep], v[keep], scale, rows)


def merge_lse(o_a, lse_a, o_b, lse_b):
    """Attention over two disjoint key sets from their partial results.

    o_a, o_b: [R, H, d]; lse_a, lse_b: [H, R] (as ``attention`` returns
    them).  Returns (o [R, H, d], lse [H, R]) in float64.  A part with
    lse = -inf (no keys) has Z = 0; two such parts give o = 0, lse = -inf.
    """
    o_a, o_b = np.asarray(o_a, np.float64), np.asarray(o_b, np.float64)
    lse_a, lse_b = np.asarray(lse_a, np.float64), np.asarray(lse_b, np.float64)
    m = np.maximum(lse_a, lse_b)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    z_a = np.exp(lse_a - m_safe)           # Z_a / e^m  (0 for an empty part)
    z_b = np.exp(lse_b - m_safe)
    z = z_a + z_b
    z_safe = np.where(empty, 1.0, z)
    w_a = (z_a / z_safe).T[:, :, None]     # [R, H, 1]
    w_b = (z_b / z_safe).T[:, :, None]
    o = w_a * o_a + w_b * o_b
    lse = np.where(empty, -np.inf, m_safe + np.log(z_safe))
    return o, lse


def attention_rope(q, k, v, grid, split, theta=10000.0, n_prefix=0, scale=0.0,
                   rows=None, pairing=0):
    """RoPE on Q and K, then attention; one head at a time.

    Arguments as in ``attention``; returns (o [R, H, d], lse [H, R]).
    """
    n, heads, d = k.shape
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.empty((rows.size, heads, d), dtype=np.float64)
    lse = np.empty((heads, rows.size), dtype=np.float64)
    for h in range(heads):
        kr = rope3d_apply(k[:, h:h + 1, :], grid, split, theta, n_prefix, pairing=pairing)
        qr = rope3d_apply(q[rows, h:h + 1, :], grid, split, theta, n_prefix, tokens=rows,
                          pairing=pairing)
        # attention() indexes q by token, so place the rotated rows at 0..R-1
        oh, lh = attention(qr, kr, v[:, h:h + 1, :], scale)
        o[:, h:h + 1, :] = oh
        lse[h:h + 1, :] = lh
    return o, lse
