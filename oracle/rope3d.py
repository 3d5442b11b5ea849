"""3D rotary position embedding, fp64 (oracle; test infrastructure only).

Source: the vidax paper (arXiv 2609.18077), §2 "3D RoPE, 3D VAEs, and flash
attention", and its agihunt.info summary: each family rotates Q and K with a
3D RoPE whose time, height and width parts use separate frequency bands, and
the families' conventions differ, so each keeps its own.  §3.1 ("CogVideoX")
describes joint text+video attention, where text tokens carry no 3D
position.  §2 "Spatiotemporal tensor and sequence sharding" splits tokens
along time, which yields contiguous shards only when time is the outermost
token axis.

The pages print no formula.  Readings taken here (one convention, stated):
* token order: ``n_prefix`` text tokens first, then the video grid with t
  outermost, then h, then w; video positions restart at 0 after the prefix;
  positions are the integer grid indices;
* the head dimension is split into contiguous bands [t | h | w] of widths
  (d_t, d_h, d_w);
* within a band of width d_a, pair j turns by angle
  pos_a * theta ** (-2 j / d_a); the angles of all bands, listed t, h, w,
  form the head's d/2 angles;
* which two elements form pair j depends on the family's convention
  (``pairing``): 0, adjacent elements 2j, 2j+1 of the band; 1, the head
  split in halves, the k-th angle of the [t | h | w] list turning elements
  k and k + d/2 of the head; 2, each band split in halves, elements j and
  j + d_a/2 of the band;
* a pair (a, b) read as the complex number a + i b is multiplied by
  exp(i * angle);
* the same angles apply to every head and to Q and K; V is not rotated;
  text tokens are left unchanged.
"""
from __future__ import annotations

import numpy as np


def token_positions(grid, n_prefix: int = 0):
    """(t, h, w) integer positions of the video tokens, in token order."""
    T, H, W = (int(g) for g in grid)
    v = np.arange(T * H * W, dtype=np.int64)
    return v // (H * W), (v // W) % H, v % W


def rope_angles(grid, split, theta: float = 10000.0, n_prefix: int = 0) -> np.ndarray:
    """Angles [T*H*W, head_dim // 2] for the video tokens (float64)."""
    pos = token_positions(grid, n_prefix)
    cols = []
    for p, width in zip(pos, split):
        j = np.arange(width // 2, dtype=np.float64)
        freq = np.power(float(theta), -2.0 * j / float(width))
        cols.append(np.outer(p.astype(np.float64), freq))
    return np.concatenate(cols, axis=1)


def pair_elements(split, pairing: int = 0):
    """(first, second) element indices of the head's d/2 pairs, in angle order."""
    d = int(sum(split))
    k = np.arange(d // 2)
    if pairing == 0:
        return 2 * k, 2 * k + 1
    if pairing == 1:
        return k, k + d // 2
    if pairing == 2:
        firsts, seconds, start = [], [], 0
        for width in split:
            j = np.arange(width // 2)
            firsts.append(start + j)
            seconds.append(start + j + width // 2)
            start += width
        return np.concatenate(firsts), np.concatenate(seconds)
    raise ValueError(f"unknown pairing {pairing}")


def rope3d_apply(x, grid, split, theta: float = 10000.0, n_prefix: int = 0,
                 tokens=None, pairing: int = 0) -> np.ndarray:
    """Rotate x of shape [N, heads, head_dim]; returns a float64 copy.

    ``tokens`` (optional) lists the token indices the rows of x hold; by
    default x holds all N = n_prefix + T*H*W tokens in order.  ``pairing``
    picks which elements form each rotated pair (see the module notes).
    """
    x = np.array(x, dtype=np.float64, copy=True)
    d = x.shape[-1]
    if sum(split) != d or any(s % 2 for s in split):
        raise ValueError("band widths must be even and sum to head_dim")
    n_video = int(np.prod(grid))
    if tokens is None:
        if x.shape[0] != n_prefix + n_video:
            raise ValueError("token count does not match prefix + grid")
        tokens = np.arange(x.shape[0])
    tokens = np.asarray(tokens, dtype=np.int64)
    if tokens.size != x.shape[0] or (tokens.size and (tokens.min() < 0 or
                                                      tokens.max() >= n_prefix + n_video)):
        raise ValueError("token indices out of range")
    video = tokens >= n_prefix
    ang = rope_angles(grid, split, theta, n_prefix)[tokens[video] - n_prefix]
    rot = np.exp(1j * ang)[:, None, :]                         # [Nv, 1, d/2]
    first, second = pair_elements(split, pairing)
    vid = x[video]
    z = (vid[..., first] + 1j * vid[..., second]) * rot
    vid[..., first] = z.real
    vid[..., second] = z.imag
    x[video] = vid
    return x
