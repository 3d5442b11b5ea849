"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle runs.

This module draws random numbers and rounds them to the storage type; it
holds none of the attention, RoPE or LayerNorm arithmetic.

Recipe
------
* Every tensor is a row-major ``[rows, width]`` float32 draw from numpy's
  PCG64, split into chunks of ``CHUNK_ROWS`` rows.  Chunk ``c`` of tensor
  ``tensor_id`` for workload ``config_id`` comes from
  ``SeedSequence([seed, config_id, tensor_id, c])``, so any subset of rows
  can be regenerated without drawing the rest, and the result does not
  depend on how many rows are drawn at once.
* Values are ``N(0, std)`` with ``std`` the standard deviation (1 for x, Q,
  K, V; 0.1 for the modulation shift and scale).
* bf16 tensors are rounded from float32 to bfloat16 on the host with
  round-to-nearest-even, before they reach the device: the vidax paper
  (arXiv 2609.18077, §2, "JIT compilation and memory ergonomics") casts
  precision down on the host before placement.  The device and the oracle
  then see the same rounded values; the oracle upcasts them exactly.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

CHUNK_ROWS = 4096

# tensor ids entering the seed
T_X, T_SHIFT, T_SCALE, T_Q, T_K, T_V, T_ROWS = range(7)


def _chunk(seed, config_id, tensor_id, c, n_rows, width):
    lo = c * CHUNK_ROWS
    hi = min(lo + CHUNK_ROWS, n_rows)
    g = np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([seed, config_id, tensor_id, c])))
    return g.standard_normal((hi - lo, width), dtype=np.float32)


def _workers():
    return max(1, min(16, os.cpu_count() or 1))


def normal_rows(seed: int, config_id: int, tensor_id: int, n_rows: int,
                width: int, std: float = 1.0, rows=None, dtype: str = "f32") -> np.ndarray:
    """N(0, std) draw of shape [n_rows, width] (or [len(rows), width]).

    Returned in storage form for ``dtype``: float32, or bf16 bits (uint16).
    Chunks are drawn in worker threads (numpy releases the GIL while it
    fills an array); the result does not depend on the thread count.
    """
    out_dt = np.uint16 if dtype == "bf16" else np.float32
    if rows is None:
        out = np.empty((n_rows, width), dtype=out_dt)

        def fill(c):
            a = _chunk(seed, config_id, tensor_id, c, n_rows, width)
            if std != 1.0:
                a *= np.float32(std)
            out[c * CHUNK_ROWS:c * CHUNK_ROWS + a.shape[0]] = storage(a, dtype)

        n_chunks = (n_rows + CHUNK_ROWS - 1) // CHUNK_ROWS
        with cf.ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(n_chunks)))
        return out
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, width), dtype=np.float32)
    chunk_of = rows // CHUNK_ROWS
    for c in np.unique(chunk_of):
        block = _chunk(seed, config_id, tensor_id, int(c), n_rows, width)
        sel = chunk_of == c
        out[sel] = block[rows[sel] - int(c) * CHUNK_ROWS]
    if std != 1.0:
        out *= np.float32(std)
    return storage(out, dtype)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); uint16 bits.

    NaN stays NaN (quiet bit forced); infinities and overflow go to inf.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | np.uint32(0x40)).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """Host storage form of a float32 draw: float32, or bf16 bits as uint16."""
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        return to_bf16_bits(a)
    raise ValueError(f"unknown dtype {dtype!r}")


def values(a: np.ndarray) -> np.ndarray:
    """The float32 values a storage array holds (bf16 bits are widened)."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a)
    return np.asarray(a, dtype=np.float32)


def tensor(wl, seed: int, tensor_id: int, std: float = 1.0, rows=None) -> np.ndarray:
    """One [rows, heads*head_dim] input of workload ``wl`` in storage form.

    Batch entries are stacked along rows (row b*N + n is token n of batch b).
    """
    n = wl.n_tokens * wl.batch
    return normal_rows(seed, wl.config_id, tensor_id, n, wl.hidden, std, rows, wl.dtype)


def attention_inputs(wl, seed: int = 0):
    """Q, K, V in storage form, each shaped [batch, N, heads, head_dim]."""
    shape = (wl.batch, wl.n_tokens, wl.heads, wl.head_dim)
    return tuple(tensor(wl, seed, t).reshape(shape) for t in (T_Q, T_K, T_V))


def adaln_inputs(wl, seed: int = 0):
    """x ~ N(0,1), shift ~ N(0,0.1), scale ~ N(0,0.1); each [batch*rows, width].

    rows and width are the tokens and model width one GPU modulates
    (``wl.adaln_rows``, ``wl.adaln_hidden``): N and heads*head_dim unless
    ``wl`` is one GPU's share of a sequence-parallel run.
    """
    n = wl.adaln_rows * wl.batch
    return tuple(normal_rows(seed, wl.config_id, t, n, wl.adaln_hidden, std, None, wl.dtype)
                 for t, std in ((T_X, 1.0), (T_SHIFT, 0.1), (T_SCALE, 0.1)))


def adaln_inputs_ex(wl, x_dtype: str, mod_dtype: str, per_sample: bool, seed: int = 0):
    """AdaLN inputs with per-tensor storage types and optional per-sample tables.

    x ~ N(0,1) as [batch, rows, width] in ``x_dtype``; shift, scale ~
    N(0,0.1) in ``mod_dtype`` as [batch, rows, width], or [batch, 1, width]
    when ``per_sample`` (rows and width as for ``adaln_inputs``).  The x
    draw is the same as ``adaln_inputs``'s, before its storage rounding.
    """
    rows, width, b = wl.adaln_rows, wl.adaln_hidden, wl.batch
    x = normal_rows(seed, wl.config_id, T_X, rows * b, width, 1.0, None, x_dtype)
    mrows = b if per_sample else rows * b
    tabs = tuple(normal_rows(seed, wl.config_id, t, mrows, width, 0.1, None, mod_dtype)
                 for t in (T_SHIFT, T_SCALE))
    mshape = (b, 1 if per_sample else rows, width)
    return (x.reshape(b, rows, width),) + tuple(t.reshape(mshape) for t in tabs)


def sample_rows(wl, seed: int = 0, count: int = 0) -> np.ndarray:
    """Sorted query rows the oracle checks on a large workload.

    Always holds the first and last token and, with a text prefix, the last
    text token and the first video token, so the prefix/video boundary is
    covered; the rest is a seeded uniform draw without replacement.
    """
    n = wl.n_tokens
    count = count or wl.oracle_rows
    if count <= 0 or count >= n:
        return np.arange(n)
    fixed = {0, n - 1}
    if wl.n_prefix > 0:
        fixed |= {wl.n_prefix - 1, wl.n_prefix}
    g = np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([seed, wl.config_id, T_ROWS])))
    pool = np.setdiff1d(np.arange(n), np.fromiter(fixed, dtype=np.int64))
    extra = g.choice(pool, size=count - len(fixed), replace=False)
    return np.sort(np.concatenate([np.fromiter(fixed, dtype=np.int64), extra]))
