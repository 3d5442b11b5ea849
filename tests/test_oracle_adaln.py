"""Pins for the AdaLN oracle (CPU only).

Each check ties the oracle to something other than itself: a library
LayerNorm, rows whose normalised value is known in closed form, and
invariants of the definition.
"""
import numpy as np
import pytest
import torch

import oracle
from spatiotemporal_attention_vx_amd import configs, inputs


def _rng(seed=1):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("eps", [1e-6, 1e-2])
def test_zero_modulation_is_library_layer_norm(eps):
    # Includes rows of tiny variance, where eps placement matters.
    g = _rng()
    x = g.standard_normal((64, 128))
    x[:8] *= 1e-4
    x += 3.0 * g.standard_normal((64, 1))
    z = np.zeros_like(x)
    y = oracle.adaln_modulate(x, z, z, eps)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (128,), eps=eps).numpy()
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12)


def test_closed_form_plus_minus_one_row():
    # Row alternating +-c around mean m has mean m and variance c^2, so
    # LN(x)_i = +-c / sqrt(c^2 + eps); modulation then is explicit.
    D, c, m, eps = 16, 2.0, 0.75, 1e-6
    x = m + c * np.array([1.0, -1.0] * (D // 2))[None, :]
    g = _rng(2)
    shift = g.normal(0, 0.1, (1, D))
    scale = g.normal(0, 0.1, (1, D))
    y = oracle.adaln_modulate(x, shift, scale, eps)
    sign = np.array([1.0, -1.0] * (D // 2))
    expect = sign * c / np.sqrt(c * c + eps) * (1.0 + scale) + shift
    np.testing.assert_allclose(y, expect, rtol=0, atol=1e-14)


def test_constant_row_gives_shift():
    g = _rng(3)
    x = np.full((4, 32), 5.5)
    shift, scale = g.normal(0, 0.1, (4, 32)), g.normal(0, 0.1, (4, 32))
    y = oracle.adaln_modulate(x, shift, scale, 1e-6)
    np.testing.assert_array_equal(y, shift)


def test_affine_invariance_of_normalisation():
    g = _rng(4)
    x = g.standard_normal((8, 96))
    z = np.zeros_like(x)
    a, b = 3.7, -1.25
    y1 = oracle.adaln_modulate(x, z, z, 0.0)
    y2 = oracle.adaln_modulate(a * x + b, z, z, 0.0)
    np.testing.assert_allclose(y1, y2, rtol=0, atol=1e-12)


def test_zero_modulation_moments():
    g = _rng(5)
    x = g.standard_normal((16, 64)) * 0.01
    eps = 1e-4
    z = np.zeros_like(x)
    y = oracle.adaln_modulate(x, z, z, eps)
    var = x.var(axis=1)
    np.testing.assert_allclose(y.sum(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose((y * y).mean(axis=1), var / (var + eps), rtol=1e-12)


def test_modulation_is_per_token():
    # Changing one token's scale/shift changes only that token's output.
    g = _rng(6)
    x = g.standard_normal((6, 32))
    shift, scale = g.normal(0, 0.1, (6, 32)), g.normal(0, 0.1, (6, 32))
    y1 = oracle.adaln_modulate(x, shift, scale)
    shift2, scale2 = shift.copy(), scale.copy()
    shift2[2] += 1.0
    scale2[2] *= -3.0
    y2 = oracle.adaln_modulate(x, shift2, scale2)
    rows = [r for r in range(6) if r != 2]
    np.testing.assert_array_equal(y1[rows], y2[rows])
    assert np.abs(y1[2] - y2[2]).min() > 0


def test_tiny_workload_matches_library_path():
    # Whole Tiny workload: library LayerNorm then explicit modulation.
    wl = configs.WORKLOADS["tiny"]
    x, sh, sc = (inputs.values(a).astype(np.float64) for a in inputs.adaln_inputs(wl))
    ln = torch.nn.functional.layer_norm(torch.from_numpy(x), (wl.hidden,), eps=wl.eps).numpy()
    np.testing.assert_allclose(oracle.adaln_modulate(x, sh, sc, wl.eps), ln * (1 + sc) + sh,
                               rtol=0, atol=1e-12)


# ---- one modulation row per sample (Wan2.1)

def test_per_sample_closed_form():
    # Rows of +-c: LN gives +-c / sqrt(c^2 + eps) exactly, then sample b's row.
    g = _rng(7)
    B, N, D, c, eps = 3, 5, 16, 0.75, 1e-6
    sign = np.array([1.0, -1.0] * (D // 2))
    x = np.broadcast_to(sign * c, (B, N, D)).copy()
    shift, scale = g.normal(0, 0.1, (B, D)), g.normal(0, 0.1, (B, D))
    y = oracle.adaln_modulate_per_sample(x, shift, scale, eps)
    expect = sign * c / np.sqrt(c * c + eps) * (1.0 + scale[:, None, :]) + shift[:, None, :]
    np.testing.assert_allclose(y, np.broadcast_to(expect, (B, N, D)), rtol=0, atol=1e-14)


def test_per_sample_zero_tables_is_library_layer_norm():
    g = _rng(8)
    x = g.standard_normal((2, 7, 48))
    z = np.zeros((2, 48))
    y = oracle.adaln_modulate_per_sample(x, z, z, 1e-5)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (48,), eps=1e-5).numpy()
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12)


def test_per_sample_equals_per_token_with_repeated_rows():
    g = _rng(9)
    x = g.standard_normal((3, 6, 40))
    shift, scale = g.normal(0, 0.1, (3, 40)), g.normal(0, 0.1, (3, 40))
    rep = lambda t: np.repeat(t[:, None, :], 6, axis=1)
    np.testing.assert_allclose(oracle.adaln_modulate_per_sample(x, shift, scale),
                               oracle.adaln_modulate(x, rep(shift), rep(scale)),
                               rtol=0, atol=1e-15)


def test_per_sample_row_reaches_only_its_sample():
    g = _rng(10)
    x = g.standard_normal((3, 4, 32))
    shift, scale = g.normal(0, 0.1, (3, 32)), g.normal(0, 0.1, (3, 32))
    y1 = oracle.adaln_modulate_per_sample(x, shift, scale)
    shift2, scale2 = shift.copy(), scale.copy()
    shift2[1] += 1.0
    scale2[1] *= -2.0
    y2 = oracle.adaln_modulate_per_sample(x, shift2, scale2)
    np.testing.assert_array_equal(y1[[0, 2]], y2[[0, 2]])
    assert np.abs(y1[1] - y2[1]).min() > 0          # every token of sample 1 moves
