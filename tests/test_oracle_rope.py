"""Pins for the 3D-RoPE oracle (CPU only).

Closed-form angles fix the band layout, the pairing, the per-band frequency
law and the rotation sign; invariants fix the rest.  The choice among real
families' conventions is itself a reading of the pages (parity unpinned).
"""
import math

import numpy as np
import pytest

import oracle


GRID, SPLIT = (3, 4, 4), (16, 24, 24)


def _unit(d, i):
    e = np.zeros((1, 1, d))
    e[0, 0, i] = 1.0
    return e


def test_token_order_time_outermost():
    t, h, w = oracle.token_positions((3, 4, 5))
    # token n = t*H*W + h*W + w
    assert (t[0], h[0], w[0]) == (0, 0, 0)
    assert (t[1], h[1], w[1]) == (0, 0, 1)
    assert (t[5], h[5], w[5]) == (0, 1, 0)
    assert (t[20], h[20], w[20]) == (1, 0, 0)
    assert (t[59], h[59], w[59]) == (2, 3, 4)


# (token, element index, angle) with angles fixed by the stated reading:
# t band, width 16, pair 1: theta^(-2/16) = 10000^(-1/8) = 10^(-1/2)
# t band pair 4: 10000^(-8/16) = 10^(-2);  h band (elements 16..39, width 24)
# pair 3: 10000^(-6/24) = 10^(-1), at h = 2 -> 0.2; w band (elements 40..63)
# pair 0: frequency 1, at w = 3 -> 3; w band pair 6: 10000^(-12/24) = 10^(-2).
CLOSED = [
    (16, 2, 1 * 10 ** -0.5),          # t=1: t band pair 1
    (32, 2, 2 * 10 ** -0.5),          # t=2
    (32, 8, 2 * 1e-2),                # t=2: t band pair 4
    (8, 16 + 6, 2 * 1e-1),            # h=2: h band pair 3
    (3, 40, 3.0),                     # w=3: w band pair 0
    (3, 40 + 12, 3 * 1e-2),           # w=3: w band pair 6
    (5, 0, 0.0),                      # t=0: t band untouched
]


@pytest.mark.parametrize("token,elem,angle", CLOSED)
def test_closed_form_rotation_of_unit_vector(token, elem, angle):
    d = sum(SPLIT)
    x = np.zeros((48, 1, d))
    x[token, 0, elem] = 1.0
    y = oracle.rope3d_apply(x, GRID, SPLIT)
    expect = np.zeros(d)
    expect[elem] = math.cos(angle)
    expect[elem + 1] = math.sin(angle)
    np.testing.assert_allclose(y[token, 0], expect, rtol=0, atol=1e-15)
    # odd element: (0, 1) -> (-sin, cos)
    x = np.zeros((48, 1, d))
    x[token, 0, elem + 1] = 1.0
    y = oracle.rope3d_apply(x, GRID, SPLIT)
    expect = np.zeros(d)
    expect[elem] = -math.sin(angle)
    expect[elem + 1] = math.cos(angle)
    np.testing.assert_allclose(y[token, 0], expect, rtol=0, atol=1e-15)


def test_prefix_tokens_untouched_and_positions_restart():
    g = np.random.default_rng(0)
    P = 5
    x = g.standard_normal((P + 48, 3, 64))
    y = oracle.rope3d_apply(x, GRID, SPLIT, n_prefix=P)
    np.testing.assert_array_equal(y[:P], x[:P])
    np.testing.assert_array_equal(y[P], x[P])            # position (0, 0, 0)
    y0 = oracle.rope3d_apply(x[P:], GRID, SPLIT)
    np.testing.assert_array_equal(y[P:], y0)


def test_norm_preserved_per_pair():
    g = np.random.default_rng(1)
    x = g.standard_normal((48, 2, 64))
    y = oracle.rope3d_apply(x, GRID, SPLIT)
    n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n1 = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12, atol=1e-12)


def _rot_at(vec, pos, split=SPLIT, theta=10000.0):
    """Rotate one vector [d] to position pos=(t,h,w) via a 1-token grid trick."""
    t, h, w = pos
    grid = (t + 1, h + 1, w + 1)
    n = grid[0] * grid[1] * grid[2]
    x = np.zeros((n, 1, vec.size))
    idx = t * grid[1] * grid[2] + h * grid[2] + w
    x[idx, 0] = vec
    return oracle.rope3d_apply(x, grid, split, theta)[idx, 0]


def test_scores_depend_only_on_relative_offset():
    g = np.random.default_rng(2)
    q, k = g.standard_normal(64), g.standard_normal(64)
    p, pp, delta = (1, 2, 0), (3, 0, 5), (2, 3, 1)
    s1 = _rot_at(q, p) @ _rot_at(k, pp)
    s2 = _rot_at(q, tuple(a + b for a, b in zip(p, delta))) @ \
        _rot_at(k, tuple(a + b for a, b in zip(pp, delta)))
    assert abs(s1 - s2) < 1e-12
    # and it equals <q, R(p' - p) k> when the offset is non-negative
    off = (2, 0, 5)
    p0 = (1, 0, 0)
    s3 = _rot_at(q, p0) @ _rot_at(k, tuple(a + b for a, b in zip(p0, off)))
    s4 = q @ _rot_at(k, off)
    assert abs(s3 - s4) < 1e-12


def test_composition():
    g = np.random.default_rng(3)
    v = g.standard_normal(64)
    a, b = (1, 2, 1), (1, 1, 2)
    ab = tuple(x + y for x, y in zip(a, b))
    np.testing.assert_allclose(_rot_at(_rot_at(v, a), b), _rot_at(v, ab), atol=1e-12)


def test_same_rotation_for_every_head():
    g = np.random.default_rng(4)
    x = g.standard_normal((48, 1, 64))
    y1 = oracle.rope3d_apply(x, GRID, SPLIT)
    y3 = oracle.rope3d_apply(np.repeat(x, 3, axis=1), GRID, SPLIT)
    for h in range(3):
        np.testing.assert_array_equal(y3[:, h], y1[:, 0])


def test_subset_of_tokens_matches_full():
    g = np.random.default_rng(5)
    x = g.standard_normal((7 + 48, 2, 64))
    full = oracle.rope3d_apply(x, GRID, SPLIT, n_prefix=7)
    rows = np.array([0, 6, 7, 8, 30, 54])
    sub = oracle.rope3d_apply(x[rows], GRID, SPLIT, n_prefix=7, tokens=rows)
    np.testing.assert_array_equal(sub, full[rows])


def test_rejects_bad_split():
    with pytest.raises(ValueError):
        oracle.rope3d_apply(np.zeros((48, 1, 64)), GRID, (16, 23, 25))
    with pytest.raises(ValueError):
        oracle.rope3d_apply(np.zeros((48, 1, 64)), GRID, (16, 24, 26))


# ---- half-split pairings (pairing 1: halves of the head; 2: halves of each band)

# (token, angle, (first, second) element indices under pairing 1, under pairing 2)
# for SPLIT (16, 24, 24), head_dim 64, angle list [t: 8 | h: 12 | w: 12]:
# t pair 1 is angle 1; h pair 3 is angle 8 + 3 = 11; w pair 6 is angle 26.
HALF_CLOSED = [
    (16, 1 * 10 ** -0.5, (1, 33), (1, 9)),              # t=1, t band pair 1
    (8, 2 * 1e-1, (11, 43), (19, 31)),                  # h=2, h band pair 3
    (3, 3 * 1e-2, (26, 58), (46, 58)),                  # w=3, w band pair 6
    (3, 3.0, (20, 52), (40, 52)),                       # w=3, w band pair 0
]


@pytest.mark.parametrize("token,angle,p1,p2", HALF_CLOSED)
@pytest.mark.parametrize("pairing", [1, 2])
def test_half_split_closed_form(token, angle, p1, p2, pairing):
    a, b = p1 if pairing == 1 else p2
    d = sum(SPLIT)
    for src, expect_a, expect_b in ((a, math.cos(angle), math.sin(angle)),
                                    (b, -math.sin(angle), math.cos(angle))):
        x = np.zeros((48, 1, d))
        x[token, 0, src] = 1.0
        y = oracle.rope3d_apply(x, GRID, SPLIT, pairing=pairing)
        expect = np.zeros(d)
        expect[a], expect[b] = expect_a, expect_b
        np.testing.assert_allclose(y[token, 0], expect, rtol=0, atol=1e-15)


def _to_adjacent(pairing):
    """Permutation P (written out per convention) with (P x)[2k], (P x)[2k+1] =
    the k-th pair's first and second elements."""
    if pairing == 1:
        first, second = list(range(0, 32)), list(range(32, 64))
    else:   # bands t: 0..15, h: 16..39, w: 40..63, each split in halves
        first = list(range(0, 8)) + list(range(16, 28)) + list(range(40, 52))
        second = list(range(8, 16)) + list(range(28, 40)) + list(range(52, 64))
    perm = np.empty(64, dtype=np.int64)
    perm[0::2], perm[1::2] = first, second
    return perm


@pytest.mark.parametrize("pairing", [1, 2])
def test_half_split_is_adjacent_under_a_permutation(pairing):
    g = np.random.default_rng(20 + pairing)
    x = g.standard_normal((48, 2, 64))
    perm = _to_adjacent(pairing)
    y = oracle.rope3d_apply(x, GRID, SPLIT, pairing=pairing)
    y0 = oracle.rope3d_apply(x[..., perm], GRID, SPLIT, pairing=0)
    back = np.empty_like(y0)
    back[..., perm] = y0
    np.testing.assert_allclose(y, back, rtol=0, atol=1e-14)


@pytest.mark.parametrize("pairing", [1, 2])
def test_half_split_invariants(pairing):
    g = np.random.default_rng(30 + pairing)
    q, k = g.standard_normal(64), g.standard_normal(64)

    def rot(vec, pos):
        t, h, w = pos
        grid = (t + 1, h + 1, w + 1)
        x = np.zeros((grid[0] * grid[1] * grid[2], 1, 64))
        idx = t * grid[1] * grid[2] + h * grid[2] + w
        x[idx, 0] = vec
        return oracle.rope3d_apply(x, grid, SPLIT, pairing=pairing)[idx, 0]

    # identity at the origin, norm kept, scores depend only on the offset
    np.testing.assert_array_equal(rot(q, (0, 0, 0)), q)
    assert abs(np.linalg.norm(rot(q, (2, 1, 3))) - np.linalg.norm(q)) < 1e-12
    p, pp, delta = (1, 2, 0), (3, 0, 5), (2, 3, 1)
    s1 = rot(q, p) @ rot(k, pp)
    s2 = rot(q, tuple(a + b for a, b in zip(p, delta))) @ rot(k, tuple(a + b for a, b in zip(pp, delta)))
    assert abs(s1 - s2) < 1e-12
    # text prefix rows stay as they are under every pairing
    x = g.standard_normal((3 + 48, 1, 64))
    y = oracle.rope3d_apply(x, GRID, SPLIT, n_prefix=3, pairing=pairing)
    np.testing.assert_array_equal(y[:3], x[:3])


def test_zero_width_band():
    # a band of width 0 contributes no pairs; the others keep their layout
    g = np.random.default_rng(40)
    x = g.standard_normal((48, 1, 48))
    for pairing in (0, 1, 2):
        y = oracle.rope3d_apply(x, GRID, (0, 24, 24), pairing=pairing)
        np.testing.assert_allclose((y ** 2).sum(-1), (x ** 2).sum(-1), rtol=1e-12)
        # tokens at h = w = 0 (t varies) are not rotated at all
        for tok in (0, 16, 32):
            np.testing.assert_array_equal(y[tok], x[tok])
