"""Pins for the attention oracle (CPU only).

The oracle is compared with torch's scaled_dot_product_attention and
scipy's logsumexp in float64, and with closed forms: equal keys give the
mean of V, a dominant key selects its value, N = 1 returns V, and joint
permutations of K/V leave the result unchanged.
"""
import numpy as np
import pytest
import scipy.special
import torch

import oracle


def _qkv(n=40, h=3, d=64, seed=0):
    g = np.random.default_rng(seed)
    return (g.standard_normal((n, h, d)), g.standard_normal((n, h, d)),
            g.standard_normal((n, h, d)))


@pytest.mark.parametrize("n,d", [(1, 64), (37, 64), (130, 128)])
def test_matches_library_sdpa(n, d):
    q, k, v = _qkv(n, 3, d)
    o, _ = oracle.attention(q, k, v)
    t = lambda a: torch.from_numpy(a).permute(1, 0, 2)[None]          # [1,H,N,d]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))
    np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_explicit_scale_matches_library():
    q, k, v = _qkv(50, 2, 64, seed=1)
    o, _ = oracle.attention(q, k, v, scale=0.3)
    t = lambda a: torch.from_numpy(a).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=0.3)
    np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_lse_is_library_logsumexp():
    q, k, v = _qkv(60, 2, 64, seed=2)
    _, lse = oracle.attention(q, k, v)
    for h in range(2):
        s = q[:, h] @ k[:, h].T / 8.0
        np.testing.assert_allclose(lse[h], scipy.special.logsumexp(s, axis=1), rtol=0,
                                   atol=1e-12)


def test_softmax_rows_sum_to_one():
    """The weights attention() applies sum to 1 in every row: with every value
    equal to 1 each output element is that row's sum of weights.  Scores up to
    about +-40 (q scaled by 10), so the max subtraction matters."""
    g = np.random.default_rng(3)
    q, k = g.standard_normal((20, 2, 64)) * 10, g.standard_normal((300, 2, 64))
    o, _ = oracle.attention(q, k, np.ones((300, 2, 64)))
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-12)


def test_weights_are_the_library_softmax():
    """With V the identity (d = N, value j = unit vector e_j) attention()
    returns its weight matrix itself: each row must equal scipy's softmax of
    the scaled scores, be non-negative, and sum to 1."""
    g = np.random.default_rng(13)
    n = 48
    q, k = g.standard_normal((n, 1, n)) * 3, g.standard_normal((n, 1, n))
    p, _ = oracle.attention(q, k, np.eye(n)[:, None, :], scale=0.4)
    ref = scipy.special.softmax(0.4 * (q[:, 0] @ k[:, 0].T), axis=1)
    np.testing.assert_allclose(p[:, 0], ref, rtol=0, atol=1e-14)
    assert (p >= 0).all()
    np.testing.assert_allclose(p.sum(axis=2), 1.0, rtol=0, atol=1e-12)


def test_equal_keys_give_mean_of_values():
    q, k, v = _qkv(33, 2, 64, seed=4)
    k[:] = k[0]
    o, lse = oracle.attention(q, k, v)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), atol=1e-12)
    # lse = s + ln N for identical scores
    s = np.einsum("nhd,hd->hn", q, k[0]) / 8.0
    np.testing.assert_allclose(lse, s + np.log(33), atol=1e-12)


def test_dominant_key_selects_its_value():
    q, k, v = _qkv(25, 2, 64, seed=5)
    k[11] = 200.0 * q[0]          # huge score for query 0 only
    o, _ = oracle.attention(q, k, v, rows=[0])
    np.testing.assert_allclose(o[0], v[11], atol=1e-12)


def test_single_token_returns_value():
    q, k, v = _qkv(1, 4, 128, seed=6)
    o, lse = oracle.attention(q, k, v)
    np.testing.assert_allclose(o, v, atol=0)


def test_permutation_invariance():
    q, k, v = _qkv(45, 2, 64, seed=7)
    perm = np.random.default_rng(8).permutation(45)
    o1, _ = oracle.attention(q, k, v)
    o2, _ = oracle.attention(q, k[perm], v[perm])
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    o3, _ = oracle.attention(q[perm], k, v)
    np.testing.assert_allclose(o3, o1[perm], atol=1e-12)


def test_shift_invariance_of_scores():
    # Adding c*q to every key adds c*|q|^2*scale to each score of a row.
    q, k, v = _qkv(30, 1, 64, seed=9)
    o1, _ = oracle.attention(q, k, v, rows=[4])
    o2, _ = oracle.attention(q, k + 0.7 * q[4], v, rows=[4])
    np.testing.assert_allclose(o1, o2, atol=1e-12)


def test_row_subset_matches_full():
    q, k, v = _qkv(70, 2, 64, seed=10)
    o, lse = oracle.attention(q, k, v)
    rows = np.array([0, 13, 69])
    o2, lse2 = oracle.attention(q, k, v, rows=rows, row_block=2)
    np.testing.assert_allclose(o2, o[rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse2, lse[:, rows], rtol=0, atol=1e-14)


def test_rope_then_attention_equals_composition():
    q, k, v = _qkv(48, 2, 64, seed=11)
    grid, split = (3, 4, 4), (16, 24, 24)
    o1, l1 = oracle.attention_rope(q, k, v, grid, split)
    o2, l2 = oracle.attention(oracle.rope3d_apply(q, grid, split),
                              oracle.rope3d_apply(k, grid, split), v)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    rows = [1, 20, 47]
    o3, l3 = oracle.attention_rope(q, k, v, grid, split, rows=rows)
    np.testing.assert_allclose(o3, o1[rows], atol=1e-13)
    np.testing.assert_allclose(l3, l1[:, rows], atol=1e-13)


def test_rope_with_prefix_rows():
    q, k, v = _qkv(6 + 48, 2, 64, seed=12)
    grid, split = (3, 4, 4), (16, 24, 24)
    rows = [0, 5, 6, 53]
    o, l = oracle.attention_rope(q, k, v, grid, split, n_prefix=6, rows=rows)
    qr = oracle.rope3d_apply(q, grid, split, n_prefix=6)
    kr = oracle.rope3d_apply(k, grid, split, n_prefix=6)
    o2, l2 = oracle.attention(qr, kr, v, rows=rows)
    np.testing.assert_allclose(o, o2, atol=1e-13)
    np.testing.assert_allclose(l, l2, atol=1e-13)


# ---- queries and keys from different token sets; merging key-split parts

def test_cross_attention_matches_library_sdpa():
    g = np.random.default_rng(11)
    q = g.standard_normal((23, 2, 64))
    k, v = g.standard_normal((70, 2, 64)), g.standard_normal((70, 2, 64))
    o, lse = oracle.attention(q, k, v)
    t = lambda a: torch.from_numpy(a).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))
    np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    s = np.einsum("qhd,khd->hqk", q, k) / 8.0
    np.testing.assert_allclose(lse, scipy.special.logsumexp(s, axis=-1), rtol=0, atol=1e-12)


def test_cross_attention_single_key_returns_its_value():
    g = np.random.default_rng(12)
    q = g.standard_normal((9, 3, 64))
    k, v = g.standard_normal((1, 3, 64)), g.standard_normal((1, 3, 64))
    o, lse = oracle.attention(q, k, v)
    np.testing.assert_array_equal(o, np.broadcast_to(v, o.shape))
    np.testing.assert_allclose(lse, np.einsum("qhd,hd->hq", q, k[0]) / 8.0, rtol=0, atol=1e-13)


@pytest.mark.parametrize("split", [1, 17, 39])
def test_merge_of_key_split_equals_full_attention(split):
    q, k, v = _qkv(40, 3, 64, seed=13)
    o_a, l_a = oracle.attention(q, k[:split], v[:split])
    o_b, l_b = oracle.attention(q, k[split:], v[split:])
    o, lse = oracle.merge_lse(o_a, l_a, o_b, l_b)
    ref, rl = oracle.attention(q, k, v)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


def test_merge_is_associative_and_symmetric():
    q, k, v = _qkv(45, 2, 64, seed=14)
    parts = [oracle.attention(q, k[a:b], v[a:b]) for a, b in ((0, 10), (10, 31), (31, 45))]
    left = oracle.merge_lse(*oracle.merge_lse(*parts[0], *parts[1]), *parts[2])
    right = oracle.merge_lse(*parts[0], *oracle.merge_lse(*parts[1], *parts[2]))
    swapped = oracle.merge_lse(*parts[2], *oracle.merge_lse(*parts[1], *parts[0]))
    for x in (right, swapped):
        np.testing.assert_allclose(x[0], left[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(x[1], left[1], rtol=0, atol=1e-12)


def test_merge_with_empty_part_and_with_itself():
    q, k, v = _qkv(20, 2, 64, seed=15)
    o, lse = oracle.attention(q, k, v)
    empty_o, empty_l = np.zeros_like(o), np.full_like(lse, -np.inf)
    mo, ml = oracle.merge_lse(o, lse, empty_o, empty_l)
    np.testing.assert_array_equal(mo, o)
    np.testing.assert_array_equal(ml, lse)
    mo, ml = oracle.merge_lse(empty_o, empty_l, empty_o, empty_l)
    assert np.all(mo == 0) and np.all(np.isneginf(ml))
    mo, ml = oracle.merge_lse(o, lse, o, lse)      # the same keys twice: Z doubles
    np.testing.assert_allclose(mo, o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(ml, lse + np.log(2.0), rtol=0, atol=1e-13)


# ---- key padding

@pytest.mark.parametrize("lo,hi", [(0, 10), (5, 17), (30, 40), (0, 39), (12, 12)])
def test_masked_matches_library_sdpa_with_bool_mask(lo, hi):
    q, k, v = _qkv(40, 2, 64, seed=16)
    o, lse = oracle.attention_masked(q, k, v, lo, hi)
    allow = np.ones((40, 40), dtype=bool)
    allow[:, lo:hi] = False
    t = lambda a: torch.from_numpy(a).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v),
                                                           attn_mask=torch.from_numpy(allow))
    np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    s = np.einsum("qhd,khd->hqk", q, k) / 8.0
    s[:, :, lo:hi] = -np.inf
    np.testing.assert_allclose(lse, scipy.special.logsumexp(s, axis=-1), rtol=0, atol=1e-12)


def test_masked_keys_do_not_matter():
    q, k, v = _qkv(50, 2, 64, seed=17)
    o1, l1 = oracle.attention_masked(q, k, v, 20, 35)
    k2, v2 = k.copy(), v.copy()
    k2[20:35] *= -7.0
    v2[20:35] += 100.0
    o2, l2 = oracle.attention_masked(q, k2, v2, 20, 35)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_mask_leaving_one_key_returns_its_value():
    q, k, v = _qkv(9, 2, 64, seed=18)
    o, _ = oracle.attention_masked(q, k, v, 1, 9)
    np.testing.assert_array_equal(o, np.broadcast_to(v[0], o.shape))
    with pytest.raises(ValueError):
        oracle.attention_masked(q, k, v, 0, 9)
