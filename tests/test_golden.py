"""The oracle against hand-derived worked cases (tests/golden/).

The pages print no worked numerical example, so each fixture is a case
derived by hand from the definition the pages give, with inputs chosen so
that the expected values are exact binary fractions or closed-form
constants.  Each file states its source passage and derivation.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _load("adaln_exact.json")["cases"],
                         ids=lambda c: c["derivation"][:24])
def test_adaln_worked_cases(case):
    row = lambda key: np.array([case[key]], dtype=np.float64)
    y = oracle.adaln_modulate(row("x"), row("shift"), row("scale"), case["eps"])
    np.testing.assert_allclose(y, row("y"), rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", _load("attention_exact.json")["cases"],
                         ids=lambda c: c["derivation"][:24])
def test_attention_worked_cases(case):
    as3 = lambda key: np.array(case[key], dtype=np.float64)[:, None, :]   # [N, 1 head, d]
    o, lse = oracle.attention(as3("q"), as3("k"), as3("v"))
    np.testing.assert_allclose(o[:, 0, :], np.array(case["o"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0], np.array(case["lse"]), rtol=0, atol=1e-13)


def test_rope_token_positions():
    fx = _load("rope3d_exact.json")["positions"]
    t, h, w = oracle.token_positions(fx["grid"], fx["n_prefix"])
    for token, tt, hh, ww in fx["token_twh"]:
        v = token - fx["n_prefix"]
        assert (t[v], h[v], w[v]) == (tt, hh, ww), token


@pytest.mark.parametrize("block", _load("rope3d_exact.json")["angles"],
                         ids=lambda b: f"split{b['split']}")
def test_rope_worked_angles(block):
    grid, split = tuple(block["grid"]), tuple(block["split"])
    d, n = sum(split), int(np.prod(grid))
    for token, elem, angle in block["token_element_angle"]:
        # a unit vector on the even element of the pair turns to (cos, sin)
        x = np.zeros((n, 1, d))
        x[token, 0, elem] = 1.0
        y = oracle.rope3d_apply(x, grid, split)[token, 0]
        expect = np.zeros(d)
        expect[elem], expect[elem + 1] = math.cos(angle), math.sin(angle)
        np.testing.assert_allclose(y, expect, rtol=0, atol=1e-15, err_msg=f"{token},{elem}")
