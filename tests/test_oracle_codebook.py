"""Pins of the oracle's NF4 codebook against what the page and mathematics fix."""

import math

import numpy as np
import pytest

from oracle.codebook import (
    nf4_codebook_f32,
    nf4_codebook_f64,
    nf4_midpoints_f64,
    nf4_probabilities,
    text_formula_levels,
)


def _phi(x):
    """Standard normal CDF through math.erf (independent of the inverse used by
    the oracle)."""
    return 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))


def _phi_inv_bisect(p):
    lo, hi = -10.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if _phi(mid) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def test_textual_invariants():
    # one exact zero, 8 negative levels and 7 positive ones, all in [-1, 1],
    # sorted ascending (QLoRAの理論と実装, §5-1 数学的な構成 / step 1)
    c = nf4_codebook_f32()
    assert c.dtype == np.float32 and c.shape == (16,)
    assert np.all(np.diff(c) > 0)
    assert c[0] == np.float32(-1.0)
    assert c[8] == 0.0 and not np.signbit(c[8])
    assert int((c < 0).sum()) == 8 and int((c > 0).sum()) == 7
    assert np.all(np.abs(c) <= 1.0)
    assert c[15] < 1.0  # the positive side never reaches 1: 7 levels vs 8


def test_levels_are_normal_quantiles_via_erf():
    """Each non-zero level times the normaliser |Φ⁻¹(1/18)| sits at the page's
    probability; Φ is evaluated with erf and the normaliser by bisection, so no
    step shares code with the oracle's inverse CDF."""
    norm = -_phi_inv_bisect(1.0 / 18.0)
    c = nf4_codebook_f64()
    neg, pos = nf4_probabilities()
    probs = [float(p) for p in neg] + [float(p) for p in pos]
    nonzero = [v for i, v in enumerate(c) if i != 8]
    for level, p in zip(nonzero, probs):
        assert abs(_phi(level * norm) - p) < 1e-12, (level, p)
    # equal probability mass between consecutive negative levels: 1/18 each
    for k in range(7):
        mass = _phi(c[k + 1] * norm) - _phi(c[k] * norm)
        assert abs(mass - 1.0 / 18.0) < 1e-12
    # and 1/16 between consecutive positive levels
    for k in range(9, 15):
        mass = _phi(c[k + 1] * norm) - _phi(c[k] * norm)
        assert abs(mass - 1.0 / 16.0) < 1e-12


def test_second_inverse_cdf_gives_same_float32_table():
    scipy_stats = pytest.importorskip("scipy.stats")
    neg, pos = nf4_probabilities()
    v = [scipy_stats.norm.ppf(float(p)) for p in neg] + [0.0] + \
        [scipy_stats.norm.ppf(float(p)) for p in pos]
    v = np.sort(np.array(v)) / np.max(np.abs(v))
    assert np.array_equal(v.astype(np.float32).view(np.uint32),
                          nf4_codebook_f32().view(np.uint32))


def test_page_code_probabilities_match_exact_fractions():
    # the page's code builds the probabilities with linspace; the rounded values
    # must equal the exact fractions used here
    neg, pos = nf4_probabilities()
    lin_neg = np.linspace(1 / (2 * 9), 0.5, 8, endpoint=False)
    lin_pos = np.linspace(0.5 + 1 / (2 * 8), 1 - 1 / (2 * 8), 7)
    assert np.allclose(lin_neg, [float(p) for p in neg], rtol=0, atol=1e-15)
    assert np.allclose(lin_pos, [float(p) for p in pos], rtol=0, atol=1e-15)


def test_text_formula_is_not_a_finite_codebook():
    # the prose formula's first level is −∞: the reason the code form is used
    lv = text_formula_levels()
    assert lv[0] == float("-inf")
    assert len(lv) == 16


def test_midpoints_exact_and_narrow():
    c = nf4_codebook_f32().astype(np.float64)
    m = nf4_midpoints_f64()
    assert m.shape == (15,)
    assert np.all((c[:-1] < m) & (m < c[1:]))
    # each midpoint needs at most 29 significant bits, so m * a (a float32, 24
    # bits) is exact in float64's 53
    for x in m:
        mant, exp = math.frexp(abs(x))
        bits = 0
        while mant != math.floor(mant):
            mant *= 2
            bits += 1
        assert bits <= 29, (x, bits)
    # which midpoints are themselves float32 numbers (exact ties reachable at a = 1)
    rep = [i for i, x in enumerate(m) if float(np.float32(x)) == x]
    assert rep == [1, 3, 4, 7, 8, 11, 13, 14]
