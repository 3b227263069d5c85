"""NF4 codebook, derived from the normal quantile function.

Source: "QLoRAの理論と実装" (disassemble-channel.com), §5-1 "4-bit NormalFloat
(NF4)量子化":
  * "数学的な構成": levels are quantiles of N(0, 1) at equally spaced
    probabilities, one level pinned to exactly zero, 8 levels on the negative
    side and 7 on the positive side, all normalised into [-1, 1];
  * the educational implementation ("NF4量子化の仕組みの実装", function that
    builds the codebook) fixes the probabilities: the negative side uses
    p = k/18 for k = 1..8, the positive side p = 1/2 + j/16 for j = 1..7; the
    values are divided by the largest magnitude and sorted ascending.

Reading taken: the printed text formula (q_i = Φ⁻¹(i/(2^b+1)),
c_i = (q_i + q_{i+1})/2) evaluates to c_0 = −∞ (Φ⁻¹(0)), so it cannot be the
16-level code the section describes; the code form is the only finite
construction on the page that meets the "one exact zero, 8 negative, 7
positive, inside [-1, 1]" statements, and it is the one used here.  The data
type is that table rounded once to float32: every decision and every
dequantisation uses exactly those 16 float32 values.

Parity: pinned (tests/test_oracle_codebook.py) by Φ(level·norm) = p through
math.erf (a routine independent of the inverse used here), by the textual
invariants, and by a second inverse-CDF implementation (scipy's ndtri).
"""

from fractions import Fraction
from statistics import NormalDist

import numpy as np


def nf4_probabilities():
    """The 15 non-zero quantile probabilities as exact fractions (negative side
    first), following the page's construction."""
    neg = [Fraction(k, 18) for k in range(1, 9)]
    pos = [Fraction(1, 2) + Fraction(j, 16) for j in range(1, 8)]
    return neg, pos


def nf4_codebook_f64():
    """16 levels in float64, ascending: Φ⁻¹ at the page's probabilities plus an
    exact 0, divided by the largest magnitude."""
    phi_inv = NormalDist(0.0, 1.0).inv_cdf
    neg, pos = nf4_probabilities()
    vals = [phi_inv(float(p)) for p in neg] + [0.0] + [phi_inv(float(p)) for p in pos]
    vals.sort()
    norm = max(abs(v) for v in vals)
    return np.array([v / norm for v in vals], dtype=np.float64)


def nf4_codebook_f32():
    """The NF4 data type: the float64 levels rounded once to float32."""
    return nf4_codebook_f64().astype(np.float32)


def nf4_midpoints_f64():
    """m_i = (c_i + c_{i+1}) / 2 for the float32 levels, i = 0..14, in float64.

    Exact: the levels are float32 numbers within [-1, 1], so their sum and the
    halving lose nothing in float64.  The nearest level to a real x is the
    number of midpoints strictly below x (a tie at a midpoint goes to the lower
    index, as a first-index argmin over ascending levels does)."""
    c = nf4_codebook_f32().astype(np.float64)
    return (c[:-1] + c[1:]) / 2.0


def text_formula_levels(bits=4):
    """The codebook exactly as the page's prose formula states it, kept only to
    show why that reading is rejected (its first level is −∞)."""
    phi_inv = NormalDist(0.0, 1.0).inv_cdf
    n = 2 ** bits
    q = []
    for i in range(n + 1):
        p = i / (n + 1)
        q.append(float("-inf") if p <= 0.0 else phi_inv(p))
    return [(q[i] + q[i + 1]) / 2.0 for i in range(n)]
