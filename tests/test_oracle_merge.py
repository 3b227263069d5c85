"""Pins of the oracle's adapter merge and re-quantisation."""

from fractions import Fraction

import numpy as np
import torch

from oracle.merge import merge_16bit, merge_4bit, merge_bf16, rank_r_sum, requantize
from oracle.quant import bf16_round, bf16_round64, bf16_to_f64, dequantize_nf4, double_quant, \
    quantize_nf4, unpack_nibbles


def _bf16_vals(x):
    """float32 array of the bf16 values nearest to x."""
    return bf16_to_f64(bf16_round(np.asarray(x, np.float32).ravel())).astype(np.float32).reshape(
        np.shape(x))


# every finite non-negative bf16 value, ascending with its bit pattern
_GRID_BITS = np.arange(0x7F80, dtype=np.uint16)
_GRID = [Fraction(float(v)) for v in bf16_to_f64(_GRID_BITS)]
_HALF_ULP_MAX = (_GRID[-1] - _GRID[-2]) / 2


def _nearest_bf16(x):
    """The bf16 bit pattern nearest to the rational x by a search over the
    grid; of two equally near values the one with an even pattern; past the
    largest value by half its spacing or more, infinity."""
    sign = 0x8000 if x < 0 else 0
    a = abs(Fraction(x))
    if a >= _GRID[-1] + _HALF_ULP_MAX:
        return sign | 0x7F80
    lo, hi = 0, len(_GRID) - 1
    while hi - lo > 1:  # _GRID[lo] <= a <= _GRID[hi]
        mid = (lo + hi) // 2
        if _GRID[mid] <= a:
            lo = mid
        else:
            hi = mid
    dl, dh = a - _GRID[lo], _GRID[hi] - a
    pick = lo if (dl < dh or (dl == dh and lo % 2 == 0)) else hi
    return sign | pick


def test_bf16_round64_against_grid_search():
    """float64 -> bf16 at random magnitudes, at exact midpoints between
    neighbours (ties), at their float64 neighbours, in the subnormal range and
    at the overflow boundary."""
    rng = np.random.default_rng(37)
    xs = list(rng.standard_normal(400) * np.exp2(rng.integers(-40, 40, 400)))
    xs += list(rng.standard_normal(50) * 2.0 ** -130)  # subnormal bf16
    for b in rng.integers(1, 0x7F7F, 300):
        mid = (_GRID[b] + _GRID[b + 1]) / 2
        m = float(mid)  # exact: a bf16 midpoint has 9 significant bits
        assert Fraction(m) == mid
        xs += [m, np.nextafter(m, np.inf), np.nextafter(m, -np.inf), -m]
    top = float(_GRID[-1] + _HALF_ULP_MAX)
    xs += [top, np.nextafter(top, 0.0), float(_GRID[-1]), 0.0, -0.0, 2.0 ** -133, 2.0 ** -134,
           3 * 2.0 ** -135]
    xs = np.array(xs, dtype=np.float64)
    got = bf16_round64(xs)
    for x, g in zip(xs, got):
        want = _nearest_bf16(Fraction(float(x)))
        if x == 0.0:
            want = 0x8000 if np.signbit(x) else 0
        assert int(g) == want, (x, hex(int(g)), hex(want))


def test_merge_is_the_exact_value_rounded_once():
    """m = the bf16 value nearest to the exact rational w + s·Σ B·A, for
    random bf16 bases and adapters (16-bit and decoded-4-bit magnitudes)."""
    rng = np.random.default_rng(38)
    N, K, r = 6, 24, 16
    for scale, s in ((0.02, 0.25), (0.5, 2.0), (1e-3, np.float32(16.0 / 24.0))):
        base = _bf16_vals(rng.standard_normal((N, K)) * scale)
        A = _bf16_vals(rng.standard_normal((r, K)) * 0.05)
        B = _bf16_vals(rng.standard_normal((N, r)) * 0.05)
        got = merge_bf16(base, A, B, s)
        sf = Fraction(float(np.float32(s)))
        for n in range(N):
            for k in range(K):
                exact = Fraction(float(base[n, k])) + sf * sum(
                    Fraction(float(B[n, j])) * Fraction(float(A[j, k])) for j in range(r))
                assert int(got[n, k]) == _nearest_bf16(exact), (n, k)


def test_rank_r_sum_exact_on_dyadic_inputs():
    """Small dyadic factors: every partial sum is exact, so the float64 sum
    equals the exact rational product."""
    rng = np.random.default_rng(31)
    r, N, K = 8, 5, 7
    A = (rng.integers(-16, 17, (r, K)) / 8.0).astype(np.float32)
    B = (rng.integers(-16, 17, (N, r)) / 16.0).astype(np.float32)
    got = rank_r_sum(A, B)
    for n in range(N):
        for k in range(K):
            exact = sum(Fraction(float(B[n, j])) * Fraction(float(A[j, k])) for j in range(r))
            assert Fraction(float(got[n, k])) == exact


def test_rank_r_sum_error_bound_random():
    """bf16 factors at rank 64: the float64 sum within r·2⁻⁵³·Σ|B·A| of the
    exact rational sum (exact, in practice, at these magnitudes)."""
    rng = np.random.default_rng(32)
    r, N, K = 64, 6, 8
    A = _bf16_vals(rng.standard_normal((r, K)) * 0.01)
    B = _bf16_vals(rng.standard_normal((N, r)) * 0.01)
    got = rank_r_sum(A, B)
    for n in range(N):
        for k in range(K):
            terms = [Fraction(float(B[n, j])) * Fraction(float(A[j, k])) for j in range(r)]
            bound = r * Fraction(2) ** -53 * sum(abs(t) for t in terms)
            assert abs(Fraction(float(got[n, k])) - sum(terms)) <= bound


def test_zero_adapter_leaves_the_base():
    rng = np.random.default_rng(33)
    N, K, r = 8, 128, 4
    base = _bf16_vals(rng.standard_normal((N, K)) * 0.02)
    A = _bf16_vals(rng.standard_normal((r, K)) * 0.01)
    Z = np.zeros((N, r), np.float32)
    m = merge_bf16(base, A, Z, 0.25)
    assert np.array_equal(m, bf16_round(base.ravel()).reshape(N, K))
    m2 = merge_bf16(base, np.zeros_like(A), _bf16_vals(rng.standard_normal((N, r))), 4.0)
    assert np.array_equal(m2, m)


def test_merge_formula_on_one_element():
    """m = RNE_bf16(w + s·acc) with the sum formed in float64."""
    A = np.array([[0.5], [0.25]], np.float32).T.reshape(2, 1)   # [r=2][K=1]
    B = np.array([[0.75, -1.5]], np.float32)                     # [N=1][r=2]
    base = np.array([[1.0]], np.float32)
    s = np.float32(1 / 3)
    assert 0.75 * 0.5 - 1.5 * 0.25 == 0.0                        # acc = 0: the base comes back
    assert merge_bf16(base, A, B, s)[0, 0] == bf16_round(np.array([1.0], np.float32))[0]
    B2 = np.array([[0.75, 1.5]], np.float32)
    x = 1.0 + float(s) * 0.75                                    # exact in float64
    assert merge_bf16(base, A, B2, s)[0, 0] == bf16_round64(np.array([x]))[0]
    assert merge_bf16(base, A, B2, s)[0, 0] == _nearest_bf16(1 + Fraction(float(s)) * Fraction(3, 4))


def test_requantized_decode_is_stable_and_tiny_adapters_vanish_in_4bit():
    """The page's warning: merging into the 4-bit base re-rounds onto the
    4-bit grid.  Re-quantising a decoded NF4 weight returns its own codes, so
    an adapter far below the level spacing is lost entirely."""
    rng = np.random.default_rng(34)
    N, K, r = 64, 512, 8
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    packed, absmax = quantize_nf4(W.ravel())
    q, c2 = double_quant(absmax)
    # without an adapter the re-quantised decode returns the original codes
    z = np.zeros((N, r), np.float32)
    _, (p0, _, _, _) = merge_4bit(packed, q, c2, (N, K), np.zeros((r, K), np.float32), z, 0.25)
    assert np.array_equal(unpack_nibbles(p0), unpack_nibbles(packed))
    # an adapter of ~6e-4 per weight: above the bf16 step of these weights,
    # well below the NF4 level gaps (~5e-3)
    A = _bf16_vals(rng.standard_normal((r, K)) * 3e-2)
    B = _bf16_vals(rng.standard_normal((N, r)) * 3e-2)
    m, (p4, q4, c24, d4) = merge_4bit(packed, q, c2, (N, K), A, B, 0.25)
    base = dequantize_nf4(packed, q, c2, N * K).reshape(N, K)
    # the delta is real in 16 bits (most merged bf16 values moved) ...
    assert np.mean(m != base) > 0.5
    # ... and gone after re-quantisation: nearly every code is the original one,
    # and the decoded change keeps under 15 % of the delta (its projection on
    # the delta; the rest is scale noise from the re-quantised absmax)
    assert np.mean(unpack_nibbles(p4) != unpack_nibbles(packed)) < 0.01
    D = 0.25 * (B.astype(np.float64) @ A.astype(np.float64))
    d = bf16_to_f64(d4) - bf16_to_f64(base)
    assert np.sum(d * D) / np.sum(D * D) < 0.15


def test_16bit_path_is_closer_to_the_merged_weight():
    rng = np.random.default_rng(35)
    N, K, r = 64, 1024, 16
    W16 = _bf16_vals(rng.standard_normal((N, K)) * 0.02)
    A = _bf16_vals(rng.standard_normal((r, K)) * 0.05)
    B = _bf16_vals(rng.standard_normal((N, r)) * 0.05)
    s = 0.25
    target = W16.astype(np.float64) + s * (B.astype(np.float64) @ A.astype(np.float64))
    m16, (_, _, _, d16) = merge_16bit(bf16_round(W16.ravel()).reshape(N, K), A, B, s)
    packed, absmax = quantize_nf4(W16.ravel())
    q, c2 = double_quant(absmax)
    m4, (_, _, _, d4) = merge_4bit(packed, q, c2, (N, K), A, B, s)
    e16 = np.linalg.norm(bf16_to_f64(d16) - target)
    e4 = np.linalg.norm(bf16_to_f64(d4) - target)
    assert e4 > 1.2 * e16, (e4, e16)
    # the merged 16-bit weight itself is within bf16 rounding of the target
    assert np.all(np.abs(bf16_to_f64(m16) - target) <= 2.0 ** -8 * np.abs(target) + 1e-12)


def test_requantize_goes_through_the_quantiser():
    rng = np.random.default_rng(36)
    m = bf16_round((rng.standard_normal(64 * 300) * 0.03).astype(np.float32)).reshape(75, 256)
    packed, q, c2, dec = requantize(m)
    p2, a2 = quantize_nf4(bf16_to_f64(m).astype(np.float32).ravel())
    q2, c22 = double_quant(a2)
    assert np.array_equal(packed, p2) and np.array_equal(q, q2) and np.array_equal(c2, c22)
    assert dec.shape == (75, 256)
    t = torch.from_numpy(bf16_to_f64(dec))
    assert torch.all(torch.isfinite(t))
