"""Pins of the oracle's QLoRA linear forward and backward."""

from fractions import Fraction

import numpy as np
import pytest

from oracle.linear import linear_bwd, linear_fwd, lora_scale


def _rand(rng, shape, scale=1.0):
    # small dyadic rationals: exact in float64 and in Fraction
    return (rng.integers(-64, 65, size=shape) / 32.0 * scale).astype(np.float64)


def _mat(a):
    return [[Fraction(float(x)) for x in row] for row in np.atleast_2d(a)]


def _mm(a, b):
    n, k, m = len(a), len(b), len(b[0])
    return [[sum((a[i][t] * b[t][j] for t in range(k)), Fraction(0)) for j in range(m)]
            for i in range(n)]


def _t(a):
    return [list(x) for x in zip(*a)]


def _add(a, b, s=Fraction(1)):
    return [[x + s * y for x, y in zip(ra, rb)] for ra, rb in zip(a, b)]


def _scal(a, s):
    return [[s * x for x in r] for r in a]


@pytest.mark.parametrize("M,K,N,r", [(1, 1, 1, 1), (2, 3, 2, 1), (3, 64, 2, 2), (2, 128, 3, 8),
                                     (64, 2, 3, 2)])
def test_fwd_bwd_against_exact_rationals(M, K, N, r):
    rng = np.random.default_rng(M * 1000 + K * 10 + N + r)
    X, W, A, B, dY = (_rand(rng, (M, K)), _rand(rng, (N, K)), _rand(rng, (r, K)),
                      _rand(rng, (N, r)), _rand(rng, (M, N)))
    s = lora_scale(16.0, r)
    Y, U = linear_fwd(X, W, A, B, s)
    dX, dA, dB = linear_bwd(X, dY, W, A, B, s)
    Xq, Wq, Aq, Bq, dYq = map(_mat, (X, W, A, B, dY))
    sq = Fraction(s)
    Uq = _mm(Xq, _t(Aq))
    Yq = _add(_mm(Xq, _t(Wq)), _mm(Uq, _t(Bq)), sq)
    Vq = _mm(dYq, Bq)
    dXq = _add(_mm(dYq, Wq), _mm(Vq, Aq), sq)
    dAq = _scal(_mm(_t(Vq), Xq), sq)
    dBq = _scal(_mm(_t(dYq), Uq), sq)
    for got, want in [(Y, Yq), (U, Uq), (dX, dXq), (dA, dAq), (dB, dBq)]:
        want = np.array([[float(x) for x in row] for row in want])
        assert np.allclose(got, want, rtol=1e-13, atol=1e-13)


def test_gradients_by_finite_differences():
    """Central differences of L = <dY, Y(X, A, B)> (L is linear in X and in each
    of A, B separately, so the difference quotient is exact up to rounding)."""
    rng = np.random.default_rng(11)
    M, K, N, r = 5, 16, 7, 3
    X = rng.standard_normal((M, K))
    W = rng.standard_normal((N, K)) * 0.1
    A = rng.standard_normal((r, K)) * 0.1
    B = rng.standard_normal((N, r)) * 0.1
    dY = rng.standard_normal((M, N))
    s = lora_scale(32.0, r)

    def loss(X_, A_, B_):
        return float(np.sum(dY * linear_fwd(X_, W, A_, B_, s)[0]))

    dX, dA, dB = linear_bwd(X, dY, W, A, B, s)
    h = 1e-3
    for name, P, G in [("X", X, dX), ("A", A, dA), ("B", B, dB)]:
        for idx in [(0, 0), (P.shape[0] - 1, P.shape[1] - 1), (P.shape[0] // 2, 1)]:
            Pp, Pm = P.copy(), P.copy()
            Pp[idx] += h
            Pm[idx] -= h
            args_p = dict(X_=X, A_=A, B_=B)
            args_m = dict(X_=X, A_=A, B_=B)
            args_p[name + "_"] = Pp
            args_m[name + "_"] = Pm
            fd = (loss(**args_p) - loss(**args_m)) / (2 * h)
            assert abs(fd - G[idx]) <= 1e-8 * max(1.0, abs(G[idx])), (name, idx, fd, G[idx])


def test_zero_init_adapter_reduces_to_quantised_base():
    # adapters start with B = 0, so the first step equals the quantised base
    # (issoh.co.jp guide, LoftQ paragraph)
    rng = np.random.default_rng(12)
    X, W, A = rng.standard_normal((4, 8)), rng.standard_normal((6, 8)), rng.standard_normal((2, 8))
    B = np.zeros((6, 2))
    Y, U = linear_fwd(X, W, A, B, 0.5)
    assert np.array_equal(Y, X @ W.T)
    dY = rng.standard_normal((4, 6))
    dX, dA, dB = linear_bwd(X, dY, W, A, B, 0.5)
    assert np.all(dA == 0)
    assert np.array_equal(dX, dY @ W)
    Y2, U2 = linear_fwd(X, W, np.zeros_like(A), rng.standard_normal((6, 2)), 0.5)
    dX2, dA2, dB2 = linear_bwd(X, dY, W, np.zeros_like(A), rng.standard_normal((6, 2)), 0.5)
    assert np.all(dB2 == 0) and np.all(U2 == 0)


def test_identity_inputs_expose_the_weight():
    rng = np.random.default_rng(13)
    K, N = 8, 5
    W = rng.standard_normal((N, K))
    Y, _ = linear_fwd(np.eye(K), W, np.zeros((2, K)), np.zeros((N, 2)), 1.0)
    assert np.array_equal(Y, W.T)
    dX, _, _ = linear_bwd(np.zeros((N, K)), np.eye(N), W, np.zeros((2, K)), np.zeros((N, 2)), 1.0)
    assert np.array_equal(dX, W)


def test_scale_is_linear_and_rounded_in_float32():
    assert lora_scale(16.0, 64) == 0.25
    assert lora_scale(16.0, 8) == 2.0
    assert lora_scale(32.0, 16) == 2.0
    assert lora_scale(16.0, 3) == float(np.float32(16.0) / np.float32(3.0))
    rng = np.random.default_rng(14)
    X, W, A, B = (rng.standard_normal((3, 4)), rng.standard_normal((2, 4)),
                  rng.standard_normal((2, 4)), rng.standard_normal((2, 2)))
    Y1, _ = linear_fwd(X, W, A, B, 1.0)
    Y2, _ = linear_fwd(X, W, A, B, 2.0)
    Y0, _ = linear_fwd(X, W, A, B, 0.0)
    assert np.allclose(Y2 - Y0, 2 * (Y1 - Y0), rtol=1e-14, atol=1e-14)
