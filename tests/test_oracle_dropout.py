"""Pins of the oracle's LoRA dropout: the Philox generator, the mask and the
dropout linear's forward and backward."""

import numpy as np
import pytest

from oracle.dropout import (drop_threshold, element_values, keep_mask, linear_bwd_dropout,
                            linear_fwd_dropout, linear_no_dropout, mulhilo64, philox4x64_10,
                            philox4x64_10_np)
from oracle.linear import lora_scale

M64 = (1 << 64) - 1


@pytest.mark.parametrize("counter,key", [
    ((0, 0, 0, 0), (0, 0)),
    ((4, 0, 0, 0), (123, 456)),
    ((0x243F6A8885A308D3, 0x13198A2E03707344, 0xA4093822299F31D0, 0x082EFA98EC4E6C89),
     (0x452821E638D01377, 0xBE5466CF34E90C6C)),
    ((M64 - 1, 7, 0, 0), (2 ** 63, 1)),
])
def test_philox_against_numpy_bit_generator(counter, key):
    """numpy's Philox (a library Philox4x64-10) returns, as its first four raw
    words, the block of counter + 1 (it increments before generating)."""
    g = np.random.Philox(counter=np.array(counter, dtype=np.uint64),
                         key=np.array(key, dtype=np.uint64))
    raw = [int(x) for x in g.random_raw(8)]
    c = list(counter)
    for blk in range(2):
        # counter + 1 with carry across the four words
        for i in range(4):
            c[i] = (c[i] + 1) & M64
            if c[i] != 0:
                break
        assert list(philox4x64_10(tuple(c), key)) == raw[4 * blk:4 * blk + 4]


def test_vectorised_philox_matches_scalar():
    rng = np.random.default_rng(21)
    c0 = rng.integers(0, 2 ** 63, 50, dtype=np.uint64) * np.uint64(2) + np.uint64(1)
    c1 = np.uint64(987654321987)
    k0, k1 = 0xDEADBEEFCAFEF00D, 0
    w = philox4x64_10_np(c0, c1, k0, k1)
    for i in range(c0.size):
        ref = philox4x64_10((int(c0[i]), int(c1), 0, 0), (k0, k1))
        assert tuple(int(x[i]) for x in w) == ref


def test_mulhilo_against_exact_products():
    rng = np.random.default_rng(22)
    a = rng.integers(0, 2 ** 64 - 1, 2000, dtype=np.uint64, endpoint=True)
    b = rng.integers(0, 2 ** 64 - 1, 2000, dtype=np.uint64, endpoint=True)
    a[:3] = [0, M64, M64]
    b[:3] = [M64, M64, 1]
    with np.errstate(over="ignore"):
        hi, lo = mulhilo64(a, b)
    for x, y, h, l in zip(a, b, hi, lo):
        p = int(x) * int(y)
        assert int(h) == p >> 64 and int(l) == p & M64


def test_element_values_layout():
    """Element f takes 32-bit value f & 7 of block f >> 3: word (f & 7) >> 1,
    low half for even f."""
    seed, offset = 77, 5
    v = element_values(40, seed, offset)
    for f in (0, 1, 6, 7, 8, 13, 39):
        words = philox4x64_10((f >> 3, offset, 0, 0), (seed, 0))
        w = words[(f & 7) >> 1]
        assert int(v[f]) == ((w >> 32) if f & 1 else (w & 0xFFFFFFFF))


def test_threshold_and_drop_rate():
    assert drop_threshold(0.0) == 0
    assert drop_threshold(0.5) == 2 ** 31
    assert drop_threshold(np.float32(0.05)) == int(np.floor(float(np.float32(0.05)) * 2 ** 32))
    M, K, p = 512, 1024, 0.05
    keep = keep_mask(M, K, p, seed=1234, offset=0)
    n = keep.size
    q = drop_threshold(p) / 2 ** 32
    sd = np.sqrt(n * q * (1 - q))
    assert abs((~keep).sum() - n * q) < 5 * sd
    # each of the eight positions within a block drops at the same rate
    flat = (~keep).ravel().reshape(-1, 8)
    sd8 = np.sqrt(flat.shape[0] * q * (1 - q))
    assert np.all(np.abs(flat.sum(axis=0) - flat.shape[0] * q) < 5 * sd8)
    # a different offset or seed gives a different mask; p = 0 keeps everything
    assert not np.array_equal(keep, keep_mask(M, K, p, seed=1234, offset=1))
    assert not np.array_equal(keep, keep_mask(M, K, p, seed=1235, offset=0))
    assert keep_mask(8, 64, 0.0, 1, 2).all()


def test_zero_rate_reduces_to_plain_linear():
    rng = np.random.default_rng(23)
    M, K, N, r = 6, 64, 24, 4
    X, dY = rng.standard_normal((M, K)), rng.standard_normal((M, N))
    W = rng.standard_normal((N, K)) * 0.1
    A, B = rng.standard_normal((r, K)) * 0.1, rng.standard_normal((N, r)) * 0.1
    s = lora_scale(16.0, r)
    keep = keep_mask(M, K, 0.0, 9, 9)
    Y, U = linear_fwd_dropout(X, W, A, B, s, 0.0, keep)
    dX, dA, dB = linear_bwd_dropout(X, dY, W, A, B, s, 0.0, keep)
    Y0, U0, (dX0, dA0, dB0) = linear_no_dropout(X, dY, W, A, B, s)
    for a, b in ((Y, Y0), (U, U0), (dX, dX0), (dA, dA0), (dB, dB0)):
        np.testing.assert_allclose(a, b, rtol=1e-14, atol=1e-14)


def test_dropout_gradients_by_finite_differences():
    """With the mask fixed, L = <dY, Y> is linear in X and in each of A, B: the
    central difference quotient is exact up to rounding."""
    rng = np.random.default_rng(24)
    M, K, N, r, p = 5, 16, 7, 3, 0.3
    X = rng.standard_normal((M, K))
    W = rng.standard_normal((N, K)) * 0.1
    A = rng.standard_normal((r, K)) * 0.1
    B = rng.standard_normal((N, r)) * 0.1
    dY = rng.standard_normal((M, N))
    s = lora_scale(16.0, r)
    keep = keep_mask(M, K, p, seed=3, offset=4)
    assert 0 < (~keep).sum() < keep.size  # some dropped, some kept

    def loss(X_, A_, B_):
        return float(np.sum(dY * linear_fwd_dropout(X_, W, A_, B_, s, p, keep)[0]))

    dX, dA, dB = linear_bwd_dropout(X, dY, W, A, B, s, p, keep)
    h = 1e-3
    for name, P, G in [("X", X, dX), ("A", A, dA), ("B", B, dB)]:
        for idx in [(0, 0), (P.shape[0] - 1, P.shape[1] - 1), (P.shape[0] // 2, 1), (1, 2)]:
            Pp, Pm = P.copy(), P.copy()
            Pp[idx] += h
            Pm[idx] -= h
            args_p = dict(X_=X, A_=A, B_=B)
            args_m = dict(X_=X, A_=A, B_=B)
            args_p[name + "_"] = Pp
            args_m[name + "_"] = Pm
            fd = (loss(**args_p) - loss(**args_m)) / (2 * h)
            assert abs(fd - G[idx]) <= 1e-8 * max(1.0, abs(G[idx])), (name, idx, fd, G[idx])


def test_dropped_inputs_do_not_reach_the_adapter():
    """A dropped element of X changes only the frozen path: Y depends on it
    through X·Ŵᵀ alone (adapter with Ŵ = 0 gives Y independent of it)."""
    rng = np.random.default_rng(25)
    M, K, N, r, p = 3, 64, 8, 2, 0.5
    X = rng.standard_normal((M, K))
    A, B = rng.standard_normal((r, K)), rng.standard_normal((N, r))
    keep = keep_mask(M, K, p, seed=8, offset=0)
    i, k = map(int, np.argwhere(~keep)[0])
    X2 = X.copy()
    X2[i, k] += 10.0
    Z = np.zeros((N, K))
    Y1, U1 = linear_fwd_dropout(X, Z, A, B, 1.0, p, keep)
    Y2, U2 = linear_fwd_dropout(X2, Z, A, B, 1.0, p, keep)
    assert np.array_equal(Y1, Y2) and np.array_equal(U1, U2)
    # and a kept element scales by 1 / (1 − p) through the adapter
    i, k = map(int, np.argwhere(keep)[0])
    X3 = X.copy()
    X3[i, k] += 1.0
    Y3, _ = linear_fwd_dropout(X3, Z, A, B, 1.0, p, keep)
    np.testing.assert_allclose(Y3[i] - Y1[i], (B @ A[:, k]) / (1 - np.float32(p)), rtol=1e-12)
