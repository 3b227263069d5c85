"""Pins of the oracle's quantiser variants: uniform INT4, single quantisation
and the quantisation error."""

import json
import os
from fractions import Fraction

import numpy as np

from oracle.codebook import nf4_codebook_f32, nf4_codebook_f64
from oracle.quant import BLOCK, bf16_round, block_absmax, dequantize_nf4_single, unpack_nibbles
from oracle.variants import (INT4, NF4, dequantize_single, indices, int4_levels_f32,
                             int4_midpoints_f64, page_experiment, quantize_4bit,
                             reconstruct_f32, sq_error)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
L4 = int4_levels_f32()
L4_Q = [Fraction(float(c)) for c in L4]


def _argmin_exact(w, a):
    """Brute force: nearest INT4 level to the exact quotient, first index on a tie."""
    if a == 0:
        return 7
    x = Fraction(float(w)) / Fraction(float(a))
    best, best_d = None, None
    for i, c in enumerate(L4_Q):
        d = abs(x - c)
        if best_d is None or d < best_d:
            best, best_d = i, d
    return best


def _f32_neighbors(x, k):
    x = np.float32(x)
    out, up, dn = [x], x, x
    for _ in range(k):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(-np.inf))
        out += [up, dn]
    return out


def test_int4_levels():
    # the page's linspace(-1, 1, 16), rounded to float32 by the library
    assert np.array_equal(L4, np.linspace(-1, 1, 16).astype(np.float32))
    for k in range(16):
        exact = Fraction(2 * k - 15, 15)
        # nearest float32: no float32 neighbour is closer
        for nb in _f32_neighbors(L4[k], 1)[1:]:
            assert abs(Fraction(float(nb)) - exact) >= abs(L4_Q[k] - exact)
        assert L4[k] == -L4[15 - k]
    assert L4[0] == -1.0 and L4[15] == 1.0 and not np.any(L4 == 0)
    assert np.all(np.abs(np.diff(L4.astype(np.float64)) - 2 / 15) < 1e-7)
    m = int4_midpoints_f64()
    assert m[7] == 0.0 and m.size == 15


def test_int4_indices_match_brute_force_random_blocks():
    rng = np.random.default_rng(11)
    w = (rng.standard_normal(64 * 12) * 0.02).astype(np.float32)
    w[5] = 0.0
    a = block_absmax(w)
    idx = indices(w, a, INT4)
    for j in range(w.size):
        assert idx[j] == _argmin_exact(w[j], a[j // 64]), j
    assert idx[5] == 7  # a zero weight ties between ±1/15 and takes the lower index


def test_int4_indices_near_every_midpoint_with_random_scales():
    rng = np.random.default_rng(12)
    mids = int4_midpoints_f64()
    checked = 0
    for _ in range(30):
        a = np.float32(rng.uniform(0.01, 0.2))
        vals = []
        for m in mids:
            vals += _f32_neighbors(np.float32(m * float(a)), 3)
        vals = np.array(vals, dtype=np.float32)
        for s in range(0, vals.size, 63):
            chunk = vals[s:s + 63]
            block = np.concatenate([[a], chunk, np.zeros(63 - chunk.size, np.float32)]).astype(np.float32)
            got = indices(block, block_absmax(block), INT4)
            for j in range(1, 1 + chunk.size):
                assert got[j] == _argmin_exact(block[j], a)
                checked += 1
    assert checked == 15 * 7 * 30


def test_int4_exact_ties_go_to_lower_index():
    mids = int4_midpoints_f64()
    ties = [i for i, m in enumerate(mids) if float(np.float32(m)) == m]
    assert 7 in ties
    for i in ties:
        block = np.zeros(64, np.float32)
        block[0] = 1.0
        block[1] = np.float32(mids[i])
        assert indices(block, block_absmax(block), INT4)[1] == i
        assert _argmin_exact(block[1], np.float32(1.0)) == i


def test_level_multiples_round_trip_exactly():
    """A block of RN32(level_k · a) for every k (with the ±1 levels present, so
    absmax = a) quantises back to k and reconstructs to its own input."""
    for code, lv in ((INT4, L4), (NF4, nf4_codebook_f32())):
        for a in (np.float32(0.037), np.float32(1.5), np.float32(3e-5)):
            block = np.tile((lv * a).astype(np.float32), 4)
            packed, absmax = quantize_4bit(block, code)
            assert absmax[0] == a
            assert np.array_equal(unpack_nibbles(packed), np.tile(np.arange(16, dtype=np.uint8), 4))
            assert np.array_equal(reconstruct_f32(packed, absmax, block.size, code), block)
            assert np.array_equal(dequantize_single(packed, absmax, block.size, code),
                                  bf16_round(block))
            assert sq_error(block, packed, absmax, code) == 0.0


def test_int4_error_bound():
    """|w − l_idx·a| ≤ a/15 (half the level spacing; the outer levels are ±1)."""
    rng = np.random.default_rng(13)
    w = (rng.standard_normal(64 * 400) * 0.02).astype(np.float32)
    packed, absmax = quantize_4bit(w, INT4)
    rec = L4.astype(np.float64)[unpack_nibbles(packed)] * np.repeat(absmax.astype(np.float64), 64)
    err = np.abs(w.astype(np.float64) - rec)
    assert np.all(err <= np.repeat(absmax.astype(np.float64), 64) / 15 * (1 + 1e-6))


def test_zero_blocks_padding_and_single_decode():
    w = np.zeros(64 * 3 + 5, np.float32)
    w[64:128] = np.linspace(-0.1, 0.05, 64, dtype=np.float32)
    w[192:] = [0.01, -0.02, 0.0, 0.03, -0.005]
    packed, absmax = quantize_4bit(w, INT4)
    idx = unpack_nibbles(packed)
    assert absmax[0] == 0.0 and absmax[2] == 0.0 and absmax.size == 4
    assert np.all(idx[0:64] == 7) and np.all(idx[128:192] == 7) and np.all(idx[197:] == 7)
    assert idx[194] == 7
    d = dequantize_single(packed, absmax, w.size, INT4)
    # zero blocks decode to (−1/15)·0 = −0 under IEEE arithmetic
    assert d.size == w.size and np.all(d[:64] == 0x8000) and np.all(d[128:192] == 0x8000)
    # NF4 single-quantisation decode is the same function of the NF4 codes
    p2, a2 = quantize_4bit(w, NF4)
    assert np.array_equal(dequantize_single(p2, a2, w.size, NF4),
                          dequantize_nf4_single(p2, a2, w.size))


def test_sq_error_against_exact_rationals():
    rng = np.random.default_rng(14)
    for code in (NF4, INT4):
        w = (rng.standard_normal(64 * 4 + 37) * 0.3).astype(np.float32)
        w[3] = 1e-12  # a term whose float64 difference is not exact
        packed, absmax = quantize_4bit(w, code)
        r = reconstruct_f32(packed, absmax, w.size, code)
        exact = sum((Fraction(float(x)) - Fraction(float(y))) ** 2 for x, y in zip(w, r))
        got = sq_error(w, packed, absmax, code)
        assert abs(Fraction(got) - exact) <= exact * Fraction(1, 10 ** 14)


def test_page_experiment_nf4_beats_int4():
    """The page's comparison (10,000 N(0,1), legacy seed 42, block 64): inside
    the printed 10-30 % range, and within 1e-6 of the page's own float64
    procedure (float64 levels, float64 reconstruction, argmin)."""
    e = json.load(open(os.path.join(GOLDEN, "page_figures.json")))["nf4_vs_int4_mse_improvement_pct"]
    np.random.seed(e["seed"])
    w = np.random.randn(e["samples"]).astype(np.float32)
    got = page_experiment(w)
    assert got["mse_nf4"] < got["mse_int4"]
    assert e["low"] <= got["improvement_pct"] <= e["high"]
    # the page's procedure in float64
    n = w.size
    nb = -(-n // BLOCK)
    wp = np.zeros(nb * BLOCK)
    wp[:n] = w
    blocks = wp.reshape(nb, BLOCK)
    a = np.abs(blocks).max(axis=1)[:, None]
    x = blocks / np.where(a == 0, 1, a)
    for code, lv in ((NF4, nf4_codebook_f64()), (INT4, np.linspace(-1, 1, 16))):
        rec = (lv[np.argmin(np.abs(x[..., None] - lv), axis=-1)] * a).ravel()[:n]
        mse = np.mean((w.astype(np.float64) - rec) ** 2)
        assert abs(got["mse_" + code] - mse) <= 1e-6 * mse, code
