"""Pins of the oracle's quantiser, Double Quantization and dequantiser."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle.codebook import nf4_codebook_f32, nf4_midpoints_f64
from oracle.quant import (
    bf16_round,
    bf16_to_f64,
    block_absmax,
    dequant_absmax,
    dequantize_nf4,
    double_quant,
    nf4_indices,
    pack_nibbles,
    quantize_nf4,
    quantize_weight,
    storage_bits_per_param,
    unpack_nibbles,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LEVELS = nf4_codebook_f32()
LEVELS_Q = [Fraction(float(c)) for c in LEVELS]


def _argmin_exact(w, a):
    """Brute force: index of the nearest level to the exact quotient w / a,
    first index on a tie (what an argmin over ascending levels returns)."""
    if a == 0:
        return 8
    x = Fraction(float(w)) / Fraction(float(a))
    best, best_d = None, None
    for i, c in enumerate(LEVELS_Q):
        d = abs(x - c)
        if best_d is None or d < best_d:
            best, best_d = i, d
    return best


def _f32_neighbors(x, k):
    x = np.float32(x)
    out = [x]
    up, dn = x, x
    for _ in range(k):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(-np.inf))
        out += [up, dn]
    return out


def test_indices_match_brute_force_random_blocks():
    rng = np.random.default_rng(1)
    w = (rng.standard_normal(64 * 12) * 0.02).astype(np.float32)
    a = block_absmax(w)
    idx = nf4_indices(w, a)
    for j in range(w.size):
        assert idx[j] == _argmin_exact(w[j], a[j // 64]), j


def test_indices_near_every_midpoint_with_random_scales():
    """w = RN32(m_i·a) ± up to 3 ulp for random non-power-of-two a: the cases a
    rounded quotient would get wrong."""
    rng = np.random.default_rng(2)
    mids = nf4_midpoints_f64()
    checked = 0
    for trial in range(40):
        a = np.float32(rng.uniform(0.01, 0.2))
        vals = []
        for m in mids:
            vals += _f32_neighbors(np.float32(m * float(a)), 3)
        vals = np.array(vals, dtype=np.float32)
        # put a itself first so that the block absmax is a
        for s in range(0, vals.size, 63):
            chunk = vals[s:s + 63]
            block = np.concatenate([[a], chunk, np.zeros(63 - chunk.size, np.float32)])
            block = block.astype(np.float32)
            got = nf4_indices(block, block_absmax(block))
            for j in range(1, 1 + chunk.size):
                assert got[j] == _argmin_exact(block[j], a)
                checked += 1
    assert checked > 15 * 7 * 40 - 1


@pytest.mark.parametrize("a", [np.finfo(np.float32).max, np.float32(1e38), np.float32(2.0 ** 64 * 1.5),
                               np.float32(2.0 ** 126 * 1.25), np.float32(3e-39), np.float32(1e-44)])
def test_indices_near_every_midpoint_at_extreme_scales(a):
    """Block maxima at both ends of the float32 range (up to FLT_MAX, down to a
    subnormal): the decision still follows the exact quotient (the float64
    products m_i·a neither overflow nor lose bits)."""
    a = np.float32(a)
    mids = nf4_midpoints_f64()
    vals = []
    for m in mids:
        vals += [v for v in _f32_neighbors(np.float32(m * float(a)), 3) if abs(float(v)) <= float(a)]
    rng = np.random.default_rng(int(a.view(np.uint32)))
    vals += list((rng.uniform(-1, 1, 40) * float(a)).astype(np.float32))
    vals = np.array(vals, dtype=np.float32)
    for s in range(0, vals.size, 63):
        chunk = vals[s:s + 63]
        block = np.concatenate([[a], chunk, np.zeros(63 - chunk.size, np.float32)]).astype(np.float32)
        assert block_absmax(block)[0] == a
        got = nf4_indices(block, block_absmax(block))
        for j in range(1, 1 + chunk.size):
            assert got[j] == _argmin_exact(block[j], a), (float(a), float(block[j]))


def test_indices_invariant_under_power_of_two_scaling():
    """w/a does not change when both are multiplied by 2^e (exactly, inside the
    float32 range), so neither may the codes: unit-scale blocks scaled to
    2^100 and 2^-100."""
    rng = np.random.default_rng(9)
    w = (rng.standard_normal(64 * 40) * 0.02).astype(np.float32)
    ref = nf4_indices(w, block_absmax(w))
    for e in (100, -100, 127 - 4):
        ws = (w.astype(np.float64) * 2.0 ** e).astype(np.float32)
        assert np.array_equal(ws.astype(np.float64) * 2.0 ** -e, w.astype(np.float64))
        assert np.array_equal(nf4_indices(ws, block_absmax(ws)), ref), e


def test_exact_ties_go_to_lower_index():
    mids = nf4_midpoints_f64()
    for i in [1, 3, 4, 7, 8, 11, 13, 14]:
        w = np.float32(mids[i])
        assert float(w) == mids[i]
        block = np.zeros(64, np.float32)
        block[0] = 1.0
        block[1] = w
        idx = nf4_indices(block, block_absmax(block))
        assert idx[1] == i
        assert _argmin_exact(w, np.float32(1.0)) == i


def test_unit_scale_sweep_against_float64_argmin():
    """With absmax = 1 the quotient is w itself; a float64 argmin over |w − c|
    is an independent brute force (ties only occur at representable midpoints,
    where both distances are exact)."""
    mids = nf4_midpoints_f64()
    vals = []
    for m in mids:
        base = np.float32(m)
        vals.append(np.array(_f32_neighbors(base, 200), dtype=np.float32))
    rng = np.random.default_rng(3)
    vals.append(rng.uniform(-1, 1, 20000).astype(np.float32))
    vals = np.concatenate(vals)
    vals = vals[np.abs(vals) <= 1.0]
    n = vals.size
    nb = -(-n // 63)
    blocks = np.zeros((nb, 64), np.float32)
    blocks[:, 0] = 1.0
    flat = np.zeros(nb * 63, np.float32)
    flat[:n] = vals
    blocks[:, 1:] = flat.reshape(nb, 63)
    idx = nf4_indices(blocks.ravel(), block_absmax(blocks.ravel())).reshape(nb, 64)[:, 1:].ravel()[:n]
    d = np.abs(vals.astype(np.float64)[:, None] - LEVELS.astype(np.float64)[None, :])
    ref = np.argmin(d, axis=1)
    assert np.array_equal(idx, ref)


def test_codebook_values_round_trip_exactly():
    """A block holding c_k·a for every k (with c_0·a = −a present, so absmax = a)
    quantises back to k and dequantises to RN32(c_k·a) (single level)."""
    for a in [np.float32(1.0), np.float32(0.03125), np.float32(0.0371)]:
        block = np.zeros(64, np.float32)
        vals = (LEVELS * a).astype(np.float32)
        block[:16] = vals
        block[16:32] = vals[::-1]
        assert block_absmax(block)[0] == a
        idx = nf4_indices(block, block_absmax(block))
        assert list(idx[:16]) == list(range(16))
        assert list(idx[16:32]) == list(range(15, -1, -1))
        rec = (LEVELS[idx[:16]] * a).astype(np.float32)
        assert np.array_equal(rec, vals)


def test_double_quant_round_trip_power_of_two_step():
    """c2 = 2^-10 exactly (group max 127·2^-10): every block absmax that is a
    multiple q·2^-10 comes back exactly, so dequantised weights equal
    RNE_bf16(RN32(c_k · a))."""
    step = np.float32(2.0 ** -10)
    qs = np.array([127] + list(range(1, 127, 3)), dtype=np.int32)
    a_vals = (qs * step).astype(np.float32)
    blocks = []
    for a in a_vals:
        b = np.zeros(64, np.float32)
        b[:16] = (LEVELS * a).astype(np.float32)
        blocks.append(b)
    w = np.concatenate(blocks)
    packed, absmax = quantize_nf4(w)
    assert np.array_equal(absmax, a_vals)
    q, c2 = double_quant(absmax)
    assert c2[0] == np.float32(127 * 2.0 ** -10) / np.float32(127)
    assert c2[0] == step
    assert np.array_equal(q.astype(np.int32), qs)
    w_hat = dequantize_nf4(packed, q, c2, w.size)
    assert np.array_equal(w_hat, bf16_round(w))


def test_double_quant_against_brute_force():
    rng = np.random.default_rng(4)
    absmax = np.abs(rng.standard_normal(256 * 3 + 17) * 0.05).astype(np.float32)
    absmax[5] = 0.0
    q, c2 = double_quant(absmax)
    assert c2.size == 4
    for g in range(4):
        grp = absmax[g * 256:(g + 1) * 256]
        gmax = Fraction(float(grp.max()))
        exact = gmax / 127
        c = Fraction(float(c2[g]))
        # c2 is the float32 nearest to max/127
        lo = Fraction(float(np.nextafter(c2[g], np.float32(0))))
        hi = Fraction(float(np.nextafter(c2[g], np.float32(1))))
        assert abs(c - exact) <= abs(lo - exact) and abs(c - exact) <= abs(hi - exact)
        for j, a in enumerate(grp):
            x = Fraction(float(a)) / c
            best = min(range(128), key=lambda k: (abs(x - k), k))
            assert q[g * 256 + j] == best
        assert q[g * 256 + int(np.argmax(grp))] == 127


def test_double_quant_tie_goes_low():
    step = np.float32(2.0 ** -8)
    absmax = np.zeros(256, np.float32)
    absmax[0] = 127 * step
    absmax[1] = np.float32(10.5) * step   # exactly between 10 and 11
    absmax[2] = np.float32(0.5) * step    # exactly between 0 and 1
    q, c2 = double_quant(absmax)
    assert c2[0] == step
    assert q[1] == 10 and q[2] == 0 and q[0] == 127


def test_zero_blocks_and_padding():
    w = np.zeros(64 * 3 + 5, np.float32)
    w[64:128] = np.linspace(-0.1, 0.05, 64, dtype=np.float32)
    w[192:] = [0.01, -0.02, 0.0, 0.03, -0.005]
    packed, absmax = quantize_nf4(w)
    assert absmax.size == 4 and packed.size == 4 * 32
    assert absmax[0] == 0.0 and absmax[2] == 0.0
    assert absmax[3] == np.float32(0.03)
    idx = unpack_nibbles(packed)
    assert np.all(idx[0:64] == 8) and np.all(idx[128:192] == 8)
    assert np.all(idx[192 + 5:] == 8)  # padded tail slots
    q, c2 = double_quant(absmax)
    assert q[0] == 0 and q[2] == 0
    w_hat = dequantize_nf4(packed, q, c2, w.size)
    assert w_hat.size == w.size
    assert np.all(w_hat[:64] == 0) and np.all(w_hat[128:192] == 0)


def test_empty_input():
    packed, absmax = quantize_nf4(np.zeros(0, np.float32))
    assert packed.size == 0 and absmax.size == 0
    q, c2 = double_quant(absmax)
    assert q.size == 0 and c2.size == 0


def test_pack_unpack_invariant():
    rng = np.random.default_rng(5)
    idx = rng.integers(0, 16, 1000).astype(np.uint8)
    p = pack_nibbles(idx)
    assert p.size == 500
    assert p[0] == (idx[0] | (idx[1] << 4))
    assert np.array_equal(unpack_nibbles(p), idx)


def test_reconstruction_error_bound():
    """|w − c_idx·a| ≤ (local gap / 2)·a; above the top level the bound is
    (1 − c_15)·a (QLoRAの理論と実装, §5-1 step 2: nearest level)."""
    rng = np.random.default_rng(6)
    w = (rng.standard_normal(64 * 500) * 0.02).astype(np.float32)
    w[rng.random(w.size) < 1e-3] = 0.16
    packed, absmax = quantize_nf4(w)
    idx = unpack_nibbles(packed)
    a = np.repeat(absmax.astype(np.float64), 64)
    rec = LEVELS.astype(np.float64)[idx] * a
    c = LEVELS.astype(np.float64)
    gap_lo = np.concatenate([[0.0], np.diff(c)])
    gap_hi = np.concatenate([np.diff(c), [2 * (1.0 - c[15])]])
    bound = np.where(w.astype(np.float64) >= rec, gap_hi[idx], gap_lo[idx]) / 2 * a
    err = np.abs(w.astype(np.float64) - rec)
    assert np.all(err <= bound * (1 + 1e-12) + 1e-30)


def test_bf16_rounding_against_definition():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(5000).astype(np.float32) * 0.03,
        np.array([1.0, -1.0, 0.0, 1.00390625, 1.005859375, 1.001953125, 3e-39, -2e-40],
                 np.float32),
    ])
    # construct exact ties: bf16 value + half a bf16 ulp
    base = (rng.standard_normal(200).astype(np.float32).view(np.uint32) & 0xFFFF0000)
    ties = (base | 0x8000).view(np.float32)
    x = np.concatenate([x, ties])
    got = bf16_round(x)
    for v, g in zip(x, got):
        bits = int(np.float32(v).view(np.uint32))
        lo = bits & 0xFFFF0000
        hi = lo + 0x10000
        lo_v = float(np.uint32(lo).view(np.float32))
        hi_v = float(np.uint32(hi).view(np.float32))
        dl, dh = abs(float(v) - lo_v), abs(float(v) - hi_v)
        if dl < dh:
            want = lo
        elif dh < dl:
            want = hi
        else:
            want = lo if ((lo >> 16) & 1) == 0 else hi
        assert int(g) == (want >> 16), (v, hex(bits), hex(int(g)))


def test_storage_bits_per_param_closed_forms():
    figs = json.load(open(os.path.join(GOLDEN, "page_figures.json")))
    n = 64 * 256 * 100
    dq = storage_bits_per_param(n, double=True)
    sq = storage_bits_per_param(n, double=False)
    assert dq == 4 + 8 / 64 + 32 / (64 * 256) == 4.126953125
    assert sq == figs["single_quant_bits_per_param"]["value"]
    assert sq - 4 == figs["scale_overhead_bits_per_param"]["value"]
    e = figs["double_quant_bits_per_param_approx"]
    assert abs(dq - e["value"]) <= e["abs_tol"]
    e = figs["double_quant_saving_bits_approx"]
    assert abs((sq - dq) - e["value"]) <= e["abs_tol"]
    assert sq - dq == 0.373046875
    e = figs["scale_overhead_65b_gb_approx"]
    assert abs(65e9 * (sq - 4) / 8 / 1e9 - e["value"]) <= e["abs_tol"] + 0.07
    e = figs["double_quant_saving_65b_gb_approx"]
    assert abs(65e9 * (sq - dq) / 8 / 1e9 - e["value"]) <= e["abs_tol"]
    # the byte buffers the quantiser actually produces agree with the formula
    w = np.zeros(n, np.float32)
    w[::7] = 0.01
    packed, absmax = quantize_nf4(w)
    q, c2 = double_quant(absmax)
    assert (packed.nbytes + q.nbytes + c2.nbytes) * 8 / n == dq
    assert (packed.nbytes + absmax.nbytes) * 8 / n == sq


def test_nf4_beats_int4_as_the_page_measures():
    """The page's experiment: 10,000 N(0,1) samples (legacy seed 42), block 64,
    NF4 vs uniform 16-level INT4 on [-1, 1] with the same absmax blocks."""
    e = json.load(open(os.path.join(GOLDEN, "page_figures.json")))["nf4_vs_int4_mse_improvement_pct"]
    np.random.seed(e["seed"])
    w = np.random.randn(e["samples"]).astype(np.float32)
    packed, absmax = quantize_nf4(w)
    idx = unpack_nibbles(packed)[: w.size]
    a = np.repeat(absmax.astype(np.float64), 64)[: w.size]
    nf4 = LEVELS.astype(np.float64)[idx] * a
    # INT4 comparison quantiser (test-only): nearest of linspace(-1, 1, 16)
    lv = np.linspace(-1, 1, 16)
    x = w.astype(np.float64) / a
    int4 = lv[np.argmin(np.abs(x[:, None] - lv[None, :]), axis=1)] * a
    mse_nf4 = np.mean((w - nf4) ** 2)
    mse_int4 = np.mean((w - int4) ** 2)
    impr = (1 - mse_nf4 / mse_int4) * 100
    assert mse_nf4 < mse_int4
    assert e["low"] <= impr <= e["high"], impr


def test_lora_param_count_figure():
    e = json.load(open(os.path.join(GOLDEN, "page_figures.json")))["lora_params_d4096_k4096_r8"]
    from workloads import SINGLE_LINEAR as wl
    inp = wl.inputs(M=1)
    assert inp["A"].numel() + inp["B"].numel() == e["value"]
    assert wl.n_out * wl.k_in == e["full"]
    assert round(100 * e["value"] / e["full"], 1) == e["fraction_pct_approx"]


def test_dequant_order_matches_page():
    """â = RN32(c2·q) first, then RN32(c·â): differs from RN32(c·c2)·q in general
    (Qiita explainer: W ≈ (c2 · c1^quant) · W^quant)."""
    q = np.array([97], np.int8)
    c2 = np.array([np.float32(0.0013)], np.float32)
    a_hat = dequant_absmax(q, c2)
    assert a_hat[0] == np.float32(c2[0] * np.float32(97))
    packed = pack_nibbles(np.array([15, 0] * 32, np.uint8))
    w_hat = dequantize_nf4(packed, q, c2, 64)
    assert w_hat[0] == bf16_round(np.array([LEVELS[15] * a_hat[0]], np.float32))[0]
    assert bf16_to_f64(w_hat[1]) == -float(bf16_to_f64(bf16_round(np.array([a_hat[0]], np.float32)))[0])


def test_quantize_weight_shapes():
    w = (np.random.default_rng(8).standard_normal((96, 128)) * 0.02).astype(np.float32)
    r = quantize_weight(w)
    assert r["packed"].size == 96 * 128 // 2
    assert r["absmax"].size == 96 * 2 and r["q"].size == 96 * 2 and r["c2"].size == 1
    assert r["w_hat"].shape == (96, 128)
    assert np.all(np.abs(bf16_to_f64(r["w_hat"]) - w) <= np.repeat(r["absmax"], 64).reshape(96, 128) * 0.13)


def test_group_chunked_oracle_equals_whole_weight():
    """The parity harness runs the oracle on ranges of whole DQ groups in
    threads (DQ groups are independent); joined, that must be exactly the
    whole-weight result, with a ragged last chunk and a short last group."""
    from support import oracle_weight, oracle_weight_parallel
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((37, 11008)) * 0.02).astype(np.float32)
    W[rng.random(W.shape) < 1e-3] = np.float32(0.16)
    a = oracle_weight(W)
    b = oracle_weight_parallel(W, threads=3, chunk_groups=4)
    for k in ("packed", "absmax", "q", "c2", "w_hat"):
        assert a[k].dtype == b[k].dtype and np.array_equal(a[k], b[k]), k
