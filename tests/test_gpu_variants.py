"""GPU parity of the quantiser variants against the oracle: uniform INT4 codes
and single-quantisation decode bit-exact; the squared quantisation error
within 1e-12 relative (float64 terms, the sums differ only in order)."""

import numpy as np
import pytest
import torch

import workloads as wl
from oracle.variants import (INT4, NF4, dequantize_single, int4_midpoints_f64, page_experiment,
                             quantize_4bit, sq_error)

from support import bf16_bits, f32_bits, guarded, host, say, to_dev, u8

pytestmark = pytest.mark.gpu

q = pytest.importorskip("bit_nf4_quantized_blockwise_amd")

SSE_RTOL = 1e-12


def _compare(flat, code, name):
    say(f"[variants] {name}: code = {code}, n = {flat.size}")
    w = to_dev(flat)
    packed, absmax = q.quantize_4bit(w, code)
    op, oa = quantize_4bit(flat, code)
    assert np.array_equal(f32_bits(absmax), oa.view(np.uint32)), "absmax"
    gp = u8(packed)
    bad = np.nonzero(gp != op)[0]
    assert bad.size == 0, f"packed differs at {bad[:8]} ({bad.size} bytes)"
    return w, packed, absmax, op, oa


def _blocks_with_scale(a, vals):
    vals = np.asarray(vals, np.float32)
    nb = -(-vals.size // 63)
    flat = np.zeros(nb * 63, np.float32)
    flat[:vals.size] = vals
    blocks = np.zeros((nb, 64), np.float32)
    blocks[:, 0] = a
    blocks[:, 1:] = flat.reshape(nb, 63)
    return blocks.ravel()


def _sse_check(w, packed, absmax, flat, op, oa, code):
    got = float(host(q.quant_sq_error(w, packed, absmax, code))[0])
    ref = sq_error(flat, op, oa, code)
    say(f"  sse gpu {got:.17g} oracle {ref:.17g}")
    assert abs(got - ref) <= SSE_RTOL * abs(ref) + 1e-300
    return got


def test_int4_near_threshold_sweep_random_scales():
    rng = np.random.default_rng(201)
    mids = int4_midpoints_f64()
    parts = []
    for a in rng.uniform(1e-4, 0.3, 600).astype(np.float32):
        vals = []
        for m in mids:
            t = np.float32(m * float(a))
            for k in range(-3, 4):
                v = t
                step = np.float32(np.inf) if k > 0 else np.float32(-np.inf)
                for _ in range(abs(k)):
                    v = np.nextafter(v, step)
                vals.append(v)
        parts.append(_blocks_with_scale(a, vals))
    _compare(np.concatenate(parts), INT4, "midpoints ± 3 ulp, 600 random scales")


def test_int4_unit_scale_dense_sweep_and_exact_ties():
    vals = []
    for m in int4_midpoints_f64():
        bits = np.float32(m).view(np.uint32)
        off = np.arange(-2000, 2001, dtype=np.int64)
        if m == 0.0:  # around zero: both signs, denormals included
            vals.append(np.concatenate([off[off >= 0].astype(np.uint32).view(np.float32),
                                        -(off[off > 0].astype(np.uint32).view(np.float32))]))
        else:
            vals.append((np.int64(bits) + off).astype(np.uint32).view(np.float32))
    vals.append(np.random.default_rng(202).uniform(-1, 1, 400_000).astype(np.float32))
    v = np.concatenate(vals)
    v = v[np.abs(v) <= 1.0]
    _compare(_blocks_with_scale(np.float32(1.0), v), INT4, "unit scale dense sweep")


@pytest.mark.parametrize("code", [NF4, INT4])
def test_edge_blocks_ragged_decode_and_error(code):
    rng = np.random.default_rng(203)
    n = 64 * 3000 + 37
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    w[rng.random(n) < 1e-3] = np.float32(0.16)
    w[64 * 5:64 * 6] = 0.0
    w[64 * 7:64 * 8] = -0.0
    w[64 * 9:64 * 10] *= np.float32(1e-36)
    w[64 * 11:64 * 12] = np.float32(3e-41)
    w[64 * 13] = np.float32(-0.5)
    wd, packed, absmax, op, oa = _compare(w, code, "random N(0, 0.02) with edge blocks")
    out, check = guarded((n,), torch.bfloat16, 7.0)
    q.dequantize_4bit(packed, absmax, n, code, out=out)
    assert np.array_equal(bf16_bits(out), dequantize_single(op, oa, n, code))
    check()
    _sse_check(wd, packed, absmax, w, op, oa, code)


def test_nf4_code_matches_the_nf4_quantiser():
    w = (np.random.default_rng(204).standard_normal(64 * 777 + 5) * 0.02).astype(np.float32)
    wd = to_dev(w)
    p1, a1 = q.quantize_4bit(wd, NF4)
    p2, a2 = q.quantize_nf4(wd)
    assert np.array_equal(u8(p1), u8(p2)) and np.array_equal(f32_bits(a1), f32_bits(a2))


@pytest.mark.parametrize("n", [1, 7, 8, 9, 63, 65, 1000, 10000, 1_000_003])
def test_small_and_ragged_sizes(n):
    rng = np.random.default_rng(205 + n)
    w = (rng.standard_normal(n) * 0.5).astype(np.float32)
    for code in (NF4, INT4):
        wd, packed, absmax, op, oa = _compare(w, code, f"n = {n}")
        out, check = guarded((n,), torch.bfloat16, -3.0)
        q.dequantize_4bit(packed, absmax, n, code, out=out)
        assert np.array_equal(bf16_bits(out), dequantize_single(op, oa, n, code))
        check()
        _sse_check(wd, packed, absmax, w, op, oa, code)


def test_empty_and_repeatable():
    e = torch.empty(0, dtype=torch.float32, device="cuda")
    p, a = q.quantize_4bit(e, INT4)
    s = q.quant_sq_error(e, p, a, INT4)
    assert p.numel() == 0 and float(host(s)[0]) == 0.0
    assert q.dequantize_4bit(p, a, 0, INT4).numel() == 0
    w = to_dev((np.random.default_rng(206).standard_normal(3_000_017)).astype(np.float32))
    p, a = q.quantize_4bit(w, INT4)
    r1 = host(q.quant_sq_error(w, p, a, INT4)).numpy().view(np.uint64)
    r2 = host(q.quant_sq_error(w, p, a, INT4)).numpy().view(np.uint64)
    assert np.array_equal(r1, r2)


def test_page_experiment_on_the_gpu():
    """The page's comparison (10,000 N(0,1), legacy seed 42, block 64) with the
    GPU's codes and error sums: the same MSEs as the oracle and NF4 10-30 %
    better."""
    np.random.seed(42)
    w = np.random.randn(10000).astype(np.float32)
    ref = page_experiment(w)
    wd = to_dev(w)
    mse = {}
    for code in (NF4, INT4):
        p, a = q.quantize_4bit(wd, code)
        mse[code] = float(host(q.quant_sq_error(wd, p, a, code))[0]) / w.size
        assert abs(mse[code] - ref["mse_" + code]) <= SSE_RTOL * ref["mse_" + code]
    impr = (1 - mse[NF4] / mse[INT4]) * 100
    say(f"  NF4 MSE {mse[NF4]:.6f}, INT4 MSE {mse[INT4]:.6f}, improvement {impr:.2f} %")
    assert 10.0 <= impr <= 30.0


def test_llama7b_mlp_weight_full():
    """Full 11008 x 4096 LLaMA-7B MLP weight (with outliers): INT4 codes and
    absmax bit-exact, single decode bit-exact, error sums for both codes."""
    W = wl.llama7b_weight(0, 4).ravel()
    for code in (INT4, NF4):
        wd, packed, absmax, op, oa = _compare(W, code, "LLaMA-7B gate 4096->11008")
        if code == INT4:
            out = q.dequantize_4bit(packed, absmax, W.size, code)
            assert np.array_equal(bf16_bits(out), dequantize_single(op, oa, W.size, code))
            del out
        _sse_check(wd, packed, absmax, W, op, oa, code)
