"""GPU parity of the quantiser, Double Quantization and dequantiser against the
oracle: bit-exact on every byte, code and bf16 value."""

import numpy as np
import pytest
import torch

import workloads as wl
from oracle.codebook import nf4_codebook_f32, nf4_midpoints_f64
from oracle.quant import block_absmax, dequantize_nf4, double_quant, quantize_nf4

from support import bf16_bits, f32_bits, guarded, host, oracle_weight, say, to_dev, u8

pytestmark = pytest.mark.gpu

q = pytest.importorskip("bit_nf4_quantized_blockwise_amd")


def _gpu_all(flat):
    """Every GPU route: separate calls, the combined entry point with the scales
    kept (two launches) and without them (one pass) — all must agree bytewise."""
    w = to_dev(flat)
    packed, absmax = q.quantize_nf4(w)
    qa, c2 = q.double_quant(absmax)
    fp, fq, fc2, fabs = q.quantize_nf4_dq(w, want_absmax=True)
    op, oq, oc2 = q.quantize_nf4_dq(w, one_pass=True)
    torch.cuda.synchronize()
    for p_, q_, c_ in ((fp, fq, fc2), (op, oq, oc2)):
        assert np.array_equal(u8(packed), u8(p_))
        assert np.array_equal(u8(qa), u8(q_))
        assert np.array_equal(f32_bits(c2), f32_bits(c_))
    assert np.array_equal(f32_bits(absmax), f32_bits(fabs))
    return packed, absmax, qa, c2


def _compare(flat, name):
    say(f"[quant] {name}: n = {flat.size}")
    packed, absmax, qa, c2 = _gpu_all(flat)
    op, oa = quantize_nf4(flat)
    oq, oc2 = double_quant(oa)
    assert np.array_equal(f32_bits(absmax), oa.view(np.uint32)), "absmax"
    gp = u8(packed)
    bad = np.nonzero(gp != op)[0]
    assert bad.size == 0, f"packed differs at {bad[:8]} ({bad.size} bytes)"
    assert np.array_equal(u8(qa).view(np.int8), oq), "qabsmax"
    assert np.array_equal(f32_bits(c2), oc2.view(np.uint32)), "c2"
    return packed, qa, c2, op, oq, oc2


def _blocks_with_scale(a, vals):
    """Blocks of 64 whose first element is a (so absmax = a) and the rest vals."""
    vals = np.asarray(vals, np.float32)
    nb = -(-vals.size // 63)
    flat = np.zeros(nb * 63, np.float32)
    flat[:vals.size] = vals
    blocks = np.zeros((nb, 64), np.float32)
    blocks[:, 0] = a
    blocks[:, 1:] = flat.reshape(nb, 63)
    return blocks.ravel()


def test_near_threshold_sweep_random_scales():
    rng = np.random.default_rng(101)
    mids = nf4_midpoints_f64()
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
    flat = np.concatenate(parts)
    _compare(flat, "midpoints ± 3 ulp, 600 random scales")


def test_unit_scale_dense_sweep_and_exact_ties():
    mids = nf4_midpoints_f64()
    vals = []
    for m in mids:
        base = np.float32(m)
        bits = base.view(np.uint32)
        # 4001 consecutive float32 values centred on the midpoint
        off = np.arange(-2000, 2001, dtype=np.int64)
        cand = (np.int64(bits) + off).astype(np.uint32).view(np.float32)
        vals.append(cand)
    rng = np.random.default_rng(102)
    vals.append(rng.uniform(-1, 1, 400_000).astype(np.float32))
    v = np.concatenate(vals)
    v = v[np.abs(v) <= 1.0]
    _compare(_blocks_with_scale(np.float32(1.0), v), "unit scale dense sweep")


def test_random_weights_edge_blocks_ragged():
    rng = np.random.default_rng(103)
    n = 64 * 3000 + 37
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    w[rng.random(n) < 1e-3] = np.float32(0.16)
    w[64 * 5:64 * 6] = 0.0                       # an all-zero block
    w[64 * 7:64 * 8] = -0.0                      # negative zeros
    w[64 * 9:64 * 10] *= np.float32(1e-36)       # tiny (subnormal products)
    w[64 * 11:64 * 12] = np.float32(3e-41)       # subnormal inputs
    w[64 * 13] = np.float32(-0.5)                # negative absmax
    w[64 * 256 * 2:64 * 256 * 3] = 0.0          # an all-zero DQ group (c2 = 0)
    packed, qa, c2, op, oq, oc2 = _compare(w, "random N(0, 0.02) with edge blocks")
    # dequantiser: bf16 bit-exact (n must be a multiple of 64: drop the tail)
    m = (n // 64) * 64
    wq = q.NF4Tensor(packed, qa, c2, m // 64, 64)
    out, check = guarded((m // 64, 64), torch.bfloat16, 7.0)
    q.dequantize_nf4(wq, out=out)
    ref = dequantize_nf4(op, oq, oc2, m)
    assert np.array_equal(bf16_bits(out).ravel(), ref)
    check()


@pytest.mark.parametrize("n", [0, 1, 63, 64, 65, 16384, 16385])
def test_small_and_empty_sizes(n):
    rng = np.random.default_rng(104 + n)
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    if n == 0:
        wt = torch.zeros(0, dtype=torch.float32, device="cuda")
        p, a = q.quantize_nf4(wt)
        qa, c2 = q.double_quant(a)
        torch.cuda.synchronize()
        assert p.numel() == 0 and qa.numel() == 0 and c2.numel() == 0
        return
    _compare(w, f"n = {n}")


def test_single_linear_weight_full():
    W = wl.SINGLE_LINEAR.inputs()["W"]
    packed, qa, c2, op, oq, oc2 = _compare(W.ravel(), "single linear 4096x4096")
    wq = q.NF4Tensor(packed, qa, c2, 4096, 4096)
    out = q.dequantize_nf4(wq)
    ref = dequantize_nf4(op, oq, oc2, W.size)
    assert np.array_equal(bf16_bits(out).ravel(), ref)


@pytest.mark.parametrize("matrix", [0, 4, 6])  # q 4096x4096, gate 4096->11008, down 11008->4096
def test_llama7b_shapes_full(matrix):
    W = wl.llama7b_weight(0, matrix)
    say(f"[quant] llama7b layer 0 matrix {matrix}: {W.shape}")
    wt = to_dev(W)
    wq = q.quantize_weight(wt)
    out = q.dequantize_nf4(wq)
    o = oracle_weight(W)
    assert np.array_equal(u8(wq.packed), o["packed"])
    assert np.array_equal(u8(wq.qabsmax).view(np.int8), o["q"])
    assert np.array_equal(f32_bits(wq.c2), o["c2"].view(np.uint32))
    assert np.array_equal(bf16_bits(out), o["w_hat"])


def test_weight_beyond_two_to_the_31_elements():
    """524,290 x 4096 float32 (2^31 + 8192 weights, 8.6 GB): 64-bit indexing in
    the quantisers and the dequantiser.  Whole DQ groups (independent of the
    rest) at the 2^31 boundary and at the end are checked against the oracle;
    both quantiser routes must give the same bytes everywhere."""
    n_out, k_in = (1 << 31) // 4096 + 2, 4096
    n = n_out * k_in
    say(f"[quant] {n_out} x {k_in} = {n} weights")
    gen = torch.Generator(device="cuda").manual_seed(31)
    W = torch.randn(n_out, k_in, generator=gen, device="cuda", dtype=torch.float32) * 0.02
    W.view(-1)[n - 64:] = 0.0                      # an all-zero last block
    packed, qa, c2, absmax = q.quantize_nf4_dq(W, want_absmax=True)
    p1, q1, c21 = q.quantize_nf4_dq(W, one_pass=True)
    assert torch.equal(packed, p1) and torch.equal(qa, q1) and torch.equal(c2.view(torch.int32),
                                                                         c21.view(torch.int32))
    del p1, q1, c21
    out = q.dequantize_nf4(q.NF4Tensor(packed, qa, c2, n_out, k_in))
    G = 64 * 256
    ngroups = n // G
    for g in (0, (1 << 31) // G - 1, (1 << 31) // G, ngroups - 1):
        s0, s1 = g * G, (g + 1) * G
        flat = host(W.view(-1)[s0:s1]).numpy()
        op, oa = quantize_nf4(flat)
        oq, oc2 = double_quant(oa)
        assert np.array_equal(u8(packed[s0 // 2:s1 // 2]), op), g
        assert np.array_equal(u8(qa[s0 // 64:s1 // 64]).view(np.int8), oq), g
        assert f32_bits(c2[g:g + 1])[0] == oc2.view(np.uint32)[0], g
        assert np.array_equal(f32_bits(absmax[s0 // 64:s1 // 64]), oa.view(np.uint32)), g
        ref = dequantize_nf4(op, oq, oc2, G)
        assert np.array_equal(bf16_bits(out.view(-1)[s0:s1]), ref), g


def test_batches_match_single_calls_and_oracle():
    """53 weights (two launches of up to 48 jobs), ragged tails and an empty one:
    every byte of the batched quantiser and decoder equals the single-matrix
    calls; one ragged weight is also compared with the oracle."""
    rng = np.random.default_rng(77)
    sizes = [64, 100, 0, 16384 + 64, 4096 * 64, 255 * 64 + 17] + \
        [64 * (1 + (i * 37) % 700) for i in range(47)]
    say(f"[quant] batches of {len(sizes)} weights")
    flats = [(rng.standard_normal(n) * 0.02).astype(np.float32) for n in sizes]
    ws = [to_dev(f) for f in flats]
    got = q.quantize_nf4_dq_batch(ws)
    torch.cuda.synchronize()
    for w, g in zip(ws, got):
        ref = q.quantize_nf4_dq(w, want_absmax=True)
        torch.cuda.synchronize()
        assert np.array_equal(u8(g[0]), u8(ref[0]))
        assert np.array_equal(u8(g[1]), u8(ref[1]))
        assert np.array_equal(f32_bits(g[2]), f32_bits(ref[2]))
        assert np.array_equal(f32_bits(g[3]), f32_bits(ref[3]))
    op, oa = quantize_nf4(flats[1])
    oq, oc2 = double_quant(oa)
    assert np.array_equal(u8(got[1][0]), op)
    assert np.array_equal(u8(got[1][1]).view(np.int8), oq)
    assert np.array_equal(f32_bits(got[1][2]), oc2.view(np.uint32))
    wqs = [q.NF4Tensor(g[0], g[1], g[2], n // 64, 64) for n, g in zip(sizes, got) if n % 64 == 0]
    outs = q.dequantize_nf4_batch(wqs)
    torch.cuda.synchronize()
    for wq, o in zip(wqs, outs):
        assert np.array_equal(bf16_bits(o), bf16_bits(q.dequantize_nf4(wq)))
    i3 = [n for n in sizes if n % 64 == 0].index(16384 + 64)
    p3, a3 = quantize_nf4(flats[3])
    q3, c3 = double_quant(a3)
    assert np.array_equal(bf16_bits(outs[i3]).ravel(), dequantize_nf4(p3, q3, c3, sizes[3]))


def test_batches_of_one_llama7b_layer_match_single_calls():
    """The seven matrices of layer 0 of the LLaMA-7B weight set (with their
    outliers) in one batch: every byte of the quantiser and every decoded
    value equals the single-weight calls."""
    say("[quant] batch of the 7 matrices of a LLaMA-7B layer")
    ws = [to_dev(wl.llama7b_weight(0, m)) for m in range(len(wl.LLAMA7B_MATRICES))]
    got = q.quantize_nf4_dq_batch([w.reshape(-1) for w in ws])
    torch.cuda.synchronize()
    wqs = []
    for w, g in zip(ws, got):
        ref = q.quantize_nf4_dq(w.reshape(-1), want_absmax=True)
        torch.cuda.synchronize()
        assert np.array_equal(u8(g[0]), u8(ref[0]))
        assert np.array_equal(u8(g[1]), u8(ref[1]))
        assert np.array_equal(f32_bits(g[2]), f32_bits(ref[2]))
        wqs.append(q.NF4Tensor(g[0], g[1], g[2], w.shape[0], w.shape[1]))
    outs = q.dequantize_nf4_batch(wqs)
    torch.cuda.synchronize()
    for wq, o in zip(wqs, outs):
        assert torch.equal(o.view(torch.int16), q.dequantize_nf4(wq).view(torch.int16))


def test_huge_and_tiny_block_maxima():
    """Block maxima from subnormal up to FLT_MAX: codes, scales, DQ codes and
    decoded bf16 (overflowing to ±Inf where RNE_bf16 does) bit-exact on every
    route.  Above 2^126 the reciprocal of the maximum is subnormal, which the
    bucket estimate must not meet."""
    mids = nf4_midpoints_f64()
    rng = np.random.default_rng(106)
    parts = []
    scales = [np.finfo(np.float32).max, 3e38, 1e38, 2.0 ** 127, 2.0 ** 126 * 1.5, 2.0 ** 64 * 1.5,
              2.0 ** 64, 1e30, 1e-30, 2.0 ** -64, 3e-39, 1e-44]
    for a in np.array(scales, dtype=np.float32):
        vals = []
        for m in mids:
            t = np.float32(m * float(a))
            for k in range(-3, 4):
                v = t
                for _ in range(abs(k)):
                    v = np.nextafter(v, np.float32(np.inf) if k > 0 else np.float32(-np.inf))
                if abs(float(v)) <= float(a):
                    vals.append(v)
        vals += list((rng.uniform(-1, 1, 300) * float(a)).astype(np.float32))
        parts.append(_blocks_with_scale(a, vals))
    # whole DQ groups of huge blocks next to ordinary ones
    big = (rng.standard_normal(64 * 256) * 0.02).astype(np.float32)
    big[::64] = np.float32(3.3e38)
    parts.append(big)
    flat = np.concatenate(parts)
    m = -(-flat.size // 64) * 64
    flat = np.concatenate([flat, np.zeros(m - flat.size, np.float32)])
    packed, qa, c2, op, oq, oc2 = _compare(flat, "block maxima from 1e-44 to FLT_MAX")
    out = q.dequantize_nf4(q.NF4Tensor(packed, qa, c2, m // 64, 64))
    got, ref = bf16_bits(out).ravel(), dequantize_nf4(op, oq, oc2, m)
    # Near FLT_MAX, RN32(c2·q) overflows to Inf and the zero level decodes to
    # 0·Inf = NaN; IEEE leaves that NaN's sign and payload to the platform, so
    # a NaN matches any NaN.  Every other value must agree bit for bit.
    is_nan = lambda b: ((b & 0x7f80) == 0x7f80) & ((b & 0x007f) != 0)
    assert np.array_equal(is_nan(got), is_nan(ref))
    assert np.array_equal(got[~is_nan(got)], ref[~is_nan(ref)])
    assert np.any(is_nan(ref)) and np.any(ref == 0x7f80)  # the overflow case is exercised


def _flag():
    return torch.zeros(1, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
@pytest.mark.parametrize("where", ["first", "middle", "tail"])
def test_nonfinite_flag_is_set_on_every_route(bad, where):
    """A NaN or ±Inf anywhere (first element, inside, in a ragged tail) sets the
    optional flag on the first-level, the two-launch, the one-pass and the
    batched quantiser; finite input leaves it untouched (a preset value
    survives); no flag (NULL) is accepted."""
    say(f"[quant] non-finite {bad} at {where}")
    rng = np.random.default_rng(107)
    n = 64 * 700 + 13
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    pos = {"first": 0, "middle": 64 * 333 + 17, "tail": n - 2}[where]
    wb = w.copy()
    wb[pos] = np.float32(bad)
    good, poisoned = to_dev(w), to_dev(wb)
    for src, expect in ((good, 0), (poisoned, 1)):
        flags = [_flag() for _ in range(5)]
        q.quantize_nf4(src, nonfinite_flag=flags[0])
        q.quantize_nf4_dq(src, nonfinite_flag=flags[1])
        q.quantize_nf4_dq(src, one_pass=True, nonfinite_flag=flags[2])
        q.quantize_nf4_dq_batch([good, src], nonfinite_flags=[None, flags[3]])
        flags[4].fill_(7)
        q.quantize_nf4_dq_batch([src], nonfinite_flags=[flags[4]])
        got = [int(host(f)[0]) for f in flags]
        assert got[:4] == [expect] * 4, got
        assert got[4] == (7 if expect == 0 else 1), got
    # without a flag the call still runs (codes of non-finite input are unspecified)
    q.quantize_nf4(poisoned)
    q.quantize_nf4_dq(poisoned, one_pass=True)
    torch.cuda.synchronize()
