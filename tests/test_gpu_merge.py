"""GPU parity of the adapter merge and re-quantisation against the oracle:
the merged bf16 weight and every re-quantised byte bit-exact, for the 16-bit
and the 4-bit base."""

import numpy as np
import pytest
import torch

import workloads as wl
from oracle.merge import merge_16bit, merge_4bit
from oracle.quant import bf16_to_f64, double_quant, quantize_nf4
from oracle.linear import lora_scale

from support import bf16_bits, f32_bits, guarded, host, say, to_dev, u8

pytestmark = pytest.mark.gpu

q = pytest.importorskip("bit_nf4_quantized_blockwise_amd")


def _adapter(N, K, r, seed, sigma=0.01):
    key = 970 + seed
    A = wl.bf16_normal(key, (r, K), sigma, tensor=wl.T_A)
    B = wl.bf16_normal(key, (N, r), sigma, tensor=wl.T_B)
    return A, B


def _f32(t):
    return t.to(torch.float32).numpy()


def _check_requant(out, ref):
    packed, qa, c2, _ = ref
    assert np.array_equal(u8(out.packed), packed), "packed"
    assert np.array_equal(u8(out.qabsmax).view(np.int8), qa), "qabsmax"
    assert np.array_equal(f32_bits(out.c2), c2.view(np.uint32)), "c2"


@pytest.mark.parametrize("N,K,r,alpha", [
    (1, 64, 1, 2.0),
    (16, 1024, 8, 16.0),
    (37, 192, 3, 16.0),       # ragged rows and columns, odd rank
    (100, 2112, 64, 16.0),
    (64, 448, 72, 16.0),      # rank not a multiple of the load batch
    (20, 256, 256, 32.0),     # largest rank
])
def test_merge_16bit_and_4bit_bit_exact(N, K, r, alpha):
    say(f"[merge] N={N} K={K} r={r}")
    W = wl.weight_f32(980 + r, N, K)
    W16 = torch.from_numpy(W).to(torch.bfloat16)
    A, B = _adapter(N, K, r, r, sigma=0.05)
    s = lora_scale(alpha, r)
    Ad, Bd = to_dev(A), to_dev(B)
    # the recommended path: 16-bit base
    merged, check = guarded((N, K), torch.bfloat16, 7.0)
    _, out = q.merge_adapter(to_dev(W16), Ad, Bd, alpha, merged=merged)
    m_ref, rq = merge_16bit(bf16_bits(W16).reshape(N, K), _f32(A), _f32(B), s)
    assert np.array_equal(bf16_bits(merged), m_ref)
    _check_requant(out, rq)
    check()
    # the 4-bit base: the NF4 + DQ storage of W
    wq = q.quantize_weight(to_dev(W))
    packed, absmax = quantize_nf4(W.ravel())
    qa, c2 = double_quant(absmax)
    m4, out4 = q.merge_adapter(wq, Ad, Bd, alpha)
    m4_ref, rq4 = merge_4bit(packed, qa, c2, (N, K), _f32(A), _f32(B), s)
    assert np.array_equal(bf16_bits(m4), m4_ref)
    _check_requant(out4, rq4)


def _merge_sweep(n, seed):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 300)), 64 * int(rng.integers(1, 40)), int(rng.integers(1, 257)),
             float(rng.choice([2.0, 16.0, 32.0]))) for _ in range(n)]


@pytest.mark.parametrize("N,K,r,alpha", _merge_sweep(6, 4711))
def test_merge_sweep(N, K, r, alpha):
    """Seeded shapes and ranks: merged bf16 and re-quantised bytes bit-exact
    against the oracle on both bases."""
    test_merge_16bit_and_4bit_bit_exact(N, K, r, alpha)


def test_merge_only_and_repeatable():
    N, K, r = 48, 640, 16
    W16 = torch.from_numpy(wl.weight_f32(990, N, K)).to(torch.bfloat16)
    A, B = _adapter(N, K, r, 1)
    a, none = q.merge_adapter(to_dev(W16), to_dev(A), to_dev(B), 16.0, requantize=False)
    b, _ = q.merge_adapter(to_dev(W16), to_dev(A), to_dev(B), 16.0, requantize=False)
    assert none is None and torch.equal(a.view(torch.int16), b.view(torch.int16))
    # a zero adapter returns the base bit for bit
    z, _ = q.merge_adapter(to_dev(W16), to_dev(A), to_dev(torch.zeros_like(B)), 16.0,
                           requantize=False)
    assert torch.equal(host(z).view(torch.int16), W16.view(torch.int16))


def test_page_warning_on_the_gpu():
    """A small adapter merged into the 4-bit base keeps under 15 % of its delta
    after re-quantisation; the 16-bit path is closer to W16 + delta."""
    N, K, r = 512, 1024, 8
    W = wl.weight_f32(991, N, K)
    W16 = torch.from_numpy(W).to(torch.bfloat16)
    A, B = _adapter(N, K, r, 2, sigma=0.03)
    s = lora_scale(2.0, r)  # 0.25
    wq = q.quantize_weight(to_dev(W))
    base4 = bf16_to_f64(bf16_bits(q.dequantize_nf4(wq)))
    _, out4 = q.merge_adapter(wq, to_dev(A), to_dev(B), 2.0)
    d4 = bf16_to_f64(bf16_bits(q.dequantize_nf4(out4)))
    D = s * (_f32(B).astype(np.float64) @ _f32(A).astype(np.float64))
    kept = np.sum((d4 - base4) * D) / np.sum(D * D)
    say(f"  4-bit merge keeps {kept:.3f} of the adapter delta")
    assert kept < 0.15
    _, out16 = q.merge_adapter(to_dev(W16), to_dev(A), to_dev(B), 2.0)
    d16 = bf16_to_f64(bf16_bits(q.dequantize_nf4(out16)))
    target = bf16_to_f64(bf16_bits(W16)) + D
    assert np.linalg.norm(d4 - target) > 1.05 * np.linalg.norm(d16 - target)


def test_llama7b_mlp_weight_full():
    """11008 x 4096 gate weight with an r = 64 adapter: both paths, every byte."""
    W = wl.llama7b_weight(0, 4)
    N, K = W.shape
    r, alpha = 64, 16.0
    A, B = _adapter(N, K, r, 3)
    s = lora_scale(alpha, r)
    W16 = torch.from_numpy(W).to(torch.bfloat16)
    say("[merge] full 11008 x 4096, r = 64, 16-bit base")
    m, out = q.merge_adapter(to_dev(W16), to_dev(A), to_dev(B), alpha)
    m_ref, rq = merge_16bit(bf16_bits(W16).reshape(N, K), _f32(A), _f32(B), s)
    assert np.array_equal(bf16_bits(m), m_ref)
    _check_requant(out, rq)
    say("[merge] full 11008 x 4096, r = 64, 4-bit base")
    packed, absmax = quantize_nf4(W.ravel())
    qa, c2 = double_quant(absmax)
    m4, out4 = q.merge_adapter(q.quantize_weight(to_dev(W)), to_dev(A), to_dev(B), alpha)
    m4_ref, rq4 = merge_4bit(packed, qa, c2, (N, K), _f32(A), _f32(B), s)
    assert np.array_equal(bf16_bits(m4), m4_ref)
    _check_requant(out4, rq4)
