"""Merging a trained adapter into the base weight and re-quantising the result
(oracle) — TEST INFRASTRUCTURE ONLY.

Sources
-------
* "QLoRAとは？4bit量子化＋LoRAの仕組み・VRAM目安・実装手順と採用判断を解説"
  (issoh.co.jp), section "学習済みアダプタのマージと配布で精度が崩れる分岐点を
  整理する": merging into a base loaded in 4 bits re-rounds
  the sum onto the 4-bit grid, so the adapter's fine differences are lost
  and generations drift; the recommended order is to merge into the 16-bit
  base (W16 + (α/r)·B·A), keep that merged 16-bit model, and quantise it again
  if inference is to run in 4 bits.
* "QLoRAの理論と実装", §3 LoRA: the adapter adds (α/r)·B·A to the frozen
  weight (h = W0·x + (α/r)·B·A·x), so merging is W0 + (α/r)·B·A.

Readings taken where the pages leave a step open
------------------------------------------------
* Merged value of element (n, k), base value w (the bf16 16-bit base, or the
  decoded NF4 weight ŵ for the 4-bit path), s = RN32(α/r):
      acc = Σ_j B[n][j]·A[j][k], summed in float32 in the order j = 0, 1, …,
            r − 1 (each bf16 × bf16 product is exact in float32, so only the
            additions round)
      t   = RN32(s · acc)
      x   = RN32(w + t)
      m   = RNE_bf16(x)          the merged 16-bit weight the page saves
  and the re-quantised weight is the NF4 + Double Quantization of m (the
  quantiser's own readings).  Fixing the order of the float32 sum makes the
  merged value — and so every code decided on it — a function of the inputs
  alone.
* The 4-bit path ("merge into the 4-bit base") is the same formula with
  w = ŵ, the decoded NF4 + DQ weight.

Parity: pinned (tests/test_oracle_merge.py): the rank-r sum against exact
rational arithmetic on dyadic inputs (no rounding) and within the float32
error bound r·2⁻²⁴·Σ|B·A| on random inputs; A = 0 or B = 0 leaves the base
(and a base on the bf16 grid) unchanged; re-quantising goes through the
pinned quantiser; the page's warning holds: with an adapter smaller than
half the local level gap the 4-bit merge returns the original codes (the
delta is lost entirely), and the 4-bit path's error against W16 + delta
exceeds the 16-bit path's.
"""

import numpy as np

from .quant import bf16_round, bf16_to_f64, dequantize_nf4, double_quant, quantize_nf4


def _f32(bits_or_vals):
    return np.asarray(bits_or_vals, dtype=np.float32)


def rank_r_sum(A, B):
    """acc[n][k] = Σ_j B[n][j]·A[j][k] in float32, j ascending (A [r][K], B [N][r],
    float32 arrays holding bf16 values)."""
    A = _f32(A)
    B = _f32(B)
    acc = np.zeros((B.shape[0], A.shape[1]), dtype=np.float32)
    for j in range(A.shape[0]):
        acc = acc + B[:, j:j + 1] * A[j:j + 1, :]  # exact products, float32 additions
    return acc


def merge_bf16(base, A, B, s):
    """m = RNE_bf16(RN32(base + RN32(s·acc))) as bf16 bit patterns [N][K]; base is
    a float32 array of bf16 values."""
    t = np.float32(s) * rank_r_sum(A, B)
    x = _f32(base) + t
    return bf16_round(x.ravel()).reshape(x.shape)


def requantize(m_bits):
    """NF4 + DQ of the merged bf16 weight: (packed, q, c2, decoded bf16 bits)."""
    m = bf16_to_f64(m_bits).astype(np.float32).ravel()
    packed, absmax = quantize_nf4(m)
    q, c2 = double_quant(absmax)
    return packed, q, c2, dequantize_nf4(packed, q, c2, m.size).reshape(np.shape(m_bits))


def merge_16bit(w16_bits, A, B, s):
    """The recommended path: merge into the 16-bit base, then re-quantise."""
    base = bf16_to_f64(w16_bits).astype(np.float32)
    m = merge_bf16(base, A, B, s)
    return m, requantize(m)


def merge_4bit(packed, q, c2, shape, A, B, s):
    """The path the page warns about: merge into the decoded 4-bit base."""
    n = int(np.prod(shape))
    base = bf16_to_f64(dequantize_nf4(packed, q, c2, n)).astype(np.float32).reshape(shape)
    m = merge_bf16(base, A, B, s)
    return m, requantize(m)
