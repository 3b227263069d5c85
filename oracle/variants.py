"""Quantiser variants: single quantisation (fp32 absmax per block), uniform
INT4, and the blockwise quantisation error (oracle) — TEST INFRASTRUCTURE ONLY.

Sources
-------
* "QLoRAの理論と実装" (disassemble-channel.com), §5-2 "メモリ削減の計算": with
  the first level only (Single Quantization) every block of 64 weights keeps
  its absmax as a float32, 4 + 32/64 = 4.5 bits per parameter.
* same page, "NF4による量子化と量子化誤差の比較": the uniform INT4 comparison
  quantiser uses 16 evenly spaced levels on [-1, 1] (linspace(-1, 1, 16)), the
  same zero-padded 64-element blocks scaled by their absmax, nearest level by
  a first-index argmin, an all-zero block left at zero; the experiment
  quantises 10,000 N(0, 1) samples (legacy numpy seed 42) both ways and
  compares the mean squared errors (NF4 lower, by roughly 10-30 %).

Readings taken where the pages leave a step open
------------------------------------------------
* The INT4 data type is the 16 levels (2k - 15)/15, k = 0..15, each rounded
  once to float32 (as the NF4 table is): decisions and reconstructions use
  exactly these float32 values.  They have no zero level: a zero weight sits
  on the midpoint between -1/15 and +1/15 and takes the lower index, 7.
* As for NF4, the nearest level is decided on the exact real quotient
  w / absmax; a tie at a midpoint goes to the lower index.
* An all-zero block (and the padded tail of a block) gets index 7 under INT4
  (the index a zero weight gets in any block; with absmax 0 every index
  reconstructs to 0).  NF4 keeps its zero level, index 8.
* Codes are stored exactly as NF4 codes are: two per byte, element 2t in the
  low nibble, with the float32 absmax per block (no second level; the page's
  INT4 quantiser has none).
* Reconstruction in the data type: RN32(level_idx · absmax); the bf16 decoded
  weight is RNE_bf16 of that.  The quantisation error reported is
  Σ (w − RN32(level_idx · absmax))² over the n real weights, each term formed
  in float64 and the sum correctly rounded (math.fsum); MSE = that / n.  The
  page forms its reconstruction in float64 from float64 levels; the
  difference is a few float32 ulps per element, far below the compared
  figures (the tests check both).

Parity: pinned (tests/test_oracle_variants.py): the INT4 levels against
numpy's linspace rounded to float32 and against exact rationals; the index
rule against brute force with fractions (random blocks, every midpoint ± 3
ulp at random scales, exact ties); exact round trips of level multiples; the
error bound (half the level spacing times absmax); the squared-error sum
against exact rational arithmetic on small inputs and 0 on level multiples;
the page's experiment against the page's printed range and against a float64
re-statement of the page's own procedure.
"""

import math
from fractions import Fraction

import numpy as np

from .codebook import nf4_codebook_f32, nf4_midpoints_f64
from .quant import BLOCK, _padded, bf16_round, block_absmax, pack_nibbles, quantize_nf4, unpack_nibbles

NF4 = "nf4"
INT4 = "int4"
ZERO_INDEX = {NF4: 8, INT4: 7}


def _nearest_f32(q):
    """The float32 nearest to the rational q (ties to even), found exactly."""
    f = np.float32(float(q))
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(c)) - q)
        if best is None or d < best[0] or (d == best[0] and (int(c.view(np.uint32)) & 1) == 0):
            best = (d, c)
    return best[1]


def int4_levels_f32():
    """The 16 uniform INT4 levels (2k − 15)/15, each rounded once to float32."""
    return np.array([_nearest_f32(Fraction(2 * k - 15, 15)) for k in range(16)], dtype=np.float32)


def int4_midpoints_f64():
    """Midpoints of consecutive float32 INT4 levels, exact in float64."""
    c = int4_levels_f32().astype(np.float64)
    return (c[:-1] + c[1:]) / 2.0


def levels_f32(code):
    return nf4_codebook_f32() if code == NF4 else int4_levels_f32()


def _midpoints(code):
    return nf4_midpoints_f64() if code == NF4 else int4_midpoints_f64()


def indices(w, absmax, code, blocksize=BLOCK):
    """Index of the nearest level to w / absmax for every element of the
    zero-padded flat weight, uint8: the number of level midpoints strictly
    below the quotient, i.e. of m with w > m · absmax (exact in float64)."""
    blocks = _padded(w, blocksize).astype(np.float64)
    a = np.asarray(absmax, dtype=np.float32).astype(np.float64)[:, None]
    idx = np.zeros(blocks.shape, dtype=np.uint8)
    for m in _midpoints(code):
        idx += (blocks > m * a).astype(np.uint8)
    idx[(a == 0.0)[:, 0], :] = ZERO_INDEX[code]
    return idx.ravel()


def quantize_4bit(w, code, blocksize=BLOCK):
    """First-level blockwise quantisation with either code: (packed uint8,
    absmax float32 per block)."""
    if code == NF4:
        return quantize_nf4(w, blocksize)
    absmax = block_absmax(w, blocksize)
    return pack_nibbles(indices(w, absmax, code, blocksize)), absmax


def reconstruct_f32(packed, absmax, n, code, blocksize=BLOCK):
    """RN32(level_idx · absmax) for the first n elements, float32."""
    idx = unpack_nibbles(packed)
    nb = idx.size // blocksize
    a = np.asarray(absmax, dtype=np.float32)[:nb]
    vals = (levels_f32(code)[idx].reshape(nb, blocksize) * a[:, None]).astype(np.float32)
    return vals.ravel()[:n]


def dequantize_single(packed, absmax, n, code, blocksize=BLOCK):
    """Single-quantisation decode to bf16 bit patterns: RNE_bf16(RN32(level · a))."""
    return bf16_round(reconstruct_f32(packed, absmax, n, code, blocksize))


def sq_error(w, packed, absmax, code, blocksize=BLOCK):
    """Σ (w − RN32(level_idx · absmax))² over the n weights: float64 terms,
    correctly rounded sum."""
    w = np.asarray(w, dtype=np.float32).ravel()
    r = reconstruct_f32(packed, absmax, w.size, code, blocksize)
    d = w.astype(np.float64) - r.astype(np.float64)
    return math.fsum((d * d).tolist())


def page_experiment(w):
    """The page's comparison on one weight vector: both codes, MSE each, and
    the improvement of NF4 over INT4 in percent."""
    w = np.asarray(w, dtype=np.float32).ravel()
    out = {}
    for code in (NF4, INT4):
        packed, absmax = quantize_4bit(w, code)
        out["mse_" + code] = sq_error(w, packed, absmax, code) / w.size
    out["improvement_pct"] = (1.0 - out["mse_nf4"] / out["mse_int4"]) * 100.0
    return out
