"""Blockwise NF4 quantisation, Double Quantization and dequantisation (oracle).

Sources
-------
* "QLoRAの理論と実装" (disassemble-channel.com), §5-1 NF4, "量子化と逆量子化の
  プロセス": step 1 (scale each block of B = 64 weights by its absolute
  maximum, so the normalised values lie in [-1, 1]), step 2 (store the index of
  the nearest level, argmin |w_norm − c_i|), step 3 (ŵ = c_{i*} · absmax).
* same page, "NF4による量子化と量子化誤差の比較": the quantiser pads the flat
  weight with zeros to a whole number of blocks, leaves an all-zero block at
  scale 0, and truncates the result back to n; its argmin over ascending levels
  returns the first (lower) index on a tie.
* same page, §5-2 Double Quantization: first level NF4 with B1 = 64 and one
  float32 absmax per block; second level quantises the absmax values 256 at a
  time to 8 bits, with one float32 constant per group.
* Qiita explainer, "Double Quantization の仕組み": W ≈ (c2 · c1^quant) · W^quant,
  which fixes the order of the two dequantisation products; "計算は壊れないのか？":
  the 4-bit weight is decoded to BF16 right before the matmul.

Readings taken where the pages leave a step open
------------------------------------------------
* Nearest level is decided on the exact real quotient w / absmax (the page's
  code promotes to float64; real-number formulas in the text).  Implemented as
  "count the level midpoints strictly below w / absmax", i.e. w > m_i · absmax,
  which float64 evaluates exactly (m_i has at most 27 significant bits and
  absmax 24).  A tie at a midpoint goes to the lower index.
* All-zero block: absmax 0, every index 8 (the exact-zero level); padded tail
  slots get index 8 as well (a zero weight maps to the zero level).
* Index packing: two indices per byte, element 2t in the low nibble.
* Second level is symmetric int8 absmax quantisation: c2 = RN32(max / 127)
  (IEEE float32 division), q = the integer in [0, 127] nearest to a / c2
  (exact, tie to the lower value; c2 = 0 gives q = 0).  Groups are 256
  consecutive blocks in block order; the last group may be short.
* Dequantisation: â = RN32(c2 · q); ŵ = RNE_bf16(RN32(c_idx · â)).

Parity: pinned (tests/test_oracle_quant.py) against brute-force rational
arithmetic (fractions) on tiny and near-tie inputs, closed forms (exact round
trips of codebook values, storage bits per parameter), the per-element error
bound (half the local level gap times absmax), and the NF4-vs-INT4 error
comparison the page runs.  The bf16 rounding step is pinned against a
nearest-neighbour search written from the definition.
"""

import numpy as np
import torch

from .codebook import nf4_codebook_f32, nf4_midpoints_f64

BLOCK = 64
GROUP = 256
ZERO_INDEX = 8


def _padded(w, blocksize):
    w = np.asarray(w, dtype=np.float32).ravel()
    nb = -(-w.size // blocksize)
    out = np.zeros(nb * blocksize, dtype=np.float32)
    out[: w.size] = w
    return out.reshape(nb, blocksize)


def block_absmax(w, blocksize=BLOCK):
    """absmax of each block of `blocksize` consecutive elements (zero-padded
    tail); float32, exact."""
    blocks = _padded(w, blocksize)
    if blocks.shape[0] == 0:
        return np.zeros(0, dtype=np.float32)
    return np.abs(blocks).max(axis=1).astype(np.float32)


def nf4_indices(w, absmax, blocksize=BLOCK):
    """Index of the nearest NF4 level to w / absmax for every element of the
    zero-padded flat weight (length nblocks * blocksize), uint8."""
    blocks = _padded(w, blocksize).astype(np.float64)
    a = np.asarray(absmax, dtype=np.float32).astype(np.float64)[:, None]
    mids = nf4_midpoints_f64()
    idx = np.zeros(blocks.shape, dtype=np.uint8)
    for m in mids:
        # w / a > m  <=>  w > m * a   (a > 0); the product is exact in float64.
        idx += (blocks > m * a).astype(np.uint8)
    idx[(a == 0.0)[:, 0], :] = ZERO_INDEX
    return idx.ravel()


def pack_nibbles(idx):
    """Two 4-bit indices per byte: element 2t in the low nibble."""
    idx = np.asarray(idx, dtype=np.uint8).ravel()
    assert idx.size % 2 == 0
    return (idx[0::2] | (idx[1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    packed = np.asarray(packed, dtype=np.uint8).ravel()
    out = np.empty(packed.size * 2, dtype=np.uint8)
    out[0::2] = packed & 0x0F
    out[1::2] = packed >> 4
    return out


def quantize_nf4(w, blocksize=BLOCK):
    """First-level quantisation: (packed uint8 [nblocks * blocksize / 2],
    absmax float32 [nblocks])."""
    absmax = block_absmax(w, blocksize)
    idx = nf4_indices(w, absmax, blocksize)
    return pack_nibbles(idx), absmax


def double_quant(absmax, group=GROUP):
    """Second-level quantisation of the block absmax values:
    (q int8 [nblocks] in [0, 127], c2 float32 [ceil(nblocks / group)])."""
    absmax = np.asarray(absmax, dtype=np.float32).ravel()
    nb = absmax.size
    ng = -(-nb // group)
    q = np.zeros(nb, dtype=np.int8)
    c2 = np.zeros(ng, dtype=np.float32)
    half_steps = np.arange(127, dtype=np.float64) + 0.5  # j + 1/2, j = 0..126
    for g in range(ng):
        a = absmax[g * group:(g + 1) * group]
        step = np.float32(a.max()) / np.float32(127.0)  # IEEE float32 division
        c2[g] = step
        if step == 0.0:
            continue
        # nearest integer to a / step, tie to the lower one:
        # q = #{ j : a > (j + 1/2) * step }, exact in float64.
        thr = half_steps * np.float64(step)
        q[g * group:(g + 1) * group] = (
            a.astype(np.float64)[:, None] > thr[None, :]
        ).sum(axis=1).astype(np.int8)
    return q, c2


def dequant_absmax(q, c2, group=GROUP):
    """â_b = RN32(c2_g · q_b), float32."""
    q = np.asarray(q, dtype=np.int8).ravel()
    c2 = np.asarray(c2, dtype=np.float32).ravel()
    g = np.arange(q.size) // group
    return (c2[g] * q.astype(np.float32)).astype(np.float32)


def bf16_round(x):
    """float32 -> bfloat16, round to nearest, ties to even; returned as uint16
    bit patterns.  (torch's CPU conversion is the library step used.)"""
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32)))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_round64(x):
    """float64 -> bfloat16 bit patterns, round to nearest, ties to even: the
    bf16 value nearest to x, and of two equally near the one whose last
    stored bit is 0.  bf16 keeps 8 significant bits, so with x = m·2^e
    (m in [0.5, 1)) its spacing near x is 2^(e−8), and 2^-133 below 2^-126
    (the subnormals); x / spacing is an exact power-of-two scaling, and its
    nearest integer (ties to even) times the spacing is the rounded value,
    which float32 holds exactly.  Values at or beyond the largest bf16 plus
    half its spacing become ±inf (float32's own overflow on the last step)."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, e = np.frexp(ax)
    q = np.maximum(e - 8, -133)
    v = np.ldexp(np.rint(np.ldexp(ax, -q)), q)
    with np.errstate(over="ignore"):
        v32 = v.astype(np.float32)
    bits = (v32.view(np.uint32) >> 16).astype(np.uint16)
    return bits | (np.signbit(x).astype(np.uint16) << 15)


def bf16_to_f64(bits):
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dequantize_nf4(packed, q, c2, n, blocksize=BLOCK, group=GROUP):
    """ŵ = RNE_bf16(RN32(c_idx · RN32(c2 · q))) for the first n elements; uint16
    bf16 bit patterns."""
    idx = unpack_nibbles(packed)
    nb = idx.size // blocksize
    a_hat = dequant_absmax(q, c2, group)[:nb]
    levels = nf4_codebook_f32()
    vals = (levels[idx].reshape(nb, blocksize) * a_hat[:, None]).astype(np.float32)
    return bf16_round(vals.ravel()[:n])


def dequantize_nf4_single(packed, absmax, n, blocksize=BLOCK):
    """Single-quantisation dequant (no second level): RNE_bf16(RN32(c_idx · a))."""
    idx = unpack_nibbles(packed)
    nb = idx.size // blocksize
    levels = nf4_codebook_f32()
    a = np.asarray(absmax, dtype=np.float32)[:nb]
    vals = (levels[idx].reshape(nb, blocksize) * a[:, None]).astype(np.float32)
    return bf16_round(vals.ravel()[:n])


def quantize_weight(w, blocksize=BLOCK, group=GROUP):
    """Full storage path of one weight: NF4 + Double Quantization.
    Returns dict(packed, absmax, q, c2, w_hat_bf16)."""
    w = np.asarray(w, dtype=np.float32)
    packed, absmax = quantize_nf4(w, blocksize)
    q, c2 = double_quant(absmax, group)
    w_hat = dequantize_nf4(packed, q, c2, w.size, blocksize, group).reshape(w.shape)
    return dict(packed=packed, absmax=absmax, q=q, c2=c2, w_hat=w_hat)


def storage_bits_per_param(n, blocksize=BLOCK, group=GROUP, double=True):
    """Bits per parameter actually stored for n weights (codes + scales)."""
    nb = -(-n // blocksize)
    code_bits = nb * blocksize * 4
    if double:
        ng = -(-nb // group)
        scale_bits = nb * 8 + ng * 32
    else:
        scale_bits = nb * 32
    return (code_bits + scale_bits) / n
