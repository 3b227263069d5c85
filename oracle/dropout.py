"""LoRA dropout on the adapter input, with a counter-based random mask (oracle)
— TEST INFRASTRUCTURE ONLY.

Sources
-------
* "QLoRAの理論と実装" (disassemble-channel.com), the LoraConfig of the training
  example: lora_dropout = 0.05 on every adapted projection; the same value in
  the PEFT configuration of the Qiita explainer.
* same page, §3 LoRA: h = W0·x + (α/r)·B·A·x, the adapter being the only
  trainable path (so dropout, a training-time regulariser of the adapter, acts
  on the adapter branch only).

Readings taken where the pages leave a step open
------------------------------------------------
* The pages give only the rate.  Dropout is taken as inverted dropout on the
  adapter's input: x̃ = mask ⊙ x / (1 − p), mask ~ Bernoulli(1 − p) per element
  of X [tokens][k_in]; the frozen path sees x unchanged:
      Y  = X·Ŵᵀ + s·(X̃·Aᵀ)·Bᵀ
      dX = dY·Ŵ + s·mask ⊙ ((dY·B)·A) / (1 − p)
      dA = s·(dY·B)ᵀ·X̃,   dB = s·dYᵀ·(X̃·Aᵀ)
  Equivalently, with Xd = mask ⊙ X (exact in bf16) and s' = s / (1 − p):
  U = Xd·Aᵀ is what the forward saves, Y = X·Ŵᵀ + s'·U·Bᵀ, dA = s'·Vᵀ·Xd,
  dB = s'·dYᵀ·U, dX = dY·Ŵ + s'·mask ⊙ (V·A), V = dY·B.
* The mask is a pure function of (seed, offset, element index), so the
  backward regenerates it instead of storing it.  Generator: Philox4x64-10
  (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
  SC 2011) with key (seed, 0) and counter (f >> 3, offset, 0, 0) for the
  element at flat index f = token · k_in + k; its four 64-bit outputs are
  eight 32-bit values, the element taking value (f & 7) — word (f & 7) >> 1,
  the low half for even f.  The element is dropped when that value is below
  T = floor(p · 2^32) (p as the float32 the entry point receives), so the
  drop probability is T / 2^32.

Parity: pinned (tests/test_oracle_dropout.py): the generator against numpy's
Philox bit generator (a library implementation of Philox4x64-10, whose first
block is that of counter + 1), the vectorised 64-bit multiply against exact
integer products, the drop rate and its uniformity over the eight positions
within 5 sigma, p = 0 reducing to the plain linear (pinned on its own), and
finite differences of <dY, Y> for dX, dA, dB with the mask held fixed.
"""

import numpy as np

from .linear import linear_bwd, linear_fwd

PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B
_MASK64 = (1 << 64) - 1


def philox4x64_10(counter, key):
    """One Philox4x64-10 block (Python integers): four 64-bit words."""
    c0, c1, c2, c3 = counter
    k0, k1 = key
    for _ in range(10):
        p0 = PHILOX_M0 * c0
        p1 = PHILOX_M1 * c2
        c0, c1, c2, c3 = ((p1 >> 64) ^ c1 ^ k0, p1 & _MASK64, (p0 >> 64) ^ c3 ^ k1, p0 & _MASK64)
        k0 = (k0 + PHILOX_W0) & _MASK64
        k1 = (k1 + PHILOX_W1) & _MASK64
    return c0, c1, c2, c3


def mulhilo64(a, b):
    """(high, low) 64-bit halves of the 128-bit products of uint64 arrays,
    from 32-bit pieces (numpy has no 128-bit integers)."""
    a = np.asarray(a, dtype=np.uint64)
    b = np.asarray(b, dtype=np.uint64)
    m32 = np.uint64(0xFFFFFFFF)
    s32 = np.uint64(32)
    ah, al = a >> s32, a & m32
    bh, bl = b >> s32, b & m32
    t = al * bl
    m1 = ah * bl
    m2 = al * bh
    mid = (t >> s32) + (m1 & m32) + (m2 & m32)
    hi = ah * bh + (m1 >> s32) + (m2 >> s32) + (mid >> s32)
    lo = (mid << s32) | (t & m32)
    return hi, lo


def philox4x64_10_np(c0, c1, k0, k1):
    """Philox4x64-10 for arrays of counters (c0, c1, 0, 0) under one key;
    returns the four output words as uint64 arrays."""
    c0 = np.asarray(c0, dtype=np.uint64)
    c1 = np.broadcast_to(np.asarray(c1, dtype=np.uint64), c0.shape).copy()
    c2 = np.zeros_like(c0)
    c3 = np.zeros_like(c0)
    k0, k1 = np.uint64(k0), np.uint64(k1)
    M0, M1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
    W0, W1 = np.uint64(PHILOX_W0), np.uint64(PHILOX_W1)
    with np.errstate(over="ignore"):
        for _ in range(10):
            h0, l0 = mulhilo64(M0, c0)
            h1, l1 = mulhilo64(M1, c2)
            c0, c1, c2, c3 = h1 ^ c1 ^ k0, l1, h0 ^ c3 ^ k1, l0
            k0 = k0 + W0
            k1 = k1 + W1
    return c0, c1, c2, c3


def drop_threshold(p):
    """T = floor(p · 2^32) for the float32 rate p in [0, 1)."""
    p = float(np.float32(p))
    assert 0.0 <= p < 1.0
    return int(np.floor(p * 2.0 ** 32))


def element_values(n, seed, offset):
    """The 32-bit value each flat element f < n draws (uint64 array)."""
    f = np.arange(n, dtype=np.uint64)
    groups = np.arange(-(-n // 8), dtype=np.uint64)
    words = philox4x64_10_np(groups, offset, seed, 0)
    w = np.stack(words, axis=1).ravel()  # word index 4 g + j
    sel = w[((f >> np.uint64(3)) << np.uint64(2)) + ((f & np.uint64(7)) >> np.uint64(1))]
    return np.where((f & np.uint64(1)) == 1, sel >> np.uint64(32), sel & np.uint64(0xFFFFFFFF))


def keep_mask(M, K, p, seed, offset):
    """Boolean keep mask of X [M][K] (True = kept)."""
    T = drop_threshold(p)
    return (element_values(M * K, seed, offset) >= np.uint64(T)).reshape(M, K)


def dropped_input(X, keep):
    """Xd = mask ⊙ X (what the forward writes and the backward's dA reads)."""
    return np.where(keep, X, 0.0)


def scale_with_dropout(s, p):
    """s' = s / (1 − p) in float64."""
    return float(s) / (1.0 - float(np.float32(p)))


def linear_fwd_dropout(X, w, A, B, s, p, keep):
    """(Y, U): Y = X·Ŵᵀ + s'·U·Bᵀ with U = (mask ⊙ X)·Aᵀ; float64."""
    Xd = dropped_input(X, keep)
    U = Xd @ A.T
    Y = X @ w.T + scale_with_dropout(s, p) * (U @ B.T)
    return Y, U


def linear_bwd_dropout(X, dY, w, A, B, s, p, keep):
    """(dX, dA, dB) of the dropout forward, by the chain rule; float64."""
    sp = scale_with_dropout(s, p)
    Xd = dropped_input(X, keep)
    V = dY @ B
    dX = dY @ w + sp * np.where(keep, V @ A, 0.0)
    dA = sp * (V.T @ Xd)
    dB = sp * (dY.T @ (Xd @ A.T))
    return dX, dA, dB


def linear_no_dropout(X, dY, w, A, B, s):
    """The plain layer (p = 0 must reduce to it)."""
    Y, U = linear_fwd(X, w, A, B, s)
    return Y, U, linear_bwd(X, dY, w, A, B, s)
