"""QLoRA linear layer, forward and backward, in float64 (oracle).

Sources
-------
* "QLoRAの理論と実装" (disassemble-channel.com), §"LoRAの復習": W' = W0 + B·A with
  B ∈ R^{d×r}, A ∈ R^{r×k}; forward h = W0·x + (α/r)·B·A·x, W0 frozen.
* same page, §"QLoRAの計算フロー / 順伝播の全体像": Y = dequant(W_NF4)·X + (α/r)·B(A·X),
  computing the r×n intermediate A·X first, then summing the main and LoRA
  paths.
* same page, §"逆伝播と勾配の流れ": ∂L/∂B = (α/r)·∂L/∂Y·(A·X)ᵀ and
  ∂L/∂A = (α/r)·Bᵀ·∂L/∂Y·Xᵀ; no gradient for the frozen quantised weight,
  which is a constant of the graph.
* arXiv 2305.14314 summary (papers.plutine.com), "要約"/"手法": gradients are
  back-propagated through the frozen 4-bit model, so the layer also returns the
  input gradient; by the chain rule dX = dY·Ŵ + (α/r)·(dY·B)·A.

Layout: tokens are rows.  X [M][K_in], Ŵ [N_out][K_in], A [r][K_in],
B [N_out][r], Y and dY [M][N_out].  The pages' column-vector forms map to
Y = X·Ŵᵀ + s·(X·Aᵀ)·Bᵀ, dB = s·dYᵀ·(X·Aᵀ), dA = s·(dY·B)ᵀ·X.

Readings: s = α/r is kept in the forward (the compute-flow formula that omits
it is the shorthand of the LoRA forward that keeps it) and is taken as the
float32 quotient RN32(α / r).  All inputs are their exact bf16 values; all
arithmetic is float64 with no intermediate rounding.

Parity: pinned (tests/test_oracle_linear.py) against exact rational brute
force on tiny shapes, central finite differences of L = <dY, Y>, and the
special cases B = 0 (zero-initialised adapter: Y = X·Ŵᵀ, dA = 0), A = 0
(dB = 0), X = I (Y = Ŵᵀ) and dY = I (dX = Ŵ).
"""

import numpy as np


def lora_scale(alpha, r):
    """s = RN32(α / r), returned as a Python float (exact float32 value)."""
    return float(np.float32(alpha) / np.float32(r))


def linear_fwd(X, W_hat, A, B, s):
    """Returns (Y, U) with U = X·Aᵀ (the r-wide intermediate, saved for the
    backward) and Y = X·Ŵᵀ + s·U·Bᵀ, both float64."""
    X = np.asarray(X, dtype=np.float64)
    W_hat = np.asarray(W_hat, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    U = X @ A.T
    Y_main = X @ W_hat.T
    Y_lora = s * (U @ B.T)
    return Y_main + Y_lora, U


def linear_bwd(X, dY, W_hat, A, B, s):
    """Returns (dX, dA, dB), float64."""
    X = np.asarray(X, dtype=np.float64)
    dY = np.asarray(dY, dtype=np.float64)
    W_hat = np.asarray(W_hat, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    V = dY @ B                      # [M][r]  = (Bᵀ·∂L/∂Y) in token-row layout
    dX = dY @ W_hat + s * (V @ A)   # through the frozen weight and the adapter
    dA = s * (V.T @ X)              # (α/r)·Bᵀ·∂L/∂Y·Xᵀ
    dB = s * (dY.T @ (X @ A.T))     # (α/r)·∂L/∂Y·(A·X)ᵀ
    return dX, dA, dB
