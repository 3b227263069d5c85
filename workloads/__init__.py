"""Seeded synthetic inputs and workload shapes for the QLoRA NF4 linear.

This module holds no arithmetic of the method: it only draws random numbers
(numpy PCG64, one independent stream per tensor keyed by
SeedSequence([seed, workload, layer, matrix, tensor])) and describes shapes.
Both the CPU oracle and the GPU path receive the very same host arrays.

Weights are float32 N(0, 0.02) in [N_out][K_in] row-major order (the layer
computes Y = X·Wᵀ, tokens are rows).  bf16 tensors are float32 normals times
sigma, rounded to bf16 by torch's CPU conversion.  Shapes written "AxB" in the
workload descriptions are in x out: X is [tokens, A].
"""

from dataclasses import dataclass, field

import numpy as np
import torch

SEED = 0

# tensor ids inside one (workload, layer, matrix) key
T_W, T_OUTLIER_POS, T_OUTLIER_SIGN, T_A, T_B, T_X, T_DY = range(7)


def rng(workload, layer=0, matrix=0, tensor=0, seed=SEED):
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([seed, workload, layer, matrix, tensor]))
    )


def weight_f32(workload, n_out, k_in, layer=0, matrix=0, sigma=0.02, outlier_frac=0.0,
               outlier_sigmas=8.0, seed=SEED):
    """float32 [n_out][k_in] ~ N(0, sigma²); optionally a Bernoulli(outlier_frac)
    set of positions overwritten by ±outlier_sigmas·sigma with a random sign."""
    n = n_out * k_in
    w = rng(workload, layer, matrix, T_W, seed).standard_normal(n, dtype=np.float32)
    w *= np.float32(sigma)
    if outlier_frac > 0.0:
        pos = rng(workload, layer, matrix, T_OUTLIER_POS, seed).random(n, dtype=np.float32) \
            < np.float32(outlier_frac)
        k = int(pos.sum())
        sign = rng(workload, layer, matrix, T_OUTLIER_SIGN, seed).integers(0, 2, k) * 2 - 1
        w[pos] = (sign * (outlier_sigmas * sigma)).astype(np.float32)
    return w.reshape(n_out, k_in)


def bf16_normal(workload, shape, sigma, layer=0, matrix=0, tensor=T_X, seed=SEED):
    """torch.bfloat16 CPU tensor ~ N(0, sigma²) (float32 draw, then RNE to bf16)."""
    n = int(np.prod(shape))
    x = rng(workload, layer, matrix, tensor, seed).standard_normal(n, dtype=np.float32)
    x *= np.float32(sigma)
    return torch.from_numpy(x.reshape(shape)).to(torch.bfloat16)


def bf16_bits(t):
    """uint16 numpy view of a bf16 tensor's bit patterns."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_as_f64(t):
    return t.to(torch.float64).numpy()


@dataclass
class LinearWorkload:
    """One QLoRA linear: W [n_out][k_in], rank r, scale alpha, M tokens."""
    name: str
    workload: int
    M: int
    k_in: int
    n_out: int
    r: int
    alpha: float
    fwd_only: bool = False
    layer: int = 0
    matrix: int = 0

    def inputs(self, M=None, with_dy=True, with_w=True):
        """Seeded inputs: dict(W fp32 numpy, A, B, X, dY bf16 torch CPU)."""
        M = self.M if M is None else M
        key = dict(layer=self.layer, matrix=self.matrix)
        out = dict(
            A=bf16_normal(self.workload, (self.r, self.k_in), 0.01, tensor=T_A, **key),
            B=bf16_normal(self.workload, (self.n_out, self.r), 0.01, tensor=T_B, **key),
            X=bf16_normal(self.workload, (M, self.k_in), 1.0, tensor=T_X, **key),
        )
        if with_w:
            out["W"] = weight_f32(self.workload, self.n_out, self.k_in, **key)
        if with_dy and not self.fwd_only:
            out["dY"] = bf16_normal(self.workload, (M, self.n_out), 1.0, tensor=T_DY, **key)
        return out

    @property
    def flops_fwd(self):
        M, K, N, r = self.M, self.k_in, self.n_out, self.r
        return 2 * M * K * N + 2 * M * K * r + 2 * M * r * N

    @property
    def flops_bwd(self):
        M, K, N, r = self.M, self.k_in, self.n_out, self.r
        # dX main, V = dY·B, s·V·A, dA = s·Vᵀ·X, dB = s·dYᵀ·U
        return 2 * M * N * K + 2 * M * N * r + 2 * M * r * K + 2 * r * M * K + 2 * N * M * r


# Workload 1: single QLoRA linear, W 4096x4096, r = 8, alpha = 16, X [16, 4096], forward only.
SINGLE_LINEAR = LinearWorkload("single_linear_4096x4096_r8_m16", 1, 16, 4096, 4096, 8, 16.0,
                               fwd_only=True)

# Workload 2: LLaMA-7B-shaped weights, 32 layers x (q, k, v, o 4096x4096; gate, up
# 4096x11008; down 11008x4096), fp32 N(0, 0.02) with 0.1% outliers at +-8 sigma.
LLAMA7B_LAYERS = 32
LLAMA7B_MATRICES = [  # (name, n_out, k_in)
    ("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
    ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008),
]


def llama7b_weight(layer, matrix):
    name, n_out, k_in = LLAMA7B_MATRICES[matrix]
    return weight_f32(2, n_out, k_in, layer=layer, matrix=matrix, outlier_frac=1e-3)


# Workload 3: LLaMA-7B MLP linear 4096 -> 11008, r = 64, alpha = 16, 4096 tokens, fwd + bwd.
LLAMA7B_MLP = LinearWorkload("llama7b_mlp_4096x11008_r64_m4096", 3, 4096, 4096, 11008, 64, 16.0)

# Workload 4: few-token GEMV, 8192 -> 28672, r = 16, alpha = 32, 1..8 tokens, forward only.
GEMV_70B = LinearWorkload("gemv_8192x28672_r16", 4, 8, 8192, 28672, 16, 32.0, fwd_only=True)
GEMV_TOKENS = list(range(1, 9))

# Workload 5: one LLaMA-65B-shaped decoder layer, 7 projections, r = 64, alpha = 16,
# 2048 tokens, fwd + bwd.
LLAMA65B_LAYER = [
    LinearWorkload(f"llama65b_{name}_{k}x{n}_r64_m2048", 5, 2048, k, n, 64, 16.0, matrix=i)
    for i, (name, k, n) in enumerate([
        ("q", 8192, 8192), ("k", 8192, 8192), ("v", 8192, 8192), ("o", 8192, 8192),
        ("gate", 8192, 22016), ("up", 8192, 22016), ("down", 22016, 8192),
    ])
]

# Workload 6: the AdamW step over LLaMA-7B's LoRA factors on the four attention
# projections at r = 64: 32 layers x 4 matrices x (A, B) = 256 tensors of
# 64 x 4096, 67,108,864 parameters in all.
ADAMW_TENSORS = 32 * 4 * 2
ADAMW_TENSOR_SIZE = 64 * 4096
