"""32-bit AdamW step on the LoRA factors, with global gradient-norm clipping
(oracle) — TEST INFRASTRUCTURE ONLY.

Sources
-------
* "QLoRAの理論と実装" (disassemble-channel.com), §5-3 Paged Optimizers: the
  optimizer states are Adam's first and second moments, held on the GPU (and
  paged to host memory under memory pressure); only the LoRA parameters carry
  Adam states, 12 bytes per parameter in FP32 ("Adamオプティマイザ状態のメモリ":
  67M parameters -> about 804 MB).
* same page, the TrainingArguments of the training example: optim =
  "paged_adamw_32bit", learning_rate = 2e-4, weight_decay = 0.001,
  max_grad_norm = 0.3.

Readings taken where the pages leave a step open
------------------------------------------------
* The pages name AdamW but do not print its update.  It is taken from its
  published definition (Loshchilov & Hutter, "Decoupled Weight Decay
  Regularization", Algorithm 2, with the learning rate as the schedule
  multiplier), in the order the PyTorch implementation uses:
      p <- p * (1 - lr * wd)                       (decoupled decay)
      m <- beta1 * m + (1 - beta1) * g
      v <- beta2 * v + (1 - beta2) * g^2
      p <- p - lr * (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
  with t the 1-based step count.  beta1 = 0.9, beta2 = 0.999 and eps = 1e-8
  (not on the pages) are that implementation's defaults.
* "32-bit": the parameter the optimizer updates is an FP32 master copy, and the
  moments are FP32 — 12 bytes per parameter, the page's figure.  The BF16
  factors the layer computes with are RNE_bf16 of the master after the step.
* max_grad_norm clips by the global L2 norm over all trainable gradients:
  g <- g * min(1, max_norm / (norm + 1e-6)) (the referenced trainer's rule).
* Paging itself (moving the states between host and device memory) changes
  where the states live, not what the step computes; it is not part of this
  arithmetic.

Everything here is float64 with no intermediate rounding.

Parity: pinned (tests/test_oracle_optim.py) against torch.optim.AdamW and
torch.nn.utils.clip_grad_norm_ run on the CPU in float64 (library routines),
and against closed forms: the first step from zero moments moves each weight by
lr * g / (|g| + eps); a constant gradient keeps doing so at every step (the bias
corrections cancel exactly); a zero gradient only decays p by (1 - lr * wd)
per step; without eps the update is invariant to the gradient's scale.
"""

import numpy as np

BETA1 = 0.9
BETA2 = 0.999
EPS = 1e-8
CLIP_EPS = 1e-6


def global_grad_norm(grads):
    """L2 norm over every element of every gradient."""
    return float(np.sqrt(sum(float(np.sum(np.asarray(g, dtype=np.float64) ** 2)) for g in grads)))


def clip_coefficient(norm, max_norm):
    """The factor every gradient is multiplied by before the step (1 without clipping)."""
    if max_norm is None or max_norm <= 0:
        return 1.0
    return min(1.0, max_norm / (norm + CLIP_EPS))


def adamw_step(p, g, m, v, step, lr, beta1=BETA1, beta2=BETA2, eps=EPS, weight_decay=0.0,
               coef=1.0):
    """One AdamW update of one tensor; returns new (p, m, v) as float64 arrays."""
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64) * coef
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    p = p * (1.0 - lr * weight_decay)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v


def adamw_multi(params, grads, ms, vs, step, lr, beta1=BETA1, beta2=BETA2, eps=EPS,
                weight_decay=0.0, max_grad_norm=0.0):
    """The step over a list of tensors sharing one clipping coefficient.
    Returns (new params, new ms, new vs, norm before clipping)."""
    norm = global_grad_norm(grads)
    coef = clip_coefficient(norm, max_grad_norm)
    out = [adamw_step(p, g, m, v, step, lr, beta1, beta2, eps, weight_decay, coef)
           for p, g, m, v in zip(params, grads, ms, vs)]
    return [o[0] for o in out], [o[1] for o in out], [o[2] for o in out], norm
