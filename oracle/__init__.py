"""CPU oracle for the QLoRA NF4 linear hot path — TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, deliberately unoptimised CPU statement of what
the hot path computes, written from the QLoRA pages:

* "QLoRAの理論と実装 — 4bit量子化＋LoRAで大規模LLMを効率的にファインチューニング"
  (disassemble-channel.com): LoRA forward, NF4 construction and the
  quantise / dequantise process, Double Quantization, the compute flow and the
  LoRA gradients, and the educational NF4 code.
* The Qiita explainer on why QLoRA does not break at 4 bits
  (qiita.com/TaiyoYamada): the Double Quantization dequant order
  W ≈ (c2 · c1^quant) · W^quant, and the storage/compute split (decode to BF16
  right before the matmul).
* The arXiv 2305.14314 summary (papers.plutine.com): gradients are
  back-propagated through the frozen 4-bit model into the adapters.

It shares no code, table or constant with the HIP library: it derives its own
codebook, does every decision in exact float64 arithmetic and uses numpy /
torch-CPU library primitives (matmul, float->bfloat16 rounding) as single
steps.  Only the test-suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path never
does.

Parity status of every function is stated in its module header.
"""

from .codebook import nf4_codebook_f64, nf4_codebook_f32, nf4_midpoints_f64
from .quant import (
    block_absmax,
    nf4_indices,
    pack_nibbles,
    unpack_nibbles,
    quantize_nf4,
    double_quant,
    dequant_absmax,
    dequantize_nf4,
    bf16_round,
)
from .linear import lora_scale, linear_fwd, linear_bwd

__all__ = [
    "nf4_codebook_f64",
    "nf4_codebook_f32",
    "nf4_midpoints_f64",
    "block_absmax",
    "nf4_indices",
    "pack_nibbles",
    "unpack_nibbles",
    "quantize_nf4",
    "double_quant",
    "dequant_absmax",
    "dequantize_nf4",
    "bf16_round",
    "lora_scale",
    "linear_fwd",
    "linear_bwd",
]
