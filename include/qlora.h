/*
 * qlora.h — C ABI of the MI355X (gfx950) QLoRA NF4 linear library (libqlora.so).
 *
 * What the library computes, and where it is defined:
 *   * NF4 blockwise quantisation of a float32 weight: blocks of 64 consecutive
 *     elements scaled by their absolute maximum, each element replaced by the
 *     index of the nearest of 16 NormalFloat levels ("QLoRAの理論と実装",
 *     disassemble-channel.com, §5-1 NF4: construction, and the three-step
 *     quantise / dequantise process).
 *   * Double Quantization of the per-block float32 absmax values: 8-bit codes in
 *     groups of 256 blocks with one float32 second-level constant per group
 *     (same page, §5-2 Double Quantization), dequantised in the order
 *     W ≈ (c2 · c1^quant) · W^quant (Qiita explainer, "Double Quantization の仕組み").
 *   * The QLoRA linear: Y = dequant(W_NF4)·X + (α/r)·B·(A·X), the 4-bit weight
 *     decoded to BF16 right before the matmul (same page, "QLoRAの計算フロー";
 *     Qiita explainer, storage/compute split), and its backward: gradients for
 *     A and B only ("逆伝播と勾配の流れ") plus the input gradient through the
 *     frozen weight (arXiv 2305.14314 summary, papers.plutine.com).
 *
 * Conventions (every entry point):
 *   * Pointers are DEVICE pointers unless marked (host).  Every device pointer
 *     must be 16-byte aligned (unless its entry point states otherwise).  The caller owns every buffer; the library never
 *     allocates, frees or keeps a pointer past the call.
 *   * `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously on it; no call synchronises, except
 *     qlora_adamw_plan_init (a one-time copy of its list from host memory).
 *   * Arguments are validated on the host before anything is enqueued.  On any
 *     error status nothing is launched and no output is touched.  A failed
 *     launch returns QLORA_ERR_LAUNCH.  Faults during execution surface at the
 *     caller's next synchronisation of the stream.
 *   * Inputs must be finite; non-finite input gives unspecified output.
 *   * bf16 tensors are passed as raw 16-bit patterns (qlora_bf16).
 *   * Weight layout: W is [n_out][k_in] row-major (the layer computes
 *     Y = X·Wᵀ with tokens as rows); quantisation blocks run along k_in.
 *   * Calls are reentrant; concurrent calls on different streams are safe.
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QLORA_ABI_VERSION 3
#define QLORA_BLOCKSIZE 64   /* first-level block (NF4), elements */
#define QLORA_DQ_GROUP 256   /* second-level group, blocks */
#define QLORA_MAX_RANK 256

typedef uint16_t qlora_bf16; /* raw bfloat16 bits */

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_NULL = 1,        /* a required pointer is NULL */
  QLORA_ERR_SHAPE = 2,       /* a size is negative, out of range or not a required multiple */
  QLORA_ERR_ALIGN = 3,       /* a device pointer is not 16-byte aligned */
  QLORA_ERR_UNSUPPORTED = 4, /* a parameter outside what is supported: blocksize != 64,
                                group != 256, r outside [1, 256], an unknown 4-bit code,
                                an optimizer or dropout setting out of range, or host
                                states that are not page-locked */
  QLORA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than qlora_workspace_size() */
  QLORA_ERR_DEVICE = 6,      /* no device, or the current device is not gfx950 */
  QLORA_ERR_LAUNCH = 7       /* a kernel launch failed */
} qlora_status;

/* Non-owning view of one frozen NF4 + Double-Quantized weight W[n_out][k_in].
 *   packed  : n_out*k_in/2 bytes; byte t = idx[2t] | idx[2t+1] << 4 (flat order)
 *   qabsmax : n_out*k_in/64 second-level codes, values in [0, 127]
 *   c2      : ceil(n_out*k_in/64/256) float32 second-level constants
 *   k_in % 64 == 0 for the linear entry points (any n_out >= 1). */
typedef struct {
  const uint8_t *packed;
  const int8_t *qabsmax;
  const float *c2;
  int64_t n_out;
  int64_t k_in;
} qlora_nf4_weight;

/* ---- quantisation ------------------------------------------------------- */

/* First level ("QLoRAの理論と実装", §5-1, steps 1 and 2).  For each block of 64
 * consecutive elements of the flat w[0..n) (the tail zero-padded):
 *   absmax[b] = max |w| over the block (exact);
 *   idx       = nearest NF4 level to the exact quotient w / absmax[b], a tie
 *               going to the lower index; an all-zero block and every padded
 *               slot get index 8 (the exact-zero level).
 * Outputs: packed[ceil(n/64)*32] bytes (two indices per byte, even element in
 * the low nibble) and absmax[ceil(n/64)] float32.  n >= 0; blocksize must be 64.
 * Block maxima anywhere in the finite float32 range (subnormal up to FLT_MAX)
 * get the exact decision.
 * nonfinite_flag (optional device int32, 4-byte aligned; NULL = not wanted):
 * set to 1 when any w[i] is NaN or ±Inf, left untouched otherwise — the caller
 * zeroes it beforehand.  Non-finite input breaks the finite-input
 * precondition: its codes and scales are unspecified, the flag is the only
 * defined result. */
qlora_status qlora_quantize_nf4(const float *w, int64_t n, int32_t blocksize, uint8_t *packed,
                                float *absmax, int32_t *nonfinite_flag, void *stream);

/* Second level ("QLoRAの理論と実装", §5-2; Qiita explainer, DQ formula).  Groups of
 * 256 consecutive blocks (the last may be short):
 *   c2[g]    = RN32(max absmax over the group / 127)   (IEEE float32 division)
 *   qabsmax  = integer in [0, 127] nearest to absmax / c2 (exact, tie to the
 *              lower integer); 0 when c2 == 0.
 * Inputs absmax[nblocks] (non-negative); outputs qabsmax[nblocks],
 * c2[ceil(nblocks/256)].  group must be 256. */
qlora_status qlora_double_quant(const float *absmax, int64_t nblocks, int32_t group,
                                int8_t *qabsmax, float *c2, void *stream);

/* Both levels.  Produces exactly the bytes that qlora_quantize_nf4 followed by
 * qlora_double_quant produce.  absmax (float32 [ceil(n/64)], optional)
 * receives the first-level scales; given it, the two levels run as those two
 * launches (the faster route), without it as one pass over w.
 * nonfinite_flag: optional, as for qlora_quantize_nf4. */
qlora_status qlora_quantize_nf4_dq(const float *w, int64_t n, uint8_t *packed, int8_t *qabsmax,
                                   float *c2, float *absmax, int32_t *nonfinite_flag,
                                   void *stream);

/* Dequantisation ("QLoRAの理論と実装", §5-1 step 3, in the DQ order):
 *   â = RN32(c2[b/256] · qabsmax[b]);  out = RNE_bf16(RN32(c[idx] · â)).
 * out[n_out*k_in] bf16, row-major.  Any n_out, k_in >= 0 with n_out*k_in % 64 == 0. */
qlora_status qlora_dequantize_nf4(const qlora_nf4_weight *w /* host struct */, qlora_bf16 *out,
                                  void *stream);

/* Lists of weights, for quantising or decoding a whole model's weight set
 * (the LLaMA-7B set of "QLoRAの理論と実装" §5-2 is 224 matrices) without a
 * launch per matrix, whose fixed cost dominates for 4096x4096 weights.
 *
 * qlora_quantize_nf4_dq_batch: for each job, exactly the bytes of
 *   qlora_quantize_nf4_dq(w, n, packed, qabsmax, c2, absmax, stream); absmax
 *   is required here (it carries the first-level scales between the two
 *   levels).  Two launches per up to 48 jobs.
 * qlora_dequantize_nf4_batch: for each i, exactly qlora_dequantize_nf4(
 *   &weights[i], outs[i], stream).  One launch per up to 48 weights.
 * jobs, weights and outs are HOST arrays of count entries (count >= 0, else
 * QLORA_ERR_SHAPE; NULL with count > 0: QLORA_ERR_NULL); the buffers they
 * name are device memory with the shapes, alignment and error behaviour of
 * the single-matrix calls.  Every entry is validated before anything is
 * enqueued; entries with n = 0 are skipped.  The outputs of different jobs
 * must not overlap. */
typedef struct {
  const float *w;     /* n float32 weights                          */
  int64_t n;
  uint8_t *packed;    /* ceil(n/64)*32 bytes                        */
  int8_t *qabsmax;    /* ceil(n/64) DQ codes                        */
  float *c2;          /* ceil(n/16384) second-level steps           */
  float *absmax;      /* ceil(n/64) first-level scales (written)    */
  int32_t *nonfinite_flag; /* optional (NULL): set to 1 on NaN / Inf  */
} qlora_quant_job;
qlora_status qlora_quantize_nf4_dq_batch(const qlora_quant_job *jobs /* host */, int32_t count,
                                         void *stream);
qlora_status qlora_dequantize_nf4_batch(const qlora_nf4_weight *weights /* host */,
                                        qlora_bf16 *const *outs /* host array of device pointers */,
                                        int32_t count, void *stream);

/* ---- LoRA dropout -------------------------------------------------------- */

/* The training example's lora_dropout ("QLoRAの理論と実装", LoraConfig: 0.05)
 * as inverted dropout on the adapter's input: the adapter sees
 * X̃ = mask ⊙ X / (1 − p), the frozen path sees X.  The mask is a pure
 * function of (seed, offset, element): element f = token·k_in + k draws the
 * 32-bit value f & 7 of Philox4x64-10 block f >> 3 (key (seed, 0), counter
 * (f >> 3, offset, 0, 0); word (f & 7) >> 1, low half for even f) and is
 * dropped when that value is below floor(p · 2^32).  p must lie in [0, 1)
 * (else QLORA_ERR_UNSUPPORTED).  With s' = RN32(α/r) / (1 − p):
 *
 * qlora_lora_dropout:        Xd = mask ⊙ X (bf16, bit copies and +0), X and Xd
 *                            [M][k_in], k_in % 8 == 0.
 * qlora_linear_fwd_dropout:  Xd as above, U = Xd·Aᵀ (saved), Y = RNE_bf16(X·Ŵᵀ +
 *                            s'·U·Bᵀ).  Workspace: qlora_workspace_size(0, ...).
 * qlora_linear_bwd_dropout:  V = dY·B;  dX = RNE_bf16(dY·Ŵ + s'·mask ⊙ (V·A));
 *                            dA = s'·Vᵀ·Xd;  dB = s'·dYᵀ·U, with the same
 *                            (p, seed, offset) as the forward (the mask is
 *                            regenerated, not stored).  Workspace:
 *                            qlora_workspace_size(2, ...).
 * Shapes, dtypes and layouts otherwise as qlora_linear_fwd / qlora_linear_bwd. */
qlora_status qlora_lora_dropout(const qlora_bf16 *X, int64_t M, int64_t k_in, float p,
                                uint64_t seed, uint64_t offset, qlora_bf16 *Xd, void *stream);
qlora_status qlora_linear_fwd_dropout(const qlora_nf4_weight *w /* host struct */,
                                      const qlora_bf16 *X, int64_t M, const qlora_bf16 *A,
                                      const qlora_bf16 *B, int32_t r, float alpha, float p,
                                      uint64_t seed, uint64_t offset, qlora_bf16 *Y,
                                      qlora_bf16 *U, qlora_bf16 *Xd, void *workspace,
                                      size_t ws_bytes, void *stream);
qlora_status qlora_linear_bwd_dropout(const qlora_nf4_weight *w /* host struct */,
                                      const qlora_bf16 *Xd, const qlora_bf16 *dY, int64_t M,
                                      const qlora_bf16 *A, const qlora_bf16 *B, int32_t r,
                                      float alpha, float p, uint64_t seed, uint64_t offset,
                                      const qlora_bf16 *U, qlora_bf16 *dX, float *dA, float *dB,
                                      void *workspace, size_t ws_bytes, void *stream);

/* ---- adapter merge ------------------------------------------------------- */

/* Merge a trained adapter into the base weight and (optionally) re-quantise
 * it ("QLoRAとは？4bit量子化＋LoRAの仕組み・VRAM目安・実装手順と採用判断を解説",
 * issoh.co.jp, section on merging and distributing the adapter: merge into the
 * 16-bit base, keep the merged 16-bit model, quantise it again for 4-bit
 * inference; merging into the 4-bit base re-rounds the sum onto the 4-bit
 * grid).  Exactly one base: w16 (bf16 [n_out][k_in], the recommended path) or
 * w4 (the NF4 + DQ weight, decoded as qlora_dequantize_nf4 does; the path the
 * page warns about).  With s = RN32(alpha / r), for every element the page's
 * W + s·B·A in float64, rounded once to bf16:
 *   acc = Σ_j B[n][j]·A[j][k]   float64 (exact products; exact sums at the
 *                               magnitudes of weights and adapters)
 *   merged[n][k] = RNE_bf16(RN64(base + RN64(s·acc)))
 * A [r][k_in], B [n_out][r] bf16; merged bf16 [n_out][k_in] (required).  When
 * packed is not NULL, merged is then quantised exactly as
 * qlora_quantize_nf4_dq would quantise its float32 values: packed
 * [n_out*k_in/2], qabsmax [n_out*k_in/64], c2 [ceil(n_out*k_in/16384)].
 * k_in % 64 == 0, ceil(n_out/16) <= 65535, 1 <= r <= 256.  Both bases NULL:
 * QLORA_ERR_NULL; both given: QLORA_ERR_UNSUPPORTED. */
qlora_status qlora_merge_adapter(const qlora_bf16 *w16, const qlora_nf4_weight *w4 /* host struct */,
                                 int64_t n_out, int64_t k_in, const qlora_bf16 *A,
                                 const qlora_bf16 *B, int32_t r, float alpha, qlora_bf16 *merged,
                                 uint8_t *packed, int8_t *qabsmax, float *c2, void *stream);

/* ---- quantiser variants -------------------------------------------------- */

#define QLORA_CODE_NF4 0   /* the 16 NormalFloat levels */
#define QLORA_CODE_INT4 1  /* 16 uniform levels (2k − 15)/15, k = 0..15, each RN32 */

/* First level with either code, one float32 absmax per block kept as is:
 * single quantisation, 4 + 32/64 = 4.5 bits per weight ("QLoRAの理論と実装",
 * §5-2 "メモリ削減の計算"; the uniform INT4 code is the page's comparison
 * quantiser, "NF4による量子化と量子化誤差の比較", levels linspace(−1, 1, 16)).
 * Blocks, absmax, exact nearest-level decision and packing as for
 * qlora_quantize_nf4 (QLORA_CODE_NF4 gives the same bytes).  INT4 has no zero
 * level: a zero weight ties between ∓1/15 and takes the lower index, 7, which
 * is also the index of an all-zero block and of padded slots.
 * Outputs packed[ceil(n/64)*32], absmax[ceil(n/64)].  n >= 0. */
qlora_status qlora_quantize_4bit(const float *w, int64_t n, int32_t code, uint8_t *packed,
                                 float *absmax, void *stream);

/* Single-quantisation decode: out[i] = RNE_bf16(RN32(level[idx_i] · absmax[i/64]))
 * for i < n (any n >= 0), levels of `code`.  packed and absmax as written by
 * qlora_quantize_4bit for the same n. */
qlora_status qlora_dequantize_4bit(const uint8_t *packed, const float *absmax, int64_t n,
                                   int32_t code, qlora_bf16 *out, void *stream);

/* Quantisation error of a single-quantised weight (the page's NF4-vs-INT4
 * comparison measures its mean, "NF4による量子化と量子化誤差の比較"):
 *   *sse = Σ_{i<n} (w[i] − RN32(level[idx_i] · absmax[i/64]))²
 * each term formed in float64, summed in float64 in a fixed order (repeated
 * calls give the same bits).  sse is one device double (8-byte aligned); n = 0
 * writes 0.  workspace: at least qlora_quant_error_workspace_size(n) bytes. */
qlora_status qlora_quant_sq_error(const float *w, int64_t n, int32_t code, const uint8_t *packed,
                                  const float *absmax, double *sse, void *workspace,
                                  size_t ws_bytes, void *stream);

/* Bytes of workspace qlora_quant_sq_error needs for n weights (0 if n < 0). */
size_t qlora_quant_error_workspace_size(int64_t n);

/* ---- QLoRA linear ------------------------------------------------------- */

/* Forward ("QLoRAの理論と実装", QLoRAの計算フロー, steps 1-4), s = RN32(alpha / r):
 *   U = X·Aᵀ                       (bf16, [M][r], saved for the backward)
 *   Y = RNE_bf16(X·Ŵᵀ + s·U·Bᵀ)    (fp32 accumulation; Ŵ decoded tile by tile,
 *                                   never materialised)
 * X [M][k_in], A [r][k_in], B [n_out][r], Y [M][n_out] bf16.  M >= 0.
 * Every path decodes Ŵ as qlora_dequantize_nf4 does and accumulates in fp32;
 * paths differ only in the order of the fp32 sums, except that for at most
 * 16 tokens on weights too wide for the one-launch kernel (more than 16
 * output columns per compute unit, r > 16 or k_in > 4096) each 64-block's
 * scale multiplies that block's fp32 partial sum of the bf16-rounded levels
 * (a rounding difference of about 5e-4 relative).  Each path repeats its own
 * bits exactly.
 * workspace: at least qlora_workspace_size(0, M, n_out, k_in, r) bytes. */
qlora_status qlora_linear_fwd(const qlora_nf4_weight *w /* host struct */, const qlora_bf16 *X,
                              int64_t M, const qlora_bf16 *A, const qlora_bf16 *B, int32_t r,
                              float alpha, qlora_bf16 *Y, qlora_bf16 *U, void *workspace,
                              size_t ws_bytes, void *stream);

/* Backward ("QLoRAの理論と実装", 逆伝播と勾配の流れ; arXiv 2305.14314 summary):
 *   V  = dY·B
 *   dX = RNE_bf16(dY·Ŵ + s·V·A)   bf16 [M][k_in]
 *   dA = s·Vᵀ·X                    fp32 [r][k_in]
 *   dB = s·dYᵀ·U                   fp32 [n_out][r]   (U as saved by the forward)
 * No gradient for the frozen weight.  workspace: at least
 * qlora_workspace_size(1, M, n_out, k_in, r) bytes. */
qlora_status qlora_linear_bwd(const qlora_nf4_weight *w /* host struct */, const qlora_bf16 *X,
                              const qlora_bf16 *dY, int64_t M, const qlora_bf16 *A,
                              const qlora_bf16 *B, int32_t r, float alpha, const qlora_bf16 *U,
                              qlora_bf16 *dX, float *dA, float *dB, void *workspace,
                              size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory or hand over a workspace:
 * code under HIP graph capture that must not allocate, tight serving loops,
 * harnesses that forbid hipMalloc.  Exactly qlora_linear_fwd (same kernels,
 * same results bit for bit), its workspace taken from a buffer of
 * QLORA_NOALLOC_SCRATCH_BYTES that the library keeps in each GPU's memory
 * until the process ends; nothing is allocated or freed by the call.  Returns
 * QLORA_ERR_WORKSPACE, with nothing launched, when
 * qlora_workspace_size(0, M, n_out, k_in, r) exceeds that size (4096 tokens
 * of a LLaMA-7B MLP or 2048 of a LLaMA-65B projection need 8.4 MB, 16 tokens
 * or fewer at most a few MB; 17..127 tokens with n_out above ~130,000 do not
 * fit).  Every call on one GPU shares that GPU's buffer:
 * calls that can overlap on one GPU (several streams, or threads without an
 * order between them) race and must be serialised by the caller.  Nothing in
 * the buffer has to start at zero; it keeps the last call's contents. */
#define QLORA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
qlora_status qlora_linear_fwd_noalloc(const qlora_nf4_weight *w /* host struct */,
                                      const qlora_bf16 *X, int64_t M, const qlora_bf16 *A,
                                      const qlora_bf16 *B, int32_t r, float alpha, qlora_bf16 *Y,
                                      qlora_bf16 *U, void *stream);

/* The forward's two parts, callable on their own:
 *   qlora_lora_down:      U = X·Aᵀ, bf16 [M][r]
 *   qlora_nf4_matmul_fwd: Y = RNE_bf16(X·Ŵᵀ + s·U·Bᵀ), U given
 * qlora_linear_fwd is exactly these two calls, except on the weights its
 * one-launch kernel takes (at most 16 tokens, r <= 16, k_in <= 4096, at most
 * 16 output columns per compute unit), where it forms U and Y in one launch:
 * there the two routes differ in the order of their fp32 sums, and the
 * second uses the few-token path's per-block scaling described above.
 * Same shapes, preconditions and workspace as qlora_linear_fwd. */
qlora_status qlora_lora_down(const qlora_bf16 *X, int64_t M, int64_t k_in, const qlora_bf16 *A,
                             int32_t r, qlora_bf16 *U, void *workspace, size_t ws_bytes,
                             void *stream);
qlora_status qlora_nf4_matmul_fwd(const qlora_nf4_weight *w /* host struct */,
                                  const qlora_bf16 *X, int64_t M, const qlora_bf16 *U,
                                  const qlora_bf16 *B, int32_t r, float alpha, qlora_bf16 *Y,
                                  void *workspace, size_t ws_bytes, void *stream);

/* ---- optimizer step on the adapter factors ------------------------------ */

/* One trainable tensor of the AdamW step.  param, m and v are float32 and
 * updated in place; grad is read; param_bf16 (optional, may be NULL) receives
 * RNE_bf16 of the updated param — the bf16 factor the linear computes with. */
typedef struct {
  float *param;
  const float *grad;
  float *m;
  float *v;
  qlora_bf16 *param_bf16;
  int64_t n;
} qlora_adamw_tensor;

/* 32-bit AdamW over a list of tensors ("QLoRAの理論と実装", §5-3 Paged
 * Optimizers: Adam's first and second moments in FP32, with the FP32 master
 * weight 12 bytes per trainable parameter; the training example's
 * paged_adamw_32bit with max_grad_norm).  AdamW as published (decoupled decay),
 * t = step >= 1:
 *   coef = min(1, max_grad_norm / (||g||_2 + 1e-6)), the norm over every element
 *          of every tensor in the list (coef = 1 when max_grad_norm <= 0)
 *   p <- p·(1 − lr·weight_decay);  m <- β1·m + (1−β1)·coef·g;
 *   v <- β2·v + (1−β2)·(coef·g)²;  p <- p − lr/(1−β1^t) · m / (sqrt(v)/sqrt(1−β2^t) + eps)
 * Arithmetic in float32 (the bias corrections in float64 on the host); the
 * norm is a fixed-order float64 reduction, so repeated steps are bitwise
 * equal.  grad_norm (optional device float) receives the norm before
 * clipping.  workspace (at least qlora_adamw_workspace_size(count) bytes) is
 * needed when max_grad_norm > 0 or grad_norm != NULL, else may be NULL.
 * tensors is a host array; tensors with n == 0 may have NULL pointers.
 * Requires 0 <= β1, β2 < 1, eps > 0, lr >= 0, weight_decay >= 0. */
qlora_status qlora_adamw_step(const qlora_adamw_tensor *tensors /* host array */, int32_t count,
                              float lr, float beta1, float beta2, float eps, float weight_decay,
                              int64_t step, float max_grad_norm, float *grad_norm,
                              void *workspace, size_t ws_bytes, void *stream);

/* Bytes of workspace qlora_adamw_step needs for `count` tensors (0 if count < 0). */
size_t qlora_adamw_workspace_size(int32_t count);

/* Paged optimizer states ("QLoRAの理論と実装", §5-3 Paged Optimizers: the
 * optimizer states leave GPU memory when it runs short and come back to the
 * GPU when the update needs them).  Exactly qlora_adamw_step (same bits),
 * except that every tensor's m and v are HOST pointers into page-locked
 * memory (hipHostMalloc, or a tensor made with pin_memory; else
 * QLORA_ERR_UNSUPPORTED) that the caller owns and that stays the states'
 * home: the update kernel reads and writes them there, across the host
 * link, at the device addresses of their mappings, on `stream` (the host
 * must not touch m and v until the stream has passed the call).  The
 * device holds only p and g: 8 bytes per parameter less than the resident
 * step.  Reads and writes cross the link at the same time, so this moves
 * the states faster than paging them in and out with copies on one stream.
 * Workspace as for qlora_adamw_step. */
qlora_status qlora_adamw_step_paged(const qlora_adamw_tensor *tensors /* host array; m, v host */,
                                    int32_t count, float lr, float beta1, float beta2, float eps,
                                    float weight_decay, int64_t step, float max_grad_norm,
                                    float *grad_norm, void *workspace, size_t ws_bytes,
                                    void *stream);

/* A prepared tensor list for a training loop that steps the same tensors
 * every iteration: the descriptors and a chunk -> tensor map copied once into
 * a caller-owned device buffer, so that a step is one norm pass, one clip and
 * one update launch over all tensors whatever their number (qlora_adamw_step
 * takes 48 tensors per launch), with nothing marshalled per tensor. */
typedef struct {
  void *device;   /* the prepared list (caller-owned device memory) */
  int32_t count;  /* tensors */
  int64_t chunks; /* 2048-element chunks over all tensors */
} qlora_adamw_plan;

/* Device bytes of the prepared list of these tensors (0 if invalid). */
size_t qlora_adamw_plan_size(const qlora_adamw_tensor *tensors /* host array */, int32_t count);

/* Validates the tensors as qlora_adamw_step does and writes the prepared list
 * into `device` (at least qlora_adamw_plan_size bytes, else
 * QLORA_ERR_WORKSPACE); fills *plan (host).  Copies from host memory and
 * synchronises `stream` before returning: call it once, outside graph
 * capture.  The tensors' memory must stay where it is while the plan is used. */
qlora_status qlora_adamw_plan_init(const qlora_adamw_tensor *tensors /* host array */,
                                   int32_t count, void *device, size_t bytes,
                                   qlora_adamw_plan *plan /* host out */, void *stream);

/* Bytes of workspace qlora_adamw_step_plan needs (0 if plan is NULL). */
size_t qlora_adamw_plan_workspace_size(const qlora_adamw_plan *plan /* host */);

/* One AdamW step over a prepared list: the same arithmetic, arguments and
 * errors as qlora_adamw_step (the norm's float64 partial sums are grouped
 * differently, so the last bits of the norm and of a clipped step may differ
 * from it; each path repeats its own bits exactly). */
qlora_status qlora_adamw_step_plan(const qlora_adamw_plan *plan /* host */, float lr, float beta1,
                                   float beta2, float eps, float weight_decay, int64_t step,
                                   float max_grad_norm, float *grad_norm, void *workspace,
                                   size_t ws_bytes, void *stream);

/* Bytes of device workspace needed by op 0 (forward, also qlora_lora_down,
 * qlora_nf4_matmul_fwd and qlora_linear_fwd_dropout), op 1 (backward) or op 2
 * (qlora_linear_bwd_dropout).  Returns 0 for an invalid op. */
size_t qlora_workspace_size(int32_t op, int64_t M, int64_t n_out, int64_t k_in, int32_t r);

/* (host) The 16 float32 NF4 levels the kernels use, ascending. */
void qlora_nf4_codebook(float out[16]);

/* (host) A static string naming a status. */
const char *qlora_status_string(qlora_status s);

/* (host) QLORA_ABI_VERSION of the built library. */
int32_t qlora_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
