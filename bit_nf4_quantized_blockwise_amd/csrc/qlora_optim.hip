// 32-bit AdamW step on the rank-r adapter factors ("QLoRAの理論と実装", §5-3
// Paged Optimizers: Adam's first and second moments are the optimizer states,
// FP32, 12 bytes per trainable parameter together with the FP32 master
// weight; the training example selects paged_adamw_32bit with
// max_grad_norm = 0.3).  The update itself is AdamW's published definition
// (decoupled weight decay):
//   g <- g · coef,  coef = min(1, max_norm / (‖g‖₂ + 1e-6)) over all tensors
//   p <- p · (1 − lr·wd)
//   m <- β1·m + (1 − β1)·g
//   v <- β2·v + (1 − β2)·g²
//   p <- p − (lr / (1 − β1^t)) · m / (sqrt(v) / sqrt(1 − β2^t) + ε)
// and the bf16 copy the layer computes with is RNE_bf16(p).
//
// Both kernels stream every tensor once with 16-byte accesses (4 elements per
// lane); the work is split in units of 4 elements, a tensor's last unit
// possibly short.  The global norm is two fixed-order reductions (per
// workgroup, then over the workgroups' float64 partial sums, which every
// workgroup of the update redoes), so the step is bitwise repeatable.

#include "qlora_kernels.h"

namespace qlora {

namespace {

// Tensor of unit u (units of 4 elements, tensors back to back).
__device__ inline int tensor_of(const AdamList& L, int64_t u) {
  int t = 0;
#pragma unroll 1
  for (int i = 1; i < L.count; ++i) t = u >= L.t[i].u0 ? i : t;
  return t;
}

__device__ inline double block_sum(double v, double* sh) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
#pragma unroll
  for (int s = kAdamThreads / 2; s > 0; s >>= 1) {
    if (tid < s) sh[tid] += sh[tid + s];
    __syncthreads();
  }
  const double r = sh[0];
  __syncthreads();
  return r;
}

}  // namespace

__global__ __launch_bounds__(kAdamThreads) void adam_sqnorm_kernel(AdamList L, double* partials) {
  __shared__ double sh[kAdamThreads];
  double acc = 0.0;
  const int64_t stride = (int64_t)gridDim.x * kAdamThreads;
  for (int64_t u = (int64_t)blockIdx.x * kAdamThreads + threadIdx.x; u < L.units; u += stride) {
    const AdamTensor& T = L.t[tensor_of(L, u)];
    const int64_t i = (u - T.u0) * 4;
    if (i + 4 <= T.n) {
      const floatx4 g = *reinterpret_cast<const floatx4*>(T.g + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc += (double)g[e] * (double)g[e];
    } else {
      for (int64_t j = i; j < T.n; ++j) acc += (double)T.g[j] * (double)T.g[j];
    }
  }
  const double s = block_sum(acc, sh);
  if (threadIdx.x == 0) partials[blockIdx.x] = s;
}

__global__ __launch_bounds__(kAdamThreads) void adam_update_kernel(AdamList L, AdamHyper h,
                                                                   const double* partials,
                                                                   int32_t npart, float* norm_out) {
  __shared__ double sh[kAdamThreads];
  float coef = 1.0f;
  if (npart > 0) {
    double acc = 0.0;
    for (int i = threadIdx.x; i < npart; i += kAdamThreads) acc += partials[i];
    const double norm = sqrt(block_sum(acc, sh));
    if (h.clip) coef = (float)fmin(1.0, (double)h.max_norm / (norm + 1e-6));
    if (norm_out && blockIdx.x == 0 && threadIdx.x == 0) *norm_out = (float)norm;
  }
  const float b1 = h.beta1, b2 = h.beta2, c1 = 1.0f - h.beta1, c2 = 1.0f - h.beta2;
  auto one = [&](float& p, float g, float& m, float& v) {
    g *= coef;
    p *= h.decay;
    m = b1 * m + c1 * g;
    v = b2 * v + c2 * (g * g);
    p -= h.step_size * (m / (sqrtf(v) * h.inv_sqrt_bc2 + h.eps));
  };
  const int64_t stride = (int64_t)gridDim.x * kAdamThreads;
  for (int64_t u = (int64_t)blockIdx.x * kAdamThreads + threadIdx.x; u < L.units; u += stride) {
    const AdamTensor& T = L.t[tensor_of(L, u)];
    const int64_t i = (u - T.u0) * 4;
    if (i + 4 <= T.n) {
      floatx4 p = *reinterpret_cast<const floatx4*>(T.p + i);
      const floatx4 g = *reinterpret_cast<const floatx4*>(T.g + i);
      floatx4 m = *reinterpret_cast<const floatx4*>(T.m + i);
      floatx4 v = *reinterpret_cast<const floatx4*>(T.v + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float pe = p[e], me = m[e], ve = v[e];
        one(pe, g[e], me, ve);
        p[e] = pe;
        m[e] = me;
        v[e] = ve;
      }
      *reinterpret_cast<floatx4*>(T.p + i) = p;
      *reinterpret_cast<floatx4*>(T.m + i) = m;
      *reinterpret_cast<floatx4*>(T.v + i) = v;
      if (T.pb) *reinterpret_cast<u32x2*>(T.pb + i) = u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
    } else {
      for (int64_t j = i; j < T.n; ++j) {
        float pe = T.p[j], me = T.m[j], ve = T.v[j];
        one(pe, T.g[j], me, ve);
        T.p[j] = pe;
        T.m[j] = me;
        T.v[j] = ve;
        if (T.pb) T.pb[j] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(pe));
      }
    }
  }
}

}  // namespace qlora
