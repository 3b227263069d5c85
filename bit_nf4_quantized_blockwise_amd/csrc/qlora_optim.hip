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
// The tensors are cut into chunks of kAdamChunk elements (a tensor's last
// chunk may be short), so a workgroup step never straddles two tensors: the
// tensor of a chunk is found once per workgroup step, by a binary search over
// the tensors' first chunks, and every lane keeps kAdamUnroll 16-byte loads of
// each stream in flight; full chunks stream with nontemporal loads and stores
// (nothing is re-read).  The global norm is two fixed-order reductions (per
// workgroup in float64, then one workgroup over those partial sums, which
// also forms the clipping coefficient), so the step is bitwise repeatable.

#include "qlora_optim.h"
#include "qlora_reduce.h"

namespace qlora {

namespace {

// The tensor holding chunk c: the last tensor whose first chunk is <= c (a
// tensor of no elements shares its first chunk with the next one).
__device__ inline int chunk_tensor(const AdamList& L, int64_t c) {
  int lo = 0, hi = L.count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (L.t[mid].c0 <= c) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Where a launch finds its tensors: the list in the kernel arguments (tensor of
// a chunk by binary search), or a prepared list in device memory (tensor of a
// chunk from the chunk map: one scalar load).
struct ArgSrc {
  const AdamList& L;
  __device__ inline int64_t chunks() const { return L.chunks; }
  __device__ inline const AdamTensor& tensor(int64_t c) const { return L.t[chunk_tensor(L, c)]; }
};
struct PlanSrc {
  const AdamPlanDev& P;
  __device__ inline int64_t chunks() const { return P.chunks; }
  __device__ inline const AdamTensor& tensor(int64_t c) const { return P.t[P.tmap[c]]; }
};

__device__ inline double sq4(const floatx4& g) {
  double a = 0.0;
#pragma unroll
  for (int e = 0; e < 4; ++e) a += (double)g[e] * (double)g[e];
  return a;
}

}  // namespace

template <class Src>
__device__ inline void sqnorm_body(const Src& S, double* partials) {
  __shared__ double sh[kAdamThreads];
  double acc = 0.0;
  for (int64_t c = blockIdx.x; c < S.chunks(); c += gridDim.x) {
    const AdamTensor& T = S.tensor(c);
    const int64_t base = (c - T.c0) * kAdamChunk;
    if (base + kAdamChunk <= T.n) {
      floatx4 g[kAdamUnroll];
#pragma unroll
      for (int k = 0; k < kAdamUnroll; ++k)
        g[k] = *reinterpret_cast<const floatx4*>(T.g + base + (k * kAdamThreads + threadIdx.x) * 4);
#pragma unroll
      for (int k = 0; k < kAdamUnroll; ++k) acc += sq4(g[k]);
    } else {
#pragma unroll 1
      for (int k = 0; k < kAdamUnroll; ++k) {
        const int64_t i = base + (k * kAdamThreads + threadIdx.x) * 4;
        if (i + 4 <= T.n) {
          acc += sq4(*reinterpret_cast<const floatx4*>(T.g + i));
        } else {
          for (int64_t j = i; j < T.n; ++j) acc += (double)T.g[j] * (double)T.g[j];
        }
      }
    }
  }
  const double s = block_sum_f64<kAdamThreads>(acc, sh);
  if (threadIdx.x == 0) partials[blockIdx.x] = s;
}

__global__ __launch_bounds__(kAdamThreads) void adam_sqnorm_kernel(AdamList L, double* partials) {
  sqnorm_body(ArgSrc{L}, partials);
}

__global__ __launch_bounds__(kAdamThreads) void adam_sqnorm_plan_kernel(AdamPlanDev P,
                                                                        double* partials) {
  sqnorm_body(PlanSrc{P}, partials);
}

__global__ __launch_bounds__(kAdamThreads) void adam_clip_kernel(const double* partials,
                                                                 int32_t npart, float max_norm,
                                                                 int32_t clip, float* coef,
                                                                 float* norm_out) {
  __shared__ double sh[kAdamThreads];
  const double norm = sqrt(workgroup_sum_f64<kAdamThreads>(partials, npart, sh));
  if (threadIdx.x == 0) {
    *coef = clip ? (float)fmin(1.0, (double)max_norm / (norm + 1e-6)) : 1.0f;
    if (norm_out) *norm_out = (float)norm;
  }
}

template <class Src>
__device__ inline void update_body(const Src& S, const AdamHyper& h, const float* coef_p) {
  const float coef = coef_p ? *coef_p : 1.0f;
  const float b1 = h.beta1, b2 = h.beta2, c1 = 1.0f - h.beta1, c2 = 1.0f - h.beta2;
  auto one = [&](float& p, float g, float& m, float& v) {
    g *= coef;
    p *= h.decay;
    m = b1 * m + c1 * g;
    v = b2 * v + c2 * (g * g);
    p -= h.step_size * (m / (sqrtf(v) * h.inv_sqrt_bc2 + h.eps));
  };
  auto four = [&](floatx4& p, const floatx4& g, floatx4& m, floatx4& v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float pe = p[e], me = m[e], ve = v[e];
      one(pe, g[e], me, ve);
      p[e] = pe;
      m[e] = me;
      v[e] = ve;
    }
  };
  auto store4 = [&](const AdamTensor& T, int64_t i, const floatx4& p, const floatx4& m,
                    const floatx4& v) {
    *reinterpret_cast<floatx4*>(T.p + i) = p;
    *reinterpret_cast<floatx4*>(T.m + i) = m;
    *reinterpret_cast<floatx4*>(T.v + i) = v;
    if (T.pb)
      *reinterpret_cast<u32x2*>(T.pb + i) = u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
  };
  for (int64_t c = blockIdx.x; c < S.chunks(); c += gridDim.x) {
    const AdamTensor& T = S.tensor(c);
    const int64_t base = (c - T.c0) * kAdamChunk;
    if (base + kAdamChunk <= T.n) {
      floatx4 p[kAdamUnroll], g[kAdamUnroll], m[kAdamUnroll], v[kAdamUnroll];
#pragma unroll
      for (int k = 0; k < kAdamUnroll; ++k) {
        const int64_t i = base + (k * kAdamThreads + threadIdx.x) * 4;
        g[k] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(T.g + i));
        m[k] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(T.m + i));
        v[k] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(T.v + i));
        p[k] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(T.p + i));
      }
#pragma unroll
      for (int k = 0; k < kAdamUnroll; ++k) {
        four(p[k], g[k], m[k], v[k]);
        const int64_t i = base + (k * kAdamThreads + threadIdx.x) * 4;
        __builtin_nontemporal_store(p[k], reinterpret_cast<floatx4*>(T.p + i));
        __builtin_nontemporal_store(m[k], reinterpret_cast<floatx4*>(T.m + i));
        __builtin_nontemporal_store(v[k], reinterpret_cast<floatx4*>(T.v + i));
        if (T.pb)
          __builtin_nontemporal_store(
              u32x2{pack_bf16x2(p[k][0], p[k][1]), pack_bf16x2(p[k][2], p[k][3])},
              reinterpret_cast<u32x2*>(T.pb + i));
      }
    } else {
#pragma unroll 1
      for (int k = 0; k < kAdamUnroll; ++k) {
        const int64_t i = base + (k * kAdamThreads + threadIdx.x) * 4;
        if (i + 4 <= T.n) {
          floatx4 p = *reinterpret_cast<const floatx4*>(T.p + i);
          const floatx4 g = *reinterpret_cast<const floatx4*>(T.g + i);
          floatx4 m = *reinterpret_cast<const floatx4*>(T.m + i);
          floatx4 v = *reinterpret_cast<const floatx4*>(T.v + i);
          four(p, g, m, v);
          store4(T, i, p, m, v);
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
  }
}

__global__ __launch_bounds__(kAdamThreads) void adam_update_kernel(AdamList L, AdamHyper h,
                                                                   const float* coef_p) {
  update_body(ArgSrc{L}, h, coef_p);
}

__global__ __launch_bounds__(kAdamThreads) void adam_update_plan_kernel(AdamPlanDev P, AdamHyper h,
                                                                        const float* coef_p) {
  update_body(PlanSrc{P}, h, coef_p);
}

}  // namespace qlora
