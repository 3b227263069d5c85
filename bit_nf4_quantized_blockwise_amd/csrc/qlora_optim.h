// Argument structs and kernels of the 32-bit AdamW step over a list of tensors.
#pragma once

#include "qlora_common.h"

namespace qlora {

constexpr int kAdamThreads = 256;
constexpr int kAdamUnroll = 2;                                   // float4 units per lane per chunk
constexpr int kAdamChunk = kAdamThreads * 4 * kAdamUnroll;      // elements per workgroup step
constexpr int kAdamMaxTensors = 48;  // tensors per launch (the list travels in the kernel arguments)
constexpr int kAdamNormWgs = 2048;   // most workgroups (float64 partial sums) of one norm launch
constexpr int kAdamMaxGrid = 65536;  // most workgroups of one update launch

struct AdamTensor {
  float* p;        // fp32 master weights
  const float* g;  // fp32 gradient
  float* m;
  float* v;
  uint16_t* pb;    // bf16 copy of p after the step, or nullptr
  int64_t n;
  int64_t c0;      // first chunk of this tensor within the launch
};
struct AdamList {
  AdamTensor t[kAdamMaxTensors];
  int32_t count;
  int64_t chunks;  // chunks of all tensors (a tensor's last chunk may be short)
};
struct AdamHyper {
  float beta1, beta2, eps;
  float decay;         // 1 - lr·wd
  float step_size;     // lr / (1 - beta1^t)
  float inv_sqrt_bc2;  // 1 / sqrt(1 - beta2^t)
};

// A prepared list in device memory: the descriptors (c0 as above, over all
// tensors) and the tensor index of every chunk.
constexpr int kAdamPlanNormWgs = 8192;  // most workgroups of the norm launch over a prepared list
struct AdamPlanDev {
  const AdamTensor* t;
  const int32_t* tmap;
  int64_t chunks;
};

// partials[blockIdx.x] = Σ g² over the chunks this workgroup visits (float64)
__global__ void adam_sqnorm_kernel(AdamList L, double* partials);
// One workgroup: norm = sqrt(Σ partials) in a fixed order; *coef = min(1, max_norm/(norm+1e-6))
// (1 when clip == 0); *norm_out = norm when norm_out != nullptr.
__global__ void adam_clip_kernel(const double* partials, int32_t npart, float max_norm,
                                 int32_t clip, float* coef, float* norm_out);
// The step; coef == nullptr means no clipping.
__global__ void adam_update_kernel(AdamList L, AdamHyper h, const float* coef);
// The same two passes over a prepared list.
__global__ void adam_sqnorm_plan_kernel(AdamPlanDev P, double* partials);
__global__ void adam_update_plan_kernel(AdamPlanDev P, AdamHyper h, const float* coef);

}  // namespace qlora
