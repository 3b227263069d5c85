// Fixed-order float64 reductions shared by the kernels that produce a scalar
// (the AdamW gradient norm, the quantisation error).  The summation order
// depends only on the number of values and the workgroup size, so results
// are bitwise repeatable.
#pragma once

#include "qlora_common.h"

namespace qlora {

// Sum of one value per thread of an NT-thread workgroup (tree in LDS); every
// thread receives the sum.  sh holds NT doubles.
template <int NT>
__device__ inline double block_sum_f64(double v, double* sh) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
#pragma unroll
  for (int s = NT / 2; s > 0; s >>= 1) {
    if (tid < s) sh[tid] += sh[tid + s];
    __syncthreads();
  }
  const double r = sh[0];
  __syncthreads();
  return r;
}

// Σ p[0..n) by one NT-thread workgroup.  Eight independent accumulators per
// lane keep eight loads in flight.
template <int NT>
__device__ inline double workgroup_sum_f64(const double* p, int64_t n, double* sh) {
  constexpr int A = 8;
  double acc[A];
#pragma unroll
  for (int a = 0; a < A; ++a) acc[a] = 0.0;
  int64_t i = threadIdx.x;
  for (; i + (int64_t)(A - 1) * NT < n; i += (int64_t)A * NT) {
    double x[A];
#pragma unroll
    for (int a = 0; a < A; ++a) x[a] = p[i + (int64_t)a * NT];
#pragma unroll
    for (int a = 0; a < A; ++a) acc[a] += x[a];
  }
#pragma unroll
  for (int a = 0; a < A - 1; ++a)
    if (i + (int64_t)a * NT < n) acc[a] += p[i + (int64_t)a * NT];
  double t = 0.0;
#pragma unroll
  for (int a = 0; a < A; ++a) t += acc[a];
  return block_sum_f64<NT>(t, sh);
}

}  // namespace qlora
