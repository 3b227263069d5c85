// Kernels of the quantiser variants: uniform INT4 codes, single-quantisation
// decode (float32 absmax per block) and the squared quantisation error.
#pragma once

#include "qlora_common.h"

namespace qlora {

enum QuantCode { kCodeNF4 = 0, kCodeINT4 = 1 };

constexpr int kErrMaxWgs = 2048;  // most workgroups (float64 partial sums) of one error launch

// packed[ceil(n/64)*32], absmax[ceil(n/64)]; one lane per 16 weights.
__global__ void quantize_int4_kernel(const float* w, int64_t n, int64_t nblocks, uint8_t* packed,
                                     float* absmax);
// out[n] bf16 = RNE_bf16(RN32(level_idx · absmax_block)), any n.
template <int CODE>
__global__ void dequantize_4bit_kernel(const uint32_t* packed, const float* absmax, int64_t n,
                                       uint16_t* out);
// partials[blockIdx.x] = Σ (w − RN32(level_idx · absmax))² over the workgroup's weights.
template <int CODE>
__global__ void quant_sq_error_kernel(const float* w, int64_t n, const uint32_t* packed,
                                      const float* absmax, double* partials);
// *out = Σ partials[0..npart) in a fixed order (one workgroup).
__global__ void sum_partials_kernel(const double* partials, int32_t npart, double* out);

}  // namespace qlora
