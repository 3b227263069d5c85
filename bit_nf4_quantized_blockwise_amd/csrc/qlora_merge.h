// Kernels of the adapter merge: the merged 16-bit weight and its
// re-quantisation to NF4 + Double Quantization.
#pragma once

#include "qlora_common.h"

namespace qlora {

constexpr int kMergeRows = 16;   // rows of W per workgroup
constexpr int kMergeCols = 1024; // columns per workgroup (4 per lane)
constexpr int kMaxRankLds = 256; // largest rank (B rows staged in LDS)

struct MergeArgs {
  const uint16_t* w16;     // bf16 base [n_out][k_in], or nullptr for the NF4 base
  const uint8_t* packed;   // NF4 + DQ base (when w16 is nullptr)
  const int8_t* qabsmax;
  const float* c2;
  const uint16_t* a;       // A [r][k_in] bf16
  const uint16_t* b;       // B [n_out][r] bf16
  int64_t n_out, k_in;
  int32_t r;
  float s;
  uint16_t* merged;        // [n_out][k_in] bf16
};

// merged = RNE_bf16(RN64(base + RN64(s · Σ_j B[n][j]·A[j][k]))), the sum of
// exact float64 products formed by float64 fma over j = 0, 1, …, r − 1.
__global__ void merge_adapter_kernel(MergeArgs g);
// quantize_nf4_dq_kernel on a bf16 input.
__global__ void quantize_nf4_dq_bf16_kernel(const uint16_t* w, int64_t n, int64_t nblocks,
                                            uint8_t* packed, int8_t* qabsmax, float* c2);

}  // namespace qlora
