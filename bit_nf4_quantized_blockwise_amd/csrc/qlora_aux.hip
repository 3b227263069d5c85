// Small helper kernels around the GEMMs: deterministic reduction of split-K
// partial sums (fixed summation order, so repeated runs are bitwise equal),
// and transpose / zero-pad copies of the rank-r adapter factors.

#include "qlora_kernels.h"

namespace qlora {

// out(row, col) = scale · Σ_z part[z][row][col], for row < rows_pad, col < cols_pad;
// entries with row >= rows or col >= cols are written as zero (padding).
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float* __restrict__ part,
                                                              int64_t part_stride, int32_t nsplit,
                                                              int64_t rows, int64_t cols,
                                                              int64_t rows_pad, int64_t cols_pad,
                                                              int64_t ldp, float scale,
                                                              ReduceOut o0, ReduceOut o1) {
  const int64_t total = rows_pad * cols_pad;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
    const int64_t row = i / cols_pad, col = i % cols_pad;
    float v = 0.0f;
    if (row < rows && col < cols) {
      for (int z = 0; z < nsplit; ++z) v += part[(int64_t)z * part_stride + row * ldp + col];
      v *= scale;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const ReduceOut& o = k ? o1 : o0;
      const int64_t off = o.transposed ? col * o.ld + row : row * o.ld + col;
      if (o.bf16) o.bf16[off] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
      if (o.f32) o.f32[off] = v;
    }
  }
}

// out[c][r] = in[r][c] for r < R, c < C; zero for r in [R, Rp) or c in [C, Cp).
__global__ __launch_bounds__(256) void transpose_pad_kernel(const uint16_t* __restrict__ in,
                                                            int64_t ldi, int64_t R, int64_t C,
                                                            int64_t Rp, int64_t Cp,
                                                            uint16_t* __restrict__ out,
                                                            int64_t ldo) {
  const int64_t total = Rp * Cp;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
    const int64_t c = i / Rp, r = i % Rp;
    out[c * ldo + r] = (r < R && c < C) ? in[r * ldi + c] : (uint16_t)0;
  }
}

// out[r][c] = in[r][c] for c < C, zero for c in [C, Cp): pads the row pitch.
__global__ __launch_bounds__(256) void pad_cols_kernel(const uint16_t* __restrict__ in, int64_t ldi,
                                                       int64_t R, int64_t C, int64_t Cp,
                                                       uint16_t* __restrict__ out, int64_t ldo) {
  const int64_t total = R * Cp;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
    const int64_t r = i / Cp, c = i % Cp;
    out[r * ldo + c] = (c < C) ? in[r * ldi + c] : (uint16_t)0;
  }
}

}  // namespace qlora
