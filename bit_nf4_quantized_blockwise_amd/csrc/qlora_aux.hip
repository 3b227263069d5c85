// Small helper kernels around the GEMMs: deterministic reduction of split-K
// partial sums (fixed summation order, so repeated runs are bitwise equal),
// zero-padded copies that give rows a 16-byte aligned pitch, and the LoRA
// dropout of the adapter input.

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
      const int64_t off = row * o.ld + col;
      if (o.bf16) o.bf16[off] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
      if (o.f32) o.f32[off] = v;
    }
  }
}

// The same reduction, four columns per thread: float4 partial loads (cols_pad,
// ldp and part_stride multiples of 4, part 16-byte aligned).  blockIdx.y picks
// one of two jobs, so two reductions share a launch.
__global__ __launch_bounds__(256) void reduce_partials4_kernel(ReduceJob j0, ReduceJob j1) {
  const ReduceJob& j = blockIdx.y ? j1 : j0;
  const int64_t cq = j.cols_pad >> 2;
  const int64_t total = j.rows_pad * cq;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
    const int64_t row = i / cq, col = (i % cq) * 4;
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if (row < j.rows && col < j.cols) {
      const floatx4* p = reinterpret_cast<const floatx4*>(j.part + row * j.ldp + col);
      const int64_t zs = j.part_stride >> 2;
      // sixteen loads in flight, then the adds in split order (the same sums
      // as one split at a time)
      for (int z0 = 0; z0 < j.nsplit; z0 += 16) {
        floatx4 t[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (z0 + u < j.nsplit) t[u] = p[(int64_t)(z0 + u) * zs];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (z0 + u < j.nsplit) v += t[u];
      }
      v *= j.scale;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (col + e >= j.cols) v[e] = 0.0f;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const ReduceOut& o = k ? j.o1 : j.o0;
      const int64_t off = row * o.ld + col;
      if (o.bf16) {
        const uint32_t lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<u32x2*>(o.bf16 + off) = u32x2{lo, hi};
      }
      if (o.f32) *reinterpret_cast<floatx4*>(o.f32 + off) = v;
    }
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

// LoRA dropout of the adapter input: each lane takes blocks of 8 consecutive
// elements (one generator block, one 16-byte load and store); a dropped
// element becomes +0, a kept one is copied bit for bit.
__global__ __launch_bounds__(256) void lora_dropout_kernel(const uint16_t* __restrict__ x,
                                                           int64_t nblk, DropoutKey d,
                                                           uint16_t* __restrict__ xd) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nblk; b += stride) {
    u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x) + b);
    const uint32_t keep = keep_bits8(d, (uint64_t)b);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = ((keep >> (2 * e)) & 1u) ? 0x0000ffffu : 0u;
      const uint32_t hi = ((keep >> (2 * e + 1)) & 1u) ? 0xffff0000u : 0u;
      v[e] &= lo | hi;
    }
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(xd) + b);
  }
}

}  // namespace qlora
