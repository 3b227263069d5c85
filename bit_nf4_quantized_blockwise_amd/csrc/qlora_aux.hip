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

// The same reduction, four columns per thread: float4 partial loads (cols_pad,
// ldp and part_stride multiples of 4, part 16-byte aligned).
__global__ __launch_bounds__(256) void reduce_partials4_kernel(const float* __restrict__ part,
                                                               int64_t part_stride, int32_t nsplit,
                                                               int64_t rows, int64_t cols,
                                                               int64_t rows_pad, int64_t cols_pad,
                                                               int64_t ldp, float scale,
                                                               ReduceOut o0, ReduceOut o1) {
  const int64_t cq = cols_pad >> 2;
  const int64_t total = rows_pad * cq;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
    const int64_t row = i / cq, col = (i % cq) * 4;
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if (row < rows && col < cols) {
      const floatx4* p = reinterpret_cast<const floatx4*>(part + row * ldp + col);
      const int64_t zs = part_stride >> 2;
      for (int z = 0; z < nsplit; ++z) v += p[(int64_t)z * zs];
      v *= scale;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (col + e >= cols) v[e] = 0.0f;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const ReduceOut& o = k ? o1 : o0;
      if (!o.bf16 && !o.f32) continue;
      if (o.transposed) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t off = (col + e) * o.ld + row;
          if (o.bf16) o.bf16[off] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[e]));
          if (o.f32) o.f32[off] = v[e];
        }
      } else {
        const int64_t off = row * o.ld + col;
        if (o.bf16) {
          const uint32_t lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<u32x2*>(o.bf16 + off) = u32x2{lo, hi};
        }
        if (o.f32) *reinterpret_cast<floatx4*>(o.f32 + off) = v;
      }
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

// Up to three transpose_pad jobs in one launch (blockIdx.y picks the job),
// through 64 x 64 LDS tiles so that both the reads and the writes are
// row-contiguous.
__global__ __launch_bounds__(256) void transpose_pad3_kernel(TransposeJob j0, TransposeJob j1,
                                                             TransposeJob j2) {
  __shared__ uint32_t tile[64][65];
  const TransposeJob& j = blockIdx.y == 0 ? j0 : (blockIdx.y == 1 ? j1 : j2);
  if (!j.out) return;
  const int t = threadIdx.x;
  const int64_t tr = (j.Rp + 63) / 64, tc = (j.Cp + 63) / 64;
  for (int64_t tile_id = blockIdx.x; tile_id < tr * tc; tile_id += gridDim.x) {
    const int64_t r0 = (tile_id / tc) * 64, c0 = (tile_id % tc) * 64;
    // read: rows r0.., 64 columns each, 4 rows per pass of 256 threads
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int rr = p * 4 + (t >> 6), cc = t & 63;
      const int64_t r = r0 + rr, c = c0 + cc;
      tile[rr][cc] = (r < j.R && c < j.C) ? j.in[r * j.ldi + c] : 0u;
    }
    __syncthreads();
    // write: out rows c0.. (input columns), 64 entries each (input rows)
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int cc = p * 4 + (t >> 6), rr = t & 63;
      const int64_t c = c0 + cc, r = r0 + rr;
      if (c < j.Cp && r < j.Rp) j.out[c * j.ldo + r] = (uint16_t)tile[rr][cc];
    }
    __syncthreads();
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
