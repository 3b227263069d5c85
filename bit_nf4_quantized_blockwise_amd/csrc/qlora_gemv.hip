// Few-token QLoRA forward (M <= 16 tokens) for gfx950: stream the NF4 weight
// once from HBM with 16-byte loads and contract it on the matrix cores.
//
//   Y[m][n] = Σ_b â_b · Σ_{k in block b} X[m][k] · c_bf16[idx(n, k)]  +  s · Σ_j U[m][j] · B[n][j]
//
// ("QLoRAの理論と実装", QLoRAの計算フロー: the main path plus the rank-r adapter
// path, here for decode-sized batches.)  The block scale â_b = RN32(c2 · q)
// (Qiita explainer, DQ formula) multiplies the fp32 partial sum of its block
// instead of every weight: this keeps the per-weight work to one table lookup
// per two weights.  The codebook enters the bf16 MFMA rounded to bf16, so the
// result differs from "decode each weight to bf16, then multiply" only by
// rounding (well inside the forward's tolerance); the many-token GEMMs decode
// every weight exactly.
//
// Layout of one v_mfma_f32_16x16x32_bf16 (a chunk = 128 k = two 64-blocks):
//   B operand: lane (c = l%16, q = l/16) holds 8 consecutive weights of W row
//     n0 + c, taken from its own 16-byte load of 32 weights at k = kb + 32q
//     (the four MFMAs of a chunk take bytes 4j..4j+3, j = 0..3).
//   A operand: rows 0..7 carry tokens 0..7 restricted to the lanes with q < 2
//     (block kb/64), rows 8..15 the same tokens restricted to q >= 2 (block
//     kb/64 + 1); the other entries are zero.  So C rows 0..7 hold the first
//     block's partial sums and rows 8..15 the second's, and every lane scales
//     the rows it holds by the scale of the block it loaded itself.
// 8 waves split the reduction; each wave walks all of its workgroup's column
// groups and the partial sums meet in LDS once, at the end.

#include "qlora_kernels.h"

namespace qlora {

namespace {

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9)

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffffLL : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kRsrcWord3);
}

__device__ inline uint16_t bf16_rne_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

}  // namespace

template <int CPW, int MG, int G>
__global__ __launch_bounds__(512) void nf4_gemv_kernel(GemvArgs g) {
  __shared__ uint32_t lut[256 * 32];        // byte -> two bf16 levels, one copy per bank
  __shared__ float red[8][G][MG][32][4];    // per-wave partial sums, reduced once at the end

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c16 = lane & 15, qd = lane >> 4;

  for (int i = tid; i < 256 * 32; i += 512) {
    const int e = i >> 5;
    const float lo = bits_to_float(kNF4Bits[e & 15]);
    const float hi = bits_to_float(kNF4Bits[e >> 4]);
    lut[i] = (uint32_t)bf16_rne_bits(lo) | ((uint32_t)bf16_rne_bits(hi) << 16);
  }

  const int64_t K = g.K, N = g.N;
  const int M = g.M;
  const int64_t chunk0 = ((int64_t)blockIdx.y * 8 + w) * CPW;

  // Token operands for this wave's chunks, kept in registers for all columns.
  u32x4 xa[MG][CPW][4];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg)
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t k = (chunk0 + c) * 128 + 32 * qd + 8 * j;
        const int tok = (c16 & 7) + 8 * mg;
        const bool valid = ((c16 < 8) == (qd < 2)) && tok < M && k < K;
        xa[mg][c][j] = valid ? *reinterpret_cast<const u32x4*>(g.x + (int64_t)tok * K + k)
                             : u32x4{0u, 0u, 0u, 0u};
      }
  __syncthreads();

  const uint32_t* lutl = lut + (lane & 31);
  const int64_t ncg = (N + 15) / 16;
  const int64_t blocks_per_row = K >> 6;
  const __amdgpu_buffer_rsrc_t c2r = make_rsrc(g.c2, ((N * blocks_per_row + 255) >> 8) * 4);
  const int64_t cg0 = (int64_t)blockIdx.x * G;

  // Every wave walks all G column groups of the workgroup on its own slice
  // of the reduction; no workgroup barrier until the end, so the waves drift
  // apart and one wave's loads overlap another's MFMAs.
  floatx4 acc[G][MG];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) acc[gi][mg] = floatx4{0.f, 0.f, 0.f, 0.f};
    const int64_t n0 = (cg0 + gi) * 16;
    if (n0 >= N) continue;  // uniform
    const __amdgpu_buffer_rsrc_t pr = make_rsrc(g.packed + n0 * (K >> 1), (N - n0) * (K >> 1));
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(g.qabsmax + n0 * blocks_per_row,
                                                (N - n0) * blocks_per_row);
    u32x4 pk[CPW];
    float ah[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int64_t kq = (chunk0 + c) * 128 + 32 * qd;
      const int off = (int)((c16 * K + kq) >> 1);
      pk[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(pr, off, 0, 0));
      const int64_t lb = (c16 * K + kq) >> 6;  // block index relative to row n0
      const uint32_t qv = __builtin_amdgcn_raw_buffer_load_b8(qr, (int)lb, 0, 0);
      const int64_t gb = n0 * blocks_per_row + lb;
      const float c2v = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(c2r, (int)((gb >> 8) * 4), 0, 0));
      ah[c] = c2v * (float)qv;
    }
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      floatx4 cb[MG];
#pragma unroll
      for (int mg = 0; mg < MG; ++mg) cb[mg] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t p = pk[c][j];
        u32x4 bop;
#pragma unroll
        for (int t = 0; t < 4; ++t) bop[t] = lutl[((p >> (8 * t)) & 0xffu) * 32];
#pragma unroll
        for (int mg = 0; mg < MG; ++mg)
          cb[mg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[mg][c][j]),
                                                           __builtin_bit_cast(bf16x8, bop), cb[mg],
                                                           0, 0, 0);
      }
#pragma unroll
      for (int mg = 0; mg < MG; ++mg)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[gi][mg][i] += ah[c] * cb[mg][i];
    }
  }
  // rows r and r + 8 hold the same token for the two blocks of each chunk
#pragma unroll
  for (int gi = 0; gi < G; ++gi)
#pragma unroll
    for (int mg = 0; mg < MG; ++mg)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[gi][mg][i] += __shfl_xor(acc[gi][mg][i], 32);
  if (lane < 32) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
#pragma unroll
      for (int mg = 0; mg < MG; ++mg)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[w][gi][mg][lane][i] = acc[gi][mg][i];
  }
  __syncthreads();
  for (int o = tid; o < G * MG * 128; o += 512) {
    const int gi = o / (MG * 128), mg = (o / 128) % MG, t = o & 127;
    const int tok8 = t >> 4, col = t & 15;
    float v = 0.0f;
#pragma unroll
    for (int ww = 0; ww < 8; ++ww) v += red[ww][gi][mg][col + 16 * (tok8 >> 2)][tok8 & 3];
    const int tok = tok8 + 8 * mg;
    const int64_t n = (cg0 + gi) * 16 + col;
    if (tok < M && n < N) {
      if (blockIdx.y == 0) {
        float l = 0.0f;
        for (int jr = 0; jr < g.r; ++jr)
          l += bf16_bits_to_float(g.u[(int64_t)tok * g.r + jr]) *
               bf16_bits_to_float(g.b[n * g.r + jr]);
        v += g.s * l;
      }
      if (g.ksplit == 1)
        g.y[(int64_t)tok * N + n] = bf16_rne_bits(v);
      else
        g.part[((int64_t)blockIdx.y * M + tok) * N + n] = v;
    }
  }
}

// U[m][j] = Σ_k X[m][k] · A[j][k] for M <= 16 tokens: one workgroup per rank
// index j; every load issued up front, then a fixed-order reduction through
// LDS (no shuffle chains).
__global__ __launch_bounds__(256) void lora_down_small_kernel(const uint16_t* __restrict__ x, int M,
                                                              int64_t K, const uint16_t* __restrict__ a,
                                                              int r, uint16_t* __restrict__ u) {
  __shared__ float red[16][257];
  const int j = blockIdx.x, tid = threadIdx.x;
  float acc[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) acc[m] = 0.0f;
  for (int64_t k0 = (int64_t)tid * 8; k0 < K; k0 += 4 * 256 * 8) {
    u32x4 av[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t k = k0 + (int64_t)s * 256 * 8;
      av[s] = k < K ? *reinterpret_cast<const u32x4*>(a + (int64_t)j * K + k) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      if (m >= M) continue;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int64_t k = k0 + (int64_t)s * 256 * 8;
        if (k >= K) continue;
        const u32x4 xv = *reinterpret_cast<const u32x4*>(x + (int64_t)m * K + k);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          acc[m] += bits_to_float(xv[d] << 16) * bits_to_float(av[s][d] << 16);
          acc[m] += bits_to_float(xv[d] & 0xffff0000u) * bits_to_float(av[s][d] & 0xffff0000u);
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < 16; ++m) red[m][tid] = acc[m];
  __syncthreads();
  {  // 256 threads: (m, part) sums 16 entries
    const int m = tid >> 4, part = tid & 15;
    float v = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) v += red[m][part * 16 + i];
    __syncthreads();
    red[m][part] = v;
  }
  __syncthreads();
  if (tid < M) {
    float v = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) v += red[tid][i];
    u[(int64_t)tid * r + j] = bf16_rne_bits(v);
  }
}

template __global__ void nf4_gemv_kernel<1, 1, 1>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 1, 2>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 1, 3>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 1, 4>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 1, 5>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 1, 6>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 1, 7>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 1, 8>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 1, 1>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 1, 2>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 1, 3>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 1, 4>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 1, 5>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 1, 6>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 1, 7>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 1, 8>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 1, 1>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 1, 2>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 1, 3>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 1, 4>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 1, 5>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 1, 6>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 1, 7>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 1, 8>(GemvArgs);
template __global__ void nf4_gemv_kernel<8, 1, 1>(GemvArgs);
template __global__ void nf4_gemv_kernel<8, 1, 2>(GemvArgs);
template __global__ void nf4_gemv_kernel<8, 1, 3>(GemvArgs);
template __global__ void nf4_gemv_kernel<8, 1, 4>(GemvArgs);
template __global__ void nf4_gemv_kernel<8, 1, 5>(GemvArgs);
template __global__ void nf4_gemv_kernel<8, 1, 6>(GemvArgs);
template __global__ void nf4_gemv_kernel<8, 1, 7>(GemvArgs);
template __global__ void nf4_gemv_kernel<8, 1, 8>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 2, 1>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 2, 2>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 2, 3>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 2, 4>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 2, 5>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 2, 6>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 2, 7>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 2, 8>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 2, 1>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 2, 2>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 2, 3>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 2, 4>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 2, 5>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 2, 6>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 2, 7>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 2, 8>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 2, 1>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 2, 2>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 2, 3>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 2, 4>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 2, 5>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 2, 6>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 2, 7>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 2, 8>(GemvArgs);

}  // namespace qlora
