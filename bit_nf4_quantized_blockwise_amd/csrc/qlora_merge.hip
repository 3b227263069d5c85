// Merging a trained adapter into the base weight ("QLoRAとは？4bit量子化＋LoRAの
// 仕組み・VRAM目安・実装手順と採用判断を解説", section on merging and
// distributing the adapter: merge into the 16-bit base, keep the merged
// 16-bit model, re-quantise it for 4-bit inference; merging into the 4-bit
// base re-rounds the sum onto the 4-bit grid).  The adapter adds s·B·A,
// s = α/r ("QLoRAの理論と実装", §3 LoRA).
//
// Each element is the same fixed sequence of float32 operations on both the
// 16-bit base and the decoded 4-bit one: acc = Σ_j B[n][j]·A[j][k], j
// ascending (a bf16 × bf16 product is exact in float32, so each fma is the
// rounding of one addition), t = RN32(s·acc), x = RN32(w + t), merged =
// RNE_bf16(x).  A fixed order makes the merged value, and every code the
// re-quantiser decides on it, a function of the inputs alone.
//
// Work: n_out·k_in·r fused multiply-adds on the vector ALU (the rank-r
// product is tiny next to the weight, but it is not a GEMM that the matrix
// cores could run in this order); each lane owns four columns of 16 rows and
// reads B's 16 rows of the current j from LDS as broadcasts (four 16-byte
// reads per 64 fma).

#include "qlora_merge.h"

namespace qlora {

__global__ __launch_bounds__(256) void merge_adapter_kernel(MergeArgs g) {
  __shared__ floatx4 bs[kMaxRankLds][kMergeRows / 4];  // B[n0 + i][j] as float, [j][i]
  const int tid = threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.y * kMergeRows;
  const int64_t c = (int64_t)blockIdx.x * kMergeCols + 4 * tid;  // this lane's four columns
  const int rows = (int)min<int64_t>(kMergeRows, g.n_out - n0);

  float* bsf = reinterpret_cast<float*>(bs);
  for (int e = tid; e < g.r * kMergeRows; e += 256) {
    const int j = e / kMergeRows, i = e % kMergeRows;
    bsf[e] = (i < rows) ? bits_to_float((uint32_t)g.b[(n0 + i) * g.r + j] << 16) : 0.0f;
  }
  __syncthreads();
  if (c >= g.k_in) return;

  float acc[kMergeRows][4];
#pragma unroll
  for (int i = 0; i < kMergeRows; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[i][e] = 0.0f;
  // one rank step: acc[i][e] += B[n0 + i][j] · A[j][c + e] (an exact product:
  // the fma rounds only the addition)
  auto step = [&](const u32x2& av, int j) {
    float a[4];
    a[0] = bits_to_float(av[0] << 16);
    a[1] = bits_to_float(av[0] & 0xffff0000u);
    a[2] = bits_to_float(av[1] << 16);
    a[3] = bits_to_float(av[1] & 0xffff0000u);
#pragma unroll
    for (int q = 0; q < kMergeRows / 4; ++q) {
      const floatx4 b = bs[j][q];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[4 * q + i][e] = __builtin_fmaf(b[i], a[e], acc[4 * q + i][e]);
    }
  };
  const u32x2* ap = reinterpret_cast<const u32x2*>(g.a + c);  // A[j][c .. c + 3]
  const int64_t astride = g.k_in / 4;                        // in groups of four bf16
  constexpr int JB = 8;                                       // A loads in flight
  int j = 0;
  for (; j + JB <= g.r; j += JB) {
    u32x2 av[JB];
#pragma unroll
    for (int u = 0; u < JB; ++u) av[u] = ap[(int64_t)(j + u) * astride];
#pragma unroll
    for (int u = 0; u < JB; ++u) step(av[u], j + u);
  }
  for (; j < g.r; ++j) step(ap[(int64_t)j * astride], j);

  // (a guarded body, not an early exit: the accumulators stay in registers)
#pragma unroll
  for (int i = 0; i < kMergeRows; ++i) {
    if (i < rows) {
      const int64_t f = (n0 + i) * g.k_in + c;  // multiple of 4: one block, two packed bytes
      float w[4];
      if (g.w16) {
        const u32x2 wv = *reinterpret_cast<const u32x2*>(g.w16 + f);
        w[0] = bits_to_float(wv[0] << 16);
        w[1] = bits_to_float(wv[0] & 0xffff0000u);
        w[2] = bits_to_float(wv[1] << 16);
        w[3] = bits_to_float(wv[1] & 0xffff0000u);
      } else {
        const uint32_t bytes = *reinterpret_cast<const uint16_t*>(g.packed + (f >> 1));
        const int64_t blk = f >> 6;
        const float ah = g.c2[blk >> 8] * (float)g.qabsmax[blk];
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          const uint32_t d = pack_bf16x2(bits_to_float(kNF4Bits[(bytes >> (4 * e)) & 15u]) * ah,
                                         bits_to_float(kNF4Bits[(bytes >> (4 * e + 4)) & 15u]) * ah);
          w[e] = bits_to_float(d << 16);
          w[e + 1] = bits_to_float(d & 0xffff0000u);
        }
      }
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = w[e] + g.s * acc[i][e];  // RN32(w + RN32(s·acc))
      *reinterpret_cast<u32x2*>(g.merged + f) = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    }
  }
}

}  // namespace qlora
