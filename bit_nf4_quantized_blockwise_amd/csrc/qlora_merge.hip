// Merging a trained adapter into the base weight ("QLoRAとは？4bit量子化＋LoRAの
// 仕組み・VRAM目安・実装手順と採用判断を解説", section on merging and
// distributing the adapter: merge into the 16-bit base, keep the merged
// 16-bit model, re-quantise it for 4-bit inference; merging into the 4-bit
// base re-rounds the sum onto the 4-bit grid).  The adapter adds s·B·A,
// s = α/r ("QLoRAの理論と実装", §3 LoRA).
//
// Each element is W + s·B·A evaluated in float64 and rounded once to bf16,
// on the 16-bit base and on the decoded 4-bit one alike: acc = Σ_j
// B[n][j]·A[j][k] (a bf16 × bf16 product is exact in float64, so each fma
// rounds only an addition, and for these magnitudes the sum is exact),
// t = RN64(s·acc), x = RN64(w + t), merged = RNE_bf16(x) — one rounding from
// float64 straight to bf16.
//
// Work: n_out·k_in·r float64 fused multiply-adds on the vector ALU (peak
// 78.6 TFLOP/s on this GPU; the rank-r product is tiny next to the weight);
// each lane owns four columns of 16 rows and reads B's 16 rows of the current
// j from LDS as broadcasts (eight 16-byte reads per 64 fma).

#include "qlora_merge.h"

namespace qlora {

// RNE_bf16 of a float64 value: with x = m·2^e (m in [0.5, 1)) the bf16
// spacing near x is 2^(e−8), and 2^-133 below 2^-126 (the subnormals);
// x / spacing is an exact power-of-two scaling, its nearest integer (ties to
// even) times the spacing is the rounded value, which float32 holds exactly
// (2^128, the rounding of values at or past the largest bf16 plus half its
// spacing, becomes infinity).  Finite inputs.
__device__ inline uint32_t bf16_rne_from_f64(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
  const int e = (int)((u >> 52) & 0x7ffu) - 1022;
  const int q = max(e - 8, -133);
  const double k = __builtin_rint(__builtin_ldexp(__builtin_fabs(x), -q));
  const float v = (float)__builtin_ldexp(k, q);
  return sign | (__builtin_bit_cast(uint32_t, v) >> 16);
}

__device__ inline double bf16_to_f64(uint32_t bits16) { return (double)bits_to_float(bits16 << 16); }

__global__ __launch_bounds__(256) void merge_adapter_kernel(MergeArgs g) {
  __shared__ double2 bs[kMaxRankLds][kMergeRows / 2];  // B[n0 + i][j] as float64, [j][i]
  const int tid = threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.y * kMergeRows;
  const int64_t c = (int64_t)blockIdx.x * kMergeCols + 4 * tid;  // this lane's four columns
  const int rows = (int)min<int64_t>(kMergeRows, g.n_out - n0);

  double* bsd = reinterpret_cast<double*>(bs);
  for (int e = tid; e < g.r * kMergeRows; e += 256) {
    const int j = e / kMergeRows, i = e % kMergeRows;
    bsd[e] = (i < rows) ? bf16_to_f64(g.b[(n0 + i) * g.r + j]) : 0.0;
  }
  __syncthreads();
  if (c >= g.k_in) return;

  double acc[kMergeRows][4];
#pragma unroll
  for (int i = 0; i < kMergeRows; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[i][e] = 0.0;
  // one rank step: acc[i][e] += B[n0 + i][j] · A[j][c + e] (an exact product:
  // the fma rounds only the addition)
  auto step = [&](const u32x2& av, int j) {
    double a[4];
    a[0] = bf16_to_f64(av[0] & 0xffffu);
    a[1] = bf16_to_f64(av[0] >> 16);
    a[2] = bf16_to_f64(av[1] & 0xffffu);
    a[3] = bf16_to_f64(av[1] >> 16);
#pragma unroll
    for (int q = 0; q < kMergeRows / 2; ++q) {
      const double2 b = bs[j][q];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * q][e] = __builtin_fma(b.x, a[e], acc[2 * q][e]);
        acc[2 * q + 1][e] = __builtin_fma(b.y, a[e], acc[2 * q + 1][e]);
      }
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

  const double s = (double)g.s;
  // (a guarded body, not an early exit: the accumulators stay in registers)
#pragma unroll
  for (int i = 0; i < kMergeRows; ++i) {
    if (i < rows) {
      const int64_t f = (n0 + i) * g.k_in + c;  // multiple of 4: one block, two packed bytes
      uint32_t wb[4];                           // the base's bf16 bits
      if (g.w16) {
        const u32x2 wv = *reinterpret_cast<const u32x2*>(g.w16 + f);
        wb[0] = wv[0] & 0xffffu;
        wb[1] = wv[0] >> 16;
        wb[2] = wv[1] & 0xffffu;
        wb[3] = wv[1] >> 16;
      } else {
        const uint32_t bytes = *reinterpret_cast<const uint16_t*>(g.packed + (f >> 1));
        const int64_t blk = f >> 6;
        const float ah = g.c2[blk >> 8] * (float)g.qabsmax[blk];
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          const uint32_t d = pack_bf16x2(bits_to_float(kNF4Bits[(bytes >> (4 * e)) & 15u]) * ah,
                                         bits_to_float(kNF4Bits[(bytes >> (4 * e + 4)) & 15u]) * ah);
          wb[e] = d & 0xffffu;
          wb[e + 1] = d >> 16;
        }
      }
      uint32_t m[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double t = s * acc[i][e];          // RN64(s·acc)
        const double x = bf16_to_f64(wb[e]) + t; // RN64(w + t)
        m[e] = bf16_rne_from_f64(x);
      }
      *reinterpret_cast<u32x2*>(g.merged + f) = u32x2{m[0] | (m[1] << 16), m[2] | (m[3] << 16)};
    }
  }
}

}  // namespace qlora
