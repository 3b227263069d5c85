// NF4 blockwise quantisation, Double Quantization and dequantisation for gfx950.
//
// Method ("QLoRAの理論と実装", disassemble-channel.com, §5-1 NF4 process steps
// 1-3, §5-2 Double Quantization; Qiita explainer, DQ formula
// W ≈ (c2 · c1^quant) · W^quant):
//   absmax_b = max |w| over 64 consecutive elements (zero-padded tail)
//   idx      = nearest of the 16 NF4 levels to w / absmax_b (tie -> lower index)
//   c2_g     = RN32(max absmax over 256 blocks / 127), q_b = nearest int to absmax_b / c2_g
//   ŵ        = RNE_bf16(RN32(c_idx · RN32(c2_g · q_b)))
//
// Exact decisions without a per-element division: for a > 0 and the level
// midpoints m_i (i = 0..14), "w / a > m_i" is equivalent to "w > T_i" with
// T_i = RD32(m_i · a): m_i · a is exact in float64 and, w being a float32,
// w exceeds the real product exactly when it exceeds the largest float32 not
// above it.  idx = #{i : w > T_i}, ties at a midpoint go to the lower index.
//
// The same exact-threshold quantiser serves the uniform INT4 comparison code
// of the same page ("NF4による量子化と量子化誤差の比較": 16 evenly spaced
// levels on [-1, 1], here each rounded once to float32), stored like NF4 with
// a float32 absmax per block (single quantisation, 4 + 32/64 = 4.5 bits per
// weight, §5-2 "メモリ削減の計算").  INT4 has no zero level: a zero weight
// ties between ±1/15 and takes the lower index, 7, which is also the index of
// an all-zero block.
//
// These kernels are HBM-bound: 4 B read + 0.5 B written per weight for the
// quantiser, 0.52 B read + 2 B written per weight for the dequantiser.

#include "qlora_kernels.h"
#include "qlora_merge.h"
#include "qlora_quant_variants.h"
#include "qlora_reduce.h"

namespace qlora {

namespace {

// RN32((2k − 15)/15), k = 0..15: the uniform INT4 levels, ascending.
constexpr uint32_t kINT4Bits[16] = {
    0xbf800000u, 0xbf5ddddeu, 0xbf3bbbbcu, 0xbf19999au, 0xbeeeeeefu, 0xbeaaaaabu,
    0xbe4ccccdu, 0xbd888889u, 0x3d888889u, 0x3e4ccccdu, 0x3eaaaaabu, 0x3eeeeeefu,
    0x3f19999au, 0x3f3bbbbcu, 0x3f5ddddeu, 0x3f800000u,
};

template <int CODE>
struct Code;
template <>
struct Code<kCodeNF4> {
  static constexpr const uint32_t* bits = kNF4Bits;
  static constexpr uint32_t zero_word = 0x88888888u;  // eight codes of the zero level
};
template <>
struct Code<kCodeINT4> {
  static constexpr const uint32_t* bits = kINT4Bits;
  static constexpr uint32_t zero_word = 0x77777777u;  // eight codes 7 (a zero weight's code)
};

struct Midpoints {
  double m[15];
};

constexpr Midpoints make_midpoints(const uint32_t* bits) {
  Midpoints r{};
  for (int i = 0; i < 15; ++i)
    r.m[i] = ((double)__builtin_bit_cast(float, bits[i]) +
              (double)__builtin_bit_cast(float, bits[i + 1])) * 0.5;
  return r;
}

template <int CODE>
constexpr Midpoints kMid = make_midpoints(Code<CODE>::bits);

// RD32(m * a): the largest float32 not above the exact product.
__device__ inline float rd32_mul(double m, float a) {
  const double p = m * (double)a;  // exact: m has <= 29 significant bits, a 24
  float f = (float)p;              // round to nearest
  if ((double)f > p) {
    uint32_t b = float_to_bits(f);
    if (f > 0.0f)
      b -= 1u;                                          // toward zero
    else
      b = ((b & 0x7fffffffu) == 0u) ? 0x80000001u : b + 1u;  // away from zero (negative side)
    f = bits_to_float(b);
  }
  return f;
}

// Second-level code: integer in [0, 127] nearest to a / step, tie to the lower.
__device__ inline int dq_code(float a, float step) {
  if (!(step > 0.0f)) return 0;
  const double s = (double)step, ad = (double)a;
  int q = (int)rint(ad / s);
  q = q < 0 ? 0 : (q > 127 ? 127 : q);
  // (q ± 1/2) · s is exact in float64; one step each way fixes any rounding of ad / s.
  if (q < 127 && ad > ((double)q + 0.5) * s) ++q;
  if (q > 0 && ad <= ((double)q - 0.5) * s) --q;
  return q;
}

__device__ inline float dq_step(float gmax) {
  // IEEE float32 division max / 127, via float64 (double rounding is harmless
  // for a quotient of two float32 numbers).
  return (float)((double)gmax / 127.0);
}

// Bucket table for the exact decision.  With x = w / a in [-1, 1], bucket
// j = floor((x + 1) · 32) spans [j/32 − 1, (j+1)/32 − 1); j = 64 is x = 1 (the
// estimate never leaves [0, 64], so no clamp is needed).
// kBucketMargin exceeds the error of the float32 quotient w · RN(1/a) by orders
// of magnitude and, because consecutive midpoints are more than 0.088 apart
// (NF4; 2/15 for INT4),
// a bucket widened by the margin on both sides still holds at most one
// midpoint.  first[j] = #{i : m_i < j/32 − 1 − margin}: the exact index is
// first[j] or first[j] + 1, decided by one exact compare w > T_first[j].
constexpr double kBucketMargin = 1.0 / 1024.0;

constexpr int kNBuckets = 65;

struct BucketTable {
  uint8_t first[kNBuckets];
};

constexpr BucketTable make_buckets(const Midpoints& mid) {
  BucketTable t{};
  for (int j = 0; j < kNBuckets; ++j) {
    const double lo = j / 32.0 - 1.0 - kBucketMargin;
    int c = 0;
    for (int i = 0; i < 15; ++i) c += (mid.m[i] < lo) ? 1 : 0;
    t.first[j] = (uint8_t)c;
  }
  return t;
}

template <int CODE>
constexpr BucketTable kBuckets = make_buckets(kMid<CODE>);

constexpr int kTStride = 17;  // floats per block in the LDS threshold table (bank spread)

// Power of two that brings a block maximum m > 0 into [2^-64, 2^64] for the
// bucket estimate: 1/(m·sc) is then a normal float32.  x·sc is exact for
// normal results; a value that underflows in it is below 2^-85 of m and lands
// in the zero bucket either way.
__device__ inline float estimate_scale(float m) {
  return (m < 0x1p-64f) ? 0x1p64f : ((m > 0x1p64f) ? 0x1p-64f : 1.0f);
}

// 1 when any of the values is NaN or ±Inf (the precondition is finite input).
__device__ inline bool any_nonfinite4(const floatx4& x) {
  bool bad = false;
#pragma unroll
  for (int u = 0; u < 4; ++u) bad |= !__builtin_isfinite(x[u]);
  return bad;
}

// Flags non-finite input: every lane that saw one stores 1 (a vector store;
// the flag is never cleared here, the caller zeroes it beforehand).
__device__ inline void flag_nonfinite(int32_t* flag, bool bad) {
  if (flag != nullptr && bad) *reinterpret_cast<volatile int32_t*>(flag) = 1;
}

// One lane handles 16 consecutive elements; 4 lanes form one 64-block.
// T: this block's 16-entry threshold row in LDS (T[15] = +inf); bk: bucket table.
// Block absmax (over the block's 4 lanes) and the codes of 16 loaded values.
template <int CODE>
__device__ inline float quantize_16v(const float (&v)[16], int sub, float* __restrict__ T,
                                     const uint8_t* __restrict__ bk, u32x2& out_bytes) {
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(v[j]));
  m = fmaxf(m, __shfl_xor(m, 1));
  m = fmaxf(m, __shfl_xor(m, 2));

  // the 4 lanes of the block write its 15 thresholds (+ the +inf sentinel)
#pragma unroll
  for (int i = sub; i < 16; i += 4) T[i] = (i < 15) ? rd32_mul(kMid<CODE>.m[i], m) : __builtin_inff();
  // the block's 4 lanes share one wave, whose LDS accesses complete in order;
  // the barrier only keeps the compiler from moving the reads above the writes
  __builtin_amdgcn_wave_barrier();

  uint32_t lo = Code<CODE>::zero_word, hi = Code<CODE>::zero_word;  // all-zero block
  if (m > 0.0f) {
    // the estimate only picks a bucket; a power-of-two rescale keeps 1/m a
    // normal float32 for subnormal and for huge block maxima (v_rcp_f32
    // returns no subnormal results) without changing any ratio
    const float sc = estimate_scale(m);
    // 32 / (m·sc) to within a couple of ulp (v_rcp: the estimate only picks a
    // bucket): b = trunc(32 x + 32) in one fma, and |x| <= 1 + 2^-21 keeps b
    // in [0, 64]
    const float k32 = 32.0f * __builtin_amdgcn_rcpf(m * sc);
    lo = 0u;
    hi = 0u;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int b = (int)__builtin_fmaf(v[j] * sc, k32, 32.0f);
      const int k0 = bk[b];
      const uint32_t idx = (uint32_t)k0 + ((v[j] > T[k0]) ? 1u : 0u);
      if (j < 8)
        lo |= idx << (4 * j);
      else
        hi |= idx << (4 * (j - 8));
    }
  }
  out_bytes = u32x2{lo, hi};
  return m;
}

// The 16 values of lane `sub` of block blk (zero past n).
__device__ inline void load_16(const float* __restrict__ w, int64_t n, int64_t blk, int sub,
                               float (&v)[16]) {
  const int64_t base = blk * kBlock + (int64_t)sub * 16;
  if (base + 16 <= n) {
    const floatx4* p = reinterpret_cast<const floatx4*>(w + base);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // plain loads: the four lanes of a block read the same cache lines in
      // four instructions, which only cached loads serve from one fetch
      const floatx4 x = p[j];
      v[4 * j + 0] = x[0];
      v[4 * j + 1] = x[1];
      v[4 * j + 2] = x[2];
      v[4 * j + 3] = x[3];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = (base + j < n) ? w[base + j] : 0.0f;
  }
}

// The 16 values of lane `sub` of block blk from a bf16 input (exact in float32).
__device__ inline void load_16(const uint16_t* __restrict__ w, int64_t n, int64_t blk, int sub,
                               float (&v)[16]) {
  const int64_t base = blk * kBlock + (int64_t)sub * 16;
  if (base + 16 <= n) {
    const u32x4* p = reinterpret_cast<const u32x4*>(w + base);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const u32x4 x = p[j];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        v[8 * j + 2 * d] = bits_to_float(x[d] << 16);
        v[8 * j + 2 * d + 1] = bits_to_float(x[d] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = (base + j < n) ? bits_to_float((uint32_t)w[base + j] << 16) : 0.0f;
  }
}

// packed[nblocks*32], absmax[nblocks]; 64 blocks per 256-thread workgroup,
// workgroup wg taking blocks 64 wg .. 64 wg + 63.  The workgroup's 4096
// elements come in as 4 loads per lane, load j of lane t being the float4 at
// element 4 (256 j + t): every load is contiguous across the wave, and 16
// consecutive lanes hold one block.  Lane i of a block computes threshold i
// (T_15 = +inf) and each value reads the one it needs from that lane.
template <int CODE>
__device__ inline void quantize_blocks(const float* __restrict__ w, int64_t n, int64_t nblocks,
                                       uint8_t* __restrict__ packed, float* __restrict__ absmax,
                                       int64_t wg, int32_t* __restrict__ nonfinite) {
  __shared__ uint8_t bk[kNBuckets];
  const int t = threadIdx.x;
  if (t < kNBuckets) bk[t] = kBuckets<CODE>.first[t];
  __syncthreads();
  const int64_t e0 = wg * 4096;
  floatx4 x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t e = e0 + 4 * (256 * j + t);
    if (e + 4 <= n) {
      x[j] = *reinterpret_cast<const floatx4*>(w + e);
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) x[j][u] = (e + u < n) ? w[e + u] : 0.0f;
    }
  }
  if (nonfinite != nullptr) {
    bool bad = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) bad |= any_nonfinite4(x[j]);
    flag_nonfinite(nonfinite, bad);
  }
  const int lb = t & 15;                     // lane within its block
  const int src0 = t & 48;                   // the block's first lane within the wave
  const double mid = lb < 15 ? kMid<CODE>.m[lb] : 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t blk = (e0 >> 6) + 16 * j + (t >> 4);
    float m = fmaxf(fmaxf(fabsf(x[j][0]), fabsf(x[j][1])), fmaxf(fabsf(x[j][2]), fabsf(x[j][3])));
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));
    m = fmaxf(m, __shfl_xor(m, 8));
    const float thr = lb < 15 ? rd32_mul(mid, m) : __builtin_inff();
    // the estimate only picks a bucket; a power-of-two rescale keeps 1/m finite
    // for subnormal block maxima without changing any ratio.  32 / (m·sc) to
    // within a couple of ulp: b = trunc(32 x + 32) in one fma, and
    // |x| <= 1 + 2^-21 keeps b in [0, 64] (an all-zero block uses bucket 32
    // and its codes are replaced below)
    const bool nz = m > 0.0f;
    const float sc = estimate_scale(m);
    const float k32 = nz ? 32.0f * __builtin_amdgcn_rcpf(m * sc) : 0.0f;
    uint32_t code = 0u;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int bkt = (int)__builtin_fmaf(x[j][u] * sc, k32, 32.0f);
      const int k0 = bk[bkt];
      const float tk = __shfl(thr, src0 | k0);
      code |= ((uint32_t)k0 + ((x[j][u] > tk) ? 1u : 0u)) << (4 * u);
    }
    if (!nz) code = Code<CODE>::zero_word & 0xffffu;
    if (blk < nblocks) {
      *reinterpret_cast<uint16_t*>(packed + blk * 32 + lb * 2) = (uint16_t)code;
      if (lb == 0) absmax[blk] = m;
    }
  }
}

}  // namespace

__global__ __launch_bounds__(256) void quantize_nf4_kernel(const float* __restrict__ w, int64_t n,
                                                           int64_t nblocks,
                                                           uint8_t* __restrict__ packed,
                                                           float* __restrict__ absmax,
                                                           int32_t* __restrict__ nonfinite) {
  quantize_blocks<kCodeNF4>(w, n, nblocks, packed, absmax, blockIdx.x, nonfinite);
}

__global__ __launch_bounds__(256) void quantize_int4_kernel(const float* __restrict__ w, int64_t n,
                                                            int64_t nblocks,
                                                            uint8_t* __restrict__ packed,
                                                            float* __restrict__ absmax) {
  quantize_blocks<kCodeINT4>(w, n, nblocks, packed, absmax, blockIdx.x, nullptr);
}

namespace {

// The second level of DQ group g (256 blocks) by one 256-thread workgroup.
__device__ inline void double_quant_group(const float* __restrict__ absmax, int64_t nblocks,
                                          int8_t* __restrict__ qabsmax, float* __restrict__ c2,
                                          int64_t g) {
  __shared__ float red[4];
  const int t = threadIdx.x;
  const int64_t b = g * kGroup + t;
  const float a = (b < nblocks) ? absmax[b] : 0.0f;
  float m = a;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float step = dq_step(m);
  if (t == 0) c2[g] = step;
  if (b < nblocks) qabsmax[b] = (int8_t)dq_code(a, step);
}

// The job of workgroup `wg` in a batch: the last job whose first workgroup is
// at or before it (jobs without workgroups are never picked: a later job
// starts at the same workgroup).  Uniform, so the descriptor stays scalar.
__device__ inline int batch_job(const int64_t* wg0, int count, int64_t wg) {
  int lo = 0, hi = count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (wg0[mid] <= wg)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

}  // namespace

// One workgroup per group of 256 blocks.
__global__ __launch_bounds__(256) void double_quant_kernel(const float* __restrict__ absmax,
                                                           int64_t nblocks,
                                                           int8_t* __restrict__ qabsmax,
                                                           float* __restrict__ c2) {
  double_quant_group(absmax, nblocks, qabsmax, c2, blockIdx.x);
}

__global__ __launch_bounds__(256) void quantize_nf4_batch_kernel(QuantBatch b) {
  const int i = batch_job(b.wg0, b.count, blockIdx.x);
  const QuantJob1& J = b.j[i];
  quantize_blocks<kCodeNF4>(J.w, J.n, (J.n + kBlock - 1) / kBlock, J.packed, J.absmax,
                            blockIdx.x - b.wg0[i], J.nonfinite);
}

__global__ __launch_bounds__(256) void double_quant_batch_kernel(DqBatch b) {
  const int i = batch_job(b.wg0, b.count, blockIdx.x);
  const DqJob& J = b.j[i];
  double_quant_group(J.absmax, J.nblocks, J.qabsmax, J.c2, blockIdx.x - b.wg0[i]);
}

// Fused: one workgroup per DQ group (256 blocks = 16384 elements), four passes
// of 64 blocks, then the second level from the absmax values kept in LDS.
namespace {

template <typename In>
__device__ inline void quantize_dq_groups(const In* __restrict__ w, int64_t n, int64_t nblocks,
                                          uint8_t* __restrict__ packed,
                                          int8_t* __restrict__ qabsmax, float* __restrict__ c2,
                                          float* __restrict__ absmax_out,
                                          int32_t* __restrict__ nonfinite) {
  __shared__ float amax[kGroup];
  __shared__ float red[4];
  __shared__ float thr[64 * kTStride];
  __shared__ uint8_t bk[kNBuckets];
  const int t = threadIdx.x;
  if (t < kNBuckets) bk[t] = kBuckets<kCodeNF4>.first[t];
  __syncthreads();
  const int sub = t & 3;
  const int64_t ngroups = (nblocks + kGroup - 1) / kGroup;
  // Workgroups stride over the groups; each group is four passes of 64
  // blocks, and the next pass (of this group or the next one) is always in
  // flight while the current one is quantized.
  auto blk_of = [&](int64_t g, int pass) { return g * kGroup + pass * 64 + (t >> 2); };
  float vA[16], vB[16];
  int64_t g = blockIdx.x;
  if (g < ngroups && blk_of(g, 0) < nblocks) load_16(w, n, blk_of(g, 0), sub, vA);
  for (; g < ngroups; g += gridDim.x) {
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      float(&cur)[16] = (pass & 1) ? vB : vA;
      float(&nxt)[16] = (pass & 1) ? vA : vB;
      const int64_t gn = pass < 3 ? g : g + gridDim.x;
      const int64_t bn = blk_of(gn, (pass + 1) & 3);
      if (gn < ngroups && bn < nblocks) load_16(w, n, bn, sub, nxt);
      const int lb = pass * 64 + (t >> 2);
      const int64_t blk = g * kGroup + lb;
      float m = 0.0f;
      if (blk < nblocks) {
        if (nonfinite != nullptr) {  // (registers of blocks past the end were never loaded)
          bool bad = false;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            bad |= any_nonfinite4(floatx4{cur[4 * j], cur[4 * j + 1], cur[4 * j + 2], cur[4 * j + 3]});
          flag_nonfinite(nonfinite, bad);
        }
        u32x2 bytes;
        m = quantize_16v<kCodeNF4>(cur, sub, thr + (t >> 2) * kTStride, bk, bytes);
        *reinterpret_cast<u32x2*>(packed + blk * 32 + sub * 8) = bytes;
      }
      if (sub == 0) amax[lb] = m;
    }
    __syncthreads();
    const int64_t b = g * kGroup + t;
    const float a = amax[t];
    float m = a;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float step = dq_step(m);
    if (t == 0) c2[g] = step;
    if (b < nblocks) {
      qabsmax[b] = (int8_t)dq_code(a, step);
      if (absmax_out) absmax_out[b] = a;
    }
    __syncthreads();  // amax and red are rewritten by the next group
  }
}

}  // namespace

__global__ __launch_bounds__(256) void quantize_nf4_dq_kernel(const float* __restrict__ w, int64_t n,
                                                              int64_t nblocks,
                                                              uint8_t* __restrict__ packed,
                                                              int8_t* __restrict__ qabsmax,
                                                              float* __restrict__ c2,
                                                              float* __restrict__ absmax_out,
                                                              int32_t* __restrict__ nonfinite) {
  quantize_dq_groups(w, n, nblocks, packed, qabsmax, c2, absmax_out, nonfinite);
}

// The same from a bf16 weight (the merged 16-bit weight of an adapter merge).
__global__ __launch_bounds__(256) void quantize_nf4_dq_bf16_kernel(const uint16_t* __restrict__ w,
                                                                   int64_t n, int64_t nblocks,
                                                                   uint8_t* __restrict__ packed,
                                                                   int8_t* __restrict__ qabsmax,
                                                                   float* __restrict__ c2) {
  quantize_dq_groups(w, n, nblocks, packed, qabsmax, c2, static_cast<float*>(nullptr),
                     static_cast<int32_t*>(nullptr));
}

// Standalone dequantisation to bf16.  A workgroup decodes 1024 consecutive
// packed dwords (8192 weights); lane t takes dwords t, t + 256, t + 512,
// t + 768, so every load (4 B per lane) and every store (16 B per lane) is
// contiguous across the wave.  n is a multiple of 64.
namespace {

__device__ inline void dequant_chunk(const uint32_t* __restrict__ packed,
                                     const int8_t* __restrict__ qabsmax,
                                     const float* __restrict__ c2, int64_t ndwords,
                                     u32x4* __restrict__ out, int64_t base, const float* cb) {
  uint32_t p[4];
  float ah[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t i = base + threadIdx.x + 256 * u;
    p[u] = (i < ndwords) ? packed[i] : 0u;
    const int64_t b = (i < ndwords ? i : 0) >> 3;  // 8 dwords per 64-block
    ah[u] = c2[b >> 8] * (float)qabsmax[b];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t i = base + threadIdx.x + 256 * u;
    u32x4 o;
    o = decode8(p[u], ah[u], cb);
    if (i < ndwords) out[i] = o;
  }
}

}  // namespace

__global__ __launch_bounds__(256) void dequantize_nf4_kernel(const uint32_t* __restrict__ packed,
                                                             const int8_t* __restrict__ qabsmax,
                                                             const float* __restrict__ c2,
                                                             int64_t ndwords,
                                                             u32x4* __restrict__ out) {
  __shared__ float cb[16];
  if (threadIdx.x < 16) cb[threadIdx.x] = bits_to_float(kNF4Bits[threadIdx.x]);
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * 1024;
  for (int64_t base = (int64_t)blockIdx.x * 1024; base < ndwords; base += stride)
    dequant_chunk(packed, qabsmax, c2, ndwords, out, base, cb);
}

// A list of weights in one launch: workgroup wg decodes dwords 1024 (wg − first
// workgroup of its job) onward of its job.
__global__ __launch_bounds__(256) void dequantize_nf4_batch_kernel(DeqBatch b) {
  __shared__ float cb[16];
  if (threadIdx.x < 16) cb[threadIdx.x] = bits_to_float(kNF4Bits[threadIdx.x]);
  __syncthreads();
  const int i = batch_job(b.wg0, b.count, blockIdx.x);
  const DeqJob& J = b.j[i];
  dequant_chunk(J.packed, J.qabsmax, J.c2, J.ndwords, J.out, (blockIdx.x - b.wg0[i]) * 1024, cb);
}

// Single-quantisation decode of n weights (any n): ŵ = RNE_bf16(RN32(level · a)).
// Lane layout as in dequantize_nf4_kernel; the last dword may be partial.
template <int CODE>
__global__ __launch_bounds__(256) void dequantize_4bit_kernel(const uint32_t* __restrict__ packed,
                                                              const float* __restrict__ absmax,
                                                              int64_t n,
                                                              uint16_t* __restrict__ out) {
  __shared__ float cb[16];
  if (threadIdx.x < 16) cb[threadIdx.x] = bits_to_float(Code<CODE>::bits[threadIdx.x]);
  __syncthreads();
  const int64_t ndw = (n + 7) >> 3;
  const int64_t stride = (int64_t)gridDim.x * 1024;
  for (int64_t base = (int64_t)blockIdx.x * 1024; base < ndw; base += stride) {
    uint32_t p[4];
    float a[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = base + threadIdx.x + 256 * u;
      p[u] = (i < ndw) ? packed[i] : 0u;
      a[u] = (i < ndw) ? absmax[i >> 3] : 0.0f;  // 8 dwords per 64-block
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = base + threadIdx.x + 256 * u;
      if (i >= ndw) continue;
      const u32x4 o = decode8(p[u], a[u], cb);
      if (8 * i + 8 <= n) {
        *reinterpret_cast<u32x4*>(out + 8 * i) = o;
      } else {
        for (int e = 0; 8 * i + e < n; ++e) out[8 * i + e] = (uint16_t)(o[e >> 1] >> (16 * (e & 1)));
      }
    }
  }
}

// Partial sums of (w − RN32(level_idx · a))², float64, one per workgroup.
// Lane t takes dwords (8 weights) base + t + 256u, u = 0..3, like the decoder.
template <int CODE>
__global__ __launch_bounds__(256) void quant_sq_error_kernel(const float* __restrict__ w, int64_t n,
                                                             const uint32_t* __restrict__ packed,
                                                             const float* __restrict__ absmax,
                                                             double* __restrict__ partials) {
  __shared__ float cb[16];
  __shared__ double sh[256];
  if (threadIdx.x < 16) cb[threadIdx.x] = bits_to_float(Code<CODE>::bits[threadIdx.x]);
  __syncthreads();
  const int64_t ndw = (n + 7) >> 3;
  const int64_t stride = (int64_t)gridDim.x * 1024;
  double acc = 0.0;
  for (int64_t base = (int64_t)blockIdx.x * 1024; base < ndw; base += stride) {
    uint32_t p[4];
    float a[4];
    floatx4 x[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = base + threadIdx.x + 256 * u;
      const bool full = 8 * i + 8 <= n;
      p[u] = (i < ndw) ? packed[i] : 0u;
      a[u] = (i < ndw) ? absmax[i >> 3] : 0.0f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (full) {
          x[u][h] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(w + 8 * i + 4 * h));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t j = 8 * i + 4 * h + e;
            x[u][h][e] = (i < ndw && j < n) ? w[j] : 0.0f;
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = base + threadIdx.x + 256 * u;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float r = cb[(p[u] >> (4 * e)) & 15u] * a[u];
        const double d = (double)x[u][e >> 2][e & 3] - (double)r;
        if (i < ndw && 8 * i + e < n) acc += d * d;
      }
    }
  }
  const double s = block_sum_f64<256>(acc, sh);
  if (threadIdx.x == 0) partials[blockIdx.x] = s;
}

__global__ __launch_bounds__(256) void sum_partials_kernel(const double* __restrict__ partials,
                                                           int32_t npart, double* __restrict__ out) {
  __shared__ double sh[256];
  const double s = workgroup_sum_f64<256>(partials, npart, sh);
  if (threadIdx.x == 0) *out = s;
}

template __global__ void dequantize_4bit_kernel<kCodeNF4>(const uint32_t*, const float*, int64_t,
                                                          uint16_t*);
template __global__ void dequantize_4bit_kernel<kCodeINT4>(const uint32_t*, const float*, int64_t,
                                                           uint16_t*);
template __global__ void quant_sq_error_kernel<kCodeNF4>(const float*, int64_t, const uint32_t*,
                                                         const float*, double*);
template __global__ void quant_sq_error_kernel<kCodeINT4>(const float*, int64_t, const uint32_t*,
                                                          const float*, double*);

}  // namespace qlora
