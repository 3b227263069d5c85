// Shared device definitions for the gfx950 QLoRA NF4 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qlora.h"

namespace qlora {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = QLORA_BLOCKSIZE;  // NF4 block, elements along k_in
constexpr int kGroup = QLORA_DQ_GROUP;   // DQ group, blocks
constexpr int kZeroIndex = 8;            // index of the exact-zero level

// The 16 NF4 levels as float32 bit patterns, ascending.  They are the
// float32 roundings of Φ⁻¹(k/18), k = 1..8, 0, Φ⁻¹(1/2 + j/16), j = 1..7,
// divided by |Φ⁻¹(1/18)| ("QLoRAの理論と実装", §5-1 NF4, the page's
// educational codebook construction).
constexpr uint32_t kNF4Bits[16] = {
    0xbf800000u, 0xbf44223bu, 0xbf1b723fu, 0xbef5bfa7u, 0xbebd6dbfu, 0xbe8a6b5du,
    0xbe356319u, 0xbdb39720u, 0x00000000u, 0x3dca36f7u, 0x3e4ccc13u, 0x3e9d12fdu,
    0x3ed8c161u, 0x3f0e8c30u, 0x3f38d6dcu, 0x3f768108u,
};

__host__ __device__ inline float bits_to_float(uint32_t b) { return __builtin_bit_cast(float, b); }
__host__ __device__ inline uint32_t float_to_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32;
// `lo` lands in the low half.
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{lo, hi}, bf16x2));
}

// Decode 8 NF4 codes (one packed dword, element 2t in the low nibble of byte t)
// with block scale ah into 4 dwords of bf16 pairs: RNE_bf16(RN32(c[idx] * ah)).
// cb is the 16-entry float codebook in LDS; the nibbles are spread to byte
// offsets (4 * idx) once per dword so that each lookup costs one extract.
__device__ inline u32x4 decode8(uint32_t p, float ah, const float* cb) {
  const uint32_t ev = (p << 2) & 0x3c3c3c3cu;  // 4 * idx of elements 0, 2, 4, 6
  const uint32_t od = (p >> 2) & 0x3c3c3c3cu;  // 4 * idx of elements 1, 3, 5, 7
  const char* base = reinterpret_cast<const char*>(cb);
  u32x4 o;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float lo = *reinterpret_cast<const float*>(base + ((ev >> (8 * d)) & 0xffu)) * ah;
    const float hi = *reinterpret_cast<const float*>(base + ((od >> (8 * d)) & 0xffu)) * ah;
    o[d] = pack_bf16x2(lo, hi);
  }
  return o;
}

__device__ inline float bf16_bits_to_float(uint32_t b16) { return bits_to_float(b16 << 16); }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace qlora
