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

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = static_cast<__bf16>(lo);
  __bf16 b = static_cast<__bf16>(hi);
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ inline float bf16_bits_to_float(uint32_t b16) { return bits_to_float(b16 << 16); }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace qlora
