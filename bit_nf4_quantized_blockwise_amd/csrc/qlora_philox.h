// Philox4x64-10 counter-based generator (Salmon, Moraes, Dror, Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", SC 2011) and the LoRA dropout mask
// built on it.  The mask of the element at flat index f of X [tokens][k_in]
// is a pure function of (seed, offset, f): block (f >> 3) of the generator
// under key (seed, 0) and counter (f >> 3, offset, 0, 0) gives eight 32-bit
// values, the element takes value f & 7 (word (f & 7) >> 1, low half for even
// f) and is dropped when that value is below thr = floor(p · 2^32).
#pragma once

#include "qlora_common.h"

namespace qlora {

struct Philox4 {
  uint64_t w[4];
};

__device__ inline Philox4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
  uint64_t c2 = 0, c3 = 0;
#pragma unroll 1
  for (int r = 0; r < 10; ++r) {
    const uint64_t h0 = __umul64hi(M0, c0), l0 = M0 * c0;
    const uint64_t h1 = __umul64hi(M1, c2), l1 = M1 * c2;
    const uint64_t n0 = h1 ^ c1 ^ k0, n2 = h0 ^ c3 ^ k1;
    c0 = n0;
    c1 = l1;
    c2 = n2;
    c3 = l0;
    k0 += W0;
    k1 += W1;
  }
  return Philox4{{c0, c1, c2, c3}};
}

struct DropoutKey {
  uint64_t seed, offset;
  uint32_t thr;  // drop when the element's value is below thr
};

// Keep bits of the 8 elements of block g (bit e = element 8 g + e kept).
__device__ inline uint32_t keep_bits8(const DropoutKey& d, uint64_t g) {
  const Philox4 r = philox4x64_10(g, d.offset, d.seed, 0);
  uint32_t bits = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint64_t w = r.w[e >> 1];
    const uint32_t v = (e & 1) ? (uint32_t)(w >> 32) : (uint32_t)w;
    bits |= (v >= d.thr ? 1u : 0u) << e;
  }
  return bits;
}

}  // namespace qlora
