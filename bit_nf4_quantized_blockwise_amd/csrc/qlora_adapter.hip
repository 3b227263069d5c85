// The rank-r products of the QLoRA linear as streaming kernels for gfx950.
//
//   rows:  P[s][m][j] = Σ_{k in split s} S[m][k] · F(k, j)    U = X·Aᵀ (F = A, [r][k])
//                                                              V = dY·B (F = B, [k][r])
//   cols:  P[s][l][j] = Σ_{m in split s} S[m][l] · Q[m][j]    dA = s·Vᵀ·X, dB = s·dYᵀ·U
//
// ("QLoRAの理論と実装", 逆伝播と勾配の流れ: the gradients ∂L/∂A and ∂L/∂B; the
// forward's rank-r path U = X·Aᵀ.)  S is the big operand (the tokens X or the
// output gradient dY, read once from HBM); F and Q are the small adapter
// factors (L2-resident).  The partial sums of the splits are reduced in a fixed
// order by the reduction kernel.
//
// Each workgroup (4 waves) owns 128 indices of S's non-reduced side and one
// group of up to 128 ranks, and walks its share of the reduction in stages of
// 64.  Stages travel by direct-to-LDS buffer loads through a ring of kRing
// slots, so all but one stage (≈ 48-80 KB per CU) are in flight while one is
// multiplied: the products are bound by HBM, and what they need from the
// memory system is enough bytes in flight, not registers or issue slots.
// Tiles whose reduction runs along their rows (S in `rows`, and A) sit in LDS
// as 128-byte rows read with ds_read_b128; tiles whose reduction runs down
// their columns (B, and both operands of `cols`) sit in their own row-major
// layout and are read with gfx950's transposing LDS load ds_read_b64_tr_b16.
// Both give the MFMA operand layout of v_mfma_f32_32x32x16_bf16 with the
// reduction order k = 32 (lane / 32) + 8 ks + e within a stage.

#include <type_traits>

#include "qlora_kernels.h"

namespace qlora {

namespace {

// ring slots (stages): six while a stage is 20-24 KB, four at 32 KB (128
// ranks); one workgroup per CU (shallower rings with two or three workgroups
// per CU, and so more splits, were slower)
template <int NB>
constexpr int ring_of() { return NB == 4 ? 4 : 6; }
// One stage: 16 KB of the streamed operand (128 rows x 64 k, or 64 tokens x
// 128 columns) and 4 KB per block of 32 ranks of the factor.
template <int NB>
constexpr int stage_bytes() { return 16384 + NB * 4096; }
constexpr int kOOBA = 0x7ffffff0;        // a buffer offset past every range: loads return 0
constexpr int kRsrcWord3A = 0x00020000;  // raw buffer, 32-bit data format

typedef short s4v __attribute__((ext_vector_type(4)));

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffffLL : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kRsrcWord3A);
}

__device__ inline void dma16(__amdgpu_buffer_rsrc_t r, char* lds, int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           off, 0, 0, 0);
}

// s_waitcnt vmcnt(n) with expcnt and lgkmcnt left alone (gfx9 encoding).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

// Workgroup barrier for the ring: each wave first waits for its own
// direct-to-LDS loads of the stage (an explicit vmcnt), so the barrier itself
// must not wait for the later stages still in flight, as the release fence of
// __syncthreads() would.  The empty asm statements keep the compiler from
// moving LDS accesses across it.
__device__ inline void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Calls f(integral_constant<int, P>) for P = 0 .. N - 1 (ring slots as
// compile-time constants, so that the compiler can tell the slot being
// loaded from the slot being read and adds no wait between them).
template <int P, int N, class F>
__device__ inline void static_for(F&& f) {
  if constexpr (P < N) {
    f(std::integral_constant<int, P>{});
    static_for<P + 1, N>(f);
  }
}

// 128-byte rows (64 reduction values): chunk c of row n at c ^ (n mod 8) ^ ((n / 8) mod 8).
__device__ inline int swz128(int n, int c) { return n * 128 + ((c ^ (n & 7) ^ ((n >> 3) & 7)) << 4); }

// Row-major tile of 64 rows x C 16-byte chunks: chunk c of row n at c ^ 2 (n mod 4)
// when C >= 8 (the four rows of one transposing read then fall on distinct banks).
template <int C>
__device__ inline int swz_rm(int n, int c) {
  return n * (16 * C) + ((C >= 8 ? (c ^ ((n & 3) << 1)) : c) << 4);
}

// One wave's direct-to-LDS loads of a 128-byte-row tile: load j covers rows
// 8j .. 8j + 7 (lane l: row 8j + l / 8, LDS chunk l mod 8, which holds logical
// chunk (l mod 8) ^ (l / 8) ^ (j mod 8)).  Reduction values at or past kend
// read as zero; rows past the buffer too.
__device__ inline void load_rows128(__amdgpu_buffer_rsrc_t r, int64_t ld, char* dst, int j,
                                    int64_t k0, int64_t kend, int lane) {
  const int c = (lane & 7) ^ (lane >> 3) ^ (j & 7);
  const bool ok = k0 + 8 * c < kend;
  const int off = (8 * j + (lane >> 3)) * (int)ld * 2 + (int)k0 * 2 + 16 * c;
  dma16(r, dst + j * 1024, ok ? off : kOOBA);
}

// One wave's direct-to-LDS load j of a row-major tile of 64 rows x C chunks
// (rows r0 + 1024 j / (16 C) ..): rows at or past rend read as zero.
template <int C>
__device__ inline void load_rm(__amdgpu_buffer_rsrc_t r, int64_t ld, char* dst, int j, int64_t r0,
                               int64_t rend, int lane) {
  constexpr int RPL = 64 / C;  // rows per 1 KB load
  const int n = RPL * j + lane / C;
  const int pc = lane % C;
  const int c = C >= 8 ? (pc ^ ((n & 3) << 1)) : pc;
  const bool ok = r0 + n < rend;
  const int off = (int)(r0 + n) * (int)ld * 2 + 16 * c;
  dma16(r, dst + j * 1024, ok ? off : kOOBA);
}

// MFMA operand from a 128-byte-row tile: row `row0 + lane mod 32`, reduction
// values 32 (lane / 32) + 8 ks .. + 7.
__device__ inline bf16x8 frag128(const char* t, int row0, int lane, int ks) {
  return *reinterpret_cast<const bf16x8*>(t + swz128(row0 + (lane & 31), 4 * (lane >> 5) + ks));
}

// The four MFMA operands (ks = 0..3) of one 32-column block of a row-major
// tile, through ds_read_b64_tr_b16: column `col0 + lane mod 32`, rows
// 32 (lane / 32) + 8 ks .. + 7 in f[ks].  In each group of 16 lanes the
// instruction hands lane 4a + b element b of the 8-byte pieces fetched by
// lanes a, a + 4, a + 8, a + 12; lane q of a group therefore fetches row
// q / 4 (+ 4 for the second read of a pair), columns 4 (q mod 4) .. + 3 of the
// group's 16 columns.
//
// The eight reads and the wait for them are one asm statement: the compiler
// knows of no alias information for the transposing-read builtin and would
// wait for every direct-to-LDS load still in flight (the whole ring) before
// it.  Waiting inside the statement keeps every output register valid when
// the statement ends, and the early-clobber outputs never share a register
// with the address while reads are in flight.
template <int C>
__device__ inline void frags_tr(const char* t, int col0, int lane, bf16x8 (&f)[4]) {
  constexpr int ROW = 16 * C;  // bytes per tile row
  const int q = lane & 15, g = (lane >> 4) & 1;
  const int n = 32 * (lane >> 5) + (q >> 2);  // row at ks = 0 (+ 8 ks, + 4 keep n mod 4)
  const int col = col0 + 16 * g + 4 * (q & 3);
  const uint32_t addr = (uint32_t)(uintptr_t)(
      (__attribute__((address_space(3))) const char*)(t + swz_rm<C>(n, col >> 3) + 2 * (col & 7)));
  s4v r0, r1, r2, r3, r4, r5, r6, r7;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%9\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:%10\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:%11\n\t"
      "ds_read_b64_tr_b16 %3, %8 offset:%12\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:%13\n\t"
      "ds_read_b64_tr_b16 %5, %8 offset:%14\n\t"
      "ds_read_b64_tr_b16 %6, %8 offset:%15\n\t"
      "ds_read_b64_tr_b16 %7, %8 offset:%16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
      : "v"(addr), "i"(0), "i"(4 * ROW), "i"(8 * ROW), "i"(12 * ROW), "i"(16 * ROW),
        "i"(20 * ROW), "i"(24 * ROW), "i"(28 * ROW)
      : "memory");
  f[0] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
  f[1] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r2, r3, 0, 1, 2, 3, 4, 5, 6, 7));
  f[2] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r4, r5, 0, 1, 2, 3, 4, 5, 6, 7));
  f[3] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r6, r7, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Workgroup b of a job of `total` runs on XCD (b + base) mod 8.  Deal each
// XCD a contiguous run of the job's (tile, split) order, so that the
// workgroups sharing a split (the same slice of the adapter factor) share that
// XCD's L2 instead of every XCD fetching the whole factor.  A bijection on
// [0, total).
__device__ inline int xcd_order(int b, int total) {
  const int per = total >> 3, rem = total & 7, x = b & 7;
  return x * per + min(x, rem) + (b >> 3);
}

// acc += a·b with the operands swapped: lane l then holds stream index
// l mod 32 and ranks 8 g + 4 (l / 32) + c for e = 4 g + c.
__device__ inline floatx16 mma(const bf16x8& a, const bf16x8& b, const floatx16& acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc, 0, 0, 0);
}

// Partial sums of one wave: 32 stream indices (from s0) x NB blocks of 32
// ranks (from j0), in the accumulator layout of mma(): part[s][idx][j].
template <int NB>
__device__ inline void store_part(const AdapterArgs& g, const floatx16 (&acc)[NB], int64_t s0,
                                  int64_t j0, int split, int lane) {
  const int64_t idx = s0 + (lane & 31);
  if (idx >= g.nout) return;
  float* p = g.part + (int64_t)split * g.part_stride + idx * g.ldp + j0 + 4 * (lane >> 5);
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      floatx4 v;
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = acc[b][4 * q + c];
      *reinterpret_cast<floatx4*>(p + 32 * b + 8 * q) = v;
    }
}

// The same with the roles of the MFMA operands exchanged (mma_n): lane l holds
// rank j0 + 32 b + l mod 32 and stream indices s0 + 8 q + 4 (l / 32) + c,
// stored as part[s][j][idx] (runs of four indices; nout % 4 == 0).
template <int NB>
__device__ inline void store_part_t(const AdapterArgs& g, const floatx16 (&acc)[NB], int64_t s0,
                                    int64_t j0, int split, int lane) {
  float* p = g.part + (int64_t)split * g.part_stride + (j0 + (lane & 31)) * g.ldp;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t idx = s0 + 8 * q + 4 * (lane >> 5);
      if (idx >= g.nout) continue;
      floatx4 v;
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = acc[b][4 * q + c];
      *reinterpret_cast<floatx4*>(p + 32 * b * g.ldp + idx) = v;
    }
}

__device__ inline floatx16 mma_n(const bf16x8& a, const bf16x8& b, const floatx16& acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

}  // namespace

// rows: P[s][m][j] = Σ_k S[m][k]·F(k, j) for block bx of the launch (its
// stream tile and split).  FN = false: F = A [r][ldf] (row j
// holds its k); FN = true: F = B [L][ldf] (row k holds its ranks).  The
// reduction bounds are checked per 16-byte chunk: red % 8 == 0.
template <int NB, bool FN>
__device__ __attribute__((always_inline)) inline void rows_body(const AdapterArgs& g, int bx,
                                                                char* lds) {
  constexpr int S_BYTES = 128 * 128;    // 128 stream rows x 64 k
  constexpr int STAGE = stage_bytes<NB>();
  constexpr int PER_WAVE = 4 + NB;      // direct-to-LDS loads per wave per stage
  constexpr int kRing = ring_of<NB>();

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lin = xcd_order(bx, g.tiles * g.nsplit);
  const int tile = lin % g.tiles, split = lin / g.tiles;
  const int64_t m0 = (int64_t)tile * 128, j0 = (int64_t)blockIdx.y * 128;
  const int kt0 = split * g.kt_per_split;
  const int kt1 = min(g.nkt, kt0 + g.kt_per_split);
  const int64_t kend = min(g.red, (int64_t)kt1 * 64);

  const __amdgpu_buffer_rsrc_t rs = make_rsrc(g.s + m0 * g.lds, (g.nout - m0) * g.lds * 2);
  // B's buffer starts at the split's first row (its offsets then stay small)
  const int64_t kbeg = (int64_t)kt0 * 64;
  __amdgpu_buffer_rsrc_t rf;
  if constexpr (FN)  // B ends at row frows (the reduction may run on over zeros of S)
    rf = make_rsrc(g.f + kbeg * g.ldf + j0, (g.frows - kbeg) * g.ldf * 2 - j0 * 2);
  else
    rf = make_rsrc(g.f + j0 * g.ldf, ((int64_t)g.r - j0) * g.ldf * 2);

  auto issue = [&](int kt, int slot) {
    char* st = lds + slot * STAGE;
    const int64_t k0 = (int64_t)kt * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) load_rows128(rs, g.lds, st, 4 * wave + i, k0, kend, lane);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if constexpr (FN)
        load_rm<4 * NB>(rf, g.ldf, st + S_BYTES, NB * wave + i, k0 - kbeg, kend - kbeg, lane);
      else
        load_rows128(rf, g.ldf, st + S_BYTES, NB * wave + i, k0, kend, lane);
    }
  };

  floatx16 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[b][e] = 0.0f;

  const int n = kt1 - kt0;
  static_for<0, kRing - 1>([&](auto p) { issue(kt0 + p, p); });
  for (int i0 = 0; i0 < n; i0 += kRing) {
    static_for<0, kRing>([&](auto P) {
      constexpr int p = P;
      const int i = i0 + p;
      if (i >= n) return;
      wait_vmcnt<(kRing - 2) * PER_WAVE>();  // this wave's loads of stage i have landed
      ring_barrier();                        // ... and every wave's; slot p - 1 is free
      issue(kt0 + i + kRing - 1, (p + kRing - 1) % kRing);
      const char* st = lds + p * STAGE;
      if constexpr (FN) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          bf16x8 f[4];
          frags_tr<4 * NB>(st + S_BYTES, 32 * b, lane, f);
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) acc[b] = mma(frag128(st, 32 * wave, lane, ks), f[ks], acc[b]);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 a = frag128(st, 32 * wave, lane, ks);
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[b] = mma(a, frag128(st + S_BYTES, 32 * b, lane, ks), acc[b]);
        }
      }
    });
  }
  wait_vmcnt<0>();  // the loads past the range (zeros) have landed before the workgroup ends
  store_part<NB>(g, acc, m0 + 32 * wave, j0, split, lane);
}

// cols: P[s][l][j] = Σ_m S[m][l]·Q[m][j]  (S [M][lds], Q [M][ldf]); TR: the
// partial sums stored as [s][j][l].
template <int NB, bool TR>
__device__ __attribute__((always_inline)) inline void cols_body(const AdapterArgs& g, int bx,
                                                                char* lds) {
  constexpr int S_BYTES = 64 * 256;      // 64 rows (tokens) x 128 stream columns
  constexpr int STAGE = stage_bytes<NB>();
  constexpr int PER_WAVE = 4 + NB;
  constexpr int kRing = ring_of<NB>();

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lin = xcd_order(bx, g.tiles * g.nsplit);
  const int tile = lin % g.tiles, split = lin / g.tiles;
  const int64_t l0 = (int64_t)tile * 128, j0 = (int64_t)blockIdx.y * 128;
  const int kt0 = split * g.kt_per_split;
  const int kt1 = min(g.nkt, kt0 + g.kt_per_split);
  const int64_t mend = min(g.red, (int64_t)kt1 * 64);

  // Buffers start at the split's first row (the host keeps a split's rows
  // within 32-bit offsets).  Columns past the stream's (or the factor's)
  // width read the next row's values: they only reach outputs that are never
  // stored or never read.
  const int64_t mbeg = (int64_t)kt0 * 64;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(g.s + mbeg * g.lds + l0, (g.red - mbeg) * g.lds * 2 - l0 * 2);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(g.f + mbeg * g.ldf + j0, (g.red - mbeg) * g.ldf * 2 - j0 * 2);
  const int64_t mlen = mend - mbeg;

  auto issue = [&](int kt, int slot) {
    char* st = lds + slot * STAGE;
    const int64_t r0 = (int64_t)(kt - kt0) * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) load_rm<16>(rs, g.lds, st, 4 * wave + i, r0, mlen, lane);
#pragma unroll
    for (int i = 0; i < NB; ++i) load_rm<4 * NB>(rq, g.ldf, st + S_BYTES, NB * wave + i, r0, mlen, lane);
  };

  floatx16 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[b][e] = 0.0f;

  const int n = kt1 - kt0;
  static_for<0, kRing - 1>([&](auto p) { issue(kt0 + p, p); });
  for (int i0 = 0; i0 < n; i0 += kRing) {
    static_for<0, kRing>([&](auto P) {
      constexpr int p = P;
      const int i = i0 + p;
      if (i >= n) return;
      wait_vmcnt<(kRing - 2) * PER_WAVE>();
      ring_barrier();
      issue(kt0 + i + kRing - 1, (p + kRing - 1) % kRing);
      const char* st = lds + p * STAGE;
      bf16x8 a[4];
      frags_tr<16>(st, 32 * wave, lane, a);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        bf16x8 f[4];
        frags_tr<4 * NB>(st + S_BYTES, 32 * b, lane, f);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc[b] = TR ? mma_n(a[ks], f[ks], acc[b]) : mma(a[ks], f[ks], acc[b]);
      }
    });
  }
  wait_vmcnt<0>();
  if constexpr (TR)
    store_part_t<NB>(g, acc, l0 + 32 * wave, j0, split, lane);
  else
    store_part<NB>(g, acc, l0 + 32 * wave, j0, split, lane);
}

template <int NB, bool FN>
__global__ __launch_bounds__(256) void adapter_rows_kernel(AdapterArgs g) {
  __shared__ __attribute__((aligned(16))) char lds[ring_of<NB>() * stage_bytes<NB>()];
  rows_body<NB, FN>(g, __builtin_amdgcn_readfirstlane((int)blockIdx.x), lds);
}

template <int NB, bool TR>
__global__ __launch_bounds__(256) void adapter_cols_kernel(AdapterArgs g) {
  __shared__ __attribute__((aligned(16))) char lds[ring_of<NB>() * stage_bytes<NB>()];
  cols_body<NB, TR>(g, __builtin_amdgcn_readfirstlane((int)blockIdx.x), lds);
}

// The two products that stream dY, in one launch: blocks [0, nv) form V's
// partial sums (rows, F = B), the rest dB's (cols, Q = U).  Both run at once,
// each on about half of the CUs.
template <int NB>
__global__ __launch_bounds__(256) void adapter_dy_kernel(AdapterArgs gv, AdapterArgs gb, int nv) {
  __shared__ __attribute__((aligned(16))) char lds[ring_of<NB>() * stage_bytes<NB>()];
  const int bx = __builtin_amdgcn_readfirstlane((int)blockIdx.x);
  if (bx < nv)
    rows_body<NB, true>(gv, bx, lds);
  else
    cols_body<NB, false>(gb, bx - nv, lds);
}

template __global__ void adapter_rows_kernel<1, false>(AdapterArgs);
template __global__ void adapter_rows_kernel<2, false>(AdapterArgs);
template __global__ void adapter_rows_kernel<4, false>(AdapterArgs);
template __global__ void adapter_rows_kernel<1, true>(AdapterArgs);
template __global__ void adapter_rows_kernel<2, true>(AdapterArgs);
template __global__ void adapter_rows_kernel<4, true>(AdapterArgs);
template __global__ void adapter_cols_kernel<1, false>(AdapterArgs);
template __global__ void adapter_cols_kernel<2, false>(AdapterArgs);
template __global__ void adapter_cols_kernel<4, false>(AdapterArgs);
template __global__ void adapter_cols_kernel<1, true>(AdapterArgs);
template __global__ void adapter_cols_kernel<2, true>(AdapterArgs);
template __global__ void adapter_cols_kernel<4, true>(AdapterArgs);
template __global__ void adapter_dy_kernel<1>(AdapterArgs, AdapterArgs, int);
template __global__ void adapter_dy_kernel<2>(AdapterArgs, AdapterArgs, int);
template __global__ void adapter_dy_kernel<4>(AdapterArgs, AdapterArgs, int);

}  // namespace qlora
