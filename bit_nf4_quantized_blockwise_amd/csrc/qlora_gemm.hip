// bf16 MFMA GEMM for gfx950 with in-tile NF4 dequantisation and a LoRA
// prologue.
//
//   C[rows][cols] = s · L·Rᵀ (optional, rank-r prologue)  +  Σ_red A[row][red] · Bop[red][col]
//
// A is always a row-major bf16 matrix with the reduction contiguous (X, dY, or
// a transposed skinny factor).  The B operand comes from one of four loaders:
//   B_NF4_COLS  — the frozen weight, W[n_out][k_in] NF4+DQ, output col = W row,
//                 reduction along k_in (forward: Y = X·Ŵᵀ)
//   B_NF4_RED   — the frozen weight traversed transposed: output col = W column
//                 (k_in), reduction along W rows (input gradient: dX = dY·Ŵ)
//   B_BF16_CR   — bf16 [cols][red] row-major (A or Bᵀ of the adapter)
//   B_BF16_RC   — bf16 [red][cols] row-major (X or dY when the reduction runs
//                 over tokens: the adapter gradients)
// Dequantisation happens in the loader, right before the tile is written to
// LDS, in the order of the Qiita explainer's DQ formula:
// ŵ = RNE_bf16(RN32(c_idx · RN32(c2 · q))) — bit-identical to the standalone
// dequantiser; the dense Ŵ never exists outside one LDS tile ("QLoRAの理論と実装",
// QLoRAの計算フロー step 1: Ŵ only exists transiently).
//
// Tiling: K-tile 64 (= one NF4 block along k_in), 256 threads = 4 wave64s in
// a WM×WN grid, v_mfma_f32_32x32x16_bf16, fp32 accumulators, LDS double
// buffer with the next tile's global loads in flight during the MFMAs.  LDS
// rows are 128 B (64 bf16) split in eight 16-byte chunks, chunk c of row r
// stored at c ^ (r & 7) so that the 32 rows of one MFMA operand read hit
// distinct banks.

#include <type_traits>

#include "qlora_kernels.h"

namespace qlora {

namespace {

constexpr int KT = 64;
constexpr int ROWB = KT * 2;  // bytes per LDS row

__device__ inline int swz(int row, int chunk) { return (row * ROWB) + ((chunk ^ (row & 7)) << 4); }

// ---- A-style loader: [rows][ld] bf16, reduction contiguous ---------------------
template <int T_ROWS>
struct RowTile {
  static constexpr int PER_T = T_ROWS * 8 / 256;
  static_assert(PER_T >= 1, "tile too small");
  u32x4 r[PER_T];

  __device__ inline void load(const uint16_t* __restrict__ p, int64_t ld, int64_t nrows,
                              int64_t nred, int64_t row0, int64_t k0, int tid) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int id = tid + 256 * i;
      const int row = id >> 3, c = id & 7;
      const int64_t gr = row0 + row, gk = k0 + c * 8;
      if (gr < nrows && gk < nred)
        r[i] = *reinterpret_cast<const u32x4*>(p + gr * ld + gk);
      else
        r[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ inline void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int id = tid + 256 * i;
      const int row = id >> 3, c = id & 7;
      *reinterpret_cast<u32x4*>(lds + swz(row, c)) = r[i];
    }
  }
};

// 8x8 transpose of 16-bit elements: in[i] is row i (8 values along the
// reduction-major source), out[c] = column c.
__device__ inline void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int d = 0; d < 4; ++d)
      out[c][d] = __builtin_amdgcn_perm(in[2 * d + 1][c >> 1], in[2 * d][c >> 1], sel);
  }
}

// ---- B_BF16_RC: source [red][cols] row-major, NT == 256 -------------------------
// Thread t owns an 8(red) x 8(cols) sub-block: red rows 8*(t/32).., cols 8*(t%32)..
template <int NT>
struct RcTile {
  static_assert(NT == 256, "RC loader assumes 256 columns");
  u32x4 r[8];
  __device__ inline void load(const uint16_t* __restrict__ p, int64_t ld, int64_t nred,
                              int64_t ncols, int64_t red0, int64_t col0, int tid) {
    const int rb = tid >> 5, cb = tid & 31;
    const int64_t gc = col0 + cb * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t gr = red0 + rb * 8 + i;
      if (gr < nred && gc < ncols)
        r[i] = *reinterpret_cast<const u32x4*>(p + gr * ld + gc);
      else
        r[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ inline void store(char* lds, int tid) const {
    const int rb = tid >> 5, cb = tid & 31;
    u32x4 o[8];
    transpose8x8(r, o);
#pragma unroll
    for (int c = 0; c < 8; ++c) *reinterpret_cast<u32x4*>(lds + swz(cb * 8 + c, rb)) = o[c];
  }
};

__device__ inline u32x4 dequant8(uint32_t p, float ah, const float* __restrict__ cb) {
  u32x4 o;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float lo = cb[(p >> (8 * d)) & 15u] * ah;
    const float hi = cb[(p >> (8 * d + 4)) & 15u] * ah;
    o[d] = pack_bf16x2(lo, hi);
  }
  return o;
}

// ---- B_NF4_COLS: tile = NT rows of W (output cols) x 64 k --------------------------
template <int NT>
struct Nf4ColsTile {
  static constexpr int TPR = 256 / NT;        // threads per W row: 1 (NT=256) or 2 (NT=128)
  static constexpr int DW = 8 / TPR;          // packed dwords per thread
  static_assert(NT == 256 || NT == 128, "NF4 column loader: NT in {128, 256}");
  uint32_t p[DW];
  float ah;

  __device__ inline void load(const GemmArgs& g, int64_t n0, int64_t k0, int tid) {
    const int row = tid / TPR, part = tid % TPR;
    const int64_t n = n0 + row;
    if (n < g.cols) {
      const int64_t e0 = n * g.w_kin + k0 + part * (64 / TPR);
      const uint32_t* src = reinterpret_cast<const uint32_t*>(g.packed + (e0 >> 1));
      if constexpr (DW == 8) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(src);
        const u32x4 b = *reinterpret_cast<const u32x4*>(src + 4);
        p[0] = a[0]; p[1] = a[1]; p[2] = a[2]; p[3] = a[3];
        p[4] = b[0]; p[5] = b[1]; p[6] = b[2]; p[7] = b[3];
      } else {
        const u32x4 a = *reinterpret_cast<const u32x4*>(src);
        p[0] = a[0]; p[1] = a[1]; p[2] = a[2]; p[3] = a[3];
      }
      const int64_t blk = (n * g.w_kin + k0) >> 6;
      ah = g.c2[blk >> 8] * (float)g.qabsmax[blk];
    } else {
#pragma unroll
      for (int d = 0; d < DW; ++d) p[d] = 0x88888888u;
      ah = 0.0f;
    }
  }
  __device__ inline void store(char* lds, int tid, const float* cb) const {
    const int row = tid / TPR, part = tid % TPR;
#pragma unroll
    for (int d = 0; d < DW; ++d)
      *reinterpret_cast<u32x4*>(lds + swz(row, part * DW + d)) = dequant8(p[d], ah, cb);
  }
};

// ---- B_NF4_RED: tile = 64 rows of W (reduction) x NT columns of W (output) -------
// Thread t owns 8 W rows x 8 W columns: rows 8*(t/32).., cols 8*(t%32)..  (NT == 256)
template <int NT>
struct Nf4RedTile {
  static_assert(NT == 256, "NF4 reduction-major loader assumes 256 columns");
  uint32_t p[8];
  float ah[8];

  __device__ inline void load(const GemmArgs& g, int64_t r0, int64_t c0, int tid) {
    const int rb = tid >> 5, cb = tid & 31;
    const int64_t k = c0 + cb * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t n = r0 + rb * 8 + i;
      if (n < g.red && k < g.cols) {
        const int64_t e = n * g.w_kin + k;
        p[i] = *reinterpret_cast<const uint32_t*>(g.packed + (e >> 1));
        const int64_t blk = e >> 6;
        ah[i] = g.c2[blk >> 8] * (float)g.qabsmax[blk];
      } else {
        p[i] = 0x88888888u;
        ah[i] = 0.0f;
      }
    }
  }
  __device__ inline void store(char* lds, int tid, const float* cbk) const {
    const int rb = tid >> 5, cb = tid & 31;
    u32x4 rows[8], cols[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) rows[i] = dequant8(p[i], ah[i], cbk);
    transpose8x8(rows, cols);
#pragma unroll
    for (int c = 0; c < 8; ++c) *reinterpret_cast<u32x4*>(lds + swz(cb * 8 + c, rb)) = cols[c];
  }
};

template <int MT, int NT, int WM, int WN>
struct Mma {
  static constexpr int WTM = MT / WM, WTN = NT / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(FM >= 1 && FN >= 1, "wave tile must be a multiple of 32x32");
  floatx16 acc[FM][FN];

  __device__ inline void zero() {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  }
  __device__ inline void scale(float s) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] *= s;
  }
  // One 64-deep K tile from LDS.
  __device__ inline void run(const char* As, const char* Bs, int wm, int wn, int lane) {
    const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int chunk = ks * 2 + lh;
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * WTM + i * 32 + lr;
        af[i] = *reinterpret_cast<const bf16x8*>(As + swz(row, chunk));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = wn * WTN + j * 32 + lr;
        bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + swz(row, chunk));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }
};

}  // namespace

template <int MT, int NT, int WM, int WN, int BMODE, bool PROLOGUE, int OMODE>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  static_assert(WM * WN == 4, "4 waves");
  __shared__ __attribute__((aligned(16))) char lds[2 * (MT + NT) * ROWB];
  __shared__ float cb[16];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  if constexpr (BMODE == B_NF4_COLS || BMODE == B_NF4_RED) {
    if (tid < 16) cb[tid] = bits_to_float(kNF4Bits[tid]);
  }

  const int tile = blockIdx.x;
  const int tm = tile % g.tiles_m, tn = tile / g.tiles_m;
  const int64_t row0 = (int64_t)tm * MT, col0 = (int64_t)tn * NT;
  const int nkt_total = (int)((g.red + KT - 1) / KT);
  const int kt_begin = blockIdx.y * g.kt_per_split;
  const int kt_end = min(nkt_total, kt_begin + g.kt_per_split);

  // stage st: A tile at lds + st * STAGE, B tile right after it
  constexpr int STAGE = (MT + NT) * ROWB;
  auto As = [&](int st) { return lds + st * STAGE; };
  auto Bs = [&](int st) { return lds + st * STAGE + MT * ROWB; };

  Mma<MT, NT, WM, WN> mma;
  mma.zero();

  if constexpr (PROLOGUE) {
    if (blockIdx.y == 0 && g.rl > 0) {
      for (int64_t j0 = 0; j0 < g.rl; j0 += KT) {
        RowTile<MT> lt;
        RowTile<NT> rt;
        lt.load(g.pl, g.ldpl, g.rows, g.rl, row0, j0, tid);
        rt.load(g.pr, g.ldpr, g.cols, g.rl, col0, j0, tid);
        lt.store(As(0), tid);
        rt.store(Bs(0), tid);
        __syncthreads();
        mma.run(As(0), Bs(0), wm, wn, lane);
        __syncthreads();
      }
      mma.scale(g.s);
    }
  }

  RowTile<MT> at;
  using BTile = typename std::conditional<
      BMODE == B_NF4_COLS, Nf4ColsTile<NT>,
      typename std::conditional<BMODE == B_NF4_RED, Nf4RedTile<NT>,
                                typename std::conditional<BMODE == B_BF16_RC, RcTile<NT>,
                                                          RowTile<NT>>::type>::type>::type;
  BTile bt;

  auto load_tiles = [&](int kt) {
    const int64_t k0 = (int64_t)kt * KT;
    at.load(g.a, g.lda, g.rows, g.red, row0, k0, tid);
    if constexpr (BMODE == B_NF4_COLS) {
      bt.load(g, col0, k0, tid);
    } else if constexpr (BMODE == B_NF4_RED) {
      bt.load(g, k0, col0, tid);
    } else if constexpr (BMODE == B_BF16_RC) {
      bt.load(g.b, g.ldb, g.red, g.cols, k0, col0, tid);
    } else {
      bt.load(g.b, g.ldb, g.cols, g.red, col0, k0, tid);
    }
  };
  auto store_tiles = [&](int st) {
    at.store(As(st), tid);
    if constexpr (BMODE == B_NF4_COLS || BMODE == B_NF4_RED)
      bt.store(Bs(st), tid, cb);
    else
      bt.store(Bs(st), tid);
  };

  if (kt_begin < kt_end) {
    __syncthreads();  // codebook visible
    load_tiles(kt_begin);
    store_tiles(0);
    __syncthreads();
    for (int kt = kt_begin; kt < kt_end; ++kt) {
      const int cur = (kt - kt_begin) & 1;
      const bool more = kt + 1 < kt_end;
      if (more) load_tiles(kt + 1);
      mma.run(As(cur), Bs(cur), wm, wn, lane);
      if (more) store_tiles(cur ^ 1);
      __syncthreads();
    }
  }

  // Epilogue.  32x32 accumulator layout: lane l holds column l%32 and rows
  // 8*(e/4) + 4*(l/32) + e%4 for e = 0..15.
  constexpr int WTM = MT / WM, WTN = NT / WN;
  const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int i = 0; i < WTM / 32; ++i)
#pragma unroll
    for (int j = 0; j < WTN / 32; ++j) {
      const int64_t col = col0 + wn * WTN + j * 32 + lr;
      if (col >= g.cols) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = row0 + wm * WTM + i * 32 + (e >> 2) * 8 + lh * 4 + (e & 3);
        if (row >= g.rows) continue;
        const float v = mma.acc[i][j][e];
        if constexpr (OMODE == O_BF16) {
          g.out_bf16[row * g.ldo + col] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
        } else {
          g.out_f32[(int64_t)blockIdx.y * g.part_stride + row * g.ldo + col] = v;
        }
      }
    }
}

// Instantiations used by the library.
#define QLORA_GEMM(MT, NT, WM, WN, BM, PRO, OM) \
  template __global__ void gemm_kernel<MT, NT, WM, WN, BM, PRO, OM>(GemmArgs);

QLORA_GEMM(256, 256, 2, 2, B_NF4_COLS, true, O_BF16)   // forward, many tokens
QLORA_GEMM(256, 256, 2, 2, B_NF4_RED, true, O_BF16)    // input gradient, many tokens
QLORA_GEMM(64, 256, 1, 4, B_NF4_COLS, true, O_F32)     // forward, few tokens (split-K)
QLORA_GEMM(64, 256, 1, 4, B_NF4_RED, true, O_F32)      // input gradient, few tokens
QLORA_GEMM(128, 64, 4, 1, B_BF16_CR, false, O_F32)     // U = X·Aᵀ, V = dY·B (split-K)
QLORA_GEMM(64, 256, 2, 2, B_BF16_RC, false, O_F32)     // dA, dB: reduction over tokens

}  // namespace qlora
