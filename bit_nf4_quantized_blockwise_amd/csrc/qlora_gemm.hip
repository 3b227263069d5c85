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
constexpr int kOOB = 0x7ffffff0;         // a buffer offset past every range: loads return 0
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9)

__device__ inline int swz(int row, int chunk) { return (row * ROWB) + ((chunk ^ (row & 7)) << 4); }

// A raw buffer resource: loads at offsets outside [0, bytes) return zero, so
// ragged tiles need no branches.
struct Buf {
  __amdgpu_buffer_rsrc_t r;
  __device__ inline void init(const void* base, int64_t bytes) {
    const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffffLL : bytes);
    r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kRsrcWord3);
  }
  __device__ inline u32x4 ld16(int off) const {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
  __device__ inline uint32_t ld4(int off) const {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
  __device__ inline uint32_t ld1(int off) const {
    return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
  }
};

// ---- A-style loader: [rows][ld] bf16, reduction contiguous ---------------------
// Thread t moves 16-byte chunks id = t + 256 i: row id / 8, chunk id % 8.
template <int T_ROWS>
struct RowTile {
  static constexpr int PER_T = T_ROWS * 8 / 256;
  static_assert(PER_T >= 1, "tile too small");
  u32x4 r[PER_T];
  Buf buf;
  int voff;      // byte offset of chunk i = 0 from the tile's first row
  int rstride;   // bytes between chunk i and i + 1 (32 rows)

  __device__ inline void init(const uint16_t* p, int64_t ld, int64_t nrows, int64_t row0,
                              int tid) {
    buf.init(p + row0 * ld, (nrows - row0) * ld * 2);
    voff = (tid >> 3) * (int)ld * 2 + (tid & 7) * 16;
    rstride = 32 * (int)ld * 2;
  }
  __device__ inline void load(int64_t k0, int64_t nred, int tid) {
    const bool ok = k0 + (tid & 7) * 8 < nred;
    const int base = ok ? voff + (int)k0 * 2 : kOOB;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) r[i] = buf.ld16(ok ? base + i * rstride : kOOB);
  }
  __device__ inline void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int id = tid + 256 * i;
      *reinterpret_cast<u32x4*>(lds + swz(id >> 3, id & 7)) = r[i];
    }
  }
  // Quarter q of store(): chunks i with i % 4 == q (all of them when PER_T < 4
  // and q == 0).
  __device__ inline void store_part(char* lds, int tid, int q) const {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      if (i % 4 != q) continue;
      const int id = tid + 256 * i;
      *reinterpret_cast<u32x4*>(lds + swz(id >> 3, id & 7)) = r[i];
    }
  }
  // Stores RNE_bf16(s·v) (part 0) or RNE_bf16(s·v − part 0) (part 1) for the
  // eight bf16 values v of each chunk: s·v ≈ part 0 + part 1 to ~2^-16.
  __device__ inline void store_scaled(char* lds, int tid, float s, int part) const {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float a = bits_to_float(r[i][d] << 16) * s;
        const float b = bits_to_float(r[i][d] & 0xffff0000u) * s;
        uint32_t h = pack_bf16x2(a, b);
        if (part) h = pack_bf16x2(a - bits_to_float(h << 16), b - bits_to_float(h & 0xffff0000u));
        o[d] = h;
      }
      const int id = tid + 256 * i;
      *reinterpret_cast<u32x4*>(lds + swz(id >> 3, id & 7)) = o;
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
  __device__ inline void load(const uint16_t* p, int64_t ld, int64_t nred, int64_t ncols,
                              int64_t red0, int64_t col0, int tid) {
    Buf b;
    b.init(p + red0 * ld, (nred - red0) * ld * 2);
    const int rb = tid >> 5, cb = tid & 31;
    const int64_t gc = col0 + cb * 8;
    const int base = (gc < ncols) ? (rb * 8) * (int)ld * 2 + (int)gc * 2 : kOOB;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = b.ld16(gc < ncols ? base + i * (int)ld * 2 : kOOB);
  }
  __device__ inline void store(char* lds, int tid) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) store_part(lds, tid, q);
  }
  // Quarter q: output columns 2q and 2q + 1 of this thread's 8x8 sub-block,
  // each the 8 reduction values of one source column (an 8x8 transpose).
  __device__ inline void store_part(char* lds, int tid, int q) const {
    const int rb = tid >> 5, cb = tid & 31;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 2 * q + h;
      const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        o[d] = __builtin_amdgcn_perm(r[2 * d + 1][c >> 1], r[2 * d][c >> 1], sel);
      *reinterpret_cast<u32x4*>(lds + swz(cb * 8 + c, rb)) = o;
    }
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
  u32x4 p[DW / 4];
  float ah;
  Buf pk, qa, c2;
  int row_off, q_off;
  int64_t gblk0;  // global block index of this thread's row at k = 0

  __device__ inline void init(const GemmArgs& g, int64_t n0, int tid) {
    const int row = tid / TPR, part = tid % TPR;
    const int64_t bpr = g.w_kin >> 6;  // blocks per W row
    pk.init(g.packed + n0 * (g.w_kin >> 1), (g.cols - n0) * (g.w_kin >> 1));
    qa.init(g.qabsmax + n0 * bpr, (g.cols - n0) * bpr);
    c2.init(g.c2, ((g.cols * bpr + 255) >> 8) * 4);
    row_off = row * (int)(g.w_kin >> 1) + part * 16 * (DW / 4);
    q_off = row * (int)bpr;
    gblk0 = (n0 + row) * bpr;
  }
  __device__ inline void load(int64_t k0, int64_t kend) {
    const int kb = (int)(k0 >> 6);
    const bool ok = k0 < kend;  // uniform: tiles past this split's range read as zero
#pragma unroll
    for (int d = 0; d < DW / 4; ++d) p[d] = pk.ld16(ok ? row_off + (int)(k0 >> 1) + 16 * d : kOOB);
    const uint32_t q = qa.ld1(ok ? q_off + kb : kOOB);
    const float s2 = bits_to_float(c2.ld4((int)(((gblk0 + kb) >> 8) * 4)));
    ah = s2 * (float)q;
  }
  __device__ inline void store(char* lds, int tid, const float* cb) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) store_part(lds, tid, cb, q);
  }
  // Quarter q: packed dwords d with d % 4 == q (8 weights -> one 16-byte chunk each).
  __device__ inline void store_part(char* lds, int tid, const float* cb, int q) const {
    const int row = tid / TPR, part = tid % TPR;
#pragma unroll
    for (int d = 0; d < DW; ++d) {
      if (d % 4 != q) continue;
      *reinterpret_cast<u32x4*>(lds + swz(row, part * DW + d)) = dequant8(p[d >> 2][d & 3], ah, cb);
    }
  }
};

// ---- B_NF4_RED: tile = 64 rows of W (reduction) x NT columns of W (output) -------
// Thread t owns 8 W rows x 8 W columns: rows 8*(t/32).., cols 8*(t%32)..  (NT == 256)
template <int NT>
struct Nf4RedTile {
  static_assert(NT == 256, "NF4 reduction-major loader assumes 256 columns");
  uint32_t p[8];
  float ah[8];
  Buf c2;
  int64_t k;  // first W column of this thread

  __device__ inline void init(const GemmArgs& g, int64_t c0, int tid) {
    k = c0 + (tid & 31) * 8;
    c2.init(g.c2, ((g.red * (g.w_kin >> 6) + 255) >> 8) * 4);
  }
  __device__ inline void load(const GemmArgs& g, int64_t r0, int64_t rend, int tid) {
    const int rb = tid >> 5;
    const int64_t bpr = g.w_kin >> 6;
    Buf pk, qa;
    pk.init(g.packed + r0 * (g.w_kin >> 1), (rend - r0) * (g.w_kin >> 1));
    qa.init(g.qabsmax + r0 * bpr, (rend - r0) * bpr);
    const bool ok = k < g.cols;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = rb * 8 + i;
      p[i] = pk.ld4(ok ? n * (int)(g.w_kin >> 1) + (int)(k >> 1) : kOOB);
      const int lb = n * (int)bpr + (int)(k >> 6);
      const uint32_t q = qa.ld1(ok ? lb : kOOB);
      const float s2 = bits_to_float(c2.ld4((int)((((r0 + n) * bpr + (k >> 6)) >> 8) * 4)));
      ah[i] = s2 * (float)q;
    }
  }
  __device__ inline void store(char* lds, int tid, const float* cbk) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) store_part(lds, tid, cbk, q);
  }
  // Quarter q: output columns c = 2q, 2q + 1 — W column k + c decoded from
  // nibble c of each of the 8 W rows (the transpose falls out of the lookup).
  __device__ inline void store_part(char* lds, int tid, const float* cbk, int q) const {
    const int rb = tid >> 5, cb = tid & 31;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 2 * q + h;
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float lo = cbk[(p[2 * d] >> (4 * c)) & 15u] * ah[2 * d];
        const float hi = cbk[(p[2 * d + 1] >> (4 * c)) & 15u] * ah[2 * d + 1];
        o[d] = pack_bf16x2(lo, hi);
      }
      *reinterpret_cast<u32x4*>(lds + swz(cb * 8 + c, rb)) = o;
    }
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
  struct Frags {
    bf16x8 a[FM], b[FN];
  };
  __device__ inline void load_frags(Frags& f, const char* As, const char* Bs, int wm, int wn,
                                    int lane, int ks) const {
    const int lr = lane & 31, lh = lane >> 5;
    const int chunk = ks * 2 + lh;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      f.a[i] = *reinterpret_cast<const bf16x8*>(As + swz(wm * WTM + i * 32 + lr, chunk));
#pragma unroll
    for (int j = 0; j < FN; ++j)
      f.b[j] = *reinterpret_cast<const bf16x8*>(Bs + swz(wn * WTN + j * 32 + lr, chunk));
  }
  __device__ inline void mfma(const Frags& f) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
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
    // acc = s · L·Rᵀ over the rank dimension.  s is applied to L while it is
    // staged (two bf16 parts when s·L is not exact in one), never to acc.
    if (blockIdx.y == 0 && g.rl > 0) {
      RowTile<MT> lt;
      RowTile<NT> rt;
      lt.init(g.pl, g.ldpl, g.rows, row0, tid);
      rt.init(g.pr, g.ldpr, g.cols, col0, tid);
      // one flat loop over (rank chunk, part): nested loops around the MFMAs
      // make the register allocator spill the accumulators
      const int nparts = 1 + g.s_split;
      const int nsteps = (int)((g.rl + KT - 1) / KT) * nparts;
      for (int st = 0; st < nsteps; ++st) {
        const int64_t j0 = (int64_t)(st / nparts) * KT;
        const int part = st % nparts;
        lt.load(j0, g.rl, tid);
        rt.load(j0, g.rl, tid);
        lt.store_scaled(As(0), tid, g.s, part);
        rt.store(Bs(0), tid);
        __syncthreads();
        mma.run(As(0), Bs(0), wm, wn, lane);
        __syncthreads();
      }
    }
  }

  using BTile = typename std::conditional<
      BMODE == B_NF4_COLS, Nf4ColsTile<NT>,
      typename std::conditional<BMODE == B_NF4_RED, Nf4RedTile<NT>,
                                typename std::conditional<BMODE == B_BF16_RC, RcTile<NT>,
                                                          RowTile<NT>>::type>::type>::type;
  // Two register sets: while the MFMAs consume one LDS stage, the tile loaded
  // one half-iteration earlier is decoded into the other stage and the next
  // tile is in flight from memory.
  RowTile<MT> a0, a1;
  BTile b0, b1;
  a0.init(g.a, g.lda, g.rows, row0, tid);
  a1.init(g.a, g.lda, g.rows, row0, tid);
  if constexpr (BMODE == B_NF4_COLS || BMODE == B_NF4_RED) {
    b0.init(g, col0, tid);
    b1.init(g, col0, tid);
  } else if constexpr (BMODE == B_BF16_CR) {
    b0.init(g.b, g.ldb, g.cols, col0, tid);
    b1.init(g.b, g.ldb, g.cols, col0, tid);
  }
  const int64_t kend = min(g.red, (int64_t)kt_end * KT);  // this split's reduction bound

  auto load_tiles = [&](RowTile<MT>& at, BTile& bt, int kt) {
    const int64_t k0 = (int64_t)kt * KT;
    at.load(k0, kend, tid);
    if constexpr (BMODE == B_NF4_COLS) {
      bt.load(k0, kend);
    } else if constexpr (BMODE == B_NF4_RED) {
      bt.load(g, k0, kend, tid);
    } else if constexpr (BMODE == B_BF16_RC) {
      bt.load(g.b, g.ldb, kend, g.cols, k0, col0, tid);
    } else {
      bt.load(k0, kend, tid);
    }
  };
  auto store_part = [&](const RowTile<MT>& at, const BTile& bt, int st, int q) {
    at.store_part(As(st), tid, q);
    if constexpr (BMODE == B_NF4_COLS || BMODE == B_NF4_RED)
      bt.store_part(Bs(st), tid, cb, q);
    else
      bt.store_part(Bs(st), tid, q);
  };
  using MmaT = Mma<MT, NT, WM, WN>;
  // One K tile of MFMAs from stage `cur`, with a quarter of the next tile's
  // decode + LDS writes (into stage cur ^ 1) after each 64-deep quarter of
  // MFMAs; fragments are read one quarter ahead.  sched_barrier keeps the
  // compiler from regrouping the quarters.
  auto step = [&](int cur, const RowTile<MT>& at, const BTile& bt) {
    typename MmaT::Frags f0, f1;
    mma.load_frags(f0, As(cur), Bs(cur), wm, wn, lane, 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      typename MmaT::Frags& fc = (ks & 1) ? f1 : f0;
      typename MmaT::Frags& fn = (ks & 1) ? f0 : f1;
      if (ks < 3) mma.load_frags(fn, As(cur), Bs(cur), wm, wn, lane, ks + 1);
      mma.mfma(fc);
      store_part(at, bt, cur ^ 1, ks);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (kt_begin < kt_end) {
    __syncthreads();  // codebook visible
    load_tiles(a0, b0, kt_begin);
    load_tiles(a1, b1, kt_begin + 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) store_part(a0, b0, 0, q);
    __syncthreads();
    // Branch-free: tiles past kt_end load as zeros, so an odd count ends with
    // one MFMA pass over a zero tile.
    for (int kt = kt_begin; kt < kt_end; kt += 2) {
      load_tiles(a0, b0, kt + 2);
      step(0, a1, b1);
      __syncthreads();
      load_tiles(a1, b1, kt + 3);
      step(1, a0, b0);
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
