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
//   B_BF16_RC   — bf16 [red][cols] row-major (A, for the dropout backward's
//                 masked rank-r term T = s·mask ⊙ (V·A))
// The rank-r products of the layer itself (U, V, dA, dB) run on their own
// streaming kernels (qlora_adapter.hip).
// Dequantisation happens in the loader, right before the tile is written to
// LDS, in the order of the Qiita explainer's DQ formula:
// ŵ = RNE_bf16(RN32(c_idx · RN32(c2 · q))) — bit-identical to the standalone
// dequantiser; the dense Ŵ never exists outside one LDS tile ("QLoRAの理論と実装",
// QLoRAの計算フロー step 1: Ŵ only exists transiently).
//
// Tiling: K-tile 64 (= one NF4 block along k_in), 256 threads = 4 wave64s in
// a WM×WN grid, v_mfma_f32_32x32x16_bf16, fp32 accumulators.  The A operand
// goes from memory straight into MFMA registers; only the B tile (decoded
// weight or adapter factor) is staged in LDS, double-buffered, with the next
// tile decoded while the MFMAs of the current one run.  LDS rows are 128 B
// (64 bf16) in eight 16-byte chunks, swizzled so that the MFMA operand reads
// and every loader's stores are free of bank conflicts.

#include <type_traits>

#include "qlora_kernels.h"

namespace qlora {

namespace {

constexpr int KT = 64;
constexpr int ROWB = KT * 2;  // bytes per LDS row
constexpr int kOOB = 0x7ffffff0;         // a buffer offset past every range: loads return 0
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9)

// chunk c of row r sits at position c ^ (r mod 8) ^ ((r / 8) mod 8): eight
// consecutive rows (the MFMA operand reads and the row-wise stores) and eight
// rows 8 apart (the transposing stores) both land on eight distinct positions.
__device__ inline int swz(int row, int chunk) {
  return (row * ROWB) + ((chunk ^ (row & 7) ^ ((row >> 3) & 7)) << 4);
}

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

// ---- [rows][ld] bf16 with the reduction contiguous (the prologue's R = B) --------
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
};

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

// ---- B_NF4_COLS: tile = NT rows of W (output cols) x 64 k --------------------------
template <int NT>
struct Nf4ColsTile {
  static constexpr int TPR = 256 / NT;        // threads per W row: 1 (NT=256) or 2 (NT=128)
  static constexpr int DW = 8 / TPR;          // packed dwords per thread
  static_assert(NT == 256 || NT == 128, "NF4 column loader: NT in {128, 256}");
  u32x4 p[DW / 4];
  uint32_t qraw;  // DQ code of this thread's block
  float s2;       // its group's second-level step
  float ah;       // c2 · q, set by prep()
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
  // Issues the loads only; nothing here waits for them.
  __device__ inline void load(int64_t k0, int64_t kend) {
    const int kb = (int)(k0 >> 6);
    const bool ok = k0 < kend;  // uniform: tiles past this split's range read as zero
#pragma unroll
    for (int d = 0; d < DW / 4; ++d) p[d] = pk.ld16(ok ? row_off + (int)(k0 >> 1) + 16 * d : kOOB);
    qraw = qa.ld1(ok ? q_off + kb : kOOB);
    s2 = bits_to_float(c2.ld4((int)(((gblk0 + kb) >> 8) * 4)));
  }
  __device__ inline void prep() { ah = s2 * (float)qraw; }
  __device__ inline void store(char* lds, int tid, const float* cb) {
    prep();
#pragma unroll
    for (int q = 0; q < 4; ++q) store_part(lds, tid, cb, q);
  }
  // Quarter q: packed dwords d with d % 4 == q (8 weights -> one 16-byte chunk each).
  __device__ inline void store_part(char* lds, int tid, const float* cb, int q) const {
    const int row = tid / TPR, part = tid % TPR;
#pragma unroll
    for (int d = 0; d < DW; ++d) {
      if (d % 4 != q) continue;
      *reinterpret_cast<u32x4*>(lds + swz(row, part * DW + d)) = decode8(p[d >> 2][d & 3], ah, cb);
    }
  }
  // The same quarter in two phases, so the codebook reads can be issued a
  // quarter before their use: lookup() gathers c[idx] (fp32), finish() scales,
  // rounds to bf16 and stores.  The nibbles are first spread to byte offsets
  // 4·idx (even elements in one dword, odd in another); the empty asm keeps
  // the compiler from folding that back into a shift-and-mask per element, so
  // each lookup address is a single byte extract.
  __device__ inline void lookup(int q, float (&v)[16], const float* cb) const {
    const char* base = reinterpret_cast<const char*>(cb);
#pragma unroll
    for (int d = 0, n = 0; d < DW; ++d) {
      if (d % 4 != q) continue;
      const uint32_t w = p[d >> 2][d & 3];
      uint32_t ev = (w << 2) & 0x3c3c3c3cu, od = (w >> 2) & 0x3c3c3c3cu;
      asm("" : "+v"(ev), "+v"(od));
#pragma unroll
      for (int b = 0; b < 4; ++b, n += 2) {
        v[n] = *reinterpret_cast<const float*>(base + ((ev >> (8 * b)) & 0xffu));
        v[n + 1] = *reinterpret_cast<const float*>(base + ((od >> (8 * b)) & 0xffu));
      }
    }
  }
  __device__ inline void finish(int q, const float (&v)[16], char* lds, int tid) const {
    const int row = tid / TPR, part = tid % TPR;
#pragma unroll
    for (int d = 0, n = 0; d < DW; ++d) {
      if (d % 4 != q) continue;
      u32x4 o;
#pragma unroll
      for (int b = 0; b < 4; ++b, n += 2) o[b] = pack_bf16x2(v[n] * ah, v[n + 1] * ah);
      *reinterpret_cast<u32x4*>(lds + swz(row, part * DW + d)) = o;
    }
  }
};

// ---- B_NF4_RED: tile = 64 rows of W (reduction) x NT columns of W (output) -------
// Thread t owns 8 W rows x 8 W columns: rows 8*(t/32).., cols 8*(t%32)..  (NT == 256)
template <int NT>
struct Nf4RedTile {
  static_assert(NT == 256, "NF4 reduction-major loader assumes 256 columns");
  uint32_t p[8];     // packed dword of each of the 8 rows; after prep(): 4·idx of even nibbles
  uint32_t od[8];    // after prep(): 4·idx of odd nibbles
  uint32_t qraw[8];  // DQ codes; after prep() the block scales (float bits)
  Buf c2;
  int64_t k;  // first W column of this thread

  __device__ inline void init(const GemmArgs& g, int64_t c0, int tid) {
    k = c0 + (tid & 31) * 8;
    c2.init(g.c2, ((g.red * (g.w_kin >> 6) + 255) >> 8) * 4);
  }
  // Issues the loads only.  The DQ code and the step of each row are folded
  // into the row's block scale by prep(), once they have arrived.
  float s2[8];
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
      qraw[i] = qa.ld1(ok ? lb : kOOB);
      s2[i] = bits_to_float(c2.ld4((int)((((r0 + n) * bpr + (k >> 6)) >> 8) * 4)));
    }
  }
  __device__ inline void prep() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w = p[i];
      uint32_t e = (w << 2) & 0x3c3c3c3cu, o = (w >> 2) & 0x3c3c3c3cu;
      asm("" : "+v"(e), "+v"(o));
      p[i] = e;
      od[i] = o;
      qraw[i] = float_to_bits(s2[i] * (float)qraw[i]);
    }
  }
  __device__ inline float ah(int i) const { return bits_to_float(qraw[i]); }
  __device__ inline void store(char* lds, int tid, const float* cbk) {
    prep();
    float v[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      lookup(q, v, cbk);
      finish(q, v, lds, tid);
    }
  }
  __device__ inline void store_part(char* lds, int tid, const float* cbk, int q) const {
    float v[16];
    lookup(q, v, cbk);
    finish(q, v, lds, tid);
  }
  // Quarter q: output columns c = 2q, 2q + 1 — W column k + c decoded from
  // nibble c of each of the 8 W rows (the transpose falls out of the lookup).
  __device__ inline void lookup(int q, float (&v)[16], const float* cbk) const {
    const char* base = reinterpret_cast<const char*>(cbk);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = *reinterpret_cast<const float*>(base + ((p[i] >> (8 * q)) & 0xffu));
      v[8 + i] = *reinterpret_cast<const float*>(base + ((od[i] >> (8 * q)) & 0xffu));
    }
  }
  __device__ inline void finish(int q, const float (&v)[16], char* lds, int tid) const {
    const int rb = tid >> 5, cb = tid & 31;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 2 * q + h;
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        o[d] = pack_bf16x2(v[8 * h + 2 * d] * ah(2 * d), v[8 * h + 2 * d + 1] * ah(2 * d + 1));
      *reinterpret_cast<u32x4*>(lds + swz(cb * 8 + c, rb)) = o;
    }
  }
};

// ---- B_NF4_RED, row-major staging (NT = 256) ---------------------------------
// The tile is 64 W rows (the reduction) x 256 W columns (the output), kept in
// LDS in W's own layout: row n holds its 256 columns in 512 bytes, the 16-byte
// chunk c at position c ^ 4 (n mod 4).  Thread t decodes one NF4 block: row
// t / 4, columns 64 (t mod 4) .. +64, exactly as the column tile does, and the
// MFMA reads its operand through the transposing LDS loads.
__device__ inline int swz_rows(int n, int chunk) { return n * 512 + ((chunk ^ ((n & 3) << 2)) << 4); }

struct Nf4RowsTile {
  u32x4 p[2];
  uint32_t qraw;
  float s2, ah;
  Buf c2;
  int n, b;      // row within the tile, block within the row
  int64_t col;   // first W column of this thread's block

  __device__ inline void init(const GemmArgs& g, int64_t c0, int tid) {
    n = tid >> 2;
    b = tid & 3;
    col = c0 + 64 * b;
    c2.init(g.c2, ((g.red * (g.w_kin >> 6) + 255) >> 8) * 4);
  }
  // Issues the loads only: W row r0 + n; rows at or past rend and columns
  // past the matrix read as zero.
  __device__ inline void load(const GemmArgs& g, int64_t r0, int64_t rend) {
    const int64_t bpr = g.w_kin >> 6;
    Buf pk, qa;
    pk.init(g.packed + r0 * (g.w_kin >> 1), (rend - r0) * (g.w_kin >> 1));
    qa.init(g.qabsmax + r0 * bpr, (rend - r0) * bpr);
    const bool ok = col < g.cols;
    const int off = n * (int)(g.w_kin >> 1) + (int)(col >> 1);
    p[0] = pk.ld16(ok ? off : kOOB);
    p[1] = pk.ld16(ok ? off + 16 : kOOB);
    qraw = qa.ld1(ok ? n * (int)bpr + (int)(col >> 6) : kOOB);
    s2 = bits_to_float(c2.ld4((int)((((r0 + n) * bpr + (col >> 6)) >> 8) * 4)));
  }
  __device__ inline void prep() { ah = s2 * (float)qraw; }
  // Quarter q: packed dwords q and q + 4 (chunks q and q + 4 of the block).
  __device__ inline void lookup(int q, float (&v)[16], const float* cb) const {
    const char* base = reinterpret_cast<const char*>(cb);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int d = q + 4 * h;
      const uint32_t w = p[d >> 2][d & 3];
      uint32_t ev = (w << 2) & 0x3c3c3c3cu, od = (w >> 2) & 0x3c3c3c3cu;
      asm("" : "+v"(ev), "+v"(od));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * h + 2 * e] = *reinterpret_cast<const float*>(base + ((ev >> (8 * e)) & 0xffu));
        v[8 * h + 2 * e + 1] = *reinterpret_cast<const float*>(base + ((od >> (8 * e)) & 0xffu));
      }
    }
  }
  __device__ inline void finish(int q, const float (&v)[16], char* lds, int) const {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(v[8 * h + 2 * e] * ah, v[8 * h + 2 * e + 1] * ah);
      *reinterpret_cast<u32x4*>(lds + swz_rows(n, 8 * b + q + 4 * h)) = o;
    }
  }
  __device__ inline void store_part(char* lds, int tid, const float* cb, int q) const {
    float v[16];
    lookup(q, v, cb);
    finish(q, v, lds, tid);
  }
  // Whole tile at once (pipeline fill).
  __device__ inline void store(char* lds, const float* cb) {
    prep();
    float v[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      lookup(q, v, cb);
      finish(q, v, lds, 0);
    }
  }
};

// A tile staged by direct-to-LDS buffer loads (no VGPRs).  A wave-wide
// 16-byte load writes lane l's data at LDS offset 16 l, i.e. 8 rows x 128 B;
// the LDS swizzle is applied on the global side: the lane landing in chunk
// position pc of row r fetches logical chunk pc ^ f(r).  The tile's MT / 8
// such loads are split over the 4 waves.
template <int MT>
struct ADma {
  static constexpr int PER_W = MT / 32;
  static_assert(PER_W % 8 == 0, "A tile loads must cover whole swizzle periods");
  Buf buf;
  int vrow;   // byte offset of this lane's row in the wave's first load
  int c16;    // 16 · ((lane mod 8) ^ (lane / 8)): chunk of the first load
  int jstep;  // bytes between the rows of consecutive loads (8 rows)
  int lbase;  // LDS byte offset of the wave's first load within a stage (uniform)

  __device__ inline void init(const uint16_t* p, int64_t ld, int64_t nrows, int64_t row0,
                              int wave, int lane) {
    buf.init(p + row0 * ld, (nrows - row0) * ld * 2);
    // Load j of this wave covers rows (wave · PER_W + j) · 8 + lane / 8: r mod 8
    // is lane / 8 and (r / 8) mod 8 is j mod 8, so the lane fetches logical
    // chunk (lane mod 8) ^ (lane / 8) ^ (j mod 8) to land at its slot.
    vrow = (wave * PER_W * 8 + (lane >> 3)) * (int)ld * 2;
    c16 = ((lane & 7) ^ (lane >> 3)) << 4;
    jstep = 8 * (int)ld * 2;
    lbase = wave * PER_W * 1024;
  }
  __device__ inline void issue(char* stage, int64_t k0, int64_t kend) const {
    const int kb = (int)k0 * 2, kendb = (int)kend * 2;
    const bool full = kb + KT * 2 <= kendb;  // whole tile inside the reduction range (uniform)
#pragma unroll
    for (int j = 0; j < PER_W; ++j) {
      const int cj = c16 ^ ((j & 7) << 4);
      const int off = vrow + cj + (kb + j * jstep);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          buf.r, (__attribute__((address_space(3))) void*)(stage + lbase + j * 1024), 16,
          full || kb + cj < kendb ? off : kOOB, 0, 0, 0);
    }
  }
};

// s_waitcnt vmcnt(0) (expcnt, lgkmcnt left alone): the direct-to-LDS loads,
// which no register dependency tracks, have landed.
__device__ inline void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// A operand straight from memory into MFMA registers (no LDS round trip).
// Lane l of a wave holds row 32 i + l % 32 of the wave's rows and, for the
// four 16-deep MFMA steps ks of a 64-deep K tile, the reduction values
// k0 + 32 h + 8 ks .. + 7 with h = l / 32.  That is a permutation of k within
// the tile; the B operand reads use the same one (an MFMA sums its k slots in
// any order), so each lane's four loads of a row are 64 contiguous bytes.
template <int FM>
struct ARegs {
  u32x4 r[FM][4];
  Buf buf;
  int voff;     // byte offset of this lane's row in row block 0, at its k half
  int istride;  // bytes between row blocks i and i + 1 (32 rows)
  int h;

  __device__ inline void init(const uint16_t* p, int64_t ld, int64_t nrows, int64_t row0,
                              int lane) {
    buf.init(p + row0 * ld, (nrows - row0) * ld * 2);
    h = lane >> 5;
    voff = (lane & 31) * (int)ld * 2 + h * 64;
    istride = 32 * (int)ld * 2;
  }
  // Step ks of the K tile at k0; reduction values at or past kend read as zero.
  __device__ inline void load_ks(int64_t k0, int64_t kend, int ks) {
    const bool ok = k0 + 32 * h + 8 * ks < kend;
    const int off = voff + (int)k0 * 2 + ks * 16;
#pragma unroll
    for (int i = 0; i < FM; ++i) r[i][ks] = buf.ld16(ok ? off + i * istride : kOOB);
  }
  __device__ inline void load(int64_t k0, int64_t kend) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) load_ks(k0, kend, ks);
  }
};

// bf16 pairs of v scaled by s: RNE_bf16(s·v) (part 0) or RNE_bf16(s·v − part 0)
// (part 1); s·v ≈ part 0 + part 1 to ~2^-16.
__device__ inline u32x4 scale_part(const u32x4& v, float s, int part) {
  u32x4 o;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float a = bits_to_float(v[d] << 16) * s;
    const float b = bits_to_float(v[d] & 0xffff0000u) * s;
    uint32_t h = pack_bf16x2(a, b);
    if (part) h = pack_bf16x2(a - bits_to_float(h << 16), b - bits_to_float(h & 0xffff0000u));
    o[d] = h;
  }
  return o;
}

// Scheduling pattern for one region of the main loop: each MFMA followed by
// up to two LDS reads, one VMEM instruction and four VALU instructions, with
// the LDS writes spread in.  One wave per SIMD issues in order, so VALU work
// placed between MFMAs runs while the matrix core is busy instead of after it.
// DSR LDS reads and VALU instructions per MFMA: measured best at 2 and 4 for
// the forward tile and at 3 and 3 for the input-gradient tile (whose decode
// finishes each quarter in place); more VALU per MFMA delays the next MFMA.
template <int NMFMA, int DSR = 2, int VALU = 4>
__device__ inline void interleave() {
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, DSR, 0);   // DS read
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);     // VMEM read
    __builtin_amdgcn_sched_group_barrier(0x002, VALU, 0);  // VALU
    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);     // DS write
  }
}

// One 32x32x16 step of acc[i][j] += (A rows i)·(B cols j), issued with the
// operands swapped: the matrix core then produces the transposed block, so
// that lane l holds output row l mod 32 and, for e = 4g + c, output column
// 8g + 4 (l / 32) + c — four consecutive columns per group g, which the
// epilogue stores as one 8- or 16-byte write.
__device__ inline floatx16 mfma_t(const bf16x8& a, const bf16x8& b, const floatx16& acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc, 0, 0, 0);
}

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
  // B fragments of step ks from an LDS tile, in the k order of ARegs.
  __device__ inline void load_b(bf16x8 (&b)[FN], const char* Bs, int wn, int lane, int ks) const {
    const int chunk = 4 * (lane >> 5) + ks;
#pragma unroll
    for (int j = 0; j < FN; ++j)
      b[j] = *reinterpret_cast<const bf16x8*>(Bs + swz(wn * WTN + j * 32 + (lane & 31), chunk));
  }
  // B fragments of step ks from a row-major tile (see Nf4RowsTile), through
  // ds_read_b64_tr_b16.  In each group of 16 lanes that instruction hands
  // lane 4a + b element b of the 8-byte rows fetched by lanes a, a + 4,
  // a + 8, a + 12.  So lane r of a group fetches row n0 + r / 4, columns
  // 4 (r mod 4) .. +3 of its 16-column slice, and every lane ends up with four
  // consecutive rows (the reduction) of one column; two loads give the eight
  // rows 32 (lane / 32) + 8 ks .. +7, the A operand's k order.  tb[j] is the
  // lane's byte offset for column block j at ks = 0 (from tr_base).
  __device__ inline void load_b_tr(bf16x8 (&b)[FN], const char* Bs, const int (&tb)[FN], int ks) const {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      typedef short s4 __attribute__((ext_vector_type(4)));
      const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s4*)(Bs + tb[j] + (8 * ks) * 512));
      const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s4*)(Bs + tb[j] + (8 * ks + 4) * 512));
      b[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }
  __device__ inline void tr_base(int (&tb)[FN], int wn, int lane) const {
    const int r = lane & 15;
    const int n = 32 * (lane >> 5) + (r >> 2);  // row at ks = 0; + 8 ks (+ 4) keeps n mod 4
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int chunk = (wn * WTN + j * 32 + 16 * ((lane >> 4) & 1)) / 8 + ((r & 3) >> 1);
      tb[j] = swz_rows(n, chunk) + 8 * (r & 1);
    }
  }
  // A fragments of step ks from an LDS tile (same k order as ARegs).
  __device__ inline void load_a(bf16x8 (&a)[FM], const char* As, int wm, int lane, int ks) const {
    const int chunk = 4 * (lane >> 5) + ks;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      a[i] = *reinterpret_cast<const bf16x8*>(As + swz(wm * WTM + i * 32 + (lane & 31), chunk));
  }
  __device__ inline void mfma(const bf16x8 (&a)[FM], const bf16x8 (&b)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = mfma_t(a[i], b[j], acc[i][j]);
  }
  __device__ inline void mfma(const u32x4 (&a)[FM][4], int ks, const bf16x8 (&b)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = mfma_t(__builtin_bit_cast(bf16x8, a[i][ks]), b[j], acc[i][j]);
  }
};

}  // namespace

namespace {

// Accumulators from a float32 tile (accumulator layout: see mfma_t); rows
// past the end start at zero.
template <int FM, int FN>
__device__ inline void load_acc(floatx16 (&acc)[FM][FN], const GemmArgs& g, int64_t wrow0,
                                int64_t wcol0, int lane) {
  const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t row = wrow0 + i * 32 + lr;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = wcol0 + j * 32 + 8 * q + 4 * lh;
        floatx4 v = {0.0f, 0.0f, 0.0f, 0.0f};
        if (row < g.rows && col < g.cols)
          v = *reinterpret_cast<const floatx4*>(g.c_init + row * g.ldc + col);
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[i][j][4 * q + c] = v[c];
      }
  }
}

// Keep bits of the run of four columns col..col+3 of a row (col % 4 == 0, so
// the run lies inside one 8-element generator block).
__device__ inline uint32_t keep_bits4(const GemmArgs& g, int64_t row, int64_t col) {
  const int64_t f = row * g.cols + col;
  return keep_bits8(g.drop, (uint64_t)f >> 3) >> (f & 7);
}

}  // namespace

template <int MT, int NT, int WM, int WN, int BMODE, bool PROLOGUE, int OMODE, int AMODE>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  static_assert(WM * WN == 4, "4 waves");
  using MmaT = Mma<MT, NT, WM, WN>;
  constexpr int FM = MmaT::FM, FN = MmaT::FN, WTM = MmaT::WTM, WTN = MmaT::WTN;
  // LDS: the 16-entry codebook at offset 0, then two stages of [A tile (when
  // A is staged), B tile].
  constexpr int CB_BYTES = 64;
  constexpr int A_STAGE = AMODE == A_DMA ? MT * ROWB : 0;
  constexpr int STAGE = A_STAGE + NT * ROWB;
  __shared__ __attribute__((aligned(16))) char lds[CB_BYTES + 2 * STAGE];
  float* cb = reinterpret_cast<float*>(lds);
  auto As = [&](int st) { return lds + CB_BYTES + st * STAGE; };
  auto Bs = [&](int st) { return lds + CB_BYTES + st * STAGE + A_STAGE; };

  const int tid = threadIdx.x;
  // The wave index is uniform; saying so keeps everything derived from it
  // (tile corners, buffer resources, row offsets) in scalar registers.
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  if constexpr (BMODE == B_NF4_COLS || BMODE == B_NF4_RED) {
    if (tid < 16) cb[tid] = bits_to_float(kNF4Bits[tid]);
  }

  // Workgroups are dealt to the 8 XCDs round-robin (workgroup b runs on XCD
  // b mod 8).  Give each XCD a contiguous run of tiles, in an order that
  // walks 4 tile rows at a time (down the 4 rows, then the next column): the
  // 32 workgroups an XCD runs at once then cover about 4 x 8 tiles and share
  // both their A rows and their B columns through that XCD's L2.
  const int ntiles = g.tiles_m * g.tiles_n;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int per = ntiles >> 3, rem = ntiles & 7;
  const int tile = xcd * per + min(xcd, rem) + slot;
  // (The divisions expand to vector code; readfirstlane brings the results
  // back to scalar registers, so buffer resources built from them are too.)
  constexpr int GM = 4;
  const int grp = __builtin_amdgcn_readfirstlane(tile / (GM * g.tiles_n));
  const int gsz = min(g.tiles_m - grp * GM, GM);  // rows in this group
  const int in = tile - grp * GM * g.tiles_n;
  const int tm = __builtin_amdgcn_readfirstlane(grp * GM + in % gsz);
  const int tn = __builtin_amdgcn_readfirstlane(in / gsz);
  const int64_t row0 = (int64_t)tm * MT, col0 = (int64_t)tn * NT;
  const int64_t wrow0 = row0 + wm * WTM;  // this wave's first row
  const int nkt_total = (int)((g.red + KT - 1) / KT);
  const int kt_begin = blockIdx.y * g.kt_per_split;
  const int kt_end = min(nkt_total, kt_begin + g.kt_per_split);

  MmaT mma;
  mma.zero();

  if constexpr (PROLOGUE) {
    // acc = s · L·Rᵀ over the rank dimension, L through registers (scaled by s
    // there: two bf16 parts when s·L is not exact in one), R through LDS.
    if (blockIdx.y == 0 && g.c_init != nullptr) {
      load_acc<FM, FN>(mma.acc, g, wrow0, col0 + wn * WTN, lane);
    } else if (blockIdx.y == 0 && g.rl > 0) {
      ARegs<FM> la;
      la.init(g.pl, g.ldpl, g.rows, wrow0, lane);
      RowTile<NT> rt;
      if (!g.pr_rc) rt.init(g.pr, g.ldpr, g.cols, col0, tid);
      for (int64_t j0 = 0; j0 < g.rl; j0 += KT) {
        la.load(j0, g.rl);
        if (g.pr_rc) {  // R stored by rank: 8 x 8 transposes on the way into LDS
          RcTile<NT> rc;
          rc.load(g.pr, g.ldpr, g.rl, g.cols, j0, col0, tid);
          rc.store(Bs(0), tid);
        } else {
          rt.load(j0, g.rl, tid);
          rt.store(Bs(0), tid);
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          bf16x8 b[FN];
          mma.load_b(b, Bs(0), wn, lane, ks);
          u32x4 a[FM][4];
#pragma unroll
          for (int i = 0; i < FM; ++i) a[i][ks] = scale_part(la.r[i][ks], g.s, 0);
          mma.mfma(a, ks, b);
          if (g.s_split) {
#pragma unroll
            for (int i = 0; i < FM; ++i) a[i][ks] = scale_part(la.r[i][ks], g.s, 1);
            mma.mfma(a, ks, b);
          }
        }
        __syncthreads();
      }
    }
  }

  constexpr bool kRows = BMODE == B_NF4_RED && AMODE == A_DMA;  // row-major B, transposed reads
  static_assert(BMODE == B_NF4_COLS || BMODE == B_NF4_RED || BMODE == B_BF16_RC, "B mode");
  using BTile = typename std::conditional<
      BMODE == B_NF4_COLS, Nf4ColsTile<NT>,
      typename std::conditional<BMODE == B_NF4_RED,
                                typename std::conditional<kRows, Nf4RowsTile, Nf4RedTile<NT>>::type,
                                RcTile<NT>>::type>::type;
  ARegs<(AMODE == A_DIRECT) ? FM : 1> a;
  if constexpr (AMODE == A_DIRECT) a.init(g.a, g.lda, g.rows, wrow0, lane);
  BTile b0, b1;
  if constexpr (BMODE == B_NF4_COLS || BMODE == B_NF4_RED) {
    b0.init(g, col0, tid);
    b1.init(g, col0, tid);
  }
  const int64_t kend = min(g.red, (int64_t)kt_end * KT);  // this split's reduction bound

  auto load_b = [&](BTile& bt, int kt) {
    const int64_t k0 = (int64_t)kt * KT;
    if constexpr (BMODE == B_NF4_COLS) {
      bt.load(k0, kend);
    } else if constexpr (kRows) {
      bt.load(g, k0, kend);
    } else if constexpr (BMODE == B_NF4_RED) {
      bt.load(g, k0, kend, tid);
    } else {
      bt.load(g.b, g.ldb, kend, g.cols, k0, col0, tid);
    }
  };
  // Quarter q of a B tile into stage st; the NF4 tiles fold their scales
  // (prep) before the first quarter, once per load.
  auto store_b = [&](BTile& bt, int st, int q) {
    if constexpr (BMODE == B_NF4_COLS || BMODE == B_NF4_RED) {
      if (q == 0) bt.prep();
      bt.store_part(Bs(st), tid, cb, q);
    } else {
      bt.store_part(Bs(st), tid, q);
    }
  };
  // One K tile of MFMAs: A from registers, B from LDS stage `cur`.  After the
  // MFMAs of each 16-deep step: that step's A registers are reloaded in place
  // with tile kt_next, and a quarter of the next B tile is decoded into stage
  // cur ^ 1.  B fragments are read one step ahead.  sched_barrier keeps the
  // compiler from regrouping the steps.
  auto step = [&](int cur, BTile& bt_next, int kt_next) {
    const int64_t kn = (int64_t)kt_next * KT;
    bf16x8 f0[FN], f1[FN];
    mma.load_b(f0, Bs(cur), wn, lane, 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8(&fc)[FN] = (ks & 1) ? f1 : f0;
      bf16x8(&fn)[FN] = (ks & 1) ? f0 : f1;
      if (ks < 3) mma.load_b(fn, Bs(cur), wn, lane, ks + 1);
      if constexpr (AMODE == A_DIRECT) {
        mma.mfma(a.r, ks, fc);
        a.load_ks(kn, kend, ks);
      }
      store_b(bt_next, cur ^ 1, ks);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if constexpr (AMODE == A_DMA) {
    // A arrives by direct-to-LDS loads, B is decoded from registers into the
    // stage not being read.  Per K tile (stage cur, B registers D holding
    // the next tile, N the one after):
    //   quarters 0-2: fragments of step ks+1 and the codebook reads of
    //                 quarter ks+1 are issued, then the MFMAs of step ks run
    //                 beside the scaling/rounding/stores of quarter ks;
    //   quarter 3:    half the MFMAs beside the last quarter's decode, then the
    //                 one barrier of the tile; after it the A loads of tile +2
    //                 go to stage cur, D is reloaded with tile +3, and the first
    //                 fragments of the next stage and codebook reads of N are
    //                 issued before the second half of the MFMAs, which use
    //                 registers only.
    // The barrier needs this wave's A loads landed (vmcnt 0: they and the B
    // loads issued with them are a whole tile old by then).
    ADma<MT> adma;
    adma.init(g.a, g.lda, g.rows, row0, wave, lane);
    constexpr int kDsr = BMODE == B_NF4_RED ? 3 : 2, kValu = BMODE == B_NF4_RED ? 3 : 4;
    bf16x8 fa0[FM], fa1[FM], fb0[FN], fb1[FN];
    float lk0[16], lk1[16];
    // Codebook reads a quarter ahead where registers allow (column tiles: one
    // block per thread); the reduction-major tile, with eight block scales per
    // thread, reads and finishes each quarter in place.
    constexpr bool kAhead = BMODE == B_NF4_COLS || kRows;
    int tb[FN];
    if constexpr (kRows) mma.tr_base(tb, wn, lane);
    auto load_bf = [&](bf16x8 (&f)[FN], int st, int ks) {
      if constexpr (kRows)
        mma.load_b_tr(f, Bs(st), tb, ks);
      else
        mma.load_b(f, Bs(st), wn, lane, ks);
    };
    auto lookup = [&](const BTile& bt, int q, float (&v)[16]) {
      if constexpr (kAhead) bt.lookup(q, v, cb);
    };
    auto finish = [&](const BTile& bt, int q, const float (&v)[16], int st) {
      if constexpr (kAhead)
        bt.finish(q, v, Bs(st), tid);
      else if constexpr (BMODE == B_NF4_RED && !kRows)
        bt.store_part(Bs(st), tid, cb, q);
    };
    auto mfma_half = [&](const bf16x8 (&a)[FM], const bf16x8 (&b)[FN], int h) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          if ((i * FN + j) * 2 / (FM * FN) == h)
            mma.acc[i][j] = mfma_t(a[i], b[j], mma.acc[i][j]);
    };
    auto stepd = [&](int cur, BTile& D, BTile& N, int kt) {
      D.prep();
#pragma unroll
      for (int ks = 0; ks < 3; ++ks) {
        bf16x8(&ac)[FM] = (ks & 1) ? fa1 : fa0;
        bf16x8(&an)[FM] = (ks & 1) ? fa0 : fa1;
        bf16x8(&bc)[FN] = (ks & 1) ? fb1 : fb0;
        bf16x8(&bn)[FN] = (ks & 1) ? fb0 : fb1;
        float(&lc)[16] = (ks & 1) ? lk1 : lk0;
        float(&ln)[16] = (ks & 1) ? lk0 : lk1;
        mma.load_a(an, As(cur), wm, lane, ks + 1);
        load_bf(bn, cur, ks + 1);
        lookup(D, ks + 1, ln);
        mma.mfma(ac, bc);
        finish(D, ks, lc, cur ^ 1);
        interleave<FM * FN, kDsr, kValu>();
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma_half(fa1, fb1, 0);
      finish(D, 3, lk1, cur ^ 1);
      interleave<FM * FN / 2, kDsr, kValu>();
      __builtin_amdgcn_sched_barrier(0);
      wait_vmem_all();
      __syncthreads();
      mma.load_a(fa0, As(cur ^ 1), wm, lane, 0);
      load_bf(fb0, cur ^ 1, 0);
      lookup(N, 0, lk0);
      adma.issue(As(cur), (int64_t)(kt + 2) * KT, kend);
      load_b(D, kt + 3);
      mfma_half(fa1, fb1, 1);
      interleave<FM * FN / 2, kDsr, kValu>();
      __builtin_amdgcn_sched_barrier(0);
    };
    if (kt_begin < kt_end) {
      __syncthreads();  // codebook visible, prologue done with stage 0
      adma.issue(As(0), (int64_t)kt_begin * KT, kend);
      adma.issue(As(1), (int64_t)(kt_begin + 1) * KT, kend);
      load_b(b0, kt_begin);
      load_b(b1, kt_begin + 1);
#pragma unroll
      for (int q = 0; q < 4; ++q) store_b(b0, 0, q);
      load_b(b0, kt_begin + 2);
      wait_vmem_all();
      __syncthreads();
      mma.load_a(fa0, As(0), wm, lane, 0);
      load_bf(fb0, 0, 0);
      lookup(b1, 0, lk0);
      // Branch-free: tiles past kt_end load as zeros, so an odd count ends
      // with one MFMA pass over a zero tile.
      for (int kt = kt_begin; kt < kt_end; kt += 2) {
        stepd(0, b1, b0, kt);
        stepd(1, b0, b1, kt + 1);
      }
    }
  } else if (kt_begin < kt_end) {
    __syncthreads();  // codebook visible, prologue done with stage 0
    a.load((int64_t)kt_begin * KT, kend);
    load_b(b0, kt_begin);
    load_b(b1, kt_begin + 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) store_b(b0, 0, q);
    __syncthreads();
    // Branch-free: tiles past kt_end load as zeros, so an odd count ends with
    // one MFMA pass over a zero tile.
    for (int kt = kt_begin; kt < kt_end; kt += 2) {
      load_b(b0, kt + 2);
      step(0, b1, kt + 1);
      __syncthreads();
      load_b(b1, kt + 3);
      step(1, b0, kt + 2);
      __syncthreads();
    }
  }

  // Epilogue (accumulator layout: see mfma_t).  Lane l owns row
  // wrow0 + 32 i + l mod 32 of block i and, in column block j, the runs of
  // four columns 32 j + 8 g + 4 (l / 32) .. +3.
  const int lr = lane & 31, lh = lane >> 5;
  const int64_t wcol0 = col0 + wn * WTN;
  if (wrow0 + WTM <= g.rows && wcol0 + WTN <= g.cols && (g.ldo & 3) == 0) {
    // Whole wave tile in range, rows 8-byte aligned: one 8-byte (bf16) or
    // 16-byte (fp32) store per run, at a constant offset from the row start.
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t row = wrow0 + i * 32 + lr;
      if constexpr (OMODE == O_BF16) {
        uint16_t* o = g.out_bf16 + row * g.ldo + wcol0 + 4 * lh;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const floatx16& c = mma.acc[i][j];
            u32x2 v;
            v[0] = pack_bf16x2(c[4 * q], c[4 * q + 1]);
            v[1] = pack_bf16x2(c[4 * q + 2], c[4 * q + 3]);
            *reinterpret_cast<u32x2*>(o + 32 * j + 8 * q) = v;
          }
      } else {
        float* o = g.out_f32 + (int64_t)blockIdx.y * g.part_stride + row * g.ldo + wcol0 + 4 * lh;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const floatx16& c = mma.acc[i][j];
            floatx4 v{c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]};
            if (g.drop.thr > 0) {
              const uint32_t keep = keep_bits4(g, row, wcol0 + 32 * j + 8 * q + 4 * lh);
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = ((keep >> e) & 1u) ? g.s * v[e] : 0.0f;
            }
            *reinterpret_cast<floatx4*>(o + 32 * j + 8 * q) = v;
          }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t row = wrow0 + i * 32 + lr;
    if (row >= g.rows) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t col = wcol0 + j * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
        if (col >= g.cols) continue;
        float v = mma.acc[i][j][e];
        if constexpr (OMODE == O_BF16) {
          g.out_bf16[row * g.ldo + col] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
        } else {
          if (g.drop.thr > 0)
            v = ((keep_bits4(g, row, col & ~(int64_t)3) >> (col & 3)) & 1u) ? g.s * v : 0.0f;
          g.out_f32[(int64_t)blockIdx.y * g.part_stride + row * g.ldo + col] = v;
        }
      }
  }
}

// Instantiations used by the library.
#define QLORA_GEMM(MT, NT, WM, WN, BM, PRO, OM, AM) \
  template __global__ void gemm_kernel<MT, NT, WM, WN, BM, PRO, OM, AM>(GemmArgs);

QLORA_GEMM(256, 256, 2, 2, B_NF4_COLS, true, O_BF16, A_DMA)     // forward, many tokens
QLORA_GEMM(256, 256, 2, 2, B_NF4_RED, true, O_BF16, A_DMA)     // input gradient, many tokens
QLORA_GEMM(64, 256, 1, 4, B_NF4_COLS, true, O_F32, A_DIRECT)    // forward, 17..127 tokens (split-K)
QLORA_GEMM(64, 256, 1, 4, B_NF4_RED, true, O_F32, A_DIRECT)     // input gradient, 17..127 tokens
QLORA_GEMM(64, 256, 2, 2, B_BF16_RC, false, O_F32, A_DIRECT)    // dropout: T = s·mask ⊙ (V·A)

}  // namespace qlora
