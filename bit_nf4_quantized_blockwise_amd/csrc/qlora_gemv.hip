// Few-token QLoRA forward (M <= 16 tokens) for gfx950: stream the NF4 weight
// once from HBM with 16-byte loads and contract it on the matrix cores.
//
//   Y[m][n] = Σ_b â_b · Σ_{k in block b} X[m][k] · c_bf16[idx(n, k)]  +  s · Σ_j U[m][j] · B[n][j]
//
// ("QLoRAの理論と実装", QLoRAの計算フロー: the main path plus the rank-r adapter
// path, here for decode-sized batches.)  The block scale â_b = RN32(c2 · q)
// (Qiita explainer, DQ formula) multiplies the fp32 partial sum of its block
// instead of every weight: this keeps the per-weight work to one table lookup
// per two weights.  The codebook enters the bf16 MFMA rounded to bf16, so the
// result differs from "decode each weight to bf16, then multiply" only by
// rounding (well inside the forward's tolerance); the many-token GEMMs decode
// every weight exactly.
//
// Layout of one v_mfma_f32_16x16x32_bf16 (a chunk = 128 k = two 64-blocks):
//   B operand: lane (c = l%16, q = l/16) holds 8 consecutive weights of W row
//     n0 + c, taken from its own 16-byte load of 32 weights at k = kb + 32q
//     (the four MFMAs of a chunk take bytes 4j..4j+3, j = 0..3).
//   A operand: rows 0..7 carry tokens 0..7 restricted to the lanes with q < 2
//     (block kb/64), rows 8..15 the same tokens restricted to q >= 2 (block
//     kb/64 + 1); the other entries are zero.  So C rows 0..7 hold the first
//     block's partial sums and rows 8..15 the second's, and every lane scales
//     the rows it holds by the scale of the block it loaded itself.
// 8 waves split the reduction; each wave walks all of its workgroup's column
// groups and the partial sums meet in LDS once, at the end.

#include "qlora_kernels.h"

namespace qlora {

namespace {

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9)

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffffLL : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kRsrcWord3);
}

// Workgroup barrier that waits for this wave's LDS operations only (global
// loads stay in flight across it).
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ inline uint16_t bf16_rne_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// kNF4Bits[i] for a per-lane i, as a tree of selects between literals (no
// memory read).
template <int LO, int N>
__device__ inline uint32_t level_bits_tree(int i) {
  if constexpr (N == 1) {
    return kNF4Bits[LO];
  } else {
    return (i & (N / 2)) ? level_bits_tree<LO + N / 2, N / 2>(i) : level_bits_tree<LO, N / 2>(i);
  }
}
__device__ inline uint32_t level_bits(int i) { return level_bits_tree<0, 16>(i); }

}  // namespace

template <int CPW, int MG, int G, bool QV>
__global__ __launch_bounds__(64 * kGemvWaves) void nf4_gemv_kernel(GemvArgs g) {
  // LDS: the codebook table (64 KB), then the per-wave partial sums (reduced
  // once at the end), then the U rows of the adapter term.  The token
  // staging area (the workgroup's k range of X, all M tokens, loaded densely
  // once and read back in operand order) lies over the partial sums for up
  // to 4 tokens and over the table and the partial sums beyond, so there the
  // table is filled after the operands have been read.
  constexpr int NT = 64 * kGemvWaves;
  constexpr int kLut = 256 * 64 * 4;
  constexpr int kSpan = kGemvWaves * CPW * 128;  // k range of one workgroup
  constexpr int kRedBytes = kGemvWaves * G * MG * 32 * 4 * 4;
  constexpr int kStage4 = MG == 1 ? 4 * kSpan * 2 : 0;  // up to 4 tokens, after the table
  constexpr int kStageAll = 8 * MG * kSpan * 2;         // all token groups, from the start
  constexpr int kRedRegion = kRedBytes > kStage4 ? (kRedBytes > kStageAll - kLut ? kRedBytes : kStageAll - kLut)
                                                 : (kStage4 > kStageAll - kLut ? kStage4 : kStageAll - kLut);
  __shared__ __attribute__((aligned(16))) char smem[kLut + kRedRegion];
  // byte e -> the two bf16 levels of its nibbles, 64 copies: entry e of lane
  // l at byte 256 e + 4 l, so a lookup address is one v_perm of the packed
  // dword and the lane's offset, and the 64 lanes hit 64 different banks.
  uint32_t* lut = reinterpret_cast<uint32_t*>(smem);
  char* red_stage = smem + kLut;
  float(*red)[G][MG][32][4] = reinterpret_cast<float(*)[G][MG][32][4]>(red_stage);
  // U rows for the adapter term (M <= 16, r <= 256); its first 2 KB are the
  // zeros that token-less lanes read while the staging area is in use
  __shared__ __attribute__((aligned(16))) uint16_t ush[16 * 256];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c16 = lane & 15, qd = lane >> 4;
  const int64_t K = g.K, N = g.N;
  const int M = g.M;
  const int64_t chunk0 = ((int64_t)blockIdx.y * kGemvWaves + w) * CPW;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(g.x, (int64_t)M * K * 2);

  // The workgroup's tokens come in as dense 16-byte loads (about M·CPW / 4
  // per lane) instead of 4·CPW·MG partly empty ones per wave, so the 256
  // workgroups put far fewer requests on the same lines of X.  The loads go
  // out first.
  const bool early_lut = MG == 1 && M <= 4;  // uniform
  constexpr int kPieces = 8 * MG * kSpan / 8 / NT;  // 16-byte pieces per lane at 8·MG tokens
  const int rounds = (M * (kSpan / 8) + NT - 1) / NT;      // the rounds that carry tokens
  const int64_t kw0 = (int64_t)blockIdx.y * kSpan;
  u32x4 xs[kPieces];
  {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      if (i < rounds) {
        const int p = tid + NT * i, tok = p / (kSpan / 8);
        const int64_t k = kw0 + (int64_t)(p % (kSpan / 8)) * 8;
        const bool valid = tok < M && k < K;
        xs[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              xr, valid ? (int)(((int64_t)tok * K + k) * 2) : 0x7ffffff0, 0, 0));
      }
    }
  }

  // Table fill: thread t writes entries e = t / 16 + (NT / 16) it (four
  // copies each), whose low nibble t / 16 mod 16 is fixed and whose high
  // nibble is t / 256 + (NT / 256) it; the levels come from literals.
  static_assert(NT % 256 == 0 && 256 * 16 % NT == 0, "table fill");
  auto fill_table = [&]() {
    const uint32_t lo = bf16_rne_bits(bits_to_float(level_bits((tid >> 4) & 15)));
#pragma unroll
    for (int it = 0; it < 256 * 16 / NT; ++it) {
      const uint32_t hi = bf16_rne_bits(bits_to_float(level_bits((tid >> 8) + (NT / 256) * it)));
      const uint32_t v = lo | (hi << 16);
      *reinterpret_cast<u32x4*>(&lut[(tid + it * NT) * 4]) = u32x4{v, v, v, v};
    }
  };
  if (early_lut) fill_table();
  char* stage = early_lut ? red_stage : smem;
  {
    *reinterpret_cast<uint32_t*>(ush + 2 * tid) = 0u;  // NT · 4 B = 2 KB of zeros
#pragma unroll
    for (int i = 0; i < kPieces; ++i)
      if (i < rounds) *reinterpret_cast<u32x4*>(stage + (size_t)(tid + NT * i) * 16) = xs[i];
  }
  __syncthreads();

  // Token operands for this wave's chunks, kept in registers for all columns:
  // a lane carries token c16 mod 8 (+ 8 mg) of block (c16 >= 8) and zeros
  // elsewhere, read back from the staging area once the first weight loads
  // are out.
  u32x4 xa[MG][CPW][4];

  const char* lutb = reinterpret_cast<const char*>(lut);
  const uint32_t lane4 = (uint32_t)lane * 4;
  const int64_t blocks_per_row = K >> 6;
  const __amdgpu_buffer_rsrc_t c2r = make_rsrc(g.c2, ((N * blocks_per_row + 255) >> 8) * 4);
  const int64_t cg0 = (int64_t)blockIdx.x * G;

  // Every wave walks all G column groups of the workgroup on its own slice
  // of the reduction; no workgroup barrier until the end, so the waves drift
  // apart and one wave's loads overlap another's MFMAs.  Within a wave the
  // weight loads run one column group ahead: as soon as chunk c of group gi
  // has been turned into MFMA operands, its registers are reloaded with
  // chunk c of group gi + 1, so D 16-byte loads per lane stay in flight.
  const int64_t nw0 = cg0 * 16;  // first W row of this workgroup
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(g.packed + nw0 * (K >> 1), (N - nw0) * (K >> 1));
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(g.qabsmax + nw0 * blocks_per_row,
                                              (N - nw0) * blocks_per_row);
  // Weight chunks stream through a ring of D registers: step s = gi·CPW + c
  // consumes slot s mod D and refills it with step s + D, so D 16-byte loads
  // per lane stay in flight.  A register spill here would be worse than a
  // shallower ring: reloading it waits (in issue order) for every weight load
  // issued before it.
  constexpr int D = CPW > 6 ? 6 : CPW;  // six in flight: eight make the widest variant spill
  constexpr int S = G * CPW;
  u32x4 pk[D];
  auto load = [&](int st) {
    if (st >= S) return;
    const int gi = st / CPW, c = st % CPW;
    const int64_t kq = (chunk0 + c) * 128 + 32 * qd;
    const int64_t nl = (int64_t)gi * 16 + c16;  // W row relative to nw0
    const int off = (int)((nl * K + kq) >> 1);
    pk[st % D] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(pr, kq < K ? off : 0x7ffffff0, 0, 0));
  };
  // Block scales of one column group: the lane's chunks c = 0..CPW-1 use
  // blocks b0 + 2c + (qd >= 2) of its row, so its DQ codes are the 2·CPW
  // bytes from b0 (fetched as dwords when the row pitch in blocks is a
  // multiple of 4, else byte by byte), and they span at most two DQ groups.
  // Bytes past a row's end belong to the next row; they only ever scale
  // partial sums that are zero (weights past K meet zero tokens).
  constexpr int QW = (2 * CPW + 3) / 4;
  struct Scales {
    uint32_t q[QW];
    uint32_t c2a, c2b;
    int sw;  // first byte of the run that falls in the second DQ group
  };
  auto load_scales = [&](int gi, Scales& sc) {
    const int64_t nl = (int64_t)gi * 16 + c16;
    const int b0 = (int)(nl * blocks_per_row + 2 * chunk0);  // relative to row nw0
    if constexpr (QV) {
#pragma unroll
      for (int i = 0; i < QW; ++i) sc.q[i] = __builtin_amdgcn_raw_buffer_load_b32(qr, b0 + 4 * i, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < QW; ++i) {
        uint32_t v = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          v |= __builtin_amdgcn_raw_buffer_load_b8(qr, b0 + 4 * i + t, 0, 0) << (8 * t);
        sc.q[i] = v;
      }
    }
    const int64_t gb = nw0 * blocks_per_row + b0;
    sc.sw = 256 - (int)(gb & 255);
    sc.c2a = __builtin_amdgcn_raw_buffer_load_b32(c2r, (int)((gb >> 8) * 4), 0, 0);
    sc.c2b = __builtin_amdgcn_raw_buffer_load_b32(c2r, (int)((gb >> 8) * 4) + 4, 0, 0);
  };
  auto scale_of = [&](const Scales& sc, int c) {
    const int i = 2 * c + (qd >> 1);  // byte within the lane's run
    const uint32_t q = (sc.q[(2 * c) >> 2] >> (8 * (i & 3))) & 0xffu;
    return __builtin_bit_cast(float, i >= sc.sw ? sc.c2b : sc.c2a) * (float)q;
  };
  Scales sA, sB;
#pragma unroll
  for (int st = 0; st < D; ++st) load(st);  // rows past N read as zero
  load_scales(0, sA);
  {
    // the lane's 4·CPW operand pieces per token group are 16-byte reads at
    // fixed offsets from one base: its token's row (wave slice, k-slot qd) or
    // the zeros
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) {
      const int tok = (c16 & 7) + 8 * mg;
      const bool valid = ((c16 < 8) == (qd < 2)) && tok < M;
      const char* base = valid ? stage + ((size_t)tok * kSpan + (size_t)w * CPW * 128 + 32 * qd) * 2
                               : reinterpret_cast<const char*>(ush) + 64 * qd;
#pragma unroll
      for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          xa[mg][c][j] = *reinterpret_cast<const u32x4*>(base + c * 256 + 16 * j);
    }
    // the staging area becomes the partial sums (and the table): every wave
    // has read it first (the weight loads just issued stay in flight across
    // these barriers)
    lds_barrier();
    if (!early_lut) {
      fill_table();
      lds_barrier();
    }
  }
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    Scales& sc = (gi & 1) ? sB : sA;
    if (gi + 1 < G) load_scales(gi + 1, (gi & 1) ? sA : sB);
    floatx4 acc[MG];
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) acc[mg] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int st = gi * CPW + c;
      u32x4 bop[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t p = pk[st % D][j];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          bop[j][t] = *reinterpret_cast<const uint32_t*>(
              lutb + __builtin_amdgcn_perm(p, lane4, 0x0c0c0400u + (t << 8)));
      }
      load(st + D);  // refills the slot just read; rows past N read as zero
      floatx4 cb[MG];
#pragma unroll
      for (int mg = 0; mg < MG; ++mg) cb[mg] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int mg = 0; mg < MG; ++mg)
          cb[mg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[mg][c][j]),
                                                           __builtin_bit_cast(bf16x8, bop[j]), cb[mg],
                                                           0, 0, 0);
      const float ah = scale_of(sc, c);
#pragma unroll
      for (int mg = 0; mg < MG; ++mg)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mg][i] += ah * cb[mg][i];
    }
    // rows r and r + 8 hold the same token for the two blocks of each chunk;
    // the group's sums leave for LDS right away
#pragma unroll
    for (int mg = 0; mg < MG; ++mg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[mg][i] += __shfl_xor(acc[mg][i], 32);
        if (lane < 32) red[w][gi][mg][lane][i] = acc[mg][i];
      }
  }
  // Adapter term (split 0 only): the workgroup's G·16 rows of B and the M
  // rows of U are staged in LDS (B where the table was), so each output's
  // rank-r dot product reads LDS instead of issuing r dependent global loads.
  const bool lora = blockIdx.y == 0 && g.r > 0;
  uint16_t* bsh = reinterpret_cast<uint16_t*>(lut);  // [G·16][r]; r <= 256 fits the table
  const int nb = G * 16 * g.r;  // B rows nw0 .. nw0 + 16 G are contiguous
  const int64_t bvalid = (N - nw0) * g.r;
  const bool bvec = (g.r & 7) == 0;  // 16-byte pieces (B is 16-byte aligned)
  // The first piece of B and of U per lane is fetched before the barrier, so
  // its latency overlaps the wait for the workgroup's slowest wave.
  u32x4 b_first = u32x4{0u, 0u, 0u, 0u};
  uint16_t u_first = 0;
  if (lora) {
    if (bvec && tid * 8 < nb && tid * 8 < bvalid)
      b_first = *reinterpret_cast<const u32x4*>(g.b + nw0 * g.r + tid * 8);
    if (tid < M * g.r) u_first = g.u[tid];
  }
  __syncthreads();  // every wave is done with the table
  if (lora) {
    if (bvec) {
      if (tid * 8 < nb) *reinterpret_cast<u32x4*>(bsh + tid * 8) = b_first;
      for (int i = (tid + NT) * 8; i < nb; i += NT * 8)
        *reinterpret_cast<u32x4*>(bsh + i) =
            i < bvalid ? *reinterpret_cast<const u32x4*>(g.b + nw0 * g.r + i) : u32x4{0u, 0u, 0u, 0u};
    } else {
      for (int i = tid; i < nb; i += NT) bsh[i] = i < bvalid ? g.b[nw0 * g.r + i] : (uint16_t)0;
    }
    if (tid < M * g.r) ush[tid] = u_first;
    for (int i = tid + NT; i < M * g.r; i += NT) ush[i] = g.u[i];
  }
  __syncthreads();
  for (int o = tid; o < G * MG * 128; o += NT) {
    const int gi = o / (MG * 128), mg = (o / 128) % MG, t = o & 127;
    const int tok8 = t >> 4, col = t & 15;
    float v = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kGemvWaves; ++ww) v += red[ww][gi][mg][col + 16 * (tok8 >> 2)][tok8 & 3];
    const int tok = tok8 + 8 * mg;
    const int64_t n = (cg0 + gi) * 16 + col;
    if (tok < M && n < N) {
      if (lora) {
        const uint16_t* ur = ush + tok * g.r;
        const uint16_t* br = bsh + (n - nw0) * g.r;
        float l = 0.0f;
        for (int jr = 0; jr < g.r; ++jr) l += bf16_bits_to_float(ur[jr]) * bf16_bits_to_float(br[jr]);
        v += g.s * l;
      }
      if (g.ksplit == 1)
        g.y[(int64_t)tok * N + n] = bf16_rne_bits(v);
      else
        g.part[((int64_t)blockIdx.y * M + tok) * N + n] = v;
    }
  }
}

// U[m][j] = Σ_k X[m][k] · A[j][k] for few tokens: one workgroup per (j, m),
// 1024 lanes of 8 k each per pass, so a pass over k = 8192 is one 16-byte
// load of A and one of X per lane, all in flight together.  Each lane sums
// its products in k order; the lanes of a wave meet in a fixed butterfly and
// the 16 waves in wave order, so runs are bitwise repeatable.
__global__ __launch_bounds__(kDownThreads) void lora_down_small_kernel(
    const uint16_t* __restrict__ x, int64_t K, const uint16_t* __restrict__ a, int r,
    uint16_t* __restrict__ u) {
  constexpr int NW = kDownThreads / 64;
  __shared__ float red[NW];
  const int j = blockIdx.x, m = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float acc = 0.0f;
  for (int64_t k = (int64_t)tid * 8; k < K; k += kDownThreads * 8) {
    const u32x4 av = *reinterpret_cast<const u32x4*>(a + (int64_t)j * K + k);
    const u32x4 xv = *reinterpret_cast<const u32x4*>(x + (int64_t)m * K + k);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      acc += bits_to_float(xv[d] << 16) * bits_to_float(av[d] << 16);
      acc += bits_to_float(xv[d] & 0xffff0000u) * bits_to_float(av[d] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) red[w] = acc;
  __syncthreads();
  if (tid == 0) {
    float v = 0.0f;
#pragma unroll
    for (int i = 0; i < NW; ++i) v += red[i];
    u[(int64_t)m * r + j] = bf16_rne_bits(v);
  }
}

// ---- small weights: the whole forward in one launch ----------------------------
// Y = RNE_bf16(X·Ŵᵀ + s·U·Bᵀ) and U = RNE_bf16(X·Aᵀ) for at most 16 tokens and
// kSmallMaxRank ranks ("QLoRAの理論と実装", QLoRAの計算フロー: the main path
// and the adapter path of one layer).  Ŵ is decoded as the dequantiser decodes
// it, RNE_bf16(RN32(c_idx · â)), so the matrix cores see the same bf16 weight
// as in the many-token GEMMs.  One workgroup per 16 output rows; its 16 waves
// split k into 128-k chunks (wave w takes chunks w, w + 16, ...), and every
// lane issues all of its loads (B's rows, weight codes, block scales, tokens,
// rows of A) before its first wait, so the launch pays one memory latency.
// Each 16×16×32 MFMA takes the 16 tokens as its rows: against the decoded
// weight it accumulates Y's partial sums, against 16 rows of A (zero past r)
// U's.  The waves' sums meet in LDS in wave order; every workgroup forms the
// same U (fixed order), rounds it to bf16 and adds s·U·Bᵀ to its columns, and
// workgroup 0 writes U.
//
// Lane (c = l % 16, q = l / 16) of a chunk at k0 holds weight row n0 + c at
// k = k0 + 32q .. k0 + 32q + 31 (one 16-byte load of 32 codes), and MFMA j of
// the chunk takes k0 + 32q + 8j .. + 7 on both operands: a permutation of k
// shared by both, so the sums are those of X·Ŵᵀ.  Every workgroup reads all of
// X and A, so those loads are the ones to keep cheap: each covers 4 rows ×
// 256 contiguous bytes (whole cache lines), and the chunk's 16 rows of tokens
// and of A pass through a wave-private LDS area (row pitch 272 B, so both the
// row writes and the operand reads are conflict-free) into operand order.
template <int CPW>
__global__ __launch_bounds__(64 * kSmallWaves) void nf4_small_fwd_kernel(SmallFwdArgs g) {
  constexpr int NW = kSmallWaves;
  constexpr int RP = kSmallMaxRank + 1;  // padded pitch of the LDS rows of B and U
  constexpr int SP = 272;                // staging row pitch: 128 bf16 + 16 B
  constexpr int kStage = 2 * 16 * SP;    // one wave's tokens and rows of A for one chunk
  static_assert(kStage >= 2 * 64 * 16, "a wave's sums fit its staging area");
  __shared__ __attribute__((aligned(16))) char stage[NW * kStage];
  __shared__ float cb[16];
  __shared__ float bsh[16 * RP];  // B[n0 + c][j] at c·RP + j
  __shared__ float ush[16 * RP];  // U rounded to bf16, token t at t·RP + j
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c16 = lane & 15, qd = lane >> 4;
  const int64_t K = g.K, N = g.N;
  const int M = g.M, r = g.r;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t n = n0 + c16;
  const int64_t bpr = K >> 6;  // 64-blocks per weight row

  // Raw buffer loads: an offset past a buffer's end reads zero, so the rows
  // past N, the tokens past M, the ranks past r and the k past K need no branch.
  constexpr int kOut = 0x7ffffff0;
  const int64_t rows = N - n0 < 16 ? N - n0 : 16;
  const __amdgpu_buffer_rsrc_t br = make_rsrc(g.b + n0 * r, rows * r * 2);
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(g.packed + n0 * (K >> 1), rows * (K >> 1));
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(g.qabsmax + n0 * bpr, rows * bpr);
  const __amdgpu_buffer_rsrc_t c2r = make_rsrc(g.c2, ((N * bpr + 255) >> 8) * 4);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(g.x, (int64_t)M * K * 2);
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(g.a, (int64_t)r * K * 2);

  // B's 16 rows first: the oldest load, so the wait before its LDS store waits
  // for nothing else
  const int bi = tid / r, bj = tid - bi * r;
  const uint32_t bv =
      __builtin_amdgcn_raw_buffer_load_b16(br, tid < 16 * r ? (bi * r + bj) * 2 : kOut, 0, 0);

  // xs/as: rows 4j + q of the chunk's tokens / rows of A, 16 bytes at k0 + 8c
  u32x4 pk[CPW], xs[CPW][4], as[CPW][4];
  uint32_t qv[CPW], c2v[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int k0 = (w + NW * i) * 128;
    const int kq = k0 + 32 * qd;
    const bool kin = kq < K;  // K % 64 == 0: a lane's 32 k are all in or all out
    pk[i] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(pr, kin ? (int)((c16 * K + kq) >> 1) : kOut, 0, 0));
    const int64_t b = n * bpr + (kq >> 6);  // the lane's 64-block
    int qoff = kin ? (int)(c16 * bpr + (kq >> 6)) : kOut;
    asm volatile("" : "+v"(qoff));  // one load with a lane offset, not one per side of the select
    qv[i] = __builtin_amdgcn_raw_buffer_load_b8(qr, qoff, 0, 0);
    c2v[i] = __builtin_amdgcn_raw_buffer_load_b32(c2r, kin && n < N ? (int)((b >> 8) * 4) : kOut, 0, 0);
    const bool cin = k0 + 8 * c16 < K;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 4 * j + qd;
      const int off = (int)((row * K + k0 + 8 * c16) * 2);
      // groups of 4 rows wholly past M (past r) are not loaded (a uniform branch)
      if (4 * j < M)
        xs[i][j] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, cin && row < M ? off : kOut, 0, 0));
      if (4 * j < r)
        as[i][j] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(ar, cin && row < r ? off : kOut, 0, 0));
    }
  }
  if (tid < 16) cb[tid] = bits_to_float(level_bits(tid));
  if (tid < 16 * r) bsh[bi * RP + bj] = bf16_bits_to_float(bv);
  lds_barrier();  // the codebook is in place; the other loads stay in flight

  const char* cbb = reinterpret_cast<const char*>(cb);
  char* xst = stage + w * kStage;  // this wave's tokens, then its rows of A
  char* ast = xst + 16 * SP;
  floatx4 accY = floatx4{0.f, 0.f, 0.f, 0.f}, accU = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    if ((w + NW * i) * 128 >= K) break;  // wave-uniform: no chunk left
    // rows into the staging area, then back in operand order (a wave's LDS
    // operations complete in order, so the next chunk's writes cannot pass
    // these reads).  Rows of groups that were not loaded keep whatever the area
    // held: a token row past M only reaches outputs of that token, which are
    // not stored, and a row of A past r only U's columns past r, which are
    // neither stored nor used.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (4 * j < M) *reinterpret_cast<u32x4*>(xst + (4 * j + qd) * SP + 16 * c16) = xs[i][j];
      if (4 * j < r) *reinterpret_cast<u32x4*>(ast + (4 * j + qd) * SP + 16 * c16) = as[i][j];
    }
    const float ah = __builtin_bit_cast(float, c2v[i]) * (float)(int8_t)qv[i];  // â = RN32(c2 · q)
    // the chunk's 32 levels first, so their LDS reads share one latency; the
    // decoded weight is RNE_bf16(RN32(level · â)), element 2t in the low nibble
    // of byte t
    float lv[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t ev = (pk[i][j] << 2) & 0x3c3c3c3cu;  // 4 · code of elements 0, 2, 4, 6
      const uint32_t od = (pk[i][j] >> 2) & 0x3c3c3c3cu;  // 4 · code of elements 1, 3, 5, 7
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        lv[j][2 * d] = *reinterpret_cast<const float*>(cbb + ((ev >> (8 * d)) & 0xffu));
        lv[j][2 * d + 1] = *reinterpret_cast<const float*>(cbb + ((od >> (8 * d)) & 0xffu));
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 xo = *reinterpret_cast<const u32x4*>(xst + c16 * SP + 64 * qd + 16 * j);
      const u32x4 ao = *reinterpret_cast<const u32x4*>(ast + c16 * SP + 64 * qd + 16 * j);
      u32x4 bop;
#pragma unroll
      for (int d = 0; d < 4; ++d) bop[d] = pack_bf16x2(lv[j][2 * d] * ah, lv[j][2 * d + 1] * ah);
      accY = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xo),
                                                     __builtin_bit_cast(bf16x8, bop), accY, 0, 0, 0);
      accU = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xo),
                                                     __builtin_bit_cast(bf16x8, ao), accU, 0, 0, 0);
    }
  }
  // each wave's sums go to its own staging area (after its own last reads of
  // it: no barrier needed for that), Y's at offset 0, U's at 1 KB
  reinterpret_cast<floatx4*>(xst)[lane] = accY;
  reinterpret_cast<floatx4*>(xst + 1024)[lane] = accU;
  __syncthreads();
  // output (token t, column c) sits in lane 16·(t / 4) + c, entry t % 4
  const int t = tid >> 4, c = tid & 15;
  const int src = 16 * (t >> 2) + c, e = t & 3;
  auto red = [&](int ww, int part) {
    return reinterpret_cast<const floatx4*>(stage + ww * kStage + part * 1024)[src][e];
  };
  if (tid < 256) {
    float u = 0.0f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) u += red(ww, 1);
    const uint16_t ub = bf16_rne_bits(u);
    ush[t * RP + c] = bf16_bits_to_float(ub);
    if (blockIdx.x == 0 && t < M && c < r) g.u[t * r + c] = ub;
  }
  __syncthreads();
  if (tid < 256 && t < M && n0 + c < N) {
    float y = 0.0f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) y += red(ww, 0);
    float l = 0.0f;
    for (int j = 0; j < r; ++j) l += ush[t * RP + j] * bsh[c * RP + j];
    g.y[(int64_t)t * N + n0 + c] = bf16_rne_bits(y + g.s * l);
  }
}

template __global__ void nf4_small_fwd_kernel<1>(SmallFwdArgs);
template __global__ void nf4_small_fwd_kernel<2>(SmallFwdArgs);

template __global__ void nf4_gemv_kernel<1, 1, 1, false>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 1, 2, false>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 1, 3, false>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 1, 4, false>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 1, 5, false>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 1, 6, false>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 1, 7, false>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 1, 8, false>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 1, 1, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 1, 2, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 1, 3, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 1, 4, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 1, 5, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 1, 6, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 1, 7, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 1, 8, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 1, 1, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 1, 2, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 1, 3, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 1, 4, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 1, 5, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 1, 6, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 1, 7, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 1, 8, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<8, 1, 1, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<8, 1, 2, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<8, 1, 3, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<8, 1, 4, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<8, 1, 5, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<8, 1, 6, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<8, 1, 7, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<8, 1, 8, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 2, 1, false>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 2, 2, false>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 2, 3, false>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 2, 4, false>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 2, 5, false>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 2, 6, false>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 2, 7, false>(GemvArgs);
template __global__ void nf4_gemv_kernel<1, 2, 8, false>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 2, 1, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 2, 2, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 2, 3, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 2, 4, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 2, 5, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 2, 6, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 2, 7, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<2, 2, 8, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 2, 1, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 2, 2, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 2, 3, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 2, 4, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 2, 5, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 2, 6, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 2, 7, true>(GemvArgs);
template __global__ void nf4_gemv_kernel<4, 2, 8, true>(GemvArgs);

}  // namespace qlora
