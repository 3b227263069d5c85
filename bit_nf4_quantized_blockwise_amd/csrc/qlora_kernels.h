// Kernel declarations and argument structs shared by the kernel sources and
// the host-side entry points.
#pragma once

#include "qlora_common.h"
#include "qlora_philox.h"

namespace qlora {

enum BMode { B_NF4_COLS = 0, B_NF4_RED = 1, B_BF16_RC = 3 };
enum OMode { O_BF16 = 0, O_F32 = 1 };
// A operand: staged in LDS by direct-to-LDS loads, or loaded into MFMA registers
enum AMode { A_DMA = 0, A_DIRECT = 1 };

struct GemmArgs {
  const uint16_t* a;  // [rows][lda], reduction contiguous
  int64_t lda;
  int64_t rows, cols, red;  // valid extents (red % 8 == 0)
  const uint16_t* b;        // bf16 modes
  int64_t ldb;
  const uint8_t* packed;  // NF4 modes: W[n_out][k_in]
  const int8_t* qabsmax;
  const float* c2;
  int64_t w_kin;       // k_in of W (row pitch in elements)
  const uint16_t* pl;  // prologue: s · pl[rows][rl] · pr[cols][rl]ᵀ (pitches % 8 == 0)
  int64_t ldpl;
  const uint16_t* pr;
  int64_t ldpr;
  int32_t pr_rc;       // 1: pr is stored [rl][cols] (row-major by rank) instead
  int32_t rl;
  float s;
  int32_t s_split;     // 1: stage s·L as two bf16 parts (s·L not exact in bf16)
  DropoutKey drop;     // O_F32 with drop.thr > 0: the epilogue writes s·acc where the
                       // LoRA-dropout mask at index row·cols + col keeps, 0 where it drops
  const float* c_init;  // prologue modes: acc starts from c_init[rows][ldc] (split 0)
  int64_t ldc;          // instead of s·L·Rᵀ (fp32, ldc % 4 == 0, cols % 4 == 0)
  uint16_t* out_bf16;  // O_BF16: [rows][ldo]
  float* out_f32;      // O_F32: [split][rows][ldo] partial sums
  int64_t ldo;
  int64_t part_stride;
  int32_t tiles_m, tiles_n;
  int32_t kt_per_split;
};

struct ReduceOut {
  uint16_t* bf16;  // bf16 output or nullptr
  float* f32;      // float32 output or nullptr
  int64_t ld;
};

struct GemvArgs {
  const uint16_t* x;  // [M][K] bf16
  int32_t M;
  int64_t K, N;
  const uint8_t* packed;  // W[N][K] NF4 + DQ
  const int8_t* qabsmax;
  const float* c2;
  const uint16_t* u;  // [M][r] bf16, pitch r
  int32_t r;
  const uint16_t* b;  // [N][r] bf16, pitch r
  float s;
  uint16_t* y;   // [M][N] bf16 (ksplit == 1)
  float* part;   // [ksplit][M][N] (ksplit > 1; split 0 carries the adapter term)
  int32_t ksplit;
};

template <int MT, int NT, int WM, int WN, int BMODE, bool PROLOGUE, int OMODE, int AMODE>
__global__ void gemm_kernel(GemmArgs g);

// Rank-r products (qlora_adapter.hip): fp32 partial sums of one split each.
//   rows:  part[s][m][j] = Σ_k S[m][k]·F(k, j), F = A [r][ldf] or B [red][ldf]
//   cols:  part[s][l][j] (or [j][l]) = Σ_m S[m][l]·Q[m][j], Q [red][ldf]
struct AdapterArgs {
  const uint16_t* s;  // the streamed operand (X or dY), row-major, pitch lds
  int64_t lds;
  const uint16_t* f;  // the factor (A, B, U or V), row-major, pitch ldf
  int64_t ldf;
  int32_t r;          // rows of F when F = A
  int64_t frows;      // rows of F when F = B: rows k >= frows read as zero
  int64_t nout;       // rows: tokens; cols: columns of S
  int64_t red;        // rows: columns of S; cols: tokens
  float* part;
  int64_t ldp, part_stride;
  int32_t tiles, kt_per_split, nkt, nsplit;
};
constexpr int kAdapterTile = 128;  // stream indices per workgroup
template <int NB, bool FN>
__global__ void adapter_rows_kernel(AdapterArgs g);
template <int NB, bool TR>
__global__ void adapter_cols_kernel(AdapterArgs g);
template <int NB>
__global__ void adapter_dy_kernel(AdapterArgs gv, AdapterArgs gb, int nv);

constexpr int kGemvWaves = 8;   // waves per few-token GEMV workgroup (they split the reduction)
template <int CPW, int MG, int G, bool QV>
__global__ void nf4_gemv_kernel(GemvArgs g);

// The whole forward of a small weight for few tokens in one launch (M <= 16,
// r <= kSmallMaxRank, k_in <= 128 · kSmallWaves · kSmallMaxCpw): each
// workgroup owns 16 output rows over all of k and forms U = X·Aᵀ itself.
struct SmallFwdArgs {
  const uint16_t* x;  // [M][K] bf16
  int32_t M;
  int64_t K, N;
  const uint8_t* packed;  // W[N][K] NF4 + DQ
  const int8_t* qabsmax;
  const float* c2;
  const uint16_t* a;  // [r][K] bf16
  int32_t r;
  const uint16_t* b;  // [N][r] bf16, pitch r
  float s;
  uint16_t* y;  // [M][N] bf16
  uint16_t* u;  // [M][r] bf16, pitch r (written by workgroup 0)
};
constexpr int kSmallWaves = 16;   // waves per workgroup; they split k
constexpr int kSmallMaxCpw = 2;   // 128-k chunks per wave
constexpr int kSmallMaxRank = 16;
template <int CPW>
__global__ void nf4_small_fwd_kernel(SmallFwdArgs g);

// xd = mask ⊙ x over n / 8 blocks of 8 bf16 (LoRA dropout, see qlora_philox.h).
__global__ void lora_dropout_kernel(const uint16_t* x, int64_t nblk, DropoutKey d, uint16_t* xd);
constexpr int kDownThreads = 1024;  // lanes of the few-token U = X·Aᵀ kernel
__global__ void lora_down_small_kernel(const uint16_t* x, int64_t K, const uint16_t* a, int r,
                                       uint16_t* u);

__global__ void quantize_nf4_kernel(const float* w, int64_t n, int64_t nblocks, uint8_t* packed,
                                    float* absmax, int32_t* nonfinite);
__global__ void double_quant_kernel(const float* absmax, int64_t nblocks, int8_t* qabsmax,
                                    float* c2);

// Lists of weights in one launch (descriptors in the kernel arguments, up to
// kBatchMax per launch; wg0[i] = first workgroup of job i, wg0[count] = grid).
constexpr int kBatchMax = 48;
struct QuantJob1 {  // first level: blocks of 64 -> codes and float32 scales
  const float* w;
  int64_t n;
  uint8_t* packed;
  float* absmax;
  int32_t* nonfinite;  // optional flag, set to 1 on NaN / Inf input
};
struct QuantBatch {
  QuantJob1 j[kBatchMax];
  int64_t wg0[kBatchMax + 1];
  int32_t count;
};
struct DqJob {  // second level: groups of 256 scales -> int8 codes and steps
  const float* absmax;
  int64_t nblocks;
  int8_t* qabsmax;
  float* c2;
};
struct DqBatch {
  DqJob j[kBatchMax];
  int64_t wg0[kBatchMax + 1];
  int32_t count;
};
struct DeqJob {  // decode to bf16, 1024 packed dwords per workgroup
  const uint32_t* packed;
  const int8_t* qabsmax;
  const float* c2;
  u32x4* out;
  int64_t ndwords;
};
struct DeqBatch {
  DeqJob j[kBatchMax];
  int64_t wg0[kBatchMax + 1];
  int32_t count;
};
__global__ void quantize_nf4_batch_kernel(QuantBatch b);
__global__ void double_quant_batch_kernel(DqBatch b);
__global__ void dequantize_nf4_batch_kernel(DeqBatch b);
__global__ void quantize_nf4_dq_kernel(const float* w, int64_t n, int64_t nblocks, uint8_t* packed,
                                       int8_t* qabsmax, float* c2, float* absmax_out,
                                       int32_t* nonfinite);
__global__ void dequantize_nf4_kernel(const uint32_t* packed, const int8_t* qabsmax, const float* c2,
                                      int64_t ndwords, u32x4* out);
__global__ void reduce_partials_kernel(const float* part, int64_t part_stride, int32_t nsplit,
                                       int64_t rows, int64_t cols, int64_t rows_pad,
                                       int64_t cols_pad, int64_t ldp, float scale, ReduceOut o0,
                                       ReduceOut o1);
// One reduction: out(row, col) = scale · Σ_z part[z][row][col] (see reduce_partials_kernel).
struct ReduceJob {
  const float* part;
  int64_t part_stride;
  int32_t nsplit;
  int64_t rows, cols, rows_pad, cols_pad, ldp;
  float scale;
  ReduceOut o0, o1;
};
// Four columns per thread; blockIdx.y picks the job (one launch for two).
__global__ void reduce_partials4_kernel(ReduceJob j0, ReduceJob j1);
__global__ void pad_cols_kernel(const uint16_t* in, int64_t ldi, int64_t R, int64_t C, int64_t Cp,
                                uint16_t* out, int64_t ldo);

}  // namespace qlora
