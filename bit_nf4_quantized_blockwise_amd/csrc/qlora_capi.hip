// Host side of libqlora.so: argument validation, workspace layout, launch
// planning.  Every entry point validates all arguments before enqueuing
// anything; on an error status nothing is launched.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "qlora_kernels.h"
#include "qlora_optim.h"
#include "qlora_merge.h"
#include "qlora_quant_variants.h"

using namespace qlora;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_ok[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_dev_cus[kMaxDevices];  // compute units, once checked

qlora_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return QLORA_ERR_DEVICE;
  if (dev < kMaxDevices) {
    const int s = g_dev_ok[dev].load(std::memory_order_acquire);
    if (s == 1) return QLORA_OK;
    if (s == 2) return QLORA_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return QLORA_ERR_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) {
    // the CU count is published before the check result, so a thread that sees the
    // device checked also sees its count
    g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    g_dev_ok[dev].store(ok ? 1 : 2, std::memory_order_release);
  }
  return ok ? QLORA_OK : QLORA_ERR_DEVICE;
}

// Compute units of the current device (after check_device); 256 if unknown.
int device_cus() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  const int c = g_dev_cus[dev].load(std::memory_order_relaxed);
  return c > 0 ? c : 256;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline int64_t rup(int64_t a, int64_t b) { return (a + b - 1) / b * b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

#define QCHECK(cond, err) \
  do {                    \
    if (!(cond)) return (err); \
  } while (0)

inline qlora_status launched() {
  return hipGetLastError() == hipSuccess ? QLORA_OK : QLORA_ERR_LAUNCH;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int grid_for(int64_t n, int per = 256, int cap = 65536) {
  int64_t g = (n + per - 1) / per;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

// ---- GEMM launch plans ----------------------------------------------------------

struct Plan {
  int tiles_m, tiles_n, nkt, kt_per_split, nsplit;
};

Plan plan(int64_t rows, int64_t cols, int64_t red, int mt, int nt, bool allow_split,
          int target_wgs = 512) {
  Plan p;
  p.tiles_m = (int)ceil_div(rows, mt);
  p.tiles_n = (int)ceil_div(cols, nt);
  p.nkt = (int)ceil_div(red, 64);
  int s = 1;
  const int tiles = p.tiles_m * p.tiles_n;
  if (allow_split && tiles > 0 && tiles < target_wgs && p.nkt > 1) s = (int)std::min<int64_t>(ceil_div(target_wgs, tiles), p.nkt);
  p.kt_per_split = (int)ceil_div(std::max(p.nkt, 1), s);
  p.nsplit = (int)ceil_div(std::max(p.nkt, 1), p.kt_per_split);
  return p;
}

// Tile shapes of the instantiated kernels.
constexpr int BIG_MT = 256, BIG_NT = 256;   // NF4 GEMMs, many tokens
constexpr int SM_MT = 64, SM_NT = 256;      // NF4 GEMMs, few tokens (split-K)
constexpr int TR_MT = 64, TR_NT = 256;      // dropout's masked rank-r term T = s·mask ⊙ (V·A)
constexpr int64_t kBigM = 128;              // use the big tiles from this many tokens on
constexpr int64_t kFewM = 16;               // up to this many tokens: the streaming GEMV

bool use_big(int64_t M) { return M >= kBigM; }
bool use_gemv(int64_t M) { return M <= kFewM; }
// The one-launch forward of a small weight: few tokens, few ranks, k_in within
// the kernel's k range (two 128-k chunks per wave), and at most one workgroup
// of 16 columns per compute unit (every workgroup reads all of X and A, so a
// second round of workgroups costs more than the GEMV's second launch).
bool use_small(int64_t M, int64_t N, int64_t K, int32_t r) {
  return M >= 1 && M <= kFewM && r <= kSmallMaxRank && K <= 128 * kSmallWaves * kSmallMaxCpw &&
         ceil_div(N, 16) <= device_cus();
}

struct GemvPlan {
  int cpw, mg, ksplit, gx, groups;
};

// kGemvWaves waves per workgroup, each wave CPW chunks of 128 k; tokens in
// groups of 8 (MG groups).  The token operands live in registers, CPW · MG
// chunks' worth: at most 8 (two waves per SIMD at 256 registers).
GemvPlan gemv_plan(int64_t M, int64_t N, int64_t K) {
  GemvPlan p;
  p.mg = M <= 8 ? 1 : 2;
  const int64_t nch = ceil_div(K, 128);
  const int64_t need = ceil_div(nch, kGemvWaves);
  const int cap = 8 / p.mg;
  p.cpw = 1;
  // multi-chunk runs read the DQ codes as dwords: rows of a multiple of 4 blocks
  if ((K / 64) % 4 == 0)
    while (p.cpw < need && p.cpw < cap) p.cpw *= 2;
  p.ksplit = (int)ceil_div(nch, kGemvWaves * (int64_t)p.cpw);
  // column groups (16 outputs each) per workgroup: enough that one workgroup
  // per CU covers N, at most 8
  const int64_t ncg = ceil_div(N, 16);
  p.groups = (int)std::min<int64_t>(8, std::max<int64_t>(1, ceil_div(ncg, 256)));
  p.gx = (int)ceil_div(ncg, p.groups);
  return p;
}

// Rank-r products on the streaming kernels: stream tiles of 128, groups of up
// to 128 ranks (blocks of 32), and the reduction split so that about one
// workgroup per CU runs (each holds a 96-144 KB LDS ring).
constexpr int kAdapterWgs = 256;
struct AdPlan {
  int tiles, ncg, nb, nkt, ktps, nsplit;
  int64_t ldp;  // pitch of a partial-sum row (rows: ranks; TR: stream indices)
};

// row_pitch > 0 (the column kernel, whose reduction runs over rows): a
// split's rows of the widest operand stay below 2^31 bytes, the reach of a
// buffer offset.
// wgs: workgroups to aim for (one per CU for a launch of its own, half that
// for each of the two products sharing adapter_dy_kernel); the split count
// rounds down, so a launch never spills a few workgroups into a second round.
AdPlan ad_plan(int64_t nout, int64_t red, int32_t r, bool tr = false, int64_t row_pitch = 0,
               int wgs = kAdapterWgs) {
  AdPlan p;
  p.tiles = (int)ceil_div(nout, kAdapterTile);
  p.ncg = (int)ceil_div(r, 128);
  p.nb = p.ncg > 1 ? 4 : (r <= 32 ? 1 : (r <= 64 ? 2 : 4));
  p.nkt = (int)std::max<int64_t>(1, ceil_div(red, 64));
  const int base = p.tiles * p.ncg;  // 0 when there are no outputs (no launch then)
  const int s = (base == 0 || base >= wgs) ? 1 : std::min(p.nkt, wgs / base);
  p.ktps = (int)ceil_div(p.nkt, s);
  if (row_pitch > 0)
    p.ktps = (int)std::min<int64_t>(p.ktps, std::max<int64_t>(1, 0x7fffffffLL / (128 * row_pitch) - 1));
  p.nsplit = (int)ceil_div(p.nkt, p.ktps);
  p.ldp = tr ? (int64_t)p.tiles * kAdapterTile : (int64_t)32 * p.nb * p.ncg;
  return p;
}

// Bytes of one product's partial sums.
size_t ad_part_bytes(const AdPlan& p, int64_t nout, bool tr = false) {
  const int64_t rows = tr ? (int64_t)32 * p.nb * p.ncg : nout;
  return (size_t)p.nsplit * rows * p.ldp * 4;
}

// Forward workspace layout.
struct FwdWs {
  size_t u_part, pad_u, pad_b, y_part, total;
  AdPlan pu;
  Plan py;
  int64_t rp;
};

FwdWs fwd_ws(int64_t M, int64_t N, int64_t K, int32_t r) {
  FwdWs w{};
  w.rp = rup(r, 8);
  if (use_gemv(M)) {  // U written directly; partial sums only when K is split
    const GemvPlan g = gemv_plan(M, N, K);
    w.y_part = 0;
    w.u_part = w.pad_u = w.pad_b = 0;
    w.total = std::max<size_t>(g.ksplit > 1 ? align256((size_t)g.ksplit * M * N * 4) : 0, 256);
    return w;
  }
  w.pu = ad_plan(M, K, r);
  size_t off = 0;
  w.u_part = off;
  off += align256(ad_part_bytes(w.pu, M));
  w.pad_u = w.pad_b = off;
  if (r % 8 != 0) {
    w.pad_u = off;
    off += align256((size_t)M * w.rp * 2);
    w.pad_b = off;
    off += align256((size_t)N * w.rp * 2);
  }
  w.y_part = off;
  if (!use_big(M)) {
    w.py = plan(M, N, K, SM_MT, SM_NT, true);
    off += align256((size_t)w.py.nsplit * M * N * 4);
  }
  w.total = std::max<size_t>(off, 256);
  return w;
}

struct BwdWs {
  size_t bp, up, dyp, v, part, part_db, total;
  AdPlan pv, pda, pdb;
  Plan pdx;
  int64_t rp, Np;
};

// n_out not a multiple of 8: dY is copied to a zero-padded pitch Np (its rows
// are then 16-byte aligned for the loaders); a rank that is not a multiple of
// 8 gets padded copies of B and U for the same reason.
BwdWs bwd_ws(int64_t M, int64_t N, int64_t K, int32_t r) {
  BwdWs w{};
  w.rp = rup(r, 8);
  w.Np = rup(N, 8);
  size_t off = 0;
  w.bp = w.up = off;
  if (w.rp != r) {
    w.bp = off; off += align256((size_t)N * w.rp * 2);
    w.up = off; off += align256((size_t)M * w.rp * 2);
  }
  w.dyp = off;
  if (w.Np != N) off += align256((size_t)M * w.Np * 2);
  w.v = off; off += align256((size_t)M * w.rp * 2);
  // V's and dB's partial sums live at once (one launch forms both); dX's
  // split partials and dA's reuse V's region afterwards
  // (dB is planned first; V gets the workgroups left in one round)
  w.pdb = ad_plan(N, M, r, false, std::max<int64_t>(w.Np, w.rp), kAdapterWgs / 2);
  const int db_wgs = w.pdb.tiles * w.pdb.nsplit * w.pdb.ncg;
  w.pv = ad_plan(M, w.Np, r, false, 0, std::max(kAdapterWgs - db_wgs, kAdapterWgs / 4));
  w.pda = ad_plan(K, M, r, true, std::max<int64_t>(K, w.rp));
  size_t part = std::max(ad_part_bytes(w.pv, M), ad_part_bytes(w.pda, K, true));
  if (!use_big(M)) {
    w.pdx = plan(M, K, N, SM_MT, SM_NT, true);
    part = std::max(part, (size_t)w.pdx.nsplit * M * K * 4);
  }
  w.part = off;
  off += align256(part);
  w.part_db = off;
  off += align256(ad_part_bytes(w.pdb, N));
  w.total = std::max<size_t>(off, 256);
  return w;
}

template <int MT, int NT, int WM, int WN, int BM, bool PRO, int OM, int AM = A_DIRECT>
qlora_status run_gemm(GemmArgs g, const Plan& p, hipStream_t st) {
  g.tiles_m = p.tiles_m;
  g.tiles_n = p.tiles_n;
  g.kt_per_split = p.kt_per_split;
  dim3 grid((unsigned)(p.tiles_m * p.tiles_n), (unsigned)p.nsplit);
  hipLaunchKernelGGL((gemm_kernel<MT, NT, WM, WN, BM, PRO, OM, AM>), grid, dim3(256), 0, st, g);
  return launched();
}

// The float4 reduction needs every row of partials and outputs 16-byte
// (partials) / 8-byte (bf16 rows) aligned.
bool reduce4_ok(const ReduceJob& j) {
  auto al = [](const ReduceOut& o) {
    return (o.ld % 4) == 0 && (reinterpret_cast<uintptr_t>(o.bf16) & 7u) == 0 &&
           (reinterpret_cast<uintptr_t>(o.f32) & 15u) == 0;
  };
  return j.cols_pad % 4 == 0 && j.ldp % 4 == 0 && j.part_stride % 4 == 0 &&
         (reinterpret_cast<uintptr_t>(j.part) & 15u) == 0 && al(j.o0) && al(j.o1);
}

qlora_status run_reduce_job(const ReduceJob& j, hipStream_t st) {
  const int64_t total = j.rows_pad * j.cols_pad;
  if (total == 0) return QLORA_OK;
  if (reduce4_ok(j)) {
    const ReduceJob none{};
    hipLaunchKernelGGL(reduce_partials4_kernel, dim3(grid_for(total / 4), 1), dim3(256), 0, st, j,
                       none);
    return launched();
  }
  hipLaunchKernelGGL(reduce_partials_kernel, dim3(grid_for(total)), dim3(256), 0, st, j.part,
                     j.part_stride, j.nsplit, j.rows, j.cols, j.rows_pad, j.cols_pad, j.ldp,
                     j.scale, j.o0, j.o1);
  return launched();
}

qlora_status run_reduce(const float* part, int64_t part_stride, int nsplit, int64_t rows,
                        int64_t cols, int64_t rows_pad, int64_t cols_pad, int64_t ldp, float scale,
                        ReduceOut o0, ReduceOut o1, hipStream_t st) {
  return run_reduce_job(ReduceJob{part, part_stride, nsplit, rows, cols, rows_pad, cols_pad, ldp,
                                  scale, o0, o1},
                        st);
}

// Two reductions in one launch (separately when either needs the scalar kernel).
qlora_status run_reduce2(const ReduceJob& a, const ReduceJob& b, hipStream_t st) {
  if (!reduce4_ok(a) || !reduce4_ok(b) || a.rows_pad * a.cols_pad == 0 ||
      b.rows_pad * b.cols_pad == 0) {
    const qlora_status s = run_reduce_job(a, st);
    return s != QLORA_OK ? s : run_reduce_job(b, st);
  }
  const int64_t t = std::max(a.rows_pad * a.cols_pad, b.rows_pad * b.cols_pad) / 4;
  hipLaunchKernelGGL(reduce_partials4_kernel, dim3(grid_for(t), 2), dim3(256), 0, st, a, b);
  return launched();
}

constexpr ReduceOut kNoOut{nullptr, nullptr, 0};

AdapterArgs ad_args(const AdPlan& p, const uint16_t* S, int64_t lds, const uint16_t* F, int64_t ldf,
                    int32_t r, int64_t nout, int64_t red, float* part, bool tr = false) {
  AdapterArgs a{};
  a.s = S; a.lds = lds; a.f = F; a.ldf = ldf; a.r = r; a.nout = nout; a.red = red; a.frows = red;
  a.part = part; a.ldp = p.ldp;
  a.part_stride = (tr ? (int64_t)32 * p.nb * p.ncg : nout) * p.ldp;
  a.tiles = p.tiles; a.kt_per_split = p.ktps; a.nkt = p.nkt; a.nsplit = p.nsplit;
  return a;
}

template <bool FN>
qlora_status run_rows(const AdapterArgs& a, const AdPlan& p, hipStream_t st) {
  const dim3 grid((unsigned)(p.tiles * p.nsplit), (unsigned)p.ncg);
  switch (p.nb) {
    case 1: hipLaunchKernelGGL((adapter_rows_kernel<1, FN>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((adapter_rows_kernel<2, FN>), grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((adapter_rows_kernel<4, FN>), grid, dim3(256), 0, st, a); break;
  }
  return launched();
}

template <bool TR>
qlora_status run_cols(const AdapterArgs& a, const AdPlan& p, hipStream_t st) {
  const dim3 grid((unsigned)(p.tiles * p.nsplit), (unsigned)p.ncg);
  switch (p.nb) {
    case 1: hipLaunchKernelGGL((adapter_cols_kernel<1, TR>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((adapter_cols_kernel<2, TR>), grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((adapter_cols_kernel<4, TR>), grid, dim3(256), 0, st, a); break;
  }
  return launched();
}

// s·x is exact in bf16 for every bf16 x when s is a power of two (no
// overflow / underflow at the magnitudes of the adapter factors).
int needs_split(float s) {
  int e = 0;
  const float m = std::frexp(s, &e);
  return (m == 0.5f || m == -0.5f) ? 0 : 1;
}

qlora_status validate_weight(const qlora_nf4_weight* w) {
  QCHECK(w != nullptr, QLORA_ERR_NULL);
  QCHECK(w->n_out >= 0 && w->k_in >= 0, QLORA_ERR_SHAPE);
  if (w->n_out > 0 && w->k_in > 0) {
    QCHECK(w->packed && w->qabsmax && w->c2, QLORA_ERR_NULL);
    QCHECK(aligned16(w->packed) && aligned16(w->qabsmax) && aligned16(w->c2), QLORA_ERR_ALIGN);
  }
  return QLORA_OK;
}

qlora_status validate_linear(const qlora_nf4_weight* w, int64_t M, int32_t r) {
  qlora_status s = validate_weight(w);
  if (s != QLORA_OK) return s;
  QCHECK(M >= 0, QLORA_ERR_SHAPE);
  QCHECK(w->k_in % 64 == 0, QLORA_ERR_SHAPE);
  QCHECK(w->n_out > 0 && w->k_in > 0, QLORA_ERR_SHAPE);
  QCHECK(r >= 1 && r <= QLORA_MAX_RANK, QLORA_ERR_UNSUPPORTED);
  return QLORA_OK;
}

#define ALIGNED_OR_NULL(p) QCHECK((p) != nullptr, QLORA_ERR_NULL); QCHECK(aligned16(p), QLORA_ERR_ALIGN)

// U = X·Aᵀ (bf16 [M][r]): the rank-r streaming kernel's split partial sums in ws, then
// their reduction (few tokens: one small kernel, no partial sums).
qlora_status lora_down_impl(const uint16_t* X, int64_t M, int64_t K, const uint16_t* A, int32_t r,
                            uint16_t* U, uint16_t* Upad, int64_t rp, char* ws, const FwdWs& L,
                            hipStream_t st) {
  if (M == 0) return QLORA_OK;
  if (use_gemv(M)) {
    hipLaunchKernelGGL(lora_down_small_kernel, dim3((unsigned)r, (unsigned)M), dim3(kDownThreads), 0,
                       st, X, K, A, (int)r, U);
    return launched();
  }
  float* part = reinterpret_cast<float*>(ws + L.u_part);
  const AdapterArgs a = ad_args(L.pu, X, K, A, K, r, M, K, part);
  qlora_status s = run_rows<false>(a, L.pu, st);
  if (s != QLORA_OK) return s;
  s = run_reduce(part, a.part_stride, L.pu.nsplit, M, r, M, r, a.ldp, 1.0f,
                 ReduceOut{U, nullptr, r}, kNoOut, st);
  if (s != QLORA_OK || !Upad) return s;
  // zero-padded copy with a pitch that is a multiple of 8, for the prologue's 16-byte loads
  return run_reduce(part, a.part_stride, L.pu.nsplit, M, r, M, rp, a.ldp, 1.0f,
                    ReduceOut{Upad, nullptr, rp}, kNoOut, st);
}

template <int CPW, int MG, int G>
void launch_gemv_g(const GemvArgs& a, dim3 grid, hipStream_t st) {
  // dword reads of the DQ codes need 4-byte aligned runs: even CPW (and rows
  // a multiple of 4 blocks long, which the plan checks)
  hipLaunchKernelGGL((nf4_gemv_kernel<CPW, MG, G, (CPW > 1)>), grid, dim3(64 * kGemvWaves), 0, st, a);
}

template <int CPW, int MG>
void launch_gemv(const GemvArgs& a, dim3 grid, int groups, hipStream_t st) {
  switch (groups) {
    case 1: launch_gemv_g<CPW, MG, 1>(a, grid, st); break;
    case 2: launch_gemv_g<CPW, MG, 2>(a, grid, st); break;
    case 3: launch_gemv_g<CPW, MG, 3>(a, grid, st); break;
    case 4: launch_gemv_g<CPW, MG, 4>(a, grid, st); break;
    case 5: launch_gemv_g<CPW, MG, 5>(a, grid, st); break;
    case 6: launch_gemv_g<CPW, MG, 6>(a, grid, st); break;
    case 7: launch_gemv_g<CPW, MG, 7>(a, grid, st); break;
    default: launch_gemv_g<CPW, MG, 8>(a, grid, st); break;
  }
}

// Few-token forward: U (pitch r) and B (pitch r) are read as given.
qlora_status gemv_impl(const qlora_nf4_weight* w, const uint16_t* X, int64_t M, const uint16_t* U,
                       const uint16_t* B, int32_t r, float s, uint16_t* Y, char* ws,
                       hipStream_t st) {
  const int64_t N = w->n_out, K = w->k_in;
  const GemvPlan p = gemv_plan(M, N, K);
  GemvArgs a{};
  a.x = X; a.M = (int32_t)M; a.K = K; a.N = N;
  a.packed = w->packed; a.qabsmax = w->qabsmax; a.c2 = w->c2;
  a.u = U; a.r = r; a.b = B; a.s = s;
  a.y = Y; a.part = reinterpret_cast<float*>(ws); a.ksplit = p.ksplit;
  const dim3 grid((unsigned)p.gx, (unsigned)p.ksplit);
  if (p.mg == 1) {
    switch (p.cpw) {
      case 1: launch_gemv<1, 1>(a, grid, p.groups, st); break;
      case 2: launch_gemv<2, 1>(a, grid, p.groups, st); break;
      case 4: launch_gemv<4, 1>(a, grid, p.groups, st); break;
      default: launch_gemv<8, 1>(a, grid, p.groups, st); break;
    }
  } else {
    switch (p.cpw) {
      case 1: launch_gemv<1, 2>(a, grid, p.groups, st); break;
      case 2: launch_gemv<2, 2>(a, grid, p.groups, st); break;
      default: launch_gemv<4, 2>(a, grid, p.groups, st); break;
    }
  }
  qlora_status e = launched();
  if (e != QLORA_OK || p.ksplit == 1) return e;
  return run_reduce(a.part, M * N, p.ksplit, M, N, M, N, N, 1.0f, ReduceOut{Y, nullptr, N},
                    ReduceOut{nullptr, nullptr, 0}, st);
}

qlora_status matmul_fwd_impl(const qlora_nf4_weight* w, const uint16_t* X, int64_t M,
                             const uint16_t* Upro, int64_t ldu, const uint16_t* Bpro, int64_t ldb,
                             int32_t r, float s, uint16_t* Y, char* ws, const FwdWs& L,
                             hipStream_t st) {
  if (M == 0) return QLORA_OK;
  const int64_t N = w->n_out, K = w->k_in;
  if (use_gemv(M)) return gemv_impl(w, X, M, Upro, Bpro, r, s, Y, ws, st);
  GemmArgs g{};
  g.a = X; g.lda = K; g.rows = M; g.cols = N; g.red = K;
  g.packed = w->packed; g.qabsmax = w->qabsmax; g.c2 = w->c2; g.w_kin = K;
  g.pl = Upro; g.ldpl = ldu; g.pr = Bpro; g.ldpr = ldb; g.rl = r; g.s = s;
  g.s_split = needs_split(s);
  if (use_big(M)) {
    g.out_bf16 = Y; g.ldo = N;
    return run_gemm<BIG_MT, BIG_NT, 2, 2, B_NF4_COLS, true, O_BF16, A_DMA>(
        g, plan(M, N, K, BIG_MT, BIG_NT, false), st);
  }
  g.out_f32 = reinterpret_cast<float*>(ws + L.y_part);
  g.ldo = N;
  g.part_stride = M * N;
  qlora_status e = run_gemm<SM_MT, SM_NT, 1, 4, B_NF4_COLS, true, O_F32>(g, L.py, st);
  if (e != QLORA_OK) return e;
  return run_reduce(g.out_f32, g.part_stride, L.py.nsplit, M, N, M, N, N, 1.0f,
                    ReduceOut{Y, nullptr, N}, kNoOut, st);
}

float scale_of(float alpha, int32_t r) { return alpha / (float)r; }

// Forward with the main product on X and the adapter on Xl (X itself, or its
// dropout): U = Xl·Aᵀ, Y = X·Ŵᵀ + s·U·Bᵀ.
// Y and U of a small weight for few tokens in one launch (both products read X).
qlora_status small_fwd(const qlora_nf4_weight* w, const uint16_t* X, int64_t M, const uint16_t* A,
                       const uint16_t* B, int32_t r, float s, uint16_t* Y, uint16_t* U,
                       hipStream_t st) {
  SmallFwdArgs a{};
  a.x = X; a.M = (int32_t)M; a.K = w->k_in; a.N = w->n_out;
  a.packed = w->packed; a.qabsmax = w->qabsmax; a.c2 = w->c2;
  a.a = A; a.r = r; a.b = B; a.s = s; a.y = Y; a.u = U;
  const dim3 grid((unsigned)ceil_div(w->n_out, 16));
  if (w->k_in <= 128 * kSmallWaves)
    hipLaunchKernelGGL(nf4_small_fwd_kernel<1>, grid, dim3(64 * kSmallWaves), 0, st, a);
  else
    hipLaunchKernelGGL(nf4_small_fwd_kernel<2>, grid, dim3(64 * kSmallWaves), 0, st, a);
  return launched();
}

qlora_status linear_fwd_impl(const qlora_nf4_weight* w, const uint16_t* X, const uint16_t* Xl,
                             int64_t M, const uint16_t* A, const uint16_t* B, int32_t r, float s,
                             uint16_t* Y, uint16_t* U, char* ws, const FwdWs& L, hipStream_t st) {
  if (X == Xl && use_small(M, w->n_out, w->k_in, r)) return small_fwd(w, X, M, A, B, r, s, Y, U, st);
  const bool pad = r % 8 != 0 && !use_gemv(M);
  uint16_t* Up = pad ? reinterpret_cast<uint16_t*>(ws + L.pad_u) : nullptr;
  qlora_status e = lora_down_impl(Xl, M, w->k_in, A, r, U, Up, L.rp, ws, L, st);
  if (e != QLORA_OK) return e;
  const uint16_t* bp = B;
  if (pad) {
    uint16_t* Bp = reinterpret_cast<uint16_t*>(ws + L.pad_b);
    hipLaunchKernelGGL(pad_cols_kernel, dim3(grid_for(w->n_out * L.rp)), dim3(256), 0, st, B,
                       (int64_t)r, w->n_out, (int64_t)r, L.rp, Bp, L.rp);
    if ((e = launched()) != QLORA_OK) return e;
    bp = Bp;
  }
  return matmul_fwd_impl(w, X, M, pad ? Up : U, pad ? L.rp : r, bp, pad ? L.rp : r, r, s, Y, ws,
                         L, st);
}

// LoRA dropout key of rate p (false for p outside [0, 1)).
bool dropout_key(float p, uint64_t seed, uint64_t offset, DropoutKey* k) {
  if (!(p >= 0.0f && p < 1.0f)) return false;
  k->seed = seed;
  k->offset = offset;
  k->thr = (uint32_t)std::floor((double)p * 4294967296.0);
  return true;
}

// s' = s / (1 − p): the inverted-dropout factor folded into the adapter scale.
float scale_with_dropout(float s, float p) { return (float)((double)s / (1.0 - (double)p)); }

qlora_status run_dropout(const uint16_t* X, int64_t n, const DropoutKey& key, uint16_t* Xd,
                         hipStream_t st) {
  const int64_t nblk = n / 8;
  hipLaunchKernelGGL(lora_dropout_kernel, dim3(grid_for(nblk, 256, 1 << 16)), dim3(256), 0, st,
                     X, nblk, key, Xd);
  return launched();
}

// Arguments of both backward entry points (X: the tokens dA multiplies).
qlora_status validate_bwd(const qlora_nf4_weight* w, const uint16_t* X, const uint16_t* dY,
                          int64_t M, const uint16_t* A, const uint16_t* B, int32_t r,
                          const uint16_t* U, const uint16_t* dX, const float* dA, const float* dB) {
  qlora_status s = validate_linear(w, M, r);
  if (s != QLORA_OK) return s;
  ALIGNED_OR_NULL(A);
  ALIGNED_OR_NULL(B);
  ALIGNED_OR_NULL(dA);
  ALIGNED_OR_NULL(dB);
  if (M > 0) {
    ALIGNED_OR_NULL(X);
    ALIGNED_OR_NULL(dY);
    ALIGNED_OR_NULL(U);
    ALIGNED_OR_NULL(dX);
  }
  return QLORA_OK;
}

// Workspace of the dropout backward: the plain backward's, then the masked
// adapter term T [M][K] fp32.
size_t bwd_dropout_ws(const BwdWs& L, int64_t M, int64_t K) {
  return align256(L.total) + align256((size_t)M * K * 4);
}

// Backward; X is the input dA multiplies (the tokens, or their dropout).  With
// drop, dX = dY·Ŵ + T where T = s·mask ⊙ (V·A) is formed first (fp32, in the
// workspace after the plain backward's layout) and the dX GEMM starts its
// accumulators from it.
qlora_status linear_bwd_impl(const qlora_nf4_weight* w, const uint16_t* X, const uint16_t* dY,
                             int64_t M, const uint16_t* A, const uint16_t* B, int32_t r, float sc,
                             const DropoutKey* drop, const uint16_t* U, uint16_t* dX, float* dA,
                             float* dB, char* ws, const BwdWs& L, hipStream_t st) {
  const int64_t N = w->n_out, K = w->k_in;
  qlora_status s = QLORA_OK;

  if (M == 0) {  // no tokens: the adapter gradients are zero
    s = run_reduce(nullptr, 0, 0, 0, 0, (int64_t)r, K, 0, 0.0f, ReduceOut{nullptr, dA, K},
                   kNoOut, st);
    if (s != QLORA_OK) return s;
    return run_reduce(nullptr, 0, 0, 0, 0, N, (int64_t)r, 0, 0.0f,
                      ReduceOut{nullptr, dB, (int64_t)r}, kNoOut, st);
  }

  uint16_t* V = reinterpret_cast<uint16_t*>(ws + L.v);    // [M][rp]
  float* part = reinterpret_cast<float*>(ws + L.part);

  // dY with a 16-byte aligned row pitch (only when n_out % 8 != 0)
  const int64_t ldy = L.Np;
  const uint16_t* dYa = dY;
  if (L.Np != N) {
    uint16_t* dYp = reinterpret_cast<uint16_t*>(ws + L.dyp);
    hipLaunchKernelGGL(pad_cols_kernel, dim3(grid_for(M * L.Np)), dim3(256), 0, st, dY, N, M, N,
                       L.Np, dYp, L.Np);
    if ((s = launched()) != QLORA_OK) return s;
    dYa = dYp;
  }
  // B and U with 16-byte aligned rows (only when r % 8 != 0)
  const uint16_t *Ba = B, *Ua = U;
  if (L.rp != r) {
    uint16_t* Bp = reinterpret_cast<uint16_t*>(ws + L.bp);
    uint16_t* Up = reinterpret_cast<uint16_t*>(ws + L.up);
    hipLaunchKernelGGL(pad_cols_kernel, dim3(grid_for(N * L.rp)), dim3(256), 0, st, B,
                       (int64_t)r, N, (int64_t)r, L.rp, Bp, L.rp);
    if ((s = launched()) != QLORA_OK) return s;
    hipLaunchKernelGGL(pad_cols_kernel, dim3(grid_for(M * L.rp)), dim3(256), 0, st, U,
                       (int64_t)r, M, (int64_t)r, L.rp, Up, L.rp);
    if ((s = launched()) != QLORA_OK) return s;
    Ba = Bp;
    Ua = Up;
  }

  // One launch streams dY for both V = dY·B (over the padded pitch: dY holds
  // zeros past n_out, and B's rows past n_out read as zero) and dB = s·dYᵀ·U; one more sums
  // both products' splits: V [M][rp] bf16 (zero-padded) and dB [N][r].
  {
    float* part_db = reinterpret_cast<float*>(ws + L.part_db);
    AdapterArgs av = ad_args(L.pv, dYa, ldy, Ba, L.rp, r, M, L.Np, part);
    av.frows = N;  // B has n_out rows; dY's padding columns meet zeros, not the memory past B
    const AdapterArgs ab = ad_args(L.pdb, dYa, ldy, Ua, L.rp, r, N, M, part_db);
    const int nv = L.pv.tiles * L.pv.nsplit;
    const dim3 grid((unsigned)(nv + L.pdb.tiles * L.pdb.nsplit), (unsigned)L.pv.ncg);
    switch (L.pv.nb) {
      case 1: hipLaunchKernelGGL(adapter_dy_kernel<1>, grid, dim3(256), 0, st, av, ab, nv); break;
      case 2: hipLaunchKernelGGL(adapter_dy_kernel<2>, grid, dim3(256), 0, st, av, ab, nv); break;
      default: hipLaunchKernelGGL(adapter_dy_kernel<4>, grid, dim3(256), 0, st, av, ab, nv); break;
    }
    if ((s = launched()) != QLORA_OK) return s;
    const ReduceJob jv{part, av.part_stride, L.pv.nsplit, M, r, M, L.rp, av.ldp, 1.0f,
                       ReduceOut{V, nullptr, L.rp}, kNoOut};
    const ReduceJob jb{part_db, ab.part_stride, L.pdb.nsplit, N, r, N, r, ab.ldp, sc,
                       ReduceOut{nullptr, dB, (int64_t)r}, kNoOut};
    if ((s = run_reduce2(jv, jb, st)) != QLORA_OK) return s;
  }

  // with dropout: T = s·mask ⊙ (V·A), [M][K] fp32 (mask and scale in the epilogue)
  float* T = drop ? reinterpret_cast<float*>(ws + align256(L.total)) : nullptr;
  if (drop) {
    GemmArgs g{};
    g.a = V; g.lda = L.rp; g.rows = M; g.cols = K; g.red = r;
    g.b = A; g.ldb = K;
    g.out_f32 = T; g.ldo = K; g.part_stride = M * K;
    g.s = sc; g.drop = *drop;
    if ((s = run_gemm<TR_MT, TR_NT, 2, 2, B_BF16_RC, false, O_F32>(
             g, plan(M, K, r, TR_MT, TR_NT, false), st)) != QLORA_OK)
      return s;
  }

  // dX = dY·Ŵ + s·V·A  (with dropout: dY·Ŵ + T); W rows past n_out read as
  // zero, so a chunk of dY that straddles n_out meets zeros on both sides
  {
    GemmArgs g{};
    g.a = dYa; g.lda = ldy; g.rows = M; g.cols = K; g.red = N;
    g.packed = w->packed; g.qabsmax = w->qabsmax; g.c2 = w->c2; g.w_kin = K;
    g.pl = V; g.ldpl = L.rp; g.pr = A; g.ldpr = K; g.pr_rc = 1; g.rl = r; g.s = sc;
    g.s_split = needs_split(sc);
    if (drop) {
      g.c_init = T; g.ldc = K; g.rl = 0;
    }
    if (use_big(M)) {
      g.out_bf16 = dX; g.ldo = K;
      s = run_gemm<BIG_MT, BIG_NT, 2, 2, B_NF4_RED, true, O_BF16, A_DMA>(
          g, plan(M, K, N, BIG_MT, BIG_NT, false), st);
      if (s != QLORA_OK) return s;
    } else {
      g.out_f32 = part; g.ldo = K; g.part_stride = M * K;
      if ((s = run_gemm<SM_MT, SM_NT, 1, 4, B_NF4_RED, true, O_F32>(g, L.pdx, st)) != QLORA_OK)
        return s;
      if ((s = run_reduce(part, g.part_stride, L.pdx.nsplit, M, K, M, K, K, 1.0f,
                          ReduceOut{dX, nullptr, K}, kNoOut, st)) != QLORA_OK)
        return s;
    }
  }

  // dA = s·Vᵀ·X   [r][K] (partial sums stored rank-major)
  {
    const AdapterArgs a = ad_args(L.pda, X, K, V, L.rp, r, K, M, part, true);
    if ((s = run_cols<true>(a, L.pda, st)) != QLORA_OK) return s;
    if ((s = run_reduce(part, a.part_stride, L.pda.nsplit, r, K, r, K, a.ldp, sc,
                        ReduceOut{nullptr, dA, K}, kNoOut, st)) != QLORA_OK)
      return s;
  }
  return QLORA_OK;
}


// AdamW arguments shared by both step entry points.
qlora_status validate_adamw_tensors(const qlora_adamw_tensor* t, int32_t count) {
  QCHECK(count >= 0, QLORA_ERR_SHAPE);
  QCHECK(count == 0 || t != nullptr, QLORA_ERR_NULL);
  for (int32_t i = 0; i < count; ++i) {
    QCHECK(t[i].n >= 0, QLORA_ERR_SHAPE);
    if (t[i].n == 0) continue;
    QCHECK(t[i].param && t[i].grad && t[i].m && t[i].v, QLORA_ERR_NULL);
    QCHECK(aligned16(t[i].param) && aligned16(t[i].grad) && aligned16(t[i].m) && aligned16(t[i].v),
           QLORA_ERR_ALIGN);
    QCHECK(t[i].param_bf16 == nullptr || aligned16(t[i].param_bf16), QLORA_ERR_ALIGN);
  }
  return QLORA_OK;
}

qlora_status validate_adamw_hyper(float lr, float beta1, float beta2, float eps,
                                  float weight_decay, int64_t step, float max_grad_norm,
                                  const float* grad_norm) {
  QCHECK(step >= 1, QLORA_ERR_SHAPE);
  QCHECK(std::isfinite(lr) && lr >= 0.0f && std::isfinite(weight_decay) && weight_decay >= 0.0f,
         QLORA_ERR_UNSUPPORTED);
  QCHECK(beta1 >= 0.0f && beta1 < 1.0f && beta2 >= 0.0f && beta2 < 1.0f, QLORA_ERR_UNSUPPORTED);
  QCHECK(std::isfinite(eps) && eps > 0.0f && std::isfinite(max_grad_norm), QLORA_ERR_UNSUPPORTED);
  QCHECK(grad_norm == nullptr || aligned16(grad_norm), QLORA_ERR_ALIGN);
  return QLORA_OK;
}

// Step size and bias corrections in float64 on the host, rounded once.
AdamHyper adamw_hyper(float lr, float beta1, float beta2, float eps, float weight_decay,
                      int64_t step) {
  AdamHyper h{};
  h.beta1 = beta1;
  h.beta2 = beta2;
  h.eps = eps;
  h.decay = (float)(1.0 - (double)lr * (double)weight_decay);
  h.step_size = (float)((double)lr / (1.0 - std::pow((double)beta1, (double)step)));
  h.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(1.0 - std::pow((double)beta2, (double)step)));
  return h;
}

// Prepared list layout: the descriptors, then (from a 256-byte boundary) the
// chunk map.
size_t plan_tmap_offset(int32_t count) { return align256((size_t)count * sizeof(AdamTensor)); }

int64_t plan_chunks(const qlora_adamw_tensor* t, int32_t count) {
  int64_t c = 0;
  for (int32_t i = 0; i < count; ++i) c += ceil_div(t[i].n, kAdamChunk);
  return c;
}

}  // namespace

extern "C" {

int32_t qlora_abi_version(void) { return QLORA_ABI_VERSION; }

void qlora_nf4_codebook(float out[16]) {
  if (!out) return;
  for (int i = 0; i < 16; ++i) out[i] = bits_to_float(kNF4Bits[i]);
}

const char* qlora_status_string(qlora_status s) {
  switch (s) {
    case QLORA_OK: return "QLORA_OK";
    case QLORA_ERR_NULL: return "QLORA_ERR_NULL: a required pointer is NULL";
    case QLORA_ERR_SHAPE: return "QLORA_ERR_SHAPE: invalid size";
    case QLORA_ERR_ALIGN: return "QLORA_ERR_ALIGN: device pointer not 16-byte aligned";
    case QLORA_ERR_UNSUPPORTED: return "QLORA_ERR_UNSUPPORTED: unsupported parameter (blocksize, group, rank, code, optimizer or dropout setting, or unpinned host states)";
    case QLORA_ERR_WORKSPACE: return "QLORA_ERR_WORKSPACE: workspace missing or too small";
    case QLORA_ERR_DEVICE: return "QLORA_ERR_DEVICE: no gfx950 device current";
    case QLORA_ERR_LAUNCH: return "QLORA_ERR_LAUNCH: kernel launch failed";
  }
  return "QLORA_ERR_UNKNOWN";
}

size_t qlora_workspace_size(int32_t op, int64_t M, int64_t n_out, int64_t k_in, int32_t r) {
  if (M < 0 || n_out <= 0 || k_in <= 0 || r < 1 || r > QLORA_MAX_RANK) return 0;
  if (op == 0) return fwd_ws(M, n_out, k_in, r).total;
  if (op == 1) return bwd_ws(M, n_out, k_in, r).total;
  if (op == 2) return bwd_dropout_ws(bwd_ws(M, n_out, k_in, r), M, k_in);
  return 0;
}

qlora_status qlora_quantize_nf4(const float* w, int64_t n, int32_t blocksize, uint8_t* packed,
                                float* absmax, int32_t* nonfinite_flag, void* stream) {
  QCHECK(n >= 0, QLORA_ERR_SHAPE);
  QCHECK(blocksize == QLORA_BLOCKSIZE, QLORA_ERR_UNSUPPORTED);
  QCHECK(aligned4(nonfinite_flag), QLORA_ERR_ALIGN);
  if (n == 0) return QLORA_OK;
  ALIGNED_OR_NULL(w);
  ALIGNED_OR_NULL(packed);
  ALIGNED_OR_NULL(absmax);
  qlora_status s = check_device();
  if (s != QLORA_OK) return s;
  const int64_t nb = ceil_div(n, 64);
  const int64_t threads = nb * 4;
  QCHECK(ceil_div(threads, 256) <= 0x7fffffff, QLORA_ERR_SHAPE);
  hipLaunchKernelGGL(quantize_nf4_kernel, dim3((unsigned)ceil_div(threads, 256)), dim3(256), 0,
                     as_stream(stream), w, n, nb, packed, absmax, nonfinite_flag);
  return launched();
}

qlora_status qlora_quantize_4bit(const float* w, int64_t n, int32_t code, uint8_t* packed,
                                 float* absmax, void* stream) {
  QCHECK(n >= 0, QLORA_ERR_SHAPE);
  QCHECK(code == QLORA_CODE_NF4 || code == QLORA_CODE_INT4, QLORA_ERR_UNSUPPORTED);
  if (n == 0) return QLORA_OK;
  ALIGNED_OR_NULL(w);
  ALIGNED_OR_NULL(packed);
  ALIGNED_OR_NULL(absmax);
  qlora_status s = check_device();
  if (s != QLORA_OK) return s;
  const int64_t nb = ceil_div(n, 64);
  const int64_t grid = ceil_div(nb * 4, 256);
  QCHECK(grid <= 0x7fffffff, QLORA_ERR_SHAPE);
  if (code == QLORA_CODE_NF4)
    hipLaunchKernelGGL(quantize_nf4_kernel, dim3((unsigned)grid), dim3(256), 0, as_stream(stream),
                       w, n, nb, packed, absmax, static_cast<int32_t*>(nullptr));
  else
    hipLaunchKernelGGL(quantize_int4_kernel, dim3((unsigned)grid), dim3(256), 0,
                       as_stream(stream), w, n, nb, packed, absmax);
  return launched();
}

qlora_status qlora_dequantize_4bit(const uint8_t* packed, const float* absmax, int64_t n,
                                   int32_t code, qlora_bf16* out, void* stream) {
  QCHECK(n >= 0, QLORA_ERR_SHAPE);
  QCHECK(code == QLORA_CODE_NF4 || code == QLORA_CODE_INT4, QLORA_ERR_UNSUPPORTED);
  if (n == 0) return QLORA_OK;
  ALIGNED_OR_NULL(packed);
  ALIGNED_OR_NULL(absmax);
  ALIGNED_OR_NULL(out);
  qlora_status s = check_device();
  if (s != QLORA_OK) return s;
  const int64_t ndw = ceil_div(n, 8);
  const dim3 grid(grid_for(ndw, 1024, 1 << 20));
  const uint32_t* p = reinterpret_cast<const uint32_t*>(packed);
  if (code == QLORA_CODE_NF4)
    hipLaunchKernelGGL(dequantize_4bit_kernel<kCodeNF4>, grid, dim3(256), 0, as_stream(stream), p,
                       absmax, n, out);
  else
    hipLaunchKernelGGL(dequantize_4bit_kernel<kCodeINT4>, grid, dim3(256), 0, as_stream(stream),
                       p, absmax, n, out);
  return launched();
}

namespace {
int64_t quant_error_wgs(int64_t n) {
  return std::max<int64_t>(1, std::min<int64_t>(ceil_div(ceil_div(n, 8), 1024), kErrMaxWgs));
}
}  // namespace

size_t qlora_quant_error_workspace_size(int64_t n) {
  if (n < 0) return 0;
  return std::max<size_t>(256, (size_t)quant_error_wgs(n) * sizeof(double));
}

qlora_status qlora_quant_sq_error(const float* w, int64_t n, int32_t code, const uint8_t* packed,
                                  const float* absmax, double* sse, void* workspace,
                                  size_t ws_bytes, void* stream) {
  QCHECK(n >= 0, QLORA_ERR_SHAPE);
  QCHECK(code == QLORA_CODE_NF4 || code == QLORA_CODE_INT4, QLORA_ERR_UNSUPPORTED);
  QCHECK(sse != nullptr, QLORA_ERR_NULL);
  QCHECK((reinterpret_cast<uintptr_t>(sse) & 7) == 0, QLORA_ERR_ALIGN);
  if (n > 0) {
    ALIGNED_OR_NULL(w);
    ALIGNED_OR_NULL(packed);
    ALIGNED_OR_NULL(absmax);
  }
  QCHECK(workspace != nullptr && aligned16(workspace) &&
             ws_bytes >= qlora_quant_error_workspace_size(n),
         QLORA_ERR_WORKSPACE);
  qlora_status s = check_device();
  if (s != QLORA_OK) return s;
  hipStream_t st = as_stream(stream);
  double* partials = static_cast<double*>(workspace);
  int32_t npart = 0;
  if (n > 0) {
    npart = (int32_t)quant_error_wgs(n);
    const uint32_t* p = reinterpret_cast<const uint32_t*>(packed);
    if (code == QLORA_CODE_NF4)
      hipLaunchKernelGGL(quant_sq_error_kernel<kCodeNF4>, dim3(npart), dim3(256), 0, st, w, n, p,
                         absmax, partials);
    else
      hipLaunchKernelGGL(quant_sq_error_kernel<kCodeINT4>, dim3(npart), dim3(256), 0, st, w, n, p,
                         absmax, partials);
  }
  hipLaunchKernelGGL(sum_partials_kernel, dim3(1), dim3(256), 0, st, partials, npart, sse);
  return launched();
}

qlora_status qlora_merge_adapter(const qlora_bf16* w16, const qlora_nf4_weight* w4, int64_t n_out,
                                 int64_t k_in, const qlora_bf16* A, const qlora_bf16* B, int32_t r,
                                 float alpha, qlora_bf16* merged, uint8_t* packed, int8_t* qabsmax,
                                 float* c2, void* stream) {
  QCHECK(w16 != nullptr || w4 != nullptr, QLORA_ERR_NULL);
  QCHECK(w16 == nullptr || w4 == nullptr, QLORA_ERR_UNSUPPORTED);
  QCHECK(n_out >= 0 && k_in >= 0 && k_in % 64 == 0, QLORA_ERR_SHAPE);
  QCHECK(ceil_div(n_out, kMergeRows) <= 65535, QLORA_ERR_SHAPE);
  QCHECK(r >= 1 && r <= QLORA_MAX_RANK, QLORA_ERR_UNSUPPORTED);
  if (w4) {
    qlora_status v = validate_weight(w4);
    if (v != QLORA_OK) return v;
    QCHECK(w4->n_out == n_out && w4->k_in == k_in, QLORA_ERR_SHAPE);
  }
  if (n_out == 0 || k_in == 0) return QLORA_OK;
  if (w16) {
    ALIGNED_OR_NULL(w16);
  }
  ALIGNED_OR_NULL(A);
  ALIGNED_OR_NULL(B);
  ALIGNED_OR_NULL(merged);
  if (packed) {
    ALIGNED_OR_NULL(packed);
    ALIGNED_OR_NULL(qabsmax);
    ALIGNED_OR_NULL(c2);
  }
  qlora_status s = check_device();
  if (s != QLORA_OK) return s;
  hipStream_t st = as_stream(stream);
  MergeArgs g{};
  g.w16 = w16;
  if (w4) {
    g.packed = w4->packed;
    g.qabsmax = w4->qabsmax;
    g.c2 = w4->c2;
  }
  g.a = A; g.b = B; g.n_out = n_out; g.k_in = k_in; g.r = r; g.s = scale_of(alpha, r);
  g.merged = merged;
  hipLaunchKernelGGL(merge_adapter_kernel,
                     dim3((unsigned)ceil_div(k_in, kMergeCols), (unsigned)ceil_div(n_out, kMergeRows)),
                     dim3(256), 0, st, g);
  if ((s = launched()) != QLORA_OK || !packed) return s;
  const int64_t n = n_out * k_in, nb = n / 64, ng = ceil_div(nb, 256);
  QCHECK(ng <= 0x7fffffff, QLORA_ERR_SHAPE);
  const int64_t grid = std::min<int64_t>(ng, 4 * (int64_t)device_cus());
  hipLaunchKernelGGL(quantize_nf4_dq_bf16_kernel, dim3((unsigned)grid), dim3(256), 0, st, merged, n,
                     nb, packed, qabsmax, c2);
  return launched();
}

qlora_status qlora_double_quant(const float* absmax, int64_t nblocks, int32_t group,
                                int8_t* qabsmax, float* c2, void* stream) {
  QCHECK(nblocks >= 0, QLORA_ERR_SHAPE);
  QCHECK(group == QLORA_DQ_GROUP, QLORA_ERR_UNSUPPORTED);
  if (nblocks == 0) return QLORA_OK;
  ALIGNED_OR_NULL(absmax);
  ALIGNED_OR_NULL(qabsmax);
  ALIGNED_OR_NULL(c2);
  qlora_status s = check_device();
  if (s != QLORA_OK) return s;
  const int64_t ng = ceil_div(nblocks, 256);
  QCHECK(ng <= 0x7fffffff, QLORA_ERR_SHAPE);
  hipLaunchKernelGGL(double_quant_kernel, dim3((unsigned)ng), dim3(256), 0, as_stream(stream),
                     absmax, nblocks, qabsmax, c2);
  return launched();
}

qlora_status qlora_quantize_nf4_dq(const float* w, int64_t n, uint8_t* packed, int8_t* qabsmax,
                                   float* c2, float* absmax, int32_t* nonfinite_flag,
                                   void* stream) {
  QCHECK(n >= 0, QLORA_ERR_SHAPE);
  QCHECK(aligned4(nonfinite_flag), QLORA_ERR_ALIGN);
  if (n == 0) return QLORA_OK;
  ALIGNED_OR_NULL(w);
  ALIGNED_OR_NULL(packed);
  ALIGNED_OR_NULL(qabsmax);
  ALIGNED_OR_NULL(c2);
  QCHECK(absmax == nullptr || aligned16(absmax), QLORA_ERR_ALIGN);
  qlora_status s = check_device();
  if (s != QLORA_OK) return s;
  const int64_t nb = ceil_div(n, 64);
  const int64_t ng = ceil_div(nb, 256);
  QCHECK(ng <= 0x7fffffff && ceil_div(nb * 4, 256) <= 0x7fffffff, QLORA_ERR_SHAPE);
  hipStream_t st = as_stream(stream);
  if (absmax) {
    // With somewhere to put the first-level scales: the first level over
    // 64-block workgroups (many small workgroups keep far more loads in
    // flight than one workgroup per 256-block group can), then the second
    // level from the scales — measured faster than the one-pass kernel
    // despite writing and re-reading 4 bytes per 64 weights.
    hipLaunchKernelGGL(quantize_nf4_kernel, dim3((unsigned)ceil_div(nb * 4, 256)), dim3(256), 0, st,
                       w, n, nb, packed, absmax, nonfinite_flag);
    hipLaunchKernelGGL(double_quant_kernel, dim3((unsigned)ng), dim3(256), 0, st,
                       (const float*)absmax, nb, qabsmax, c2);
    return launched();
  }
  // one pass: four workgroups per CU stride over the groups (enough bytes in
  // flight, and every workgroup overlaps its loads with its own arithmetic)
  const int64_t grid = std::min<int64_t>(ng, 4 * (int64_t)device_cus());
  hipLaunchKernelGGL(quantize_nf4_dq_kernel, dim3((unsigned)grid), dim3(256), 0, st, w, n, nb,
                     packed, qabsmax, c2, absmax, nonfinite_flag);
  return launched();
}

qlora_status qlora_dequantize_nf4(const qlora_nf4_weight* w, qlora_bf16* out, void* stream) {
  qlora_status s = validate_weight(w);
  if (s != QLORA_OK) return s;
  const int64_t n = w->n_out * w->k_in;
  QCHECK(n % 64 == 0, QLORA_ERR_SHAPE);
  if (n == 0) return QLORA_OK;
  ALIGNED_OR_NULL(out);
  s = check_device();
  if (s != QLORA_OK) return s;
  const int64_t ndw = n / 8;
  hipLaunchKernelGGL(dequantize_nf4_kernel, dim3(grid_for(ndw, 1024, 1 << 20)), dim3(256), 0,
                     as_stream(stream), reinterpret_cast<const uint32_t*>(w->packed), w->qabsmax,
                     w->c2, ndw, reinterpret_cast<u32x4*>(out));
  return launched();
}

qlora_status qlora_quantize_nf4_dq_batch(const qlora_quant_job* jobs, int32_t count, void* stream) {
  QCHECK(count >= 0, QLORA_ERR_SHAPE);
  if (count == 0) return QLORA_OK;
  QCHECK(jobs != nullptr, QLORA_ERR_NULL);
  // every job is checked before anything is enqueued
  for (int32_t i = 0; i < count; ++i) {
    const qlora_quant_job& j = jobs[i];
    QCHECK(j.n >= 0, QLORA_ERR_SHAPE);
    if (j.n == 0) continue;
    ALIGNED_OR_NULL(j.w);
    ALIGNED_OR_NULL(j.packed);
    ALIGNED_OR_NULL(j.qabsmax);
    ALIGNED_OR_NULL(j.c2);
    ALIGNED_OR_NULL(j.absmax);
    QCHECK(aligned4(j.nonfinite_flag), QLORA_ERR_ALIGN);
    QCHECK(ceil_div(ceil_div(j.n, 64) * 4, 256) <= 0x7fffffff, QLORA_ERR_SHAPE);
  }
  qlora_status s = check_device();
  if (s != QLORA_OK) return s;
  hipStream_t st = as_stream(stream);
  // launches of up to kBatchMax jobs: the first level of all of them, then the
  // second level of all of them (each reads only its own job's scales)
  int32_t i = 0;
  while (i < count) {
    QuantBatch qb{};
    DqBatch db{};
    int64_t wq = 0, wd = 0;
    int32_t c = 0;
    for (; i < count && c < kBatchMax; ++i) {
      const qlora_quant_job& j = jobs[i];
      if (j.n == 0) continue;
      const int64_t nb = ceil_div(j.n, 64), ng = ceil_div(nb, 256), nwg = ceil_div(nb * 4, 256);
      if (wq + nwg > 0x7fffffff || wd + ng > 0x7fffffff) break;  // the next launch takes it
      qb.j[c] = QuantJob1{j.w, j.n, j.packed, j.absmax, j.nonfinite_flag};
      qb.wg0[c] = wq;
      db.j[c] = DqJob{j.absmax, nb, j.qabsmax, j.c2};
      db.wg0[c] = wd;
      wq += nwg;
      wd += ng;
      ++c;
    }
    if (c == 0) continue;
    qb.count = db.count = c;
    qb.wg0[c] = wq;
    db.wg0[c] = wd;
    hipLaunchKernelGGL(quantize_nf4_batch_kernel, dim3((unsigned)wq), dim3(256), 0, st, qb);
    hipLaunchKernelGGL(double_quant_batch_kernel, dim3((unsigned)wd), dim3(256), 0, st, db);
    if ((s = launched()) != QLORA_OK) return s;
  }
  return QLORA_OK;
}

qlora_status qlora_dequantize_nf4_batch(const qlora_nf4_weight* weights, qlora_bf16* const* outs,
                                        int32_t count, void* stream) {
  QCHECK(count >= 0, QLORA_ERR_SHAPE);
  if (count == 0) return QLORA_OK;
  QCHECK(weights != nullptr && outs != nullptr, QLORA_ERR_NULL);
  for (int32_t i = 0; i < count; ++i) {
    qlora_status s = validate_weight(&weights[i]);
    if (s != QLORA_OK) return s;
    const int64_t n = weights[i].n_out * weights[i].k_in;
    QCHECK(n % 64 == 0, QLORA_ERR_SHAPE);
    if (n == 0) continue;
    ALIGNED_OR_NULL(outs[i]);
    QCHECK(ceil_div(n / 8, 1024) <= 0x7fffffff, QLORA_ERR_SHAPE);
  }
  qlora_status s = check_device();
  if (s != QLORA_OK) return s;
  hipStream_t st = as_stream(stream);
  int32_t i = 0;
  while (i < count) {
    DeqBatch b{};
    int64_t wg = 0;
    int32_t c = 0;
    for (; i < count && c < kBatchMax; ++i) {
      const qlora_nf4_weight& w = weights[i];
      const int64_t ndw = w.n_out * w.k_in / 8;
      if (ndw == 0) continue;
      const int64_t nwg = ceil_div(ndw, 1024);
      if (wg + nwg > 0x7fffffff) break;  // the next launch takes it
      b.j[c] = DeqJob{reinterpret_cast<const uint32_t*>(w.packed), w.qabsmax, w.c2,
                      reinterpret_cast<u32x4*>(outs[i]), ndw};
      b.wg0[c] = wg;
      wg += nwg;
      ++c;
    }
    if (c == 0) continue;
    b.count = c;
    b.wg0[c] = wg;
    hipLaunchKernelGGL(dequantize_nf4_batch_kernel, dim3((unsigned)wg), dim3(256), 0, st, b);
    if ((s = launched()) != QLORA_OK) return s;
  }
  return QLORA_OK;
}

qlora_status qlora_lora_down(const qlora_bf16* X, int64_t M, int64_t k_in, const qlora_bf16* A,
                             int32_t r, qlora_bf16* U, void* workspace, size_t ws_bytes,
                             void* stream) {
  QCHECK(M >= 0 && k_in > 0 && k_in % 64 == 0, QLORA_ERR_SHAPE);
  QCHECK(r >= 1 && r <= QLORA_MAX_RANK, QLORA_ERR_UNSUPPORTED);
  if (M == 0) return QLORA_OK;
  ALIGNED_OR_NULL(X);
  ALIGNED_OR_NULL(A);
  ALIGNED_OR_NULL(U);
  // the forward's layout, with n_out taken as 8 (only the U region is used)
  const FwdWs L = fwd_ws(M, 8, k_in, r);
  if (!use_gemv(M)) {
    QCHECK(workspace != nullptr && aligned16(workspace), QLORA_ERR_WORKSPACE);
    QCHECK(ws_bytes >= L.u_part + align256(ad_part_bytes(L.pu, M)), QLORA_ERR_WORKSPACE);
  }
  qlora_status s = check_device();
  if (s != QLORA_OK) return s;
  return lora_down_impl(X, M, k_in, A, r, U, nullptr, 0, static_cast<char*>(workspace), L,
                        as_stream(stream));
}

qlora_status qlora_nf4_matmul_fwd(const qlora_nf4_weight* w, const qlora_bf16* X, int64_t M,
                                  const qlora_bf16* U, const qlora_bf16* B, int32_t r, float alpha,
                                  qlora_bf16* Y, void* workspace, size_t ws_bytes, void* stream) {
  qlora_status s = validate_linear(w, M, r);
  if (s != QLORA_OK) return s;
  if (M == 0) return QLORA_OK;
  ALIGNED_OR_NULL(X);
  ALIGNED_OR_NULL(U);
  ALIGNED_OR_NULL(B);
  ALIGNED_OR_NULL(Y);
  const FwdWs L = fwd_ws(M, w->n_out, w->k_in, r);
  QCHECK(workspace != nullptr && aligned16(workspace) && ws_bytes >= L.total, QLORA_ERR_WORKSPACE);
  s = check_device();
  if (s != QLORA_OK) return s;
  char* ws = static_cast<char*>(workspace);
  hipStream_t st = as_stream(stream);
  const uint16_t* up = U;
  const uint16_t* bp = B;
  int64_t ld = r;
  if (r % 8 != 0 && !use_gemv(M)) {
    uint16_t* Up = reinterpret_cast<uint16_t*>(ws + L.pad_u);
    uint16_t* Bp = reinterpret_cast<uint16_t*>(ws + L.pad_b);
    hipLaunchKernelGGL(pad_cols_kernel, dim3(grid_for(M * L.rp)), dim3(256), 0, st, U, (int64_t)r,
                       M, (int64_t)r, L.rp, Up, L.rp);
    hipLaunchKernelGGL(pad_cols_kernel, dim3(grid_for(w->n_out * L.rp)), dim3(256), 0, st, B,
                       (int64_t)r, w->n_out, (int64_t)r, L.rp, Bp, L.rp);
    if ((s = launched()) != QLORA_OK) return s;
    up = Up;
    bp = Bp;
    ld = L.rp;
  }
  return matmul_fwd_impl(w, X, M, up, ld, bp, ld, r, scale_of(alpha, r), Y, ws, L, st);
}

qlora_status qlora_linear_fwd(const qlora_nf4_weight* w, const qlora_bf16* X, int64_t M,
                              const qlora_bf16* A, const qlora_bf16* B, int32_t r, float alpha,
                              qlora_bf16* Y, qlora_bf16* U, void* workspace, size_t ws_bytes,
                              void* stream) {
  qlora_status s = validate_linear(w, M, r);
  if (s != QLORA_OK) return s;
  if (M == 0) return QLORA_OK;
  ALIGNED_OR_NULL(X);
  ALIGNED_OR_NULL(A);
  ALIGNED_OR_NULL(B);
  ALIGNED_OR_NULL(Y);
  ALIGNED_OR_NULL(U);
  const FwdWs L = fwd_ws(M, w->n_out, w->k_in, r);
  QCHECK(workspace != nullptr && aligned16(workspace) && ws_bytes >= L.total, QLORA_ERR_WORKSPACE);
  s = check_device();
  if (s != QLORA_OK) return s;
  return linear_fwd_impl(w, X, X, M, A, B, r, scale_of(alpha, r), Y, U,
                         static_cast<char*>(workspace), L, as_stream(stream));
}

}  // extern "C"

// ---- the forward without a caller workspace -----------------------------------
// Its scratch (split-K partial sums of U and of the 17..127-token product,
// the zero-padded copies of U and B for ranks that are not a multiple of 8)
// lives in this file-scope array, one copy per GPU, held until the process
// ends.  In host code `scratch` names a host-side stand-in, never the device
// memory: its device address is looked up once per device (with that device
// current) and only that address reaches kernels.
namespace {

static __device__ __attribute__((aligned(256))) char scratch[QLORA_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::atomic<char*> g_scratch_dev[kMaxDevices];

// Device address of the current device's copy of `scratch`.
qlora_status scratch_of_current_device(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QLORA_ERR_DEVICE;
  char* p = g_scratch_dev[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_dev[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* addr = nullptr;
      if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr)
        return QLORA_ERR_DEVICE;
      p = static_cast<char*>(addr);
      g_scratch_dev[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return QLORA_OK;
}

}  // namespace

extern "C" {

qlora_status qlora_linear_fwd_noalloc(const qlora_nf4_weight* w, const qlora_bf16* X, int64_t M,
                                      const qlora_bf16* A, const qlora_bf16* B, int32_t r,
                                      float alpha, qlora_bf16* Y, qlora_bf16* U, void* stream) {
  qlora_status s = validate_linear(w, M, r);
  if (s != QLORA_OK) return s;
  if (M == 0) return QLORA_OK;
  ALIGNED_OR_NULL(X);
  ALIGNED_OR_NULL(A);
  ALIGNED_OR_NULL(B);
  ALIGNED_OR_NULL(Y);
  ALIGNED_OR_NULL(U);
  const FwdWs L = fwd_ws(M, w->n_out, w->k_in, r);
  QCHECK(L.total <= QLORA_NOALLOC_SCRATCH_BYTES, QLORA_ERR_WORKSPACE);
  s = check_device();
  if (s != QLORA_OK) return s;
  char* ws = nullptr;
  s = scratch_of_current_device(&ws);
  if (s != QLORA_OK) return s;
  return linear_fwd_impl(w, X, X, M, A, B, r, scale_of(alpha, r), Y, U, ws, L, as_stream(stream));
}

qlora_status qlora_lora_dropout(const qlora_bf16* X, int64_t M, int64_t k_in, float p,
                                uint64_t seed, uint64_t offset, qlora_bf16* Xd, void* stream) {
  QCHECK(M >= 0 && k_in >= 0 && k_in % 8 == 0, QLORA_ERR_SHAPE);
  DropoutKey key;
  QCHECK(dropout_key(p, seed, offset, &key), QLORA_ERR_UNSUPPORTED);
  if (M == 0 || k_in == 0) return QLORA_OK;
  ALIGNED_OR_NULL(X);
  ALIGNED_OR_NULL(Xd);
  qlora_status s = check_device();
  if (s != QLORA_OK) return s;
  return run_dropout(X, M * k_in, key, Xd, as_stream(stream));
}

qlora_status qlora_linear_fwd_dropout(const qlora_nf4_weight* w, const qlora_bf16* X, int64_t M,
                                      const qlora_bf16* A, const qlora_bf16* B, int32_t r,
                                      float alpha, float p, uint64_t seed, uint64_t offset,
                                      qlora_bf16* Y, qlora_bf16* U, qlora_bf16* Xd,
                                      void* workspace, size_t ws_bytes, void* stream) {
  qlora_status s = validate_linear(w, M, r);
  if (s != QLORA_OK) return s;
  DropoutKey key;
  QCHECK(dropout_key(p, seed, offset, &key), QLORA_ERR_UNSUPPORTED);
  if (M == 0) return QLORA_OK;
  ALIGNED_OR_NULL(X);
  ALIGNED_OR_NULL(A);
  ALIGNED_OR_NULL(B);
  ALIGNED_OR_NULL(Y);
  ALIGNED_OR_NULL(U);
  ALIGNED_OR_NULL(Xd);
  const FwdWs L = fwd_ws(M, w->n_out, w->k_in, r);
  QCHECK(workspace != nullptr && aligned16(workspace) && ws_bytes >= L.total, QLORA_ERR_WORKSPACE);
  s = check_device();
  if (s != QLORA_OK) return s;
  hipStream_t st = as_stream(stream);
  if ((s = run_dropout(X, M * w->k_in, key, Xd, st)) != QLORA_OK) return s;
  return linear_fwd_impl(w, X, Xd, M, A, B, r, scale_with_dropout(scale_of(alpha, r), p), Y, U,
                         static_cast<char*>(workspace), L, st);
}

qlora_status qlora_linear_bwd(const qlora_nf4_weight* w, const qlora_bf16* X, const qlora_bf16* dY,
                              int64_t M, const qlora_bf16* A, const qlora_bf16* B, int32_t r,
                              float alpha, const qlora_bf16* U, qlora_bf16* dX, float* dA,
                              float* dB, void* workspace, size_t ws_bytes, void* stream) {
  qlora_status s = validate_bwd(w, X, dY, M, A, B, r, U, dX, dA, dB);
  if (s != QLORA_OK) return s;
  const BwdWs L = bwd_ws(M, w->n_out, w->k_in, r);
  QCHECK(workspace != nullptr && aligned16(workspace) && ws_bytes >= L.total, QLORA_ERR_WORKSPACE);
  s = check_device();
  if (s != QLORA_OK) return s;
  return linear_bwd_impl(w, X, dY, M, A, B, r, scale_of(alpha, r), nullptr, U, dX, dA, dB,
                         static_cast<char*>(workspace), L, as_stream(stream));
}

qlora_status qlora_linear_bwd_dropout(const qlora_nf4_weight* w, const qlora_bf16* Xd,
                                      const qlora_bf16* dY, int64_t M, const qlora_bf16* A,
                                      const qlora_bf16* B, int32_t r, float alpha, float p,
                                      uint64_t seed, uint64_t offset, const qlora_bf16* U,
                                      qlora_bf16* dX, float* dA, float* dB, void* workspace,
                                      size_t ws_bytes, void* stream) {
  qlora_status s = validate_bwd(w, Xd, dY, M, A, B, r, U, dX, dA, dB);
  if (s != QLORA_OK) return s;
  DropoutKey key;
  QCHECK(dropout_key(p, seed, offset, &key), QLORA_ERR_UNSUPPORTED);
  const BwdWs L = bwd_ws(M, w->n_out, w->k_in, r);
  QCHECK(workspace != nullptr && aligned16(workspace) &&
             ws_bytes >= bwd_dropout_ws(L, M, w->k_in),
         QLORA_ERR_WORKSPACE);
  s = check_device();
  if (s != QLORA_OK) return s;
  return linear_bwd_impl(w, Xd, dY, M, A, B, r, scale_with_dropout(scale_of(alpha, r), p),
                         key.thr > 0 ? &key : nullptr, U, dX, dA, dB,
                         static_cast<char*>(workspace), L, as_stream(stream));
}

// AdamW workspace: the clipping coefficient (float) at byte 0, the norm
// launches' float64 partial sums from byte kAdamPartialsOffset.
constexpr size_t kAdamPartialsOffset = 256;

size_t qlora_adamw_workspace_size(int32_t count) {
  if (count < 0) return 0;
  const int64_t groups = std::max<int64_t>(1, ceil_div(count, kAdamMaxTensors));
  return kAdamPartialsOffset + (size_t)groups * kAdamNormWgs * sizeof(double);
}

namespace {

// Arguments of both steps, checked before anything is enqueued.
qlora_status validate_adamw_step(const qlora_adamw_tensor* t, int32_t count, float lr,
                                 float beta1, float beta2, float eps, float weight_decay,
                                 int64_t step, float max_grad_norm, float* grad_norm,
                                 void* workspace, size_t ws_bytes) {
  qlora_status s = validate_adamw_tensors(t, count);
  if (s != QLORA_OK) return s;
  if ((s = validate_adamw_hyper(lr, beta1, beta2, eps, weight_decay, step, max_grad_norm,
                                grad_norm)) != QLORA_OK)
    return s;
  if (max_grad_norm > 0.0f || grad_norm != nullptr)
    QCHECK(workspace != nullptr && aligned16(workspace) &&
               ws_bytes >= qlora_adamw_workspace_size(count),
           QLORA_ERR_WORKSPACE);
  return check_device();
}

// The step itself (validated arguments): the norm passes and the clipping
// coefficient when asked for, then the update, kAdamMaxTensors tensors per
// launch.  m and v may be device memory or pinned host memory.
qlora_status adamw_step_impl(const qlora_adamw_tensor* t, int32_t count, float lr, float beta1,
                             float beta2, float eps, float weight_decay, int64_t step,
                             float max_grad_norm, float* grad_norm, void* workspace,
                             void* stream) {
  qlora_status s;
  if (count == 0) return QLORA_OK;
  const bool clip = max_grad_norm > 0.0f;
  const bool need_norm = clip || grad_norm != nullptr;
  hipStream_t st = as_stream(stream);
  const AdamHyper h = adamw_hyper(lr, beta1, beta2, eps, weight_decay, step);

  // Groups of kAdamMaxTensors tensors, each one list per launch.
  const int groups = (int)ceil_div(count, kAdamMaxTensors);
  auto list_of = [&](int gidx) {
    AdamList L{};
    const int first = gidx * kAdamMaxTensors;
    L.count = std::min(kAdamMaxTensors, count - first);
    int64_t c = 0;
    for (int i = 0; i < L.count; ++i) {
      const qlora_adamw_tensor& x = t[first + i];
      L.t[i] = AdamTensor{x.param, x.grad, x.m, x.v, x.param_bf16, x.n, c};
      c += ceil_div(x.n, kAdamChunk);
    }
    L.chunks = c;
    return L;
  };
  float* coef = static_cast<float*>(workspace);
  if (need_norm) {
    double* partials = reinterpret_cast<double*>(static_cast<char*>(workspace) +
                                                 kAdamPartialsOffset);
    int32_t npart = 0;  // partial sums packed back to back, in group order
    for (int gidx = 0; gidx < groups; ++gidx) {
      const AdamList L = list_of(gidx);
      if (L.chunks == 0) continue;
      const int grid = (int)std::min<int64_t>(L.chunks, kAdamNormWgs);
      hipLaunchKernelGGL(adam_sqnorm_kernel, dim3(grid), dim3(kAdamThreads), 0, st, L,
                         partials + npart);
      npart += grid;
    }
    hipLaunchKernelGGL(adam_clip_kernel, dim3(1), dim3(kAdamThreads), 0, st, partials, npart,
                       max_grad_norm, clip ? 1 : 0, coef, grad_norm);
    if ((s = launched()) != QLORA_OK) return s;
  }
  for (int gidx = 0; gidx < groups; ++gidx) {
    const AdamList L = list_of(gidx);
    if (L.chunks == 0) continue;
    const int grid = (int)std::min<int64_t>(L.chunks, kAdamMaxGrid);
    hipLaunchKernelGGL(adam_update_kernel, dim3(grid), dim3(kAdamThreads), 0, st, L, h,
                       clip ? coef : nullptr);
  }
  return launched();
}

}  // namespace

qlora_status qlora_adamw_step(const qlora_adamw_tensor* t, int32_t count, float lr, float beta1,
                              float beta2, float eps, float weight_decay, int64_t step,
                              float max_grad_norm, float* grad_norm, void* workspace,
                              size_t ws_bytes, void* stream) {
  const qlora_status s = validate_adamw_step(t, count, lr, beta1, beta2, eps, weight_decay, step,
                                             max_grad_norm, grad_norm, workspace, ws_bytes);
  if (s != QLORA_OK) return s;
  return adamw_step_impl(t, count, lr, beta1, beta2, eps, weight_decay, step, max_grad_norm,
                         grad_norm, workspace, stream);
}

// Paged step: m and v stay in pinned host memory and the update kernel reads
// and writes them there, across the host link (reads and writes flow at the
// same time); the norm passes read only the gradients.
qlora_status qlora_adamw_step_paged(const qlora_adamw_tensor* t, int32_t count, float lr,
                                    float beta1, float beta2, float eps, float weight_decay,
                                    int64_t step, float max_grad_norm, float* grad_norm,
                                    void* workspace, size_t ws_bytes, void* stream) {
  qlora_status s = validate_adamw_step(t, count, lr, beta1, beta2, eps, weight_decay, step,
                                       max_grad_norm, grad_norm, workspace, ws_bytes);
  if (s != QLORA_OK) return s;
  // the states must be page-locked host memory; the kernel reaches them at
  // the device addresses of their mappings (the queries' errors, if any, are
  // cleared)
  std::vector<qlora_adamw_tensor> dt(t, t + count);
  for (qlora_adamw_tensor& x : dt) {
    if (x.n == 0) continue;
    for (float** hp : {&x.m, &x.v}) {
      hipPointerAttribute_t at{};
      const hipError_t e = hipPointerGetAttributes(&at, *hp);
      (void)hipGetLastError();
      QCHECK(e == hipSuccess && at.type == hipMemoryTypeHost && at.devicePointer != nullptr,
             QLORA_ERR_UNSUPPORTED);
      QCHECK(aligned16(at.devicePointer), QLORA_ERR_ALIGN);
      *hp = static_cast<float*>(at.devicePointer);
    }
  }
  return adamw_step_impl(dt.data(), count, lr, beta1, beta2, eps, weight_decay, step,
                         max_grad_norm, grad_norm, workspace, stream);
}

size_t qlora_adamw_plan_size(const qlora_adamw_tensor* tensors, int32_t count) {
  if (count < 0 || (count > 0 && tensors == nullptr)) return 0;
  for (int32_t i = 0; i < count; ++i)
    if (tensors[i].n < 0) return 0;
  return std::max<size_t>(256, plan_tmap_offset(count) +
                                   align256((size_t)plan_chunks(tensors, count) * 4));
}

qlora_status qlora_adamw_plan_init(const qlora_adamw_tensor* tensors, int32_t count, void* device,
                                   size_t bytes, qlora_adamw_plan* plan, void* stream) {
  qlora_status s = validate_adamw_tensors(tensors, count);
  if (s != QLORA_OK) return s;
  QCHECK(plan != nullptr, QLORA_ERR_NULL);
  QCHECK(device != nullptr && aligned16(device) && bytes >= qlora_adamw_plan_size(tensors, count),
         QLORA_ERR_WORKSPACE);
  const int64_t chunks = plan_chunks(tensors, count);
  QCHECK(chunks <= 0x7fffffff, QLORA_ERR_SHAPE);
  s = check_device();
  if (s != QLORA_OK) return s;
  const size_t toff = plan_tmap_offset(count);
  std::vector<char> host(toff + (size_t)chunks * 4, 0);
  AdamTensor* d = reinterpret_cast<AdamTensor*>(host.data());
  int32_t* tmap = reinterpret_cast<int32_t*>(host.data() + toff);
  int64_t c = 0;
  for (int32_t i = 0; i < count; ++i) {
    const qlora_adamw_tensor& x = tensors[i];
    d[i] = AdamTensor{x.param, x.grad, x.m, x.v, x.param_bf16, x.n, c};
    const int64_t ci = ceil_div(x.n, kAdamChunk);
    for (int64_t k = 0; k < ci; ++k) tmap[c + k] = i;
    c += ci;
  }
  hipStream_t st = as_stream(stream);
  if (!host.empty()) {
    if (hipMemcpyAsync(device, host.data(), host.size(), hipMemcpyHostToDevice, st) != hipSuccess)
      return QLORA_ERR_LAUNCH;
    // the host copy lives only for this call
    if (hipStreamSynchronize(st) != hipSuccess) return QLORA_ERR_LAUNCH;
  }
  plan->device = device;
  plan->count = count;
  plan->chunks = chunks;
  return QLORA_OK;
}

size_t qlora_adamw_plan_workspace_size(const qlora_adamw_plan* plan) {
  if (plan == nullptr || plan->chunks < 0) return 0;
  return kAdamPartialsOffset +
         (size_t)std::max<int64_t>(1, std::min<int64_t>(plan->chunks, kAdamPlanNormWgs)) *
             sizeof(double);
}

qlora_status qlora_adamw_step_plan(const qlora_adamw_plan* plan, float lr, float beta1,
                                   float beta2, float eps, float weight_decay, int64_t step,
                                   float max_grad_norm, float* grad_norm, void* workspace,
                                   size_t ws_bytes, void* stream) {
  QCHECK(plan != nullptr, QLORA_ERR_NULL);
  QCHECK(plan->count >= 0 && plan->chunks >= 0, QLORA_ERR_SHAPE);
  QCHECK(plan->chunks == 0 || plan->device != nullptr, QLORA_ERR_NULL);
  qlora_status s = validate_adamw_hyper(lr, beta1, beta2, eps, weight_decay, step, max_grad_norm,
                                        grad_norm);
  if (s != QLORA_OK) return s;
  const bool clip = max_grad_norm > 0.0f;
  const bool need_norm = clip || grad_norm != nullptr;
  if (need_norm)
    QCHECK(workspace != nullptr && aligned16(workspace) &&
               ws_bytes >= qlora_adamw_plan_workspace_size(plan),
           QLORA_ERR_WORKSPACE);
  s = check_device();
  if (s != QLORA_OK) return s;
  hipStream_t st = as_stream(stream);
  const AdamHyper h = adamw_hyper(lr, beta1, beta2, eps, weight_decay, step);
  AdamPlanDev P{};
  P.t = static_cast<const AdamTensor*>(plan->device);
  P.tmap = reinterpret_cast<const int32_t*>(static_cast<const char*>(plan->device) +
                                            plan_tmap_offset(plan->count));
  P.chunks = plan->chunks;
  float* coef = static_cast<float*>(workspace);
  if (need_norm) {
    double* partials =
        reinterpret_cast<double*>(static_cast<char*>(workspace) + kAdamPartialsOffset);
    int32_t npart = 0;
    if (P.chunks > 0) {
      npart = (int32_t)std::min<int64_t>(P.chunks, kAdamPlanNormWgs);
      hipLaunchKernelGGL(adam_sqnorm_plan_kernel, dim3(npart), dim3(kAdamThreads), 0, st, P,
                         partials);
    }
    hipLaunchKernelGGL(adam_clip_kernel, dim3(1), dim3(kAdamThreads), 0, st, partials, npart,
                       max_grad_norm, clip ? 1 : 0, coef, grad_norm);
    if ((s = launched()) != QLORA_OK) return s;
  }
  if (P.chunks == 0) return QLORA_OK;
  hipLaunchKernelGGL(adam_update_plan_kernel, dim3((unsigned)std::min<int64_t>(P.chunks, kAdamMaxGrid)),
                     dim3(kAdamThreads), 0, st, P, h, clip ? coef : nullptr);
  return launched();
}

}  // extern "C"
