// w4a16.hip -- libw4a16.so: C ABI, argument checks and kernel selection for
// the NVFP4 W4A16 matmul on MI355X (gfx950).  See include/w4a16.h for the
// contract of every entry point.
#include "w4a16.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4a16_kernels.h"
#include "w4a16_mlp.h"
#include "w4a16_quant.h"

namespace w4a16 {
namespace {

constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices];  // 0 = not yet queried

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = __atomic_load_n(&g_cu_count[dev], __ATOMIC_RELAXED);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    __atomic_store_n(&g_cu_count[dev], n, __ATOMIC_RELAXED);
  }
  return n;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Dynamic LDS limit per workgroup (160 KiB per CU, less a little for the
// kernels' static LDS).
constexpr size_t kMaxLds = 160 * 1024 - 256;

// The split-K arrival counters (one int per row block) occupy a fixed area at
// the front of the workspace, the same for every shape, so that calls of
// different shapes can share one workspace: no call's partials ever overlap
// another call's counters.  The fp32 partials follow it.
constexpr size_t kCounterBytes = 4096;
constexpr int kMaxSplitRowBlocks = (int)(kCounterBytes / sizeof(int));
static_assert(kArgmaxSplitCounter == kMaxSplitRowBlocks - 1, "argmax counter: the last of the area");

// Activation rows up to which the VALU kernel runs; the MFMA kernel takes
// the rest.  Its cost is flat up to four rows while the VALU kernel's grows
// with every row: measured by HIP-graph replay on MI355X, M = 3 ran 8-20 %
// faster on the MFMA kernel (square 5120^2 7.07 vs 7.72 us, down 17408 ->
// 5120 14.1 vs 17.6 us, gate/up 2 x 17408 x 5120 22.3 vs 27.0 us); M = 2 was
// mixed (VALU faster on the square and gate/up shapes) and M = 1 is VALU's.
constexpr int kValuMaxM = 2;

// How one matmul call is launched.
struct Plan {
  bool mfma;   // false: VALU kernel (M <= kValuMaxM); true: 4x4x4 MFMA kernel
  int lr;      // VALU: lanes per weight row L; MFMA: row quads per task R
  int D;       // chunk loads in flight per lane (ring depth)
  int W;       // waves per workgroup
  int LB;      // launch bound the kernel was compiled for (>= 64 * W)
  int nrb;     // row blocks
  int S;       // K-slices (split-K factor); grid = nrb * S workgroups
  int rq, rr;  // rows per row block: rq, plus one for the first rr blocks
  int kmax;    // segment slots per wave
  size_t lds;  // dynamic LDS bytes per workgroup
  size_t ws;   // workspace bytes (fp32 partials) when S > 1
  int rows_cpl; // > 0: the whole-row VALU kernel for K = 1024 * rows_cpl (S = 1)
  int xr_cpl;   // > 0: the K-column MFMA kernel for K = 1024 * xr_cpl (S K-slices)
  bool xr_ring; // the K-column kernel's ring variant (partials added per iteration)
  int wide_mt;  // > 0: the wide kernel for M <= 8 * wide_mt (rq = tiles of 32 rows per row block)
  int wide_steps; // ... and its K-slice length in steps of 256 inputs (the last slice may be shorter)
};

// ---- kernel registry ---------------------------------------------------------
// Every compiled variant, keyed by its template parameters.  The planner only
// picks variants that are listed here.
struct KernEntry {
  bool mfma;
  int rows;   // VALU: MT (= M); MFMA: P (activation-row passes of 4)
  int lr, D;
  int epi;    // epilogue: kEpiPlain, kEpiSwiglu or kEpiArgmax
  int LB;
  const void* fn;
};

#define W4A16_VE(MT, L, D, F, LB) \
  {false, MT, L, D, F, LB, reinterpret_cast<const void*>(&k_gemm_valu<MT, L, D, F, LB>)},
#define W4A16_ME(P, R, D, F, LB) \
  {true, P, R, D, F, LB, reinterpret_cast<const void*>(&k_gemm_mfma<P, R, D, F, LB>)},
#define W4A16_VALU_ALL_MT(L, D, F, LB) W4A16_VE(1, L, D, F, LB) W4A16_VE(2, L, D, F, LB)
#define W4A16_MFMA_ALL_P(R, D, F, LB) \
  W4A16_ME(1, R, D, F, LB) W4A16_ME(2, R, D, F, LB) W4A16_ME(3, R, D, F, LB) W4A16_ME(4, R, D, F, LB)

#ifdef W4A16_TUNING
#define W4A16_VALU_SET(F)                                                          \
  W4A16_VALU_ALL_MT(8, 4, F, 1024) W4A16_VALU_ALL_MT(8, 8, F, 512)                 \
  W4A16_VALU_ALL_MT(16, 4, F, 1024) W4A16_VALU_ALL_MT(16, 8, F, 512)               \
  W4A16_VALU_ALL_MT(16, 8, F, 1024) W4A16_VALU_ALL_MT(16, 12, F, 512)              \
  W4A16_VALU_ALL_MT(16, 16, F, 512)                                                \
  W4A16_VALU_ALL_MT(32, 4, F, 1024) W4A16_VALU_ALL_MT(32, 8, F, 512)               \
  W4A16_VALU_ALL_MT(32, 8, F, 1024) W4A16_VALU_ALL_MT(32, 12, F, 512)              \
  W4A16_VALU_ALL_MT(32, 16, F, 512) W4A16_VALU_ALL_MT(32, 5, F, 1024)            \
  W4A16_VALU_ALL_MT(32, 2, F, 1024)
#define W4A16_MFMA_SET(F)                                                          \
  W4A16_MFMA_ALL_P(1, 8, F, 512) W4A16_MFMA_ALL_P(1, 16, F, 512)                   \
  W4A16_MFMA_ALL_P(2, 4, F, 512) W4A16_MFMA_ALL_P(2, 8, F, 512)                    \
  W4A16_MFMA_ALL_P(2, 8, F, 1024) W4A16_MFMA_ALL_P(4, 4, F, 512)                   \
  W4A16_ME(5, 1, 4, F, 512) W4A16_ME(6, 1, 4, F, 512) W4A16_ME(7, 1, 4, F, 512)     \
  W4A16_ME(8, 1, 4, F, 512) W4A16_MFMA_ALL_P(1, 4, F, 512)                         \
  W4A16_MFMA_ALL_P(1, 2, F, 1024) W4A16_MFMA_ALL_P(1, 4, F, 1024)
#endif
// the launch rules' variants (the argmax epilogue exists only in these)
#define W4A16_VALU_BASE(F)                                                         \
  W4A16_VALU_ALL_MT(8, 4, F, 1024) W4A16_VALU_ALL_MT(16, 4, F, 1024)               \
  W4A16_VALU_ALL_MT(32, 4, F, 1024)
#define W4A16_MFMA_BASE(F)                                                         \
  W4A16_MFMA_ALL_P(1, 4, F, 512) W4A16_ME(5, 1, 4, F, 512) W4A16_ME(6, 1, 4, F, 512)     \
  W4A16_ME(7, 1, 4, F, 512) W4A16_ME(8, 1, 4, F, 512)
#ifndef W4A16_TUNING
#define W4A16_VALU_SET(F) W4A16_VALU_BASE(F)
#define W4A16_MFMA_SET(F) W4A16_MFMA_BASE(F)
#endif

const KernEntry kKernels[] = {
    W4A16_VALU_SET(kEpiPlain) W4A16_VALU_SET(kEpiSwiglu) W4A16_VALU_BASE(kEpiArgmax)
    W4A16_MFMA_SET(kEpiPlain) W4A16_MFMA_SET(kEpiSwiglu) W4A16_MFMA_BASE(kEpiArgmax)};

const KernEntry* find_kernel(bool mfma, int rows, int lr, int D, int epi, int LB) {
  for (const KernEntry& e : kKernels)
    if (e.mfma == mfma && e.rows == rows && e.lr == lr && e.D == D && e.epi == epi &&
        e.LB == LB)
      return &e;
  return nullptr;
}

// Waves of kernel `fn` that fit on one CU at once as limited by its VGPR use
// (512 VGPRs per SIMD lane, allocated in granules of 8; at most 8 waves per
// SIMD).  Cached per registry entry; 32 if the attributes are unavailable.
int g_waves_per_cu[sizeof(kKernels) / sizeof(kKernels[0])];
int waves_per_cu(const KernEntry* k) {
  const size_t i = (size_t)(k - kKernels);
  int n = __atomic_load_n(&g_waves_per_cu[i], __ATOMIC_RELAXED);
  if (n > 0) return n;
  hipFuncAttributes attr{};
  n = 32;
  if (hipFuncGetAttributes(&attr, k->fn) == hipSuccess && attr.numRegs > 0) {
    const int alloc = (attr.numRegs + 7) / 8 * 8;
    const int per_simd = 512 / alloc < 8 ? 512 / alloc : 8;
    n = 4 * (per_simd > 0 ? per_simd : 1);
  }
  __atomic_store_n(&g_waves_per_cu[i], n, __ATOMIC_RELAXED);
  return n;
}

#ifdef W4A16_TUNING
struct Override {
  int enable, mfma, lr, D, W, LB, nrb, S;
};
Override g_override{};
#endif

// Whole-row VALU kernels (k_gemm_rows), by K = 1024 * CPL: 5120, the hidden
// size of the model family served here (square projections, gate/up), for
// M <= 2 and both epilogues.  Other shapes take the general kernels.  (The
// same kernel at K = 17408, the down projection, M = 1: 14.0-15.1 us at
// 4-8 waves against 10.8 us for the general VALU kernel -- ten tasks of 17
// steps per CU leave the waves unevenly loaded and the per-wave step chain
// long; measured on MI355X.)
struct RowsEntry {
  int MT, cpl, epi;
  const void* fn;
};
#define W4A16_RE(MT, CPL, F) {MT, CPL, F, reinterpret_cast<const void*>(&k_gemm_rows<MT, CPL, F>)},
const RowsEntry kRowsKernels[] = {W4A16_RE(1, 5, kEpiPlain) W4A16_RE(2, 5, kEpiPlain)
                                  W4A16_RE(1, 5, kEpiSwiglu) W4A16_RE(2, 5, kEpiSwiglu)};
#undef W4A16_RE
const void* find_rows_kernel(int MT, int cpl, int epi) {
  for (const RowsEntry& e : kRowsKernels)
    if (e.MT == MT && e.cpl == cpl && e.epi == epi) return e.fn;
  return nullptr;
}
// launch bound of k_gemm_rows<MT, CPL, ...> (as in its declaration)
int rows_launch_bound(int MT, int cpl) { return (MT == 1 && cpl <= 8) ? 640 : 512; }

// Plan for the whole-row kernel, or false if it does not apply.  One row
// block per CU; 8 waves when a block has at most 16 tasks (two rows each;
// fused: one gate/up pair), else 4 (measured on MI355X: square 5120^2 with
// 10 tasks per block 4.82 us at 8 waves, 5.04 at 10, 5.59 at 4; gate/up
// 2 x 17408 x 5120 with 68 tasks per block 17.6 us at 4 waves, 17.9 at 8).
// At M = 1 a block of 10 tasks takes 5 waves of two tasks each instead of 8
// waves of which two have a second task: square 4.94 -> 4.88 us (at M = 2
// 5.47 -> 5.73, so not there).
bool plan_rows(int M, int N, int K, int epi, Plan& pl) {
  if (M > kValuMaxM || epi == kEpiArgmax || K % 1024 != 0) return false;
#ifdef W4A16_TUNING
  if (g_override.enable) return false;
#endif
  const int cpl = K / 1024;
  if (!find_rows_kernel(M, cpl, epi)) return false;
  const int RT = epi == kEpiSwiglu ? 1 : 2;
  const long long tasks = ((long long)N + RT - 1) / RT;
  long long nrb = cu_count();
  if (nrb > tasks) nrb = tasks;
  if (nrb < 1) nrb = 1;
  const int rq = N / (int)nrb, rr = N % (int)nrb;
  const long long per_block = ((long long)rq + (rr > 0) + RT - 1) / RT;
  pl = Plan{};
  pl.mfma = false;
  pl.lr = 32;
  // the kernel stages x with >= 4 waves
  pl.W = per_block > 16 ? 4 : (M == 1 && per_block == 10) ? 5 : 8;
  pl.LB = rows_launch_bound(M, cpl);
  pl.nrb = (int)nrb;
  pl.S = 1;
  pl.rq = rq;
  pl.rr = rr;
  pl.lds = (size_t)M * (size_t)(4 * (K >> 5) + 1) * 16;
  pl.ws = 0;
  pl.rows_cpl = cpl;
  return true;
}

// K-column MFMA kernels with x in registers (k_gemm_xr), 3 <= M <= 8 at
// K = 5120 (CPL = 5; plain, SwiGLU and argmax epilogues) and at K = 17408
// (CPL = 17, the down projection; plain, in two K-slices of 17 columns);
// other shapes take the MFMA kernel.  (Measured on MI355X against the MFMA kernel,
// HIP-graph replay: 5120 x 5120 at M = 3, 4, 5, 7, 8: 5.55 / 5.61 / 6.43 /
// 6.60 / 6.68 us against 7.02 / 7.07 / 7.85 / 7.99 / 8.01; gate/up 2 x 17408
// x 5120 at M = 4, 5, 7, 8: 20.2 / 21.2 / 21.6 / 21.8 us against 22.1 / 23.3
// / 23.9 / 24.3.)
struct XrEntry {
  int M, cpl, epi, W, S;
  bool ring;
  const void* fn;
};
#define W4A16_XE(MM, C, F, WW, SS) \
  {MM, C, F, WW, SS, false, reinterpret_cast<const void*>(&k_gemm_xr<MM, C, F, WW, SS, false>)},
#define W4A16_XR(MM, F, WW) \
  {MM, 5, F, WW, 1, true, reinterpret_cast<const void*>(&k_gemm_xr<MM, 5, F, WW, 1, true>)},
#define W4A16_XR_ALL(F) \
  W4A16_XR(3, F, 5) W4A16_XR(4, F, 5) W4A16_XR(5, F, 8) W4A16_XR(6, F, 8) W4A16_XR(7, F, 8) W4A16_XR(8, F, 8)
#define W4A16_XE_P2(C, F, WW, SS) \
  W4A16_XE(5, C, F, WW, SS) W4A16_XE(6, C, F, WW, SS) W4A16_XE(7, C, F, WW, SS) W4A16_XE(8, C, F, WW, SS)
#define W4A16_XE_ALL(C, F, WW, SS) W4A16_XE(3, C, F, WW, SS) W4A16_XE(4, C, F, WW, SS) W4A16_XE_P2(C, F, WW, SS)
const XrEntry kXrKernels[] = {W4A16_XE_ALL(5, kEpiPlain, 5, 1) W4A16_XE_ALL(5, kEpiSwiglu, 5, 1)
                              W4A16_XE_P2(5, kEpiPlain, 6, 1) W4A16_XE_P2(5, kEpiSwiglu, 6, 1)
                              W4A16_XE_P2(5, kEpiPlain, 8, 1) W4A16_XE_P2(5, kEpiSwiglu, 8, 1)
                              W4A16_XE_ALL(17, kEpiPlain, 9, 2)
                              W4A16_XR_ALL(kEpiPlain) W4A16_XR_ALL(kEpiSwiglu)
                              W4A16_XR_ALL(kEpiArgmax)};
#undef W4A16_XR_ALL
#undef W4A16_XR
#undef W4A16_XE_ALL
#undef W4A16_XE_P2
#undef W4A16_XE
const void* find_xr_kernel(int M, int cpl, int epi, int W, int S, bool ring) {
  for (const XrEntry& e : kXrKernels)
    if (e.M == M && e.cpl == cpl && e.epi == epi && e.W == W && e.S == S && e.ring == ring) return e.fn;
  return nullptr;
}
// LDS bytes of k_gemm_xr<M, ..., W, S> for a row block of `rows` rows and a
// K-slice of jt columns: one fp32 partial per (quad, weight row, activation
// row, wave, 16-lane row; per activation row padded to an odd number of
// 16-byte units), the floats per (quad, weight row) padded to 4 mod 8, as in
// the kernel; at least the area the waves first stage their x in
// (per column: P passes x 4 units x 64 lanes x 16 bytes)
size_t xr_lds(int M, bool fused, long long rows, int W, int jt, bool ring = false) {
  size_t quads = (size_t)((rows + 3) / 4) * (fused ? 2 : 1);
  if (ring && quads > 8 * kXrRingIterations) quads = 8 * kXrRingIterations;  // the ring's slots
  size_t js = (size_t)M * (4 * (size_t)W + (W % 2 == 0 ? 4 : 0));
  js += js % 8 == 0 ? 4 : 0;
  const size_t partials = quads * 4 * js * sizeof(float);
  const size_t x_stage = (size_t)jt * ((M + 3) / 4) * 4 * 64 * 16;
  return partials > x_stage ? partials : x_stage;
}

// ---- wide kernel (9 <= M <= 32) ----------------------------------------------
struct WideEntry {
  int mt, epi;
  const void* fn;
};
#define W4A16_WE(MT, F) {MT, F, reinterpret_cast<const void*>(&k_gemm_wide<MT, F>)},
const WideEntry kWideKernels[] = {W4A16_WE(2, kEpiPlain) W4A16_WE(4, kEpiPlain) W4A16_WE(4, kEpiSwiglu)
#ifdef W4A16_TUNING
                                  W4A16_WE(2, kEpiSwiglu)
#endif
};
#undef W4A16_WE
const void* find_wide_kernel(int mt, int epi) {
  for (const WideEntry& e : kWideKernels)
    if (e.mt == mt && e.epi == epi) return e.fn;
  return nullptr;
}
// From 13 rows on for plain calls, 17 for gate/up (measured on MI355X by
// HIP-graph replay, wide kernel against the 4x4x4 MFMA kernel: the square
// 5120^2 at M = 12 / 13 / 16 / 24 / 32 10.7 / 10.7 / 10.8 / 12.8 / 13.1 us
// against 9.5 / 12.5 / 13.0 / 16.0 / 23.1 (the 4x4x4 kernel takes a fourth
// row pass from M = 13); down 5120 x 17408 at M = 9 / 13 / 16 / 24 / 32 19.1
// / 19.3 / 19.4 / 26.6 / 27.3 against 19.5 / 22.9 / 23.8 / 36.1 / 46.8;
// gate/up 2 x 17408 x 5120 at M = 13 / 16 / 17 / 24 / 32 43.8 / 44.8 / 41.3 /
// 42.5 / 44.7 against 40.2 / 41.7 / 48.8 / 55.3 / 82.7).  Below that the wide
// kernel's fixed costs (x staging, partial sums and their finish) outweigh
// what it saves.
constexpr int kWideMinM = 13, kWideMinMFused = 17;
// LDS bytes of k_gemm_wide<mt, ...> for a K-slice of `steps` steps of 256
// inputs: 8 * mt rows of steps * 32 units of 16 bytes, plus one unit per row
size_t wide_lds(int mt, int steps) { return (size_t)8 * mt * ((size_t)steps * 32 + 1) * 16; }

#ifdef W4A16_TUNING
// Tuning builds only: force the wide kernel's waves, slice length (units of
// 512 inputs) and smallest M (0 = the planner's choice).
int g_wide_W = 0, g_wide_u = 0, g_wide_minm = 0;
bool g_wide_any(int W, int u) { return g_wide_W == W && g_wide_u == u; }
#else
constexpr bool g_wide_any(int, int) { return false; }
#endif
// Plan for the wide kernel, or false if it does not apply.  Row blocks of W
// tiles (one per wave), W = 4 or 8; K-slices of u x 512 inputs (the slice's x
// must fit in LDS).  Rule, from a sweep of W and u on MI355X (HIP-graph
// replay; 5120 x 17408, 2 x 17408 x 5120 and 5120^2 at M = 16, 24, 32): the
// most workgroups that still run in one round, at most one per CU for a
// plain call (a second one on a CU doubles its SIMDs' work), up to 2.2 per CU
// for gate/up (whose per-workgroup work is twice as long and tolerates a
// partial second round better than an idle CU); ties go to fewer K-slices
// (fewer partial sums), then to fewer waves.  Chosen and measured: the down
// projection 8 waves x 12 slices (27.3 us at M = 32; 6 slices: 29.9), 4 x 6
// at M = 16 (19.4; 8 x 12: 23.2); the square 4 x 5 (13.0 at M = 32, 10.8 at
// M = 16; 8 x 10: 18.0 / 14.7); gate/up 4 x 4 at M = 32 (44.9; 8 x 3: 51.8).
bool plan_wide(int M, int N, int K, int epi, Plan& pl) {
  const bool fused = epi == kEpiSwiglu;
  int min_m = fused ? kWideMinMFused : kWideMinM;
#ifdef W4A16_TUNING
  if (g_override.enable) return false;
  if (g_wide_minm > 0) min_m = g_wide_minm;
#endif
  if (M < min_m || M > 32 || epi == kEpiArgmax || K % 512 != 0) return false;
  const int mt = M <= 16 ? 2 : 4;
  if (!find_wide_kernel(mt, epi)) return false;
  const int cus = cu_count();
  const long long T = ((long long)N + 31) / 32;
  const int units = K / 512;
  const long long cap = fused ? (long long)cus * 22 / 10 : cus;
  long long best_wgs = -1;
  int bW = 0, bu = 0, bS = 0;
  long long bnrb = 0;
  int Wlo = 4, Whi = 8;
#ifdef W4A16_TUNING
  if (g_wide_W > 0) Wlo = Whi = g_wide_W;
#endif
  for (int W = Wlo; W <= Whi; W += 4) {
    const long long nrb = (T + W - 1) / W;
    for (int u = 1; u <= units; ++u) {
#ifdef W4A16_TUNING
      if (g_wide_u > 0 && u != g_wide_u) continue;
#endif
      const size_t lds = wide_lds(mt, 2 * u);
      if (lds > kMaxLds) break;
      const int S = (units + u - 1) / u;
      if (S > 1 && nrb > kMaxSplitRowBlocks) continue;
      const long long wgs = nrb * S;
      const bool fits = wgs <= cap || (g_wide_any(W, u));
      if (!fits) continue;
      if (wgs > best_wgs || (wgs == best_wgs && (S < bS || (S == bS && W < bW)))) {
        best_wgs = wgs;
        bW = W;
        bu = u;
        bS = S;
        bnrb = nrb;
      }
    }
  }
  // nothing runs in one round (very wide rows): the fewest workgroups
  if (bW == 0) {
    for (int u = units; u >= 1; --u)
      if (wide_lds(mt, 2 * u) <= kMaxLds && ((T + 7) / 8 <= kMaxSplitRowBlocks || (units + u - 1) / u == 1)) {
        bW = 8;
        bu = u;
        bS = (units + u - 1) / u;
        bnrb = (T + 7) / 8;
        break;
      }
  }
  if (bW == 0) return false;
  pl = Plan{};
  pl.mfma = true;
  pl.lr = 1;
  pl.W = bW;
  pl.LB = 512;
  pl.nrb = (int)bnrb;
  pl.S = bS;
  pl.rq = bW;  // tiles per row block
  pl.rr = 0;
  pl.lds = wide_lds(mt, 2 * bu);
  pl.ws = bS > 1 ? kCounterBytes + (size_t)bS * (size_t)M * (size_t)N * sizeof(float) * (fused ? 2 : 1) : 0;
  pl.wide_mt = mt;
  pl.wide_steps = 2 * bu;
  return true;
}

// Plan for the K-column kernel, or false if it does not apply: one workgroup
// per CU.  More workgroups would each load x again: on the 5120 -> 248 320
// head at M = 7, 1024 blocks took 154.6 us against 145.6 for the MFMA kernel
// (measured on MI355X).  Where a block's partials do not all fit in LDS (K =
// 5120: N past ~63 000 plain at M = 8 with 5 waves), and for the argmax
// epilogue, the ring variant adds them every two loop iterations instead
// (for gate/up, whose blocks fit, the ring was slower: 21.3 -> 22.1 us at
// M = 7): the head
// at M = 3 / 5 / 7 / 8 in 114.6 / 122.7 / 127.1 / 130.0 us against 122.5 /
// 139.7 / 143.1 / 144.0 for the MFMA kernel.  K = 5120, waves: 2 CPL / 2 = 5 (two columns each) for
// M <= 4; for M >= 5, 6 while a block has fewer than 16 row quads and 8 from
// 16 on (the first 10 - W waves own two columns, the rest one; 5 again where
// the partials would not fit).  Waves w and w + 4 share a SIMD, so with 5
// waves SIMD 0 does four columns' work and the others two, while 6 and 8
// waves load the SIMDs 3 / 3 / 2 / 2.  Measured (HIP-graph replay): the
// square (5 quads per block) at M = 5 / 7 / 8 6.19 / 6.59 / 6.57 us with 5
// waves, 5.93 / 6.26 / 6.21 with 6, 6.02 / 6.39 / 6.20 with 7 and 6.69 at
// M = 7 with 8, but at M = 3 5.63 with 5 and 5.76 with 6; gate/up (34
// quads) at M = 7 22.5 with 5, 21.6 with 8; at M = 3 20.1 with 5, 20.3 with
// 8.  K = 17408: 34 columns
// of x do not fit one workgroup's registers at two or three per wave, so
// the row blocks are half as many and each has two workgroups, one per
// K-slice of 17 columns (split-K partials in the workspace), of 9 waves: 8
// of two columns and one of one.  (16 waves, one of two columns and 15 of
// one, would leave 128 VGPRs per wave: the two-column wave spills.)
// Measured, 5120 x 17408 at M = 3 / 4 / 5 / 7 / 8: 13.4 / 13.8 / 13.9 / 14.3 /
// 14.4 us against 14.1 / 14.4 / 16.5 / 17.0 / 17.3 for the MFMA kernel (also
// two K-slices from M = 5).
bool plan_xr(int M, int N, int K, int epi, Plan& pl) {
  if (M < 3 || M > 8 || K % 1024 != 0) return false;
#ifdef W4A16_TUNING
  if (g_override.enable) return false;
#endif
  const int cpl = K / 1024;
  const int S = cpl == 17 ? 2 : 1;
  const int jt = 2 * cpl / S;
  const bool fused = epi == kEpiSwiglu;
  long long nrb = cu_count() / S;
  if (nrb > N) nrb = N;
  if (nrb < 1) nrb = 1;
  const long long rows = N / nrb + (N % nrb > 0);
  const long long quads = (rows + 3) / 4 * (fused ? 2 : 1);
  int W;
  bool ring = false;
  if (S > 1) {
    W = 9;
  } else {
    W = M >= 5 ? (quads >= 16 ? 8 : 6) : cpl;
    if (W != cpl && xr_lds(M, fused, rows, W, jt) > kMaxLds) W = cpl;  // fewer partials per quad
    // the ring variant where the block's partials do not fit, and for argmax
    if (epi == kEpiArgmax || xr_lds(M, fused, rows, W, jt) > kMaxLds) {
      ring = true;
      W = M >= 5 ? 8 : cpl;
    }
  }
  if (!find_xr_kernel(M, cpl, epi, W, S, ring)) return false;
  if (xr_lds(M, fused, rows, W, jt, ring) > kMaxLds) return false;
  pl = Plan{};
  pl.mfma = true;
  pl.lr = 1;
  pl.W = W;
  pl.LB = 64 * W;
  pl.nrb = (int)nrb;
  pl.S = S;
  pl.rq = N / (int)nrb;
  pl.rr = N % (int)nrb;
  pl.lds = xr_lds(M, fused, pl.rq + (pl.rr > 0), W, jt, ring);
  if (epi == kEpiArgmax)  // arrival counter, then one candidate per row block and activation row
    pl.ws = kCounterBytes + (size_t)pl.nrb * (size_t)M * 2 * sizeof(float);
  else
    pl.ws = S > 1 ? kCounterBytes + (size_t)S * (size_t)M * (size_t)N * sizeof(float) * (fused ? 2 : 1) : 0;
  pl.xr_cpl = cpl;
  pl.xr_ring = ring;
  return true;
}

// Kernel selection is a pure function of (M, N, K, epilogue) and the device's
// compute-unit count.  rows_ok, xr_ok: whether the whole-row and the K-column
// kernels may be chosen.  The persistent MLP kernel runs the general kernels'
// bodies only; the MLP block's two-launch path may take the whole-row kernel
// (its sums are the VALU kernel's, bit for bit) but not the K-column kernel
// (whose sums are added in another order than the MFMA kernel's), so that
// both paths of the block give the same bits.
Plan plan_gemm(int M, int N, int K, int epi, bool rows_ok = true, bool xr_ok = true) {
  {
    Plan r;
    if (rows_ok && plan_rows(M, N, K, epi, r)) return r;
    if (xr_ok && plan_xr(M, N, K, epi, r)) return r;
    if (xr_ok && plan_wide(M, N, K, epi, r)) return r;
  }
  const bool fused = epi == kEpiSwiglu;
  Plan pl{};
  const int cus = cu_count();
  const int CR = K >> 5;  // 16-byte chunks per weight row (a multiple of 8)
  pl.mfma = M > kValuMaxM;
  // Launch rules from measured sweeps on MI355X over the benchmark shapes:
  // shallow rings (4 chunk loads in flight per lane); one workgroup of 8
  // waves per CU (x is staged into LDS once per workgroup, so fewer row
  // blocks means less x traffic); VALU rows read by 32 lanes where K/32 is a
  // multiple of 32 (512 contiguous bytes per row per load beat 256); MFMA
  // tasks of one row quad (finer stream-K tasks beat two quads sharing x
  // reads).
  pl.D = 4;
  int wmax, wg_per_cu;
  if (!pl.mfma) {
    pl.lr = (CR % 32 == 0) ? 32 : (CR % 16 == 0) ? 16 : 8;
    pl.LB = 1024;
    wmax = 8;
    wg_per_cu = 1;
  } else {
    pl.lr = 1;  // row quads per task
    pl.LB = 512;
    wmax = 8;
    wg_per_cu = 1;
  }
  bool force_w = false;
#ifdef W4A16_TUNING
  const bool ov = g_override.enable && (g_override.mfma != 0) == pl.mfma;
  if (ov) {
    pl.lr = g_override.lr;
    pl.D = g_override.D;
    pl.LB = g_override.LB;
    if (g_override.W > 0) {
      wmax = g_override.W;
      force_w = true;
    }
  }
#endif
  if (wmax > pl.LB / 64) wmax = pl.LB / 64;
  // keep wg_per_cu workgroups resident together
  const KernEntry* ke =
      find_kernel(pl.mfma, pl.mfma ? (M + 3) / 4 : M, pl.lr, pl.D, epi, pl.LB);
  if (!ke) return Plan{};
  const int wocc = waves_per_cu(ke) / wg_per_cu;
  int wcap = wmax < wocc ? wmax : wocc;
  if (wcap < 1) wcap = 1;
  const int xrows = pl.mfma ? 4 * ((M + 3) / 4) : M;        // staged x rows
  const int RT = pl.mfma ? (fused ? 2 : 4) * pl.lr : (fused ? (64 / pl.lr) / 2 : 64 / pl.lr);
  // per-wave floats: epilogue scratch (VALU G*MT*NSEG, MFMA R*P*4*16) and one
  // segment partial (VALU G*MT, MFMA R*P*4*4)
  const size_t scr_per_wave =
      pl.mfma ? (size_t)pl.lr * ((M + 3) / 4) * 4 * 16
              : (size_t)(64 / pl.lr) * M * (pl.lr < 16 ? 1 : pl.lr / 16);
  const size_t seg_vals = pl.mfma ? (size_t)pl.lr * ((M + 3) / 4) * 16 : (size_t)(64 / pl.lr) * M;
  // VALU step partial: (64 / L) row slots x (L / 16 or 1) DPP groups x M
  const size_t valu_step_vals =
      pl.mfma ? 0 : (size_t)(64 / pl.lr) * (pl.lr > 16 ? pl.lr / 16 : 1) * M;
  const long long groups = ((long long)N + RT - 1) / RT;  // row groups in total
  // Smallest K split whose x slice, scratch and segment partials fit in LDS
  // (VALU: whole chunk steps per lane) with one row block per CU and split.
  // Only when no split fits that way (wide M: the x slice forces a split of
  // few chunk steps per task, so each wave touches many tasks and their
  // segment partials outgrow LDS) are 2, 4, 8 or 16 times as many row blocks
  // tried, each with fewer tasks.
  for (int grow = 1; grow <= 16; grow *= 2)
  for (int S = 1; S <= CR; ++S) {
    if (CR % S) continue;
    const int CRS = CR / S;
    if (!pl.mfma && CRS % pl.lr) continue;
    long long nrb = (long long)cus * wg_per_cu / S > 0 ? (long long)cus * wg_per_cu / S : 1;
    nrb *= grow;
#ifdef W4A16_TUNING
    if (ov && g_override.S > 0) {
      if (S != g_override.S) continue;
    }
    if (ov && g_override.nrb > 0) nrb = g_override.nrb;
#endif
    if (nrb > groups) nrb = groups;
    if (nrb > N) nrb = N;
    // split-K arrival counters, one per row block (a K-split argmax keeps the
    // last counter for its final reduction)
    const int max_rb = kMaxSplitRowBlocks - (epi == kEpiArgmax ? 1 : 0);
    if (S > 1 && nrb > max_rb) nrb = max_rb;
    const int rq = N / (int)nrb, rr = N % (int)nrb;
    const long long ntasks = ((long long)rq + (rr > 0) + RT - 1) / RT;  // tasks of the largest block
    const int CPL = pl.mfma ? (CRS + 15) / 16 : CRS / pl.lr;
    const long long TS = ntasks * CPL;
    // LDS bytes for W waves: x slice, per-wave scratch, segment slots and
    // the task bookkeeping (two ints per segment slot, one per wave)
    auto lds_for = [&](int W, long long* kmax_out) {
      const size_t xbytes = (size_t)xrows * (size_t)(CRS * 4 + 1) * 16;
      if (!pl.mfma) {
        // VALU: one partial per step (G row slots x DPP groups x M) and the
        // batch counter
        if (kmax_out) *kmax_out = 0;
        return xbytes + (size_t)TS * (size_t)valu_step_vals * sizeof(float) + 16;
      }
      const long long steps = (TS + W - 1) / W;  // most steps of one wave
      long long kmax = (steps - 1 + CPL - 1) / CPL + 1;
      if (kmax > ntasks) kmax = ntasks;
      if (kmax_out) *kmax_out = kmax;
      return xbytes + (scr_per_wave + (size_t)kmax * seg_vals) * sizeof(float) * W +
             (2 * (size_t)kmax + 1) * sizeof(int) * W;
    };
    // the split is chosen for the largest wave count (so that it does not
    // depend on the occupancy query), the wave count then by occupancy
    const int Wfit = force_w ? wmax : (int)(TS < wmax ? TS : wmax);
    if (lds_for(Wfit, nullptr) > kMaxLds) continue;
    const int W = force_w ? wmax : (int)(TS < wcap ? TS : wcap);
    long long kmax = 0;
    const size_t lds = lds_for(W, &kmax);
    if (lds > kMaxLds) continue;
    // quotients in the kernels (div_small) are exact below 2^23
    if (TS * (W + 1) >= (1LL << 23) || (long long)xrows * CRS * 4 + 1024LL * 16 >= (1LL << 23))
      return Plan{};
    // argmax with a K split: the MFMA kernel only (M >= 3)
    if (epi == kEpiArgmax && S > 1 && !pl.mfma) break;
    pl.S = S;
    pl.nrb = (int)nrb;
    pl.rq = rq;
    pl.rr = rr;
    pl.W = W;
    pl.kmax = (int)kmax;
    pl.lds = lds;
    if (epi == kEpiArgmax) {
      // argmax: the arrival counters, the fp32 partials of a K split, then
      // one (value, index) candidate per row block and activation row
      pl.ws = kCounterBytes + (S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(float) : 0) +
              (size_t)pl.nrb * (size_t)M * 2 * sizeof(float);
    } else {
      pl.ws = S > 1 ? kCounterBytes +
                          (size_t)S * (size_t)M * (size_t)N * sizeof(float) * (fused ? 2 : 1)
                    : 0;
    }
    return pl;
  }
  return Plan{};  // no split fits (pl.S == 0): unsupported
}

hipError_t launch(const void* fn, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                  MatArgs args) {
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  void* argv[] = {&args};
  hipError_t e = hipLaunchKernel(fn, grid, block, argv, lds, stream);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

hipError_t dispatch(const Plan& pl, int epi, hipStream_t s, const MatArgs& a) {
  if (pl.wide_mt > 0) {
    const void* fn = find_wide_kernel(pl.wide_mt, epi);
    if (!fn || pl.W < 1 || pl.W > 8 || a.M > 8 * pl.wide_mt || a.K % 512 != 0 ||
        pl.wide_steps % 2 != 0 || a.CRS != pl.wide_steps || a.S != pl.S ||
        (long long)pl.S * pl.wide_steps < a.K / 256 || (long long)(pl.S - 1) * pl.wide_steps >= a.K / 256 ||
        (long long)pl.nrb * pl.rq * 32 < a.N || pl.lds != wide_lds(pl.wide_mt, pl.wide_steps) ||
        (pl.S > 1 && (a.part == nullptr || a.cnt == nullptr)))
      return hipErrorInvalidConfiguration;
    return launch(fn, dim3((unsigned)pl.nrb, (unsigned)pl.S), dim3((unsigned)(pl.W * 64)), pl.lds, s, a);
  }
  if (pl.xr_cpl > 0) {
    const void* fn = find_xr_kernel(a.M, pl.xr_cpl, epi, pl.W, pl.S, pl.xr_ring);
    if (!fn || pl.W * 64 != pl.LB || a.K != 1024 * pl.xr_cpl || a.S != pl.S ||
        (pl.S > 1 && (a.part == nullptr || a.cnt == nullptr)))
      return hipErrorInvalidConfiguration;
    return launch(fn, dim3((unsigned)pl.nrb, (unsigned)pl.S), dim3((unsigned)(pl.W * 64)), pl.lds, s, a);
  }
  if (pl.rows_cpl > 0) {
    const void* fn = find_rows_kernel(a.M, pl.rows_cpl, epi);
    if (!fn || pl.W < 4 || pl.W * 64 > pl.LB || a.K != 1024 * pl.rows_cpl)
      return hipErrorInvalidConfiguration;
    return launch(fn, dim3((unsigned)pl.nrb), dim3((unsigned)(pl.W * 64)), pl.lds, s, a);
  }
  const int rows = pl.mfma ? (a.M + 3) / 4 : a.M;
  const KernEntry* k = find_kernel(pl.mfma, rows, pl.lr, pl.D, epi, pl.LB);
  if (!k || pl.W * 64 > pl.LB) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)pl.nrb, (unsigned)pl.S), block((unsigned)(pl.W * 64));
  return launch(k->fn, grid, block, pl.lds, s, a);
}

w4a16_status_t check_shape(int M, int N, int K) {
  if (M <= 0 || N <= 0 || K <= 0) return W4A16_ERR_INVALID_VALUE;
  if (M > W4A16_MAX_M || (K % 256) != 0) return W4A16_ERR_UNSUPPORTED;
  if ((long long)K * 2 > 0x7fffffffLL) return W4A16_ERR_UNSUPPORTED;
  return W4A16_OK;
}

// Wide M: whether a call runs as two launches over activation rows [0, m1)
// and [m1, M), and m1 (a multiple of 4, at most 16; 0 for one launch).  Taken
// where the one-launch plan splits K so finely that its partial sums and
// their finish cost more than reading the weights twice: plain calls whose
// plan needs 16 or more K-slices, SwiGLU calls whose plan needs 4 or more
// (two partial sets per slice).  Measured on MI355X (HIP-graph replay): the down
// projection 5120 x 17408 at M = 32 in 75.0 us as one launch (16 slices),
// 2 x 24.2 as two of 16 rows; gate/up 2 x 17408 x 5120 at M = 24 / 28 / 32 in
// 79.4 / 92.7 / 105.9 us as one, 2 x 28.7 / 42.1 + 28.7 / 2 x 42.1 as two;
// one launch stays faster for the square 5120 x 5120 at every M and for the
// down projection up to M = 28 (8 slices).  Not for the argmax epilogue
// (whose candidates span all rows) or the MLP block (whose two paths must
// give the same bits).
int split_rows(int M, int N, int K, int epi) {
  if (M <= 16 || epi == kEpiArgmax) return 0;
  if (plan_gemm(M, N, K, epi).wide_mt > 0) return 0;  // the wide kernel takes all 32 rows at once
  int m1 = (M / 2 + 3) / 4 * 4;
  if (m1 > 16) m1 = 16;
  return plan_gemm(M, N, K, epi).S >= (epi == kEpiSwiglu ? 4 : 16) ? m1 : 0;
}

size_t workspace_bytes_for(int M, int N, int K, int epi) {
  if (check_shape(M, N, K) != W4A16_OK) return 0;
  const int m1 = split_rows(M, N, K, epi);
  if (m1 > 0) {
    const size_t w1 = plan_gemm(m1, N, K, epi).ws, w2 = plan_gemm(M - m1, N, K, epi).ws;
    return w1 > w2 ? w1 : w2;
  }
  return plan_gemm(M, N, K, epi).ws;
}

// Fill the plan-dependent launch arguments; cnt: the split-K arrival
// counters, part: the fp32 partials (or argmax candidates).
void prepare(MatArgs& a, const Plan& pl, int* cnt, float* part) {
  a.rq = pl.rq;
  a.rr = pl.rr;
  a.kmax = pl.kmax;
  a.S = pl.S;
  a.CRS = pl.wide_mt > 0 ? pl.wide_steps : (a.K >> 5) / pl.S;
  const int cpl = pl.wide_mt > 0 ? 1 : pl.mfma ? (a.CRS + 15) / 16 : a.CRS / pl.lr;
  a.rW = 1.0f / (float)pl.W;
  a.rCPL = 1.0f / (float)cpl;
  a.rUPR = 1.0f / (float)(a.CRS * 4);
  a.cnt = cnt;
  a.part = part;
  a.cand = part;
}

w4a16_status_t run_matmul_one(MatArgs a, int epi, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  const Plan pl = plan_gemm(a.M, a.N, a.K, epi);
  if (pl.S == 0 || pl.lds > kMaxLds) return W4A16_ERR_UNSUPPORTED;
  if (workspace_bytes < pl.ws || (pl.ws > 0 && workspace == nullptr))
    return W4A16_ERR_INVALID_VALUE;
  if (pl.ws > 0 && !aligned(workspace, 16)) return W4A16_ERR_UNSUPPORTED;
  prepare(a, pl, static_cast<int*>(workspace),
          reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes));
  // argmax candidates follow the partials of a K split
  if (epi == kEpiArgmax && pl.S > 1) a.cand = a.part + (size_t)pl.S * (size_t)a.M * (size_t)a.N;
  const hipError_t e = dispatch(pl, epi, stream, a);
  return e == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

// One launch, or two over row ranges of x and y (split_rows); the second
// reuses the workspace after the first on the same stream (every launch
// leaves its arrival counters at zero).
w4a16_status_t run_matmul(MatArgs a, int epi, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  const int m1 = split_rows(a.M, a.N, a.K, epi);
  if (m1 == 0) return run_matmul_one(a, epi, workspace, workspace_bytes, stream);
  MatArgs a1 = a, a2 = a;
  a1.M = m1;
  a2.M = a.M - m1;
  a2.x = a.x + (size_t)m1 * a.K;
  a2.y = a.y + (size_t)m1 * a.N;
  const w4a16_status_t st = run_matmul_one(a1, epi, workspace, workspace_bytes, stream);
  return st != W4A16_OK ? st : run_matmul_one(a2, epi, workspace, workspace_bytes, stream);
}

// ---- MLP block: gate/up + SwiGLU, then down ------------------------------------
// Workspace: the two phases' split-K counters (4 KiB each), the barrier
// words, h (bf16 [M][F]), then each phase's fp32 partials.
constexpr size_t kMlpBarrierOffset = 2 * kCounterBytes;
constexpr size_t kMlpHOffset = W4A16_MLP_H_OFFSET;
static_assert(kMlpHOffset >= kMlpBarrierOffset + (kBarFlag + 32) * sizeof(int), "barrier words");
static_assert(W4A16_MLP_TIMEOUT_OFFSET == kMlpBarrierOffset + kBarFlag * sizeof(int), "time-out flag");
static_assert(W4A16_MLP_GENERATION_OFFSET == kMlpBarrierOffset + kBarGen * sizeof(int), "generation");
size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

struct MlpKernEntry {
  bool mfma;
  int rows;    // VALU: MT; MFMA: P
  int l1, l2;  // VALU: lanes per weight row of each phase (MFMA: 1, 1)
  int D, LB;
  const void* fn;
};
#define W4A16_MLPV(MT, L1, L2) \
  {false, MT, L1, L2, 4, 1024, reinterpret_cast<const void*>(&k_mlp_valu<MT, L1, L2, 4, 1024>)},
#define W4A16_MLPV_L(L1, L2) W4A16_MLPV(1, L1, L2) W4A16_MLPV(2, L1, L2)
#define W4A16_MLPV_L2(L1) W4A16_MLPV_L(L1, 32) W4A16_MLPV_L(L1, 16) W4A16_MLPV_L(L1, 8)
#define W4A16_MLPM(P) {true, P, 1, 1, 4, 512, reinterpret_cast<const void*>(&k_mlp_mfma<P, 4, 512>)},
const MlpKernEntry kMlpKernels[] = {
    W4A16_MLPV_L2(32) W4A16_MLPV_L2(16) W4A16_MLPV_L2(8)
    W4A16_MLPM(1) W4A16_MLPM(2) W4A16_MLPM(3) W4A16_MLPM(4)
    W4A16_MLPM(5) W4A16_MLPM(6) W4A16_MLPM(7) W4A16_MLPM(8)};

// Default barrier poll limit of the one-launch MLP kernel.
constexpr int kMlpSpinDefault = 1 << 20;

struct MlpPlan {
  Plan p1, p2;              // gate/up (N = F, K = H) and down (N = H, K = F)
  Plan l1, l2;              // the same phases' plans for two launches
  size_t cap1, cap2;        // workspace bytes each phase may use (counters included)
  const MlpKernEntry* k;    // persistent kernel, or nullptr: two launches
  int grid;
  size_t lds;
  size_t part1, part2, ws;  // byte offsets of the partials, total bytes
};

// The plan of one phase of the two-launch path: the whole-row and K-column
// kernels where they apply, else the general kernels' plan.
Plan mlp_launch_plan(int M, int N, int K, int epi) { return plan_gemm(M, N, K, epi, true, true); }

MlpPlan plan_mlp(int M, int H, int F) {
  MlpPlan mp{};
  // the general kernels' plans: the persistent kernel runs their bodies, and
  // their workspace covers every variant (the whole-row kernel needs none)
  mp.p1 = plan_gemm(M, F, H, kEpiSwiglu, false, false);
  mp.p2 = plan_gemm(M, H, F, kEpiPlain, false, false);
  mp.l1 = mlp_launch_plan(M, F, H, kEpiSwiglu);
  mp.l2 = mlp_launch_plan(M, H, F, kEpiPlain);
  if (mp.p1.S == 0 || mp.p2.S == 0 || mp.l1.S == 0 || mp.l2.S == 0) return MlpPlan{};
  mp.cap1 = mp.p1.ws > mp.l1.ws ? mp.p1.ws : mp.l1.ws;
  mp.cap2 = mp.p2.ws > mp.l2.ws ? mp.p2.ws : mp.l2.ws;
  const size_t h_bytes = align256((size_t)M * F * 2);
  const size_t w1 = mp.cap1 > 0 ? align256(mp.cap1 - kCounterBytes) : 0;
  const size_t w2 = mp.cap2 > 0 ? align256(mp.cap2 - kCounterBytes) : 0;
  mp.part1 = kMlpHOffset + h_bytes;
  mp.part2 = mp.part1 + w1;
  mp.ws = mp.part2 + w2;
  // one launch: both phases on the same kernel family, block size and ring
  // depth, h addressable by 32-bit buffer offsets, and every workgroup of the
  // grid resident at once (the barrier waits for all of them)
  // Not where the two-launch path takes the K-column kernel for either phase:
  // its sums run in another order than the persistent kernel's bodies, and
  // the two paths give the same bits.
  const Plan &a = mp.p1, &b = mp.p2;
  if (a.mfma != b.mfma || a.W != b.W || a.LB != b.LB || a.D != b.D ||
      (size_t)M * F * 2 >= ((size_t)1 << 31) || mp.l1.xr_cpl > 0 || mp.l2.xr_cpl > 0 ||
      mp.l1.wide_mt > 0 || mp.l2.wide_mt > 0)
    return mp;
  const int rows = a.mfma ? (M + 3) / 4 : M;
  for (const MlpKernEntry& e : kMlpKernels)
    if (e.mfma == a.mfma && e.rows == rows && e.D == a.D && e.LB == a.LB &&
        (a.mfma || (e.l1 == a.lr && e.l2 == b.lr)) && (!a.mfma || (a.lr == 1 && b.lr == 1)))
      mp.k = &e;
  if (!mp.k) return mp;
  const int nwg1 = a.nrb * a.S, nwg2 = b.nrb * b.S;
  mp.grid = nwg1 > nwg2 ? nwg1 : nwg2;
  mp.lds = a.lds > b.lds ? a.lds : b.lds;
  return mp;
}

// Whether mp's persistent kernel can run with its whole grid resident (the
// workgroups per CU that the occupancy query allows, times the CUs); clears
// mp.k if not.  Needs the device.
void mlp_check_resident(MlpPlan& mp) {
  if (!mp.k) return;
  if (mp.lds > 64 * 1024 &&
      hipFuncSetAttribute(mp.k->fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)mp.lds) !=
          hipSuccess) {
    mp.k = nullptr;
    return;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, mp.k->fn, mp.p1.W * 64, mp.lds) !=
          hipSuccess ||
      (long long)per_cu * cu_count() < mp.grid)
    mp.k = nullptr;
}

w4a16_status_t run_mlp(const MatArgs& up0, const MatArgs& down0, void* workspace,
                       size_t workspace_bytes, const w4a16_mlp_options_t* opt,
                       hipStream_t stream) {
  const int M = up0.M, H = up0.K, F = up0.N;
  MlpPlan mp = plan_mlp(M, H, F);
  if (mp.p1.S == 0 || mp.p1.lds > kMaxLds || mp.p2.lds > kMaxLds) return W4A16_ERR_UNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < mp.ws) return W4A16_ERR_INVALID_VALUE;
  if (!aligned(workspace, 256)) return W4A16_ERR_UNSUPPORTED;
  const int launch = opt ? opt->launch : W4A16_MLP_TWO_LAUNCHES;
  if (launch != W4A16_MLP_TWO_LAUNCHES && launch != W4A16_MLP_ONE_LAUNCH)
    return W4A16_ERR_INVALID_VALUE;
  const int spin = (opt && opt->spin_limit >= 0) ? opt->spin_limit : kMlpSpinDefault;
  char* w = static_cast<char*>(workspace);
  uint16_t* h = reinterpret_cast<uint16_t*>(w + kMlpHOffset);
  MatArgs up = up0, down = down0;
  up.y = h;
  down.x = h;
  prepare(up, mp.p1, reinterpret_cast<int*>(w), reinterpret_cast<float*>(w + mp.part1));
  prepare(down, mp.p2, reinterpret_cast<int*>(w + kCounterBytes),
          reinterpret_cast<float*>(w + mp.part2));
  if (launch == W4A16_MLP_ONE_LAUNCH) {
    mlp_check_resident(mp);
    // a cooperative launch is not taken while the stream is being captured
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (mp.k && (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone))
      mp.k = nullptr;
  } else {
    mp.k = nullptr;
  }
  if (mp.k) {
    MlpArgs m{};
    m.up = up;
    m.down = down;
    m.nrb1 = mp.p1.nrb;
    m.nwg1 = mp.p1.nrb * mp.p1.S;
    m.nrb2 = mp.p2.nrb;
    m.nwg2 = mp.p2.nrb * mp.p2.S;
    m.bar = reinterpret_cast<int*>(w + kMlpBarrierOffset);
    m.spin_limit = spin;
    void* argv[] = {&m};
    // cooperative: every workgroup resident at once, or the launch is
    // refused (nothing enqueued) and the block runs as two kernels below
    const hipError_t e = hipLaunchCooperativeKernel(mp.k->fn, dim3((unsigned)mp.grid),
                                                    dim3((unsigned)(mp.p1.W * 64)), argv, mp.lds,
                                                    stream);
    if (e == hipSuccess) return W4A16_OK;
    (void)hipGetLastError();  // clear the refused launch's error
  }
  // two launches: each phase takes its own best plan (the persistent kernel
  // is planned only where that plan's sums match its own bit for bit)
  const Plan &q1 = mp.l1, &q2 = mp.l2;
  if (q1.lds > kMaxLds || q2.lds > kMaxLds || q1.ws > mp.cap1 || q2.ws > mp.cap2)
    return W4A16_ERR_UNSUPPORTED;
  prepare(up, q1, reinterpret_cast<int*>(w), reinterpret_cast<float*>(w + mp.part1));
  prepare(down, q2, reinterpret_cast<int*>(w + kCounterBytes),
          reinterpret_cast<float*>(w + mp.part2));
  hipError_t e = dispatch(q1, kEpiSwiglu, stream, up);
  if (e == hipSuccess) e = dispatch(q2, kEpiPlain, stream, down);
  return e == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

// ---- no-allocation variant of w4a16_gemm --------------------------------------
// The split-K scratch (arrival counters, then fp32 partials) in a file-scope
// device array: one copy per GPU, at a per-device address.  Host code never
// passes `scratch` itself to a kernel (in host code that name is only a
// stand-in for the symbol); it passes the address hipGetSymbolAddress returns
// for the current device, kept in g_scratch.
constexpr size_t kNoallocScratchBytes = W4A16_NOALLOC_SCRATCH_BYTES;
static_assert(kNoallocScratchBytes % 256 == 0 && kNoallocScratchBytes > kCounterBytes, "scratch size");
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];
void* g_scratch[kMaxDevices];  // device address of `scratch` per device; nullptr until set up

__global__ void __launch_bounds__(256) k_zero_words(int* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

// Once per device, with that device current: the array's device address, and
// a clear of its arrival counters enqueued on `stream` (a kernel, so that a
// call being captured into a graph records no memset node).
w4a16_status_t noalloc_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return W4A16_ERR_LAUNCH;
  void* p = __atomic_load_n(&g_scratch[dev], __ATOMIC_ACQUIRE);
  if (p == nullptr) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr)
      return W4A16_ERR_LAUNCH;
    hipLaunchKernelGGL(k_zero_words, dim3(1), dim3(256), 0, stream, static_cast<int*>(q),
                       (int)(kCounterBytes / sizeof(int)));
    if (hipGetLastError() != hipSuccess) return W4A16_ERR_LAUNCH;
    __atomic_store_n(&g_scratch[dev], q, __ATOMIC_RELEASE);
    p = q;
  }
  *out = p;
  return W4A16_OK;
}

}  // namespace
}  // namespace w4a16

using namespace w4a16;

extern "C" {

size_t w4a16_workspace_size(int M, int N, int K) { return workspace_bytes_for(M, N, K, kEpiPlain); }

size_t w4a16_workspace_size_gate_up(int M, int N, int K) {
  return workspace_bytes_for(M, N, K, kEpiSwiglu);
}

size_t w4a16_workspace_size_argmax(int M, int N, int K) {
  return workspace_bytes_for(M, N, K, kEpiArgmax);
}

w4a16_status_t w4a16_gemm(const uint8_t* wq, const uint8_t* ws, const float* g,
                          const uint16_t* x, uint16_t* y, int M, int N, int K, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  if (!wq || !ws || !g || !x || !y) return W4A16_ERR_INVALID_VALUE;
  w4a16_status_t st = check_shape(M, N, K);
  if (st != W4A16_OK) return st;
  if (!aligned(wq, 16) || !aligned(ws, 16) || !aligned(x, 16) || !aligned(g, 4) ||
      !aligned(y, 4))
    return W4A16_ERR_UNSUPPORTED;
  MatArgs a{};
  a.wq0 = wq;
  a.ws0 = ws;
  a.g0 = g;
  a.wq1 = wq;
  a.ws1 = ws;
  a.g1 = g;
  a.x = x;
  a.y = y;
  a.M = M;
  a.N = N;
  a.K = K;
  return run_matmul(a, kEpiPlain, workspace, workspace_bytes, stream);
}

w4a16_status_t w4a16_gemm_noalloc(const uint8_t* wq, const uint8_t* ws, const float* g,
                                  const uint16_t* x, uint16_t* y, int M, int N, int K,
                                  hipStream_t stream) {
  if (!wq || !ws || !g || !x || !y) return W4A16_ERR_INVALID_VALUE;
  w4a16_status_t st = check_shape(M, N, K);
  if (st != W4A16_OK) return st;
  if (!aligned(wq, 16) || !aligned(ws, 16) || !aligned(x, 16) || !aligned(g, 4) ||
      !aligned(y, 4))
    return W4A16_ERR_UNSUPPORTED;
  const Plan pl = plan_gemm(M, N, K, kEpiPlain);
  if (pl.S == 0 || pl.lds > kMaxLds || workspace_bytes_for(M, N, K, kEpiPlain) > kNoallocScratchBytes)
    return W4A16_ERR_UNSUPPORTED;
  void* work = nullptr;
  st = noalloc_scratch(stream, &work);
  if (st != W4A16_OK) return st;
  MatArgs a{};
  a.wq0 = wq;
  a.ws0 = ws;
  a.g0 = g;
  a.wq1 = wq;
  a.ws1 = ws;
  a.g1 = g;
  a.x = x;
  a.y = y;
  a.M = M;
  a.N = N;
  a.K = K;
  return run_matmul(a, kEpiPlain, work, kNoallocScratchBytes, stream);
}

w4a16_status_t w4a16_gemm_gate_up_swiglu(const uint8_t* wq_gate, const uint8_t* ws_gate,
                                         const float* g_gate, const uint8_t* wq_up,
                                         const uint8_t* ws_up, const float* g_up,
                                         const uint16_t* x, uint16_t* y, int M, int N, int K,
                                         void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
  if (!wq_gate || !ws_gate || !g_gate || !wq_up || !ws_up || !g_up || !x || !y)
    return W4A16_ERR_INVALID_VALUE;
  w4a16_status_t st = check_shape(M, N, K);
  if (st != W4A16_OK) return st;
  if (!aligned(wq_gate, 16) || !aligned(ws_gate, 16) || !aligned(wq_up, 16) ||
      !aligned(ws_up, 16) || !aligned(x, 16) || !aligned(g_gate, 4) || !aligned(g_up, 4) ||
      !aligned(y, 4))
    return W4A16_ERR_UNSUPPORTED;
  MatArgs a{};
  a.wq0 = wq_gate;
  a.ws0 = ws_gate;
  a.g0 = g_gate;
  a.wq1 = wq_up;
  a.ws1 = ws_up;
  a.g1 = g_up;
  a.x = x;
  a.y = y;
  a.M = M;
  a.N = N;
  a.K = K;
  return run_matmul(a, kEpiSwiglu, workspace, workspace_bytes, stream);
}

w4a16_status_t w4a16_gemm_argmax(const uint8_t* wq, const uint8_t* ws, const float* g,
                                 const uint16_t* x, int32_t* idx, float* val, int M, int N, int K,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!wq || !ws || !g || !x || !idx || !val) return W4A16_ERR_INVALID_VALUE;
  w4a16_status_t st = check_shape(M, N, K);
  if (st != W4A16_OK) return st;
  if (!aligned(wq, 16) || !aligned(ws, 16) || !aligned(x, 16) || !aligned(g, 4) ||
      !aligned(idx, 4) || !aligned(val, 4))
    return W4A16_ERR_UNSUPPORTED;
  MatArgs a{};
  a.wq0 = wq;
  a.ws0 = ws;
  a.g0 = g;
  a.wq1 = wq;
  a.ws1 = ws;
  a.g1 = g;
  a.x = x;
  a.y = nullptr;
  a.M = M;
  a.N = N;
  a.K = K;
  a.amax_idx = idx;
  a.amax_val = val;
  return run_matmul(a, kEpiArgmax, workspace, workspace_bytes, stream);
}

w4a16_status_t w4a16_dequant(const uint8_t* wq, const uint8_t* ws, const float* g, float* w,
                             int N, int K, hipStream_t stream) {
  if (!wq || !ws || !g || !w) return W4A16_ERR_INVALID_VALUE;
  if (N <= 0 || K <= 0) return W4A16_ERR_INVALID_VALUE;
  if ((K % 256) != 0) return W4A16_ERR_UNSUPPORTED;
  if (!aligned(wq, 16) || !aligned(ws, 16) || !aligned(w, 16) || !aligned(g, 4))
    return W4A16_ERR_UNSUPPORTED;
  const long long words = (long long)N * (K >> 3);
  long long blocks = (words + 255) / 256;
  const long long cap = (long long)cu_count() * 16;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(k_dequant, dim3((unsigned)blocks), dim3(256), 0, stream, wq, ws, g, w, words,
                     K);
  return hipGetLastError() == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

}  // extern "C"

namespace w4a16 {
namespace {

// Pass-1 workgroups of the quantiser (its workspace holds one float each).
int quant_parts(long long count) {
  long long p = (count + 255) / 256;
  const long long cap = 4LL * cu_count();
  if (p > cap) p = cap;
  return (int)(p > 0 ? p : 1);
}

template <typename T>
w4a16_status_t run_quantize(const T* w, uint8_t* wq, uint8_t* ws, float* g, int N, int K,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!w || !wq || !ws || !g || !workspace) return W4A16_ERR_INVALID_VALUE;
  if (N <= 0 || K <= 0) return W4A16_ERR_INVALID_VALUE;
  if (K % 16 != 0) return W4A16_ERR_UNSUPPORTED;
  if (!aligned(w, 16) || !aligned(wq, 16) || !aligned(g, 4) || !aligned(workspace, 16))
    return W4A16_ERR_UNSUPPORTED;
  const long long count = (long long)N * K;
  const int parts = quant_parts(count);
  if (workspace_bytes < (size_t)parts * sizeof(float)) return W4A16_ERR_INVALID_VALUE;
  float* part = static_cast<float*>(workspace);
  hipLaunchKernelGGL(k_quant_amax<T>, dim3((unsigned)parts), dim3(256), 0, stream, w, count, part);
  if (hipGetLastError() != hipSuccess) return W4A16_ERR_LAUNCH;
  const long long nblocks = count / 16;
  long long grid = (nblocks + 255) / 256;
  const long long cap = 8LL * cu_count();
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL(k_quant_encode<T>, dim3((unsigned)grid), dim3(256), 0, stream, w, nblocks,
                     part, parts, wq, ws, g);
  return hipGetLastError() == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

}  // namespace
}  // namespace w4a16

extern "C" {

size_t w4a16_quantize_workspace_size(int N, int K) {
  if (N <= 0 || K <= 0 || K % 16 != 0) return 0;
  return ((size_t)quant_parts((long long)N * K) * sizeof(float) + 255) / 256 * 256;
}

w4a16_status_t w4a16_quantize(const float* w, uint8_t* wq, uint8_t* ws, float* g, int N, int K,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run_quantize(w, wq, ws, g, N, K, workspace, workspace_bytes, stream);
}

w4a16_status_t w4a16_quantize_bf16(const uint16_t* w, uint8_t* wq, uint8_t* ws, float* g, int N,
                                   int K, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  return run_quantize(w, wq, ws, g, N, K, workspace, workspace_bytes, stream);
}

w4a16_status_t w4a16_mlp_swiglu(const uint8_t* wq_gate, const uint8_t* ws_gate,
                                const float* g_gate, const uint8_t* wq_up, const uint8_t* ws_up,
                                const float* g_up, const uint8_t* wq_down, const uint8_t* ws_down,
                                const float* g_down, const uint16_t* x, uint16_t* y, int M, int H,
                                int F, void* workspace, size_t workspace_bytes,
                                const w4a16_mlp_options_t* options, hipStream_t stream) {
  if (!wq_gate || !ws_gate || !g_gate || !wq_up || !ws_up || !g_up || !wq_down || !ws_down ||
      !g_down || !x || !y)
    return W4A16_ERR_INVALID_VALUE;
  w4a16_status_t st = check_shape(M, F, H);
  if (st != W4A16_OK) return st;
  st = check_shape(M, H, F);
  if (st != W4A16_OK) return st;
  if (!aligned(wq_gate, 16) || !aligned(ws_gate, 16) || !aligned(wq_up, 16) ||
      !aligned(ws_up, 16) || !aligned(wq_down, 16) || !aligned(ws_down, 16) || !aligned(x, 16) ||
      !aligned(g_gate, 4) || !aligned(g_up, 4) || !aligned(g_down, 4) || !aligned(y, 4))
    return W4A16_ERR_UNSUPPORTED;
  MatArgs up{}, down{};
  up.wq0 = wq_gate;
  up.ws0 = ws_gate;
  up.g0 = g_gate;
  up.wq1 = wq_up;
  up.ws1 = ws_up;
  up.g1 = g_up;
  up.x = x;
  up.M = M;
  up.N = F;
  up.K = H;
  down.wq0 = wq_down;
  down.ws0 = ws_down;
  down.g0 = g_down;
  down.y = y;
  down.M = M;
  down.N = H;
  down.K = F;
  return run_mlp(up, down, workspace, workspace_bytes, options, stream);
}

size_t w4a16_workspace_size_mlp(int M, int H, int F) {
  if (check_shape(M, F, H) != W4A16_OK || check_shape(M, H, F) != W4A16_OK) return 0;
  const MlpPlan mp = plan_mlp(M, H, F);
  if (mp.p1.S == 0 || mp.p1.lds > kMaxLds || mp.p2.lds > kMaxLds) return 0;
  return mp.ws;
}

int w4a16_mlp_one_launch(int M, int H, int F) {
  if (check_shape(M, F, H) != W4A16_OK || check_shape(M, H, F) != W4A16_OK) return -1;
  MlpPlan mp = plan_mlp(M, H, F);
  if (mp.p1.S == 0 || mp.p1.lds > kMaxLds || mp.p2.lds > kMaxLds) return -1;
  mlp_check_resident(mp);
  return mp.k ? 1 : 0;
}

const char* w4a16_status_string(w4a16_status_t status) {
  switch (status) {
    case W4A16_OK: return "ok";
    case W4A16_ERR_INVALID_VALUE: return "invalid value (null pointer, non-positive size or short workspace)";
    case W4A16_ERR_UNSUPPORTED: return "unsupported (M > 32, K % 256 != 0, misaligned pointer or shape too large)";
    case W4A16_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

int w4a16_abi_version(void) { return W4A16_ABI_VERSION; }

#ifdef W4A16_TUNING
// Tuning builds only (not part of the ABI): force launch parameters for the
// kernel family `mfma` (0 = VALU, 1 = MFMA); enable = 0 restores the planner.
// Returns 1 if the requested variant is compiled in.
__attribute__((visibility("default"))) int w4a16_tuning_set(int enable, int mfma, int lr, int D,
                                                             int W, int LB, int nrb, int S) {
  g_override = Override{enable, mfma, lr, D, W, LB, nrb, S};
  if (!enable) return 1;
  for (const KernEntry& e : kKernels)
    if (e.mfma == (mfma != 0) && e.lr == lr && e.D == D && e.LB == LB) return 1;
  return 0;
}
// Tuning builds only: the launch plan for a shape, as 12 ints
// {mfma, lr, D, W, LB, nrb, S, rq, rr, kmax, lds, ws (bytes, clamped)}.
__attribute__((visibility("default"))) void w4a16_tuning_plan(int M, int N, int K, int epi,
                                                               long long* out) {
  const Plan pl = plan_gemm(M, N, K, epi);
  const long long v[12] = {pl.mfma, pl.lr, pl.D, pl.W, pl.LB, pl.nrb, pl.S,
                           pl.rq, pl.rr, pl.kmax, (long long)pl.lds, (long long)pl.ws};
  for (int i = 0; i < 12; ++i) out[i] = v[i];
}
__attribute__((visibility("default"))) void w4a16_tuning_wide(int W, int u, int min_m) {
  g_wide_W = W;
  g_wide_u = u;
  g_wide_minm = min_m;
}
// Tuning builds only: the wide kernel's part of the plan, as 7 ints
// {wide_mt, wide_steps, W, nrb, S, lds, ws} (wide_mt = 0: another kernel).
__attribute__((visibility("default"))) void w4a16_tuning_plan_wide(int M, int N, int K, int epi,
                                                                    long long* out) {
  const Plan pl = plan_gemm(M, N, K, epi);
  const long long v[7] = {pl.wide_mt, pl.wide_steps, pl.W, pl.nrb, pl.S, (long long)pl.lds, (long long)pl.ws};
  for (int i = 0; i < 7; ++i) out[i] = v[i];
}
#endif
#ifdef W4A16_TRACE
// Trace builds only: device buffer for the per-wave timeline stamps (NULL = off).
__attribute__((visibility("default"))) int w4a16_trace_set(void* buf) {
  return hipMemcpyToSymbol(HIP_SYMBOL(w4a16_trace), &buf, sizeof(buf)) == hipSuccess ? 1 : 0;
}
#endif

}  // extern "C"
