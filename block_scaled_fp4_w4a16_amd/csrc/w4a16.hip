// w4a16.hip -- libw4a16.so: C ABI, argument checks and kernel selection for
// the NVFP4 W4A16 matmul on MI355X (gfx950).  See include/w4a16.h for the
// contract of every entry point.
#include "w4a16.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4a16_kernels.h"

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

constexpr size_t kMaxLds = 160 * 1024;

// How one matmul call is launched.
struct Plan {
  bool mfma;   // false: VALU kernel (M <= 3); true: 4x4x4 MFMA kernel
  int L;       // VALU: lanes per weight row (8, 16 or 32)
  int W;       // waves per workgroup
  int nrb;     // row blocks
  int S;       // K-slices (split-K factor); grid = nrb * S workgroups
  size_t lds;  // dynamic LDS bytes per workgroup
  size_t ws;   // workspace bytes (fp32 partials) when S > 1
};

// Waves per workgroup for `tasks` row groups: all of them when they fit,
// otherwise the count in [4, wmax] that leaves the fewest idle wave slots.
int pick_waves(long long tasks, int wmax) {
  if (tasks <= wmax) return (int)(tasks > 0 ? tasks : 1);
  int best = wmax;
  long long best_waste = -1;
  for (int w = wmax; w >= 4; --w) {
    const long long waste = (tasks + w - 1) / w * w - tasks;
    if (best_waste < 0 || waste < best_waste) {
      best = w;
      best_waste = waste;
    }
  }
  return best;
}

// Kernel selection is a pure function of (M, N, K, fused) and the device's
// compute-unit count.
Plan plan_gemm(int M, int N, int K, bool fused) {
  Plan pl{};
  const int cus = cu_count();
  const int CR = K >> 5;  // 16-byte chunks per weight row (a multiple of 8)
  int rows, RT;
  if (M <= 3) {
    pl.mfma = false;
    int L = (CR % 16 == 0) ? 16 : 8;
    if (CR % 32 == 0 && K >= 8192) L = 32;
    pl.L = L;
    rows = M;
    RT = fused ? (64 / L) / 2 : 64 / L;
  } else {
    pl.mfma = true;
    pl.L = 16;
    rows = 4 * ((M + 3) / 4);
    RT = fused ? 2 : 4;
  }
  // smallest K split whose x slice fits in LDS (and keeps whole chunks per lane)
  auto lds_bytes = [&](int S) { return (size_t)rows * (size_t)((CR / S) * 4 + 1) * 16; };
  int S = 1;
  for (; S < CR; ++S) {
    if (CR % S) continue;
    if (!pl.mfma && (CR / S) % pl.L) continue;
    if (lds_bytes(S) <= kMaxLds) break;
  }
  pl.S = S;
  pl.lds = lds_bytes(S);
  const long long groups = ((long long)N + RT - 1) / RT;  // row groups in total
  long long nrb = cus / S > 0 ? cus / S : 1;
  if (nrb > groups) nrb = groups;
  pl.nrb = (int)nrb;
  const long long tasks = (groups + nrb - 1) / nrb;        // row groups per block
  pl.W = pick_waves(tasks, 8);
  pl.ws = S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(float) * (fused ? 2 : 1) : 0;
  return pl;
}

template <typename Kern>
hipError_t launch(Kern kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                  const MatArgs& args) {
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kernel, grid, block, lds, stream, args);
  return hipGetLastError();
}

template <bool FUSED>
hipError_t dispatch(const Plan& pl, hipStream_t s, const MatArgs& a) {
  constexpr int DV = 8;  // VALU ring depth (chunk loads in flight per lane)
  constexpr int DM = 8;  // MFMA ring depth
  const dim3 grid((unsigned)(pl.nrb * pl.S)), block((unsigned)(pl.W * 64));
  hipError_t e;
  if (!pl.mfma) {
#define W4A16_VALU(MT)                                                                    \
  switch (pl.L) {                                                                         \
    case 8: e = launch(k_gemm_valu<MT, 8, DV, FUSED>, grid, block, pl.lds, s, a); break;   \
    case 16: e = launch(k_gemm_valu<MT, 16, DV, FUSED>, grid, block, pl.lds, s, a); break; \
    default: e = launch(k_gemm_valu<MT, 32, DV, FUSED>, grid, block, pl.lds, s, a); break; \
  }
    switch (a.M) {
      case 1: W4A16_VALU(1) break;
      case 2: W4A16_VALU(2) break;
      default: W4A16_VALU(3) break;
    }
#undef W4A16_VALU
  } else {
    switch ((a.M + 3) / 4) {
      case 1: e = launch(k_gemm_mfma<1, DM, FUSED>, grid, block, pl.lds, s, a); break;
      case 2: e = launch(k_gemm_mfma<2, DM, FUSED>, grid, block, pl.lds, s, a); break;
      case 3: e = launch(k_gemm_mfma<3, DM, FUSED>, grid, block, pl.lds, s, a); break;
      default: e = launch(k_gemm_mfma<4, DM, FUSED>, grid, block, pl.lds, s, a); break;
    }
  }
  if (e != hipSuccess || pl.S == 1) return e;
  const long long MN = (long long)a.M * a.N;
  long long nb = (MN + 255) / 256;
  if (nb > 4LL * cu_count()) nb = 4LL * cu_count();
  return launch(k_combine<FUSED>, dim3((unsigned)nb), dim3(256), 0, s, a);
}

w4a16_status_t check_shape(int M, int N, int K) {
  if (M <= 0 || N <= 0 || K <= 0) return W4A16_ERR_INVALID_VALUE;
  if (M > W4A16_MAX_M || (K % 256) != 0) return W4A16_ERR_UNSUPPORTED;
  if ((long long)K * 2 > 0x7fffffffLL) return W4A16_ERR_UNSUPPORTED;
  return W4A16_OK;
}

size_t workspace_bytes_for(int M, int N, int K, bool fused) {
  if (check_shape(M, N, K) != W4A16_OK) return 0;
  return plan_gemm(M, N, K, fused).ws;
}

w4a16_status_t run_matmul(MatArgs a, bool fused, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  const Plan pl = plan_gemm(a.M, a.N, a.K, fused);
  if (pl.lds > kMaxLds) return W4A16_ERR_UNSUPPORTED;
  if (workspace_bytes < pl.ws || (pl.ws > 0 && workspace == nullptr))
    return W4A16_ERR_INVALID_VALUE;
  if (pl.ws > 0 && !aligned(workspace, 16)) return W4A16_ERR_UNSUPPORTED;
  a.nrb = pl.nrb;
  a.S = pl.S;
  a.part = static_cast<float*>(workspace);
  const hipError_t e = fused ? dispatch<true>(pl, stream, a) : dispatch<false>(pl, stream, a);
  return e == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

}  // namespace
}  // namespace w4a16

using namespace w4a16;

extern "C" {

size_t w4a16_workspace_size(int M, int N, int K) { return workspace_bytes_for(M, N, K, false); }

size_t w4a16_workspace_size_gate_up(int M, int N, int K) {
  return workspace_bytes_for(M, N, K, true);
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
  return run_matmul(a, false, workspace, workspace_bytes, stream);
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
  return run_matmul(a, true, workspace, workspace_bytes, stream);
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

const char* w4a16_status_string(w4a16_status_t status) {
  switch (status) {
    case W4A16_OK: return "ok";
    case W4A16_ERR_INVALID_VALUE: return "invalid value (null pointer, non-positive size or short workspace)";
    case W4A16_ERR_UNSUPPORTED: return "unsupported (M > 16, K % 256 != 0, misaligned pointer or shape too large)";
    case W4A16_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

int w4a16_abi_version(void) { return W4A16_ABI_VERSION; }

}  // extern "C"
