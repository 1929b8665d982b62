// calib.hip -- HBM read-bandwidth calibration for the benchmark (a separate
// library, libw4a16_calib.so; not part of the matmul ABI).
//
// A plain streaming read: every lane reads NPER 16-byte units per round with
// non-temporal 128-bit loads (the matmul kernels' weight loads), grid-stride
// over the buffer, and folds them into one word that is stored only if it
// equals a value the benchmark's buffers never produce, so the loads cannot be
// removed and nothing else is written.  The benchmark times it on a buffer far
// larger than the caches (the achievable streaming rate) and on buffers of
// one matmul call's size cycled like the weight copies (the achievable rate
// for calls of that size, per-call fixed costs included).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

template <int NPER>
__global__ void __launch_bounds__(1024) k_stream_read(const u32x4_t* __restrict__ p, size_t n16,
                                                      unsigned* sink) {
  const size_t nthr = (size_t)gridDim.x * blockDim.x;
  const size_t gt = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  unsigned acc = 0;
  for (size_t base = gt; base < n16; base += nthr * NPER) {
    u32x4_t v[NPER];
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const size_t idx = base + (size_t)i * nthr;
      v[i] = idx < n16 ? __builtin_nontemporal_load(p + idx) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < NPER; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, buffer 16-byte aligned) at `buf` once with
// `grid` workgroups of `block` threads (block <= 1024), 8 loads in flight per
// lane, on `stream`.  sink: one device word, written only by the never-taken
// path.  Returns 0, or a hipError_t value (nothing enqueued on a bad argument).
__attribute__((visibility("default"))) int w4a16_calib_stream_read(const void* buf, size_t bytes,
                                                                    unsigned* sink, int grid,
                                                                    int block, hipStream_t stream) {
  if (buf == nullptr || sink == nullptr || bytes % 16 != 0 || ((uintptr_t)buf & 15) != 0 ||
      grid <= 0 || block <= 0 || block > 1024 || block % 64 != 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_stream_read<8>, dim3((unsigned)grid), dim3((unsigned)block), 0, stream,
                     static_cast<const u32x4_t*>(buf), bytes / 16, sink);
  return (int)hipGetLastError();
}

}  // extern "C"
