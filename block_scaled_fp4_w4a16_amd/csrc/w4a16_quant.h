// w4a16_quant.h -- gfx950 device code: NVFP4 encoding of fp32 / bf16 weights.
//
// Schema (FlashRT, "Qwen3.6-27B NVFP4 on RTX 5090", section 1 "Model
// dependencies"): codes u8 [N][K/2] (E2M1, two per byte, low nibble = even
// input), one E4M3 scale per 16 inputs, fp32 global scale g = 448 / amax.
// The pages give the schema, not the block-scale recipe; the recipe encoded
// here is the library's reading of it:
//   amax = max |W|;  g = fp32(448 / amax)  (g = 1 when amax = 0);
//   for each 16-input block: S = the E4M3FN value nearest to bmax * g / 6
//   (ties to the even code, saturating at 448), where bmax = max |W| over the
//   block; if S = 0 every code of the block is 0, otherwise each code is the
//   E2M1 value nearest to W * g / S (ties to the even code, saturating at 6,
//   sign kept, so -0 can occur).
// The arithmetic is fp64 in exactly that order (both products of two fp32
// values are exact in fp64; each division is rounded once), so every
// rounding decision is the same as a scalar fp64 evaluation of the recipe.
// This runs once per weight tensor, off the matmul path.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

template <typename T>
__device__ __forceinline__ float quant_load(const T* p);
template <>
__device__ __forceinline__ float quant_load<float>(const float* p) {
  return *p;
}
template <>
__device__ __forceinline__ float quant_load<uint16_t>(const uint16_t* p) {
  return __uint_as_float((uint32_t)*p << 16);  // bf16 widens exactly
}

// The 16 inputs of block b (16-byte aligned: K % 16 == 0 and the tensor is
// 16-byte aligned), widened to fp32.
__device__ __forceinline__ void quant_load16(const float* w, long long b, float (&v)[16]) {
  const float4* p = reinterpret_cast<const float4*>(w) + 4 * b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 q = p[i];
    v[4 * i] = q.x;
    v[4 * i + 1] = q.y;
    v[4 * i + 2] = q.z;
    v[4 * i + 3] = q.w;
  }
}
__device__ __forceinline__ void quant_load16(const uint16_t* w, long long b, float (&v)[16]) {
  const uint4* p = reinterpret_cast<const uint4*>(w) + 2 * b;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint4 q = p[i];
    const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = __uint_as_float(u[j] << 16);
      v[8 * i + 2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
    }
  }
}

// |v| max that ignores NaN (a NaN element never becomes amax)
__device__ __forceinline__ float quant_absmax(float m, float v) {
  const float a = fabsf(v);
  return a > m ? a : m;
}

// Pass 1: per-workgroup max |W| over a grid-stride slice -> part[blockIdx.x].
template <typename T>
__global__ void __launch_bounds__(256) k_quant_amax(const T* __restrict__ w, long long count,
                                                    float* __restrict__ part) {
  __shared__ float red[256];
  float m = 0.0f;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < count;
       i += (long long)gridDim.x * 256)
    m = quant_absmax(m, quant_load(w + i));
  red[threadIdx.x] = m;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

// Value of E4M3FN code c in [0, 0x7E] (non-negative, finite).
__device__ __forceinline__ double e4m3_value(int c) {
  const int e = c >> 3, m = c & 7;
  return e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
}

// Nearest E4M3FN code to t (ties to the even code; t >= 448 -> 448; t <= 0
// or NaN -> 0).  Normal values are 2^e (1 + m/8), e in [-6, 8]; subnormals
// are m 2^-9.  Scaling by a power of two is exact, so the rounded quantity
// q below is exact and rint (round half to even) makes the tie decision; the
// code's low bit is the low bit of the rounded mantissa, so "even mantissa"
// and "even code" agree.
__device__ __forceinline__ int e4m3_nearest(double t) {
  if (!(t > 0.0)) return 0;
  if (t >= 448.0) return 0x7E;
  int E;
  const double f = frexp(t, &E);  // t = f 2^E, f in [0.5, 1)
  const int e = E - 1;            // t = (2f) 2^e, 2f in [1, 2)
  if (e < -6) return (int)rint(ldexp(t, 9));  // subnormal grid m 2^-9 (8 -> 2^-6, code 8)
  int r = (int)rint((2.0 * f - 1.0) * 8.0);
  int ee = e;
  if (r == 8) {
    r = 0;
    ++ee;
  }
  return ((ee + 7) << 3) | r;  // t < 448 keeps this <= 0x7E
}

// Nearest E2M1 code magnitude to t >= 0 over {0, .5, 1, 1.5, 2, 3, 4, 6}
// (ties to the even code): one threshold per neighbouring pair, passed with
// '>' where the tie goes down (the lower code is even) and '>=' where it goes
// up (the upper code is even); NaN passes none.
__device__ __forceinline__ int e2m1_nearest_mag(double t) {
  return (t > 0.25) + (t >= 0.75) + (t > 1.25) + (t >= 1.75) + (t > 2.5) + (t >= 3.5) + (t > 5.0);
}

// Pass 2: one 16-input block per thread.  Every workgroup first reduces the
// pass-1 maxima to amax (max is order-independent, so all agree) and derives
// g; workgroup 0 stores g.
template <typename T>
__global__ void __launch_bounds__(256) k_quant_encode(const T* __restrict__ w, long long nblocks,
                                                      const float* __restrict__ part,
                                                      int nparts, uint8_t* __restrict__ wq,
                                                      uint8_t* __restrict__ ws,
                                                      float* __restrict__ g_out) {
  __shared__ float red[256];
  float m = 0.0f;
  for (int i = threadIdx.x; i < nparts; i += 256) m = fmaxf(m, part[i]);
  red[threadIdx.x] = m;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  const double amax = (double)red[0];
  const float g = amax > 0.0 ? (float)(448.0 / amax) : 1.0f;
  const double gd = (double)g;
  if (blockIdx.x == 0 && threadIdx.x == 0) *g_out = g;

  for (long long b = (long long)blockIdx.x * 256 + threadIdx.x; b < nblocks;
       b += (long long)gridDim.x * 256) {
    // block b: inputs 16b..16b+15 of the row-major tensor (K % 16 == 0, so a
    // block never straddles two rows); its codes at wq + 8b, its scale at ws + b
    float v[16];
    quant_load16(w, b, v);
    double bmax = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const double a = fabs((double)v[i]);
      bmax = a > bmax ? a : bmax;
    }
    const int sc = e4m3_nearest(bmax * gd / 6.0);
    const double S = e4m3_value(sc);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int code = 0;
      if (S != 0.0) {
        const double q = (double)v[i] * gd / S;
        code = e2m1_nearest_mag(fabs(q)) | (signbit(q) ? 8 : 0);
      }
      if (i < 8) lo |= (uint32_t)code << (4 * i);
      else hi |= (uint32_t)code << (4 * (i - 8));
    }
    reinterpret_cast<uint2*>(wq)[b] = make_uint2(lo, hi);
    ws[b] = (uint8_t)sc;
  }
}

}  // namespace w4a16
