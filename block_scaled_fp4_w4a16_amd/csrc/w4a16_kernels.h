// w4a16_kernels.h -- gfx950 (CDNA4) device code for the NVFP4 W4A16 matmul.
//
// Weight layout (FlashRT, "Qwen3.6-27B NVFP4 on RTX 5090", section 1 "Model
// dependencies"): codes u8 [N][K/2] (E2M1, two per byte, low nibble = even
// input), scales u8 [N][K/16] (E4M3FN, one per 16 inputs), global fp32 g;
// W[n][k] = e2m1 * e4m3 / g.
//
// Work unit: a 16-byte "chunk" of one weight row = 32 codes = two 16-input
// scale blocks, plus its two scale bytes.  Every kernel reads each chunk
// exactly once with a coalesced 128-bit load (lanes that share a row read
// consecutive chunks) and its scale pair with a 16-bit load.
//
// Decoding happens in registers with gfx950 conversion instructions:
//   v_cvt_scalef32_pk_bf16_fp4 turns one byte (two E2M1 codes) into two bf16,
//   exactly (scale operand 1.0; the instruction only applies the exponent of
//   its fp32 scale, so the E4M3 block scale cannot be folded into it);
//   v_cvt_f32_fp8 turns an E4M3FN byte into fp32 exactly.
// The block scale multiplies the fp32 partial sum of its 16 products, and the
// division by g happens once per output, so no weight is ever rounded.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;

// Launch arguments shared by all matmul kernels.  For the fused gate/up
// variant, (wq0, ws0, g0) is the gate matrix and (wq1, ws1, g1) the up matrix.
struct MatArgs {
  const uint8_t* wq0;
  const uint8_t* ws0;
  const float* g0;
  const uint8_t* wq1;
  const uint8_t* ws1;
  const float* g1;
  const uint16_t* x;
  uint16_t* y;
  int M, N, K;
  // Grid: nrb row blocks x S K-slices; workgroup b works on row block b / S
  // (rows [rb*N/nrb, (rb+1)*N/nrb)) and K-slice b % S (chunks
  // [s*CR/S, (s+1)*CR/S) of every row, CR = K/32).  With S > 1 the workgroup
  // writes fp32 partial sums part[s][M][N] (fused: gate partials, then up
  // partials at part + S*M*N) instead of y, and k_combine finishes them.
  int nrb;
  int S;
  float* part;
};

#define W4A16_DEV __device__ __forceinline__

// two E2M1 codes (byte B of w) -> two bf16 in one dword (low half = low nibble)
template <int B>
W4A16_DEV uint32_t fp4x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, B));
}

// two E2M1 codes (byte B of w) -> two fp32
template <int B>
W4A16_DEV f32x2_t fp4x2_to_f32x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
}

// E4M3FN byte B of w -> fp32 (exact; 0x7F / 0xFF give NaN)
template <int B>
W4A16_DEV float e4m3_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8(w, B);
}

// c + a.lo*b.lo + a.hi*b.hi, bf16 pairs, fp32 accumulate
W4A16_DEV float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

W4A16_DEV i16x4_t pack4(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(i16x4_t, make_uint2(lo, hi));
}

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN
W4A16_DEV uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

W4A16_DEV float silu(float v) { return v / (1.0f + expf(-v)); }

// Position of 16-byte unit q (0..3) of x-chunk c inside an LDS x row for the
// VALU kernel.  Lanes read consecutive chunks; the XOR spreads the four units
// of neighbouring chunks over distinct bank groups (for 8- and 16-lane passes).
W4A16_DEV int xsw(int c, int q) { return 4 * c + (q ^ (((c >> 1) ^ (c >> 2)) & 3)); }

// Number of 16-byte x units each thread loads before the weight prologue is
// issued (so that staging x in LDS never waits on the weight loads).
constexpr int kXPre = 8;

// Stage `rows` rows of x (K bf16 each; rows >= M are zero) into LDS units
// xs[m*RSU + pos(cu)].  Phase 1 issues the first kXPre units per thread and
// returns them in xr; phase 2 (after the caller has issued its weight loads)
// writes them and handles any remainder.
// The slice is `upr` units per row starting at unit u0 of each x row (a row
// of x has K/8 units).
W4A16_DEV void x_stage_issue(uint4 (&xr)[kXPre], const uint16_t* x, int M, int rows, int K,
                             int u0, int upr, int tid, int nthr) {
  const uint4* xg = reinterpret_cast<const uint4*>(x);
#pragma unroll
  for (int i = 0; i < kXPre; ++i) {
    const int u = tid + i * nthr;
    const int m = u / upr, cu = u - m * upr;
    xr[i] = (u < rows * upr && m < M) ? xg[(size_t)m * (K >> 3) + u0 + cu]
                                      : make_uint4(0u, 0u, 0u, 0u);
  }
}
template <typename Pos>
W4A16_DEV void x_stage_store(uint4* xs, const uint4 (&xr)[kXPre], const uint16_t* x, int M,
                             int rows, int K, int u0, int upr, int RSU, int tid, int nthr,
                             Pos pos) {
  const uint4* xg = reinterpret_cast<const uint4*>(x);
#pragma unroll
  for (int i = 0; i < kXPre; ++i) {
    const int u = tid + i * nthr;
    if (u < rows * upr) {
      const int m = u / upr, cu = u - m * upr;
      xs[m * RSU + pos(cu)] = xr[i];
    }
  }
  for (int u = tid + kXPre * nthr; u < rows * upr; u += nthr) {
    const int m = u / upr, cu = u - m * upr;
    xs[m * RSU + pos(cu)] =
        m < M ? xg[(size_t)m * (K >> 3) + u0 + cu] : make_uint4(0u, 0u, 0u, 0u);
  }
}


// ---------------------------------------------------------------------------
// VALU kernel, M = MT in {1, 2, 3}.
//
// Lane layout: a wave holds G = 64/L row slots of L lanes; lane (slot r,
// position p) reads chunks p, p+L, p+2L, ... of its row (CR/L chunks), so the
// L lanes of a row read L*16 contiguous bytes per load.  A task is one row
// group (G rows; for the fused variant G/2 gate rows plus the same G/2 up
// rows).  Workgroup b owns a contiguous row range; its waves take tasks
// round-robin.  Each lane keeps D chunk loads in flight in a register ring
// that runs across task boundaries.
//
// Per chunk and activation row: 16 bf16x2 dot products per 32 weights into
// two block partials, then acc += partial * e4m3(scale).  x rows live in LDS
// (swizzled) and are read with 128-bit LDS loads; lanes of different slots
// read the same x (broadcast).
// ---------------------------------------------------------------------------
template <int MT, int L, int D, bool FUSED>
__global__ void __launch_bounds__(512) k_gemm_valu(MatArgs a) {
  extern __shared__ uint4 xs[];
  constexpr int G = 64 / L;
  constexpr int RT = FUSED ? G / 2 : G;
  const int W = blockDim.x >> 6;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = a.K, CR = K >> 5, S = a.S;
  const int ks = blockIdx.x % S;
  const long long rb = blockIdx.x / S;
  const int CRS = CR / S;                // chunks per row in this K-slice
  const int c0 = ks * CRS;               // first chunk of the slice
  const int CPL = CRS / L, RSU = (CRS << 2) + 1;
  const int row_lo = (int)(rb * a.N / a.nrb), row_hi = (int)((rb + 1) * a.N / a.nrb);
  const int ntasks = (row_hi - row_lo + RT - 1) / RT;
  const int p = lane % L, r = lane / L;
  const int srow = FUSED ? (r % (G / 2)) : r;
  const bool is_up = FUSED && (r >= G / 2);
  const uint8_t* wq = is_up ? a.wq1 : a.wq0;
  const uint8_t* ws = is_up ? a.ws1 : a.ws0;
  const int my_tasks = wv < ntasks ? (ntasks - 1 - wv) / W + 1 : 0;
  const int T = my_tasks * CPL;  // chunk steps of this wave (uniform)
  const float g0 = *a.g0;
  const float g1 = FUSED ? *a.g1 : 1.0f;

  // ---- issue cursor: (task it_i, step jj_i) -> row pointers -------------
  const uint4* qp;
  const uint16_t* sp;
  int s_i = 0, it_i = 0, jj_i = 0;
  auto set_task = [&](int it) {
    int row = row_lo + (wv + W * it) * RT + srow;
    row = row < row_hi ? row : row_hi - 1;
    qp = reinterpret_cast<const uint4*>(wq + (size_t)row * (size_t)(K >> 1)) + c0 + p;
    sp = reinterpret_cast<const uint16_t*>(ws + (size_t)row * (size_t)(K >> 4)) + c0 + p;
  };
  set_task(0);
  uint4 qb[D];
  uint32_t sb[D];
  // load the current cursor position into slot d, then advance (the cursor
  // stops at the last step; later loads repeat it and are never used)
  auto issue = [&](int d) {
    qb[d] = qp[L * jj_i];
    sb[d] = sp[L * jj_i];
    if (s_i + 1 < T) {
      ++s_i;
      if (++jj_i == CPL) {
        jj_i = 0;
        ++it_i;
        set_task(it_i);
      }
    }
  };
  // x -> LDS (rows of K bf16; 16-byte units, swizzled): x loads first, then
  // the weight prologue, then the LDS stores
  uint4 xr[kXPre];
  auto xpos = [](int cu) { return xsw(cu >> 2, cu & 3); };
  x_stage_issue(xr, a.x, a.M, MT, K, c0 << 2, CRS << 2, tid, blockDim.x);
#pragma unroll
  for (int d = 0; d < D; ++d) issue(d);
  x_stage_store(xs, xr, a.x, a.M, MT, K, c0 << 2, CRS << 2, RSU, tid, blockDim.x, xpos);
  __syncthreads();

  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
  int it_c = 0, jj_c = 0;

  auto finish_task = [&]() {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int off = L / 2; off >= 1; off >>= 1) acc[m] += __shfl_xor(acc[m], off, 64);
    }
    const int row = row_lo + (wv + W * it_c) * RT + srow;
    if (S > 1) {
      // partial sums of this K-slice; gate and up land in separate planes
      float* dst = a.part + ((size_t)(is_up ? S : 0) + ks) * (size_t)a.M * a.N;
      if (p == 0 && row < row_hi) {
#pragma unroll
        for (int m = 0; m < MT; ++m) dst[(size_t)m * a.N + row] = acc[m];
      }
    } else if (FUSED) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float upv = __shfl(acc[m], (lane + (G / 2) * L) & 63, 64);
        if (!is_up && p == 0 && row < row_hi)
          a.y[(size_t)m * a.N + row] = f32_to_bf16(silu(acc[m] / g0) * (upv / g1));
      }
    } else {
      if (p == 0 && row < row_hi) {
#pragma unroll
        for (int m = 0; m < MT; ++m) a.y[(size_t)m * a.N + row] = f32_to_bf16(acc[m] / g0);
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
  };

  for (int s0 = 0; s0 < T; s0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      // consume slot d completely, then refill it (the refill can then reuse
      // the slot's registers: no copies and no full drain at the loop edge)
      if (s0 + d < T) {
        const uint4 q = qb[d];
        const uint32_t sc = sb[d];
        const int c = p + L * jj_c;
        uint4 xv[MT][4];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int u = 0; u < 4; ++u) xv[m][u] = xs[m * RSU + xsw(c, u)];
        const float s_lo = e4m3_to_f32<0>(sc), s_hi = e4m3_to_f32<1>(sc);
        float blo[MT], bhi[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) blo[m] = bhi[m] = 0.0f;
        // word wi holds inputs 8wi..8wi+7 of the chunk; block 0 = words 0,1
#define W4A16_DOT_WORD(word, wi, part)                                  \
  {                                                                     \
    const uint32_t d0 = fp4x2_to_bf16x2<0>(word);                       \
    const uint32_t d1 = fp4x2_to_bf16x2<1>(word);                       \
    const uint32_t d2 = fp4x2_to_bf16x2<2>(word);                       \
    const uint32_t d3 = fp4x2_to_bf16x2<3>(word);                       \
    _Pragma("unroll") for (int m = 0; m < MT; ++m) {                    \
      part[m] = dot2_bf16(d0, xv[m][wi].x, part[m]);                    \
      part[m] = dot2_bf16(d1, xv[m][wi].y, part[m]);                    \
      part[m] = dot2_bf16(d2, xv[m][wi].z, part[m]);                    \
      part[m] = dot2_bf16(d3, xv[m][wi].w, part[m]);                    \
    }                                                                   \
  }
        W4A16_DOT_WORD(q.x, 0, blo)
        W4A16_DOT_WORD(q.y, 1, blo)
        W4A16_DOT_WORD(q.z, 2, bhi)
        W4A16_DOT_WORD(q.w, 3, bhi)
#undef W4A16_DOT_WORD
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          acc[m] = fmaf(blo[m], s_lo, acc[m]);
          acc[m] = fmaf(bhi[m], s_hi, acc[m]);
        }
        if (++jj_c == CPL) {
          finish_task();
          jj_c = 0;
          ++it_c;
        }
      }
      issue(d);
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA kernel, 4 <= M <= 16 (P = ceil(M/4) passes of 4 activation rows).
//
// Uses v_mfma_f32_4x4x4_16b_bf16: 16 independent 4x4x4 products per
// instruction; lane l = 4*beta + j holds B[k=0..3][col j] and A[row j][k] of
// block beta and receives C[row r][col j] in register r.  Here block beta is
// one weight chunk column, col j one of 4 weight rows, row r one activation
// row; each MFMA covers 4 consecutive inputs, which never straddle a 16-input
// scale block, so the E4M3 scale multiplies the fp32 MFMA result of its block
// (4 MFMAs per block, one FMA per result element).
//
// Lane (beta, j) reads chunks beta, beta+16, ... of weight row j of the task
// (16 lanes x 16 B = 256 contiguous bytes per row per load) and the x slice of
// activation row 4*pp + j for the same chunk from LDS.  Tasks are 4 weight
// rows (fused: 2 gate rows and the same 2 up rows).
// ---------------------------------------------------------------------------
template <int P, int D, bool FUSED>
__global__ void __launch_bounds__(512) k_gemm_mfma(MatArgs a) {
  extern __shared__ uint4 xs[];
  constexpr int RT = FUSED ? 2 : 4;
  const int W = blockDim.x >> 6;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = a.K, CR = K >> 5, S = a.S;
  const int ks = blockIdx.x % S;
  const long long rb = blockIdx.x / S;
  const int CRS = CR / S;                // chunks per row in this K-slice
  const int c0 = ks * CRS;
  const int CPL = (CRS + 15) >> 4, RSU = (CRS << 2) + 1;
  const int row_lo = (int)(rb * a.N / a.nrb), row_hi = (int)((rb + 1) * a.N / a.nrb);
  const int ntasks = (row_hi - row_lo + RT - 1) / RT;
  const int beta = lane >> 2, j = lane & 3;
  const int srow = FUSED ? (j & 1) : j;
  const bool is_up = FUSED && (j >= 2);
  const uint8_t* wq = is_up ? a.wq1 : a.wq0;
  const uint8_t* ws = is_up ? a.ws1 : a.ws0;
  const int my_tasks = wv < ntasks ? (ntasks - 1 - wv) / W + 1 : 0;
  const int T = my_tasks * CPL;
  const bool ragged = (CRS & 15) != 0;
  const float g0 = *a.g0;
  const float g1 = FUSED ? *a.g1 : 1.0f;

  const uint4* qp;
  const uint16_t* sp;
  int s_i = 0, it_i = 0, jj_i = 0;
  auto set_task = [&](int it) {
    int row = row_lo + (wv + W * it) * RT + srow;
    row = row < row_hi ? row : row_hi - 1;
    qp = reinterpret_cast<const uint4*>(wq + (size_t)row * (size_t)(K >> 1)) + c0;
    sp = reinterpret_cast<const uint16_t*>(ws + (size_t)row * (size_t)(K >> 4)) + c0;
  };
  set_task(0);
  uint4 qb[D];
  uint32_t sb[D];
  auto issue = [&](int d) {
    int c = beta + 16 * jj_i;
    c = c < CRS ? c : CRS - 1;
    qb[d] = qp[c];
    sb[d] = sp[c];
    if (s_i + 1 < T) {
      ++s_i;
      if (++jj_i == CPL) {
        jj_i = 0;
        ++it_i;
        set_task(it_i);
      }
    }
  };
  // x -> LDS: rows 0..4P-1 (rows >= M are zero), K bf16 + 16 B pad per row
  uint4 xr[kXPre];
  auto xpos = [](int cu) { return cu; };
  x_stage_issue(xr, a.x, a.M, 4 * P, K, c0 << 2, CRS << 2, tid, blockDim.x);
#pragma unroll
  for (int d = 0; d < D; ++d) issue(d);
  x_stage_store(xs, xr, a.x, a.M, 4 * P, K, c0 << 2, CRS << 2, RSU, tid, blockDim.x, xpos);
  __syncthreads();

  float acc[P][4];
#pragma unroll
  for (int pp = 0; pp < P; ++pp)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[pp][r] = 0.0f;
  int it_c = 0, jj_c = 0;

  auto finish_task = [&]() {
#pragma unroll
    for (int pp = 0; pp < P; ++pp)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = acc[pp][r];
        v += __shfl_xor(v, 4, 64);
        v += __shfl_xor(v, 8, 64);
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        acc[pp][r] = v;
      }
    const int row = row_lo + (wv + W * it_c) * RT + srow;
#pragma unroll
    for (int pp = 0; pp < P; ++pp)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * pp + r;
        if (S > 1) {
          float* dst = a.part + ((size_t)(is_up ? S : 0) + ks) * (size_t)a.M * a.N;
          if (lane < 4 && row < row_hi && m < a.M) dst[(size_t)m * a.N + row] = acc[pp][r];
        } else if (FUSED) {
          const float upv = __shfl(acc[pp][r], (lane + 2) & 63, 64);
          if (lane < 2 && row < row_hi && m < a.M)
            a.y[(size_t)m * a.N + row] = f32_to_bf16(silu(acc[pp][r] / g0) * (upv / g1));
        } else {
          if (lane < 4 && row < row_hi && m < a.M)
            a.y[(size_t)m * a.N + row] = f32_to_bf16(acc[pp][r] / g0);
        }
        acc[pp][r] = 0.0f;
      }
  };

  for (int s0 = 0; s0 < T; s0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (s0 + d < T) {
        uint4 q = qb[d];
        const uint32_t sc = sb[d];
        int c = beta + 16 * jj_c;
        if (ragged && c >= CRS) {
          q = make_uint4(0u, 0u, 0u, 0u);
          c = CRS - 1;
        }
        uint4 xv[P][4];
#pragma unroll
        for (int pp = 0; pp < P; ++pp)
#pragma unroll
          for (int u = 0; u < 4; ++u) xv[pp][u] = xs[(4 * pp + j) * RSU + 4 * c + u];
        const float s_lo = e4m3_to_f32<0>(sc), s_hi = e4m3_to_f32<1>(sc);
        f32x4_t C[P];
        // word wi holds inputs 8wi..8wi+7 of the chunk: two MFMAs of 4 inputs
#define W4A16_MFMA_WORD(word, wi)                                              \
  {                                                                            \
    const i16x4_t b0 = pack4(fp4x2_to_bf16x2<0>(word), fp4x2_to_bf16x2<1>(word)); \
    const i16x4_t b1 = pack4(fp4x2_to_bf16x2<2>(word), fp4x2_to_bf16x2<3>(word)); \
    _Pragma("unroll") for (int pp = 0; pp < P; ++pp) {                          \
      C[pp] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(                            \
          pack4(xv[pp][wi].x, xv[pp][wi].y), b0, C[pp], 0, 0, 0);                \
      C[pp] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(                            \
          pack4(xv[pp][wi].z, xv[pp][wi].w), b1, C[pp], 0, 0, 0);                \
    }                                                                          \
  }
#pragma unroll
        for (int pp = 0; pp < P; ++pp) C[pp] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        W4A16_MFMA_WORD(q.x, 0)
        W4A16_MFMA_WORD(q.y, 1)
#pragma unroll
        for (int pp = 0; pp < P; ++pp)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[pp][r] = fmaf(C[pp][r], s_lo, acc[pp][r]);
#pragma unroll
        for (int pp = 0; pp < P; ++pp) C[pp] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        W4A16_MFMA_WORD(q.z, 2)
        W4A16_MFMA_WORD(q.w, 3)
#pragma unroll
        for (int pp = 0; pp < P; ++pp)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[pp][r] = fmaf(C[pp][r], s_hi, acc[pp][r]);
#undef W4A16_MFMA_WORD
        if (++jj_c == CPL) {
          finish_task();
          jj_c = 0;
          ++it_c;
        }
      }
      issue(d);
    }
  }
}

// ---------------------------------------------------------------------------
// Split-K epilogue: y[m][n] = f(sum over s = 0..S-1 of part[s][m][n]) in that
// fixed order (bitwise reproducible).  f = bf16(v / g), or for the fused
// variant bf16(silu(gate / g_gate) * (up / g_up)).
// ---------------------------------------------------------------------------
template <bool FUSED>
__global__ void __launch_bounds__(256) k_combine(MatArgs a) {
  const long long MN = (long long)a.M * a.N;
  const float g0 = *a.g0;
  const float g1 = FUSED ? *a.g1 : 1.0f;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < MN;
       i += (long long)gridDim.x * blockDim.x) {
    float v = 0.0f;
    for (int s = 0; s < a.S; ++s) v += a.part[(size_t)s * MN + i];
    if (FUSED) {
      float u = 0.0f;
      for (int s = 0; s < a.S; ++s) u += a.part[(size_t)(a.S + s) * MN + i];
      a.y[i] = f32_to_bf16(silu(v / g0) * (u / g1));
    } else {
      a.y[i] = f32_to_bf16(v / g0);
    }
  }
}

// ---------------------------------------------------------------------------
// Dequantisation to fp32: one thread per dword of codes (8 weights).
// w = (e2m1 * e4m3) / g: the product is exact in fp32 (at most 6 significant
// bits), the division is IEEE fp32, so the result is the correctly rounded
// quotient -- bit-identical to rounding the exact value once.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_dequant(const uint8_t* __restrict__ wq,
                                                 const uint8_t* __restrict__ ws,
                                                 const float* __restrict__ g,
                                                 float* __restrict__ w, long long words,
                                                 int K) {
  const float gv = *g;
  const int wpr = K >> 3;  // code dwords per row
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < words;
       i += (long long)gridDim.x * blockDim.x) {
    const long long n = i / wpr;
    const int wk = (int)(i - n * wpr);
    const uint32_t word = reinterpret_cast<const uint32_t*>(wq)[i];
    const uint32_t sbyte = ws[n * (K >> 4) + (wk >> 1)];
    const float s = e4m3_to_f32<0>(sbyte);
    const f32x2_t v0 = fp4x2_to_f32x2<0>(word), v1 = fp4x2_to_f32x2<1>(word);
    const f32x2_t v2 = fp4x2_to_f32x2<2>(word), v3 = fp4x2_to_f32x2<3>(word);
    float4 o0, o1;
    o0.x = (v0[0] * s) / gv;
    o0.y = (v0[1] * s) / gv;
    o0.z = (v1[0] * s) / gv;
    o0.w = (v1[1] * s) / gv;
    o1.x = (v2[0] * s) / gv;
    o1.y = (v2[1] * s) / gv;
    o1.z = (v3[0] * s) / gv;
    o1.w = (v3[1] * s) / gv;
    float4* out = reinterpret_cast<float4*>(w + i * 8);
    out[0] = o0;
    out[1] = o1;
  }
}

}  // namespace w4a16
