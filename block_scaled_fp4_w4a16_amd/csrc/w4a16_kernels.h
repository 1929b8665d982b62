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

#include <type_traits>

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
  // Grid: (row blocks) x (S K-slices).  Row block rb = blockIdx.x owns
  // rq + (rb < rr) rows starting at rb*rq + min(rb, rr); K-slice ks =
  // blockIdx.y covers chunks [ks*CRS, (ks+1)*CRS) of every row (a chunk is
  // 32 inputs).  With S > 1 the workgroup writes fp32 partial sums
  // part[ks][M][N] (fused: gate partials, then up partials at part + S*M*N)
  // instead of y, and the last workgroup of the row block to finish adds
  // them (splitk_finish); cnt[rb] counts the arrivals.
  int rq, rr;
  int S, CRS;
  float* part;
  int* cnt;
  // Segment slots per wave in the LDS area of partial sums (the most tasks
  // one wave's step range can touch; see StreamSplit).
  int kmax;
  // fp32 reciprocals of the launch's divisors (waves per workgroup, chunk
  // steps per task, x units per row), for div_small
  float rW, rCPL, rUPR;
  // argmax epilogue: per-workgroup candidates (value, index bits) [nwg][M],
  // and the results idx[M], val[M]
  float* cand;
  int* amax_idx;
  float* amax_val;
};

// Epilogue of the matmul kernels: y = bf16(x W^T / g); y = bf16(silu(gate)
// * up) from two matrices; or, instead of y, the row index of the largest
// fp32 logit x W^T / g for each activation row (greedy decoding of a head).
constexpr int kEpiPlain = 0, kEpiSwiglu = 1, kEpiArgmax = 2;

#define W4A16_DEV __device__ __forceinline__

// Weight codes and scales are read once per call: non-temporal loads keep
// them from displacing what is reused (x, partials) in the caches (measured:
// M = 1 calls 4-6 % faster, no change at larger M).
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
W4A16_DEV uint4 load_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// floor(x / d) for 0 <= x < 2^23 and d >= 1, given r = fp32(1/d): the float
// quotient is off by at most one, and one correction step makes it exact.
// Integer division proper costs ~25 instructions; the kernels' prologues run
// with a cold instruction cache, so short code there is worth having.
W4A16_DEV int div_small(int x, int d, float r) {
  const int q = (int)((float)x * r);
  const int rem = x - q * d;
  return rem < 0 ? q - 1 : (rem >= d ? q + 1 : q);
}


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

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN (gfx950's
// v_cvt_pk_bf16_f32: one instruction where the bit-level rounding took eight
// and a branch, which matters in the once-per-launch epilogue)
W4A16_DEV uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

W4A16_DEV float silu(float v) { return v / (1.0f + expf(-v)); }

// Word 3 of a gfx9 buffer descriptor for raw (untyped) dword access.
constexpr int kBufferWord3 = 0x00020000;

// Reads the fp32 at g with a vector-memory (buffer) load.  Such a load is
// counted with the weight loads, which complete in order, so it can be issued
// right after the weight prologue without delaying any later scalar-memory or
// LDS wait (a scalar load would).
W4A16_DEV float load_f32_vmem(const float* g) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(g), (short)0, 4, kBufferWord3);
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, 0, 0, 0));
}

// Coherence mode of a matmul body (template argument CO).  The persistent MLP
// kernel's first phase writes h with stores that go through to the device's
// point of coherence (the L2 caches of the eight XCDs are not coherent with
// each other), and its second phase reads h back with loads served from
// there, so that no XCD reads a stale copy.
constexpr int kCoPlain = 0, kCoLoadX = 1, kCoStoreY = 2;
constexpr int kCpolSc1 = 16;  // cache-policy bits of a memory instruction: device scope
constexpr int kCpolNt = 2;    // ... and non-temporal (the weight streams)

// 16 bytes at base[i]; with XC, read at device scope (buffer load, sc1).
// The byte offset i * 16 must stay below 2^31.
template <bool XC>
W4A16_DEV uint4 load_x16(const uint4* base, size_t i) {
  if (!XC) return base[i];
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint4*>(base), (short)0, 0x7fffffff, kBufferWord3);
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(i * 16), 0, kCpolSc1);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// y[i] = v; with YC, an agent-scope store (writes through to the device's
// point of coherence).
template <bool YC>
W4A16_DEV void store_y(uint16_t* y, size_t i, uint16_t v) {
  if (YC) __hip_atomic_store(y + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else y[i] = v;
}

// v + (v of another lane chosen by a DPP control; all lanes stay active)
template <int CTRL>
W4A16_DEV float dpp_add(float v) {
  return v + __builtin_bit_cast(
                 float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// DPP controls (gfx9): quad_perm [1,0,3,2], [2,3,0,1]; row_half_mirror; row_ror:n
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppHalfMirror = 0x141;
constexpr int kDppRor1 = 0x121, kDppRor2 = 0x122, kDppRor4 = 0x124, kDppRor8 = 0x128;

// Sum over each aligned group of `N` consecutive lanes (N = 8 or 16); every
// lane of the group receives the group total.
template <int N>
W4A16_DEV float group_allreduce(float v) {
  if (N == 8) {
    v = dpp_add<kDppQuadXor1>(v);
    v = dpp_add<kDppQuadXor2>(v);
    return dpp_add<kDppHalfMirror>(v);
  }
  v = dpp_add<kDppRor8>(v);
  v = dpp_add<kDppRor4>(v);
  v = dpp_add<kDppRor2>(v);
  return dpp_add<kDppRor1>(v);
}

#ifdef W4A16_TRACE
// Timeline probe for tuning builds: per wave, lane i < 6 stores stamp i
// (s_memrealtime, 100 MHz) to w4a16_trace[(wave id) * 8 + i] with a vector store.
__device__ unsigned long long* w4a16_trace;
#define W4A16_STAMP(var) const unsigned long long var = wall_clock64()
#define W4A16_TRACE_STORE(t0, t1, t2, t3, t4, t5)                                            \
  if (w4a16_trace) {                                                                        \
    const unsigned long long tv[6] = {t0, t1, t2, t3, t4, t5};                              \
    const int ln = threadIdx.x & 63;                                                        \
    unsigned long long mine = 0;                                                            \
    for (int i = 0; i < 6; ++i) mine = ln == i ? tv[i] : mine;                              \
    const size_t wg = (size_t)blockIdx.y * gridDim.x + blockIdx.x;                         \
    if (ln < 6) w4a16_trace[(wg * (blockDim.x >> 6) + (threadIdx.x >> 6)) * 8 + ln] = mine;  \
  }
#else
#define W4A16_STAMP(var) const unsigned long long var = 0
#define W4A16_TRACE_STORE(t0, t1, t2, t3, t4, t5)
#endif

// Orders this wave's LDS writes before its following LDS reads (a wave's LDS
// operations execute in order; this only stops the compiler reordering).
W4A16_DEV void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Keeps v computed at this point (an empty asm that takes and returns it):
// the compiler would otherwise sink 1/g to its uses after the main loop,
// where consuming the g load means waiting for the ring's last refills.
W4A16_DEV float pin(float v) {
  __asm__ volatile("" : "+v"(v));
  return v;
}

// Address read by the MFMA kernel's ring refills past a wave's last step
// (they keep every slot's load count fixed, so each wait stays exact; nothing
// reads their data): 16 bytes of the first row of x (K/8 units), unit `tid` modulo the
// largest power of two that fits, so the workgroup spreads them over up to
// 8 KiB of lines it has just staged and that are served from cache.  A phase
// that reads x coherently (x is written by the same launch) reads the first
// weight row (K/32 units) instead, which no launch writes.
template <bool XC>
W4A16_DEV const uint4* past_line(const MatArgs& a, int tid) {
  const int units = XC ? a.K >> 5 : a.K >> 3;             // >= 8, a multiple of 8
  const int mask = (1 << (31 - __builtin_clz(units))) - 1;  // largest power of two <= units, minus 1
  const uint4* base = XC ? reinterpret_cast<const uint4*>(a.wq0) : reinterpret_cast<const uint4*>(a.x);
  return base + (tid & mask);
}

// Workgroup barrier for data in LDS only: each wave waits for its own LDS
// operations, not for its global loads.  After the MFMA kernel's main loop
// its load ring still holds refills issued past the last step (past_line);
// nothing reads them, so the combine does not wait for them.  (Measured on
// the VALU kernel the same changes gained nothing: there the combine's cost
// is its own cold code path, and a g load moved ahead of x delayed the
// prologue, so that kernel keeps re-reading its last step.)
W4A16_DEV void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Position of 16-byte unit q (0..3) of x-chunk c inside an LDS x row for the
// VALU kernel.  Lanes read consecutive chunks; the XOR spreads the four units
// of neighbouring chunks over distinct bank groups (for 8- and 16-lane passes).
W4A16_DEV int xsw(int c, int q) { return 4 * c + (q ^ (((c >> 1) ^ (c >> 2)) & 3)); }

// Stage `rows` rows of x (K bf16 each; rows >= M are zero) into LDS units
// xs[m*RSU + pos(cu)].  The slice is `upr` 16-byte units per row starting at
// unit u0 of each x row (a row of x has K/8 units); unit u of the staged
// block is (row u / upr, column u % upr), and thread tid handles units tid,
// tid + nthr, ...  Phase 1 loads the first XMAX units per thread into
// registers *before* the caller issues its weight prologue, so that storing
// them (phase 2) waits only for x, since loads complete in order; units
// beyond XMAX per thread (only for very wide x) are staged after the
// prologue.  The code is straight-line: it runs at the start of every
// launch, when the instruction cache is cold, so it has no loops and only
// wave-uniform guards and short lane-masked loads.
struct XUnits {
  int total, upr;
  float rinv;  // fp32(1/upr)
  W4A16_DEV XUnits(int rows, int upr_, float rinv_) : total(rows * upr_), upr(upr_), rinv(rinv_) {}
  // (row, column) of unit u
  W4A16_DEV void split(int u, int& m, int& cu) const {
    m = div_small(u, upr, rinv);
    cu = u - m * upr;
  }
};
template <bool XC, int XMAX>
W4A16_DEV void x_stage_issue(uint4 (&xr)[XMAX], const uint16_t* x, int M, int rows, int K,
                             int u0, int upr, float rupr, int tid, int nthr) {
  const uint4* xg = reinterpret_cast<const uint4*>(x);
  const XUnits xu(rows, upr, rupr);
#pragma unroll
  for (int i = 0; i < XMAX; ++i) {
    xr[i] = make_uint4(0u, 0u, 0u, 0u);
    if (i * nthr < xu.total) {          // wave-uniform
      const int u = tid + i * nthr;
      int m, cu;
      xu.split(u, m, cu);
      if (u < xu.total && m < M) xr[i] = load_x16<XC>(xg, (size_t)m * (K >> 3) + u0 + cu);
    }
  }
}
template <bool XC, int XMAX, typename Pos>
W4A16_DEV void x_stage_store(uint4* xs, const uint4 (&xr)[XMAX], const uint16_t* x, int M,
                             int rows, int K, int u0, int upr, float rupr, int RSU, int tid,
                             int nthr, Pos pos) {
  const uint4* xg = reinterpret_cast<const uint4*>(x);
  const XUnits xu(rows, upr, rupr);
#pragma unroll
  for (int i = 0; i < XMAX; ++i) {
    if (i * nthr < xu.total) {
      const int u = tid + i * nthr;
      int m, cu;
      xu.split(u, m, cu);
      if (u < xu.total) xs[m * RSU + pos(cu)] = xr[i];
    }
  }
  for (int u = tid + XMAX * nthr; u < xu.total; u += nthr) {
    int m, cu;
    xu.split(u, m, cu);
    xs[m * RSU + pos(cu)] =
        m < M ? load_x16<XC>(xg, (size_t)m * (K >> 3) + u0 + cu) : make_uint4(0u, 0u, 0u, 0u);
  }
}

// ---------------------------------------------------------------------------
// Split-K completion inside the matmul kernel (no second launch).  Every
// workgroup (rb, ks) stores its fp32 partials part[ks][m][row] for the rows
// [row_lo, row_lo + nrows) of its row block with agent-scope stores, which
// write through to the device's point of coherence (the L2 of each XCD is
// not coherent with the others'), waits until they have completed, and then
// thread 0 adds one to cnt[rb] with a relaxed agent-scope atomic.  The
// workgroup that sees S - 1 arrivals before its own is the last one: it
// reads every slice's partials with agent-scope loads, adds them in slice
// order 0..S-1 (a fixed order, so results do not depend on which slice
// finished last), writes y, and sets cnt[rb] back to zero for the next call.
// Each counter sees S atomics per call, no cache-wide write-back or
// invalidation is needed, and nothing ever waits for another workgroup.
// ---------------------------------------------------------------------------
W4A16_DEV void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
W4A16_DEV float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// p[0] + p[st] + ... + p[(S-1) st], added in that order; the loads of eight
// slices are issued before the first of them is used (the partials live
// beyond the XCD caches, so each load costs a far round trip).
W4A16_DEV float splitk_sum(const float* p, size_t st, int S) {
  float v = 0.0f;
  int s = 0;
  for (; s + 8 <= S; s += 8) {
    float t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = load_coherent(p + (size_t)(s + j) * st);
#pragma unroll
    for (int j = 0; j < 8; ++j) v += t[j];
  }
  if (s + 4 <= S) {
    float t[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) t[j] = load_coherent(p + (size_t)(s + j) * st);
#pragma unroll
    for (int j = 0; j < 4; ++j) v += t[j];
    s += 4;
  }
  for (; s < S; ++s) v += load_coherent(p + (size_t)s * st);
  return v;
}

// Index of an argmax candidate that has seen no row yet.
constexpr int kNoIndex = 0x7fffffff;

// Counter of the argmax epilogue's final reduction when the call is split
// along K (the row blocks' split-K counters take cnt[0 .. nrb-1], nrb < this).
constexpr int kArgmaxSplitCounter = 1023;

template <int MB>
W4A16_DEV void argmax_finish(const MatArgs& a, int* cnt, int nwg, float* red, int W);
template <int MB>
W4A16_DEV void wg_argmax_rows(float (&v)[MB], int (&ix)[MB], int M, float* red, int W);
W4A16_DEV void argmax_take(float& bv, int& bi, float v, int i);

// EPI == kEpiArgmax: the finishing workgroup of each row block turns its
// rows' summed logits into one (value, index) candidate per activation row
// (MB >= M rows, side by side), stores them, and the last row block to do so
// reduces every row block's candidates (argmax_finish).  red: LDS scratch of
// 2 * MB floats per wave; W: waves per workgroup; nrb: row blocks.
template <bool FUSED, bool YC, int EPI = kEpiPlain, int MB = 1>
W4A16_DEV void splitk_finish(const MatArgs& a, int rb, int row_lo, int nrows, float ig0,
                             float ig1, float* red = nullptr, int W = 0, int nrb = 0) {
  __shared__ int is_last;
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores have completed
  __syncthreads();                // ... and so have every other wave's
  if (threadIdx.x == 0) {
    const int before = __hip_atomic_fetch_add(a.cnt + rb, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = before == a.S - 1;
    if (is_last) __hip_atomic_store(a.cnt + rb, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (EPI == kEpiArgmax) {
    // only each row block's finishing workgroup arrives at the final
    // reduction's counter (nrb arrivals in all)
    if (!is_last) return;
    const size_t MN = (size_t)a.M * a.N;
    const int M = a.M;
    float bv[MB];
    int bi[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      bv[m] = -__builtin_inff();
      bi[m] = kNoIndex;
    }
    for (int n = threadIdx.x; n < nrows; n += blockDim.x) {
#pragma unroll
      for (int m = 0; m < MB; ++m)
        if (m < M) {
          const size_t i = (size_t)m * a.N + row_lo + n;
          argmax_take(bv[m], bi[m], splitk_sum(a.part + i, MN, a.S) * ig0, row_lo + n);
        }
    }
    wg_argmax_rows<MB>(bv, bi, M, red, W);
    if ((int)threadIdx.x < M) {
      float* c = a.cand + ((size_t)rb * M + threadIdx.x) * 2;
      store_coherent(c, bv[0]);
      store_coherent(c + 1, __int_as_float(bi[0]));
    }
    argmax_finish<MB>(a, a.cnt + kArgmaxSplitCounter, nrb, red, W);
    return;
  }
  if (!is_last) return;
  const size_t MN = (size_t)a.M * a.N;
  for (int o = threadIdx.x; o < nrows * a.M; o += blockDim.x) {
    const int m = o / nrows, n = o - m * nrows;   // consecutive threads: consecutive rows
    const size_t i = (size_t)m * a.N + row_lo + n;
    const float v = splitk_sum(a.part + i, MN, a.S);
    if (FUSED) {
      const float u = splitk_sum(a.part + (size_t)a.S * MN + i, MN, a.S);
      store_y<YC>(a.y, i, f32_to_bf16(silu(v * ig0) * (u * ig1)));
    } else {
      store_y<YC>(a.y, i, f32_to_bf16(v * ig0));
    }
  }
}

// ---------------------------------------------------------------------------
// Argmax epilogue.  Order: larger value first, then the smaller row index, so
// the result does not depend on the order in which candidates meet; a NaN
// logit never wins (comparisons with NaN are false); if every logit of a row
// is NaN the index is -1.  Each workgroup reduces its rows to one candidate
// per activation row m and stores it with agent-scope stores; the last
// workgroup to finish (arrival counter cnt[0], zeroed again by that
// workgroup) reduces the candidates of all workgroups.
// ---------------------------------------------------------------------------
W4A16_DEV void argmax_take(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

// Workgroup-wide argmax of up to MB activation rows at once: every thread
// brings one candidate (v[m], ix[m]) per row m; afterwards thread m (m < M)
// holds row m's winner in v[0], ix[0].  The rows are reduced side by side
// (their wave-level exchanges are independent), with one pass through LDS
// for all of them.  red: LDS scratch of 2 * MB words per wave.
template <int MB>
W4A16_DEV void wg_argmax_rows(float (&v)[MB], int (&ix)[MB], int M, float* red, int W) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const float ov = __shfl_xor(v[m], off);
      const int oi = __shfl_xor(ix[m], off);
      argmax_take(v[m], ix[m], ov, oi);
    }
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      red[(w * MB + m) * 2] = v[m];
      red[(w * MB + m) * 2 + 1] = __int_as_float(ix[m]);
    }
  }
  __syncthreads();
  const int t = threadIdx.x;
  float bv = -__builtin_inff();
  int bi = kNoIndex;
  if (t < M)
    for (int k = 0; k < W; ++k)
      argmax_take(bv, bi, red[(k * MB + t) * 2], __float_as_int(red[(k * MB + t) * 2 + 1]));
  __syncthreads();  // red is free again
  v[0] = bv;
  ix[0] = bi;
}

// Called by every thread once the workgroup's candidates cand[rb][m] are
// stored: the last workgroup reduces all of them into idx[m], val[m].  Each
// thread issues the loads of all its candidates' rows before using any of
// them (they come from beyond the XCD caches: one round trip, not one per row).
template <int MB>
W4A16_DEV void argmax_finish(const MatArgs& a, int* cnt, int nwg, float* red, int W) {
  __shared__ int is_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int before = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = before == nwg - 1;
    if (is_last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!is_last) return;
  const int M = a.M;
  float bv[MB];
  int bi[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    bv[m] = -__builtin_inff();
    bi[m] = kNoIndex;
  }
  for (int b = threadIdx.x; b < nwg; b += W * 64) {
    const float* c = a.cand + (size_t)b * M * 2;
    float cv[MB];
    int ci[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      cv[m] = -__builtin_inff();
      ci[m] = kNoIndex;
      if (m < M) {
        cv[m] = load_coherent(c + 2 * m);
        ci[m] = __float_as_int(load_coherent(c + 2 * m + 1));
      }
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) argmax_take(bv[m], bi[m], cv[m], ci[m]);
  }
  wg_argmax_rows<MB>(bv, bi, M, red, W);
  if ((int)threadIdx.x < M) {
    a.amax_idx[threadIdx.x] = bi[0] == kNoIndex ? -1 : bi[0];
    a.amax_val[threadIdx.x] = bv[0];
  }
}

// ---------------------------------------------------------------------------
// Work split inside a workgroup (both matmul kernels).  The workgroup's rows
// form ntasks tasks (row groups); a task is CPL chunk steps along K, so the
// workgroup has TS = ntasks * CPL steps, step s = task * CPL + jj.  Wave w
// executes the contiguous steps [begin(w), begin(w + 1)), begin(w) =
// floor(w * TS / W): every wave gets the same number of steps to within one,
// whatever the row count.  A wave sums each task it touches into a segment
// partial, which it parks in LDS slot (w, task - first task of w), and notes
// in LDS which wave starts (tw0) and which finishes (tw1) each task, and each
// wave's first task (wft; a large value for a wave without steps).  After one
// barrier the workgroup adds, for every task, the segments of waves tw0..tw1
// in wave order (so results are reproducible bit for bit).
// ---------------------------------------------------------------------------
struct StreamSplit {
  int TS, W;
  float rW;
  W4A16_DEV int begin(int w) const { return div_small(w * TS, W, rW); }
};
constexpr int kNoTask = 1 << 30;

// ---------------------------------------------------------------------------
// VALU kernel, M = MT in {1, 2} (the launch rules send M >= 3 to the MFMA
// kernel; the body itself takes any small MT).
//
// Lane layout: a wave holds G = 64/L row slots of L lanes; at step (task, jj)
// lane (slot r, position p) reads chunk p + L*jj of row r of the task, so the
// L lanes of a row read L*16 contiguous bytes per load.  A task is one row
// group (G rows; for the fused variant G/2 gate rows plus the same G/2 up
// rows) and takes CPL = CRS/L steps; the workgroup has TS = ntasks*CPL steps,
// step s = task*CPL + jj.
//
// Scheduling: steps are handed out in batches of D consecutive steps.  Wave w
// starts with batch w (steps wD .. wD+D-1, so its loads can be issued before
// the x barrier); afterwards each wave takes the next batch from a workgroup
// counter in LDS (one LDS atomic per batch), so a wave whose loads return
// late takes fewer batches and the waves of a workgroup finish together.
// Each lane keeps D chunk loads in flight in a register ring: slot d holds
// step d of the current batch and is refilled with step d of the next batch
// as soon as it has been consumed.
//
// Per step and activation row: 16 bf16x2 dot products per 32 weights into
// two block partials, times their e4m3 scales; the L lanes of a row are
// summed with DPP (groups of up to 16 lanes) and the group totals are parked
// in LDS at part[step][slot][group][m].  After one barrier every output row
// adds its task's step partials in step order and group order: a fixed
// order, so results do not depend on which wave ran which step.  x rows live
// in LDS (swizzled) and are read with 128-bit LDS loads; lanes of different
// slots read the same x (broadcast).
// ---------------------------------------------------------------------------
template <int MT, int L, int D, int EPI, int LB, int CO>
W4A16_DEV void gemm_valu(const MatArgs& a, int rb, int ks, int nwg) {
  constexpr bool FUSED = EPI == kEpiSwiglu;
  constexpr bool XC = (CO & kCoLoadX) != 0, YC = (CO & kCoStoreY) != 0;
  W4A16_STAMP(t_start);
  extern __shared__ uint4 xs[];
  constexpr int G = 64 / L;
  constexpr int RT = FUSED ? G / 2 : G;   // output rows per task
  constexpr int GL = L < 16 ? L : 16;     // lanes summed by DPP
  constexpr int NSEG = L / GL;            // DPP groups per row slot
  constexpr int V = G * NSEG * MT;        // values in a step partial: [slot][group][m]
  const int W = blockDim.x >> 6, NT = blockDim.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = a.K, S = a.S, CRS = a.CRS;  // CRS: chunks per row in this K-slice
  const int c0 = ks * CRS;               // first chunk of the slice
  const int CPL = CRS / L, RSU = (CRS << 2) + 1;
  const int row_lo = rb * a.rq + (rb < a.rr ? rb : a.rr);
  const int row_hi = row_lo + a.rq + (rb < a.rr ? 1 : 0);
  const int ntasks = (row_hi - row_lo + RT - 1) / RT;
  const int TS = ntasks * CPL;
  const int p = lane % L, r = lane / L;
  const int srow = FUSED ? (r % (G / 2)) : r;
  const bool is_up = FUSED && (r >= G / 2);
  const uint8_t* wq = is_up ? a.wq1 : a.wq0;
  const uint8_t* ws = is_up ? a.ws1 : a.ws0;
  float* part = reinterpret_cast<float*>(xs + MT * RSU);  // [TS][V]
  int* next_batch = reinterpret_cast<int*>(part + (size_t)TS * V);

  // ---- issue cursor: step (task it_i, jj_i) -> row pointers ---------------
  const uint4* qp;
  const uint16_t* sp;
  int it_i, jj_i;
  auto set_task = [&](int it) {
    int row = row_lo + it * RT + srow;
    row = row < row_hi ? row : row_hi - 1;
    qp = reinterpret_cast<const uint4*>(wq + (size_t)row * (size_t)(K >> 1)) + c0 + p;
    sp = reinterpret_cast<const uint16_t*>(ws + (size_t)row * (size_t)(K >> 4)) + c0 + p;
  };
  // position the cursor at step s (steps past the end load the last step;
  // their data is never used, and they keep every slot's load count fixed so
  // that each wait stays exact)
  auto seek = [&](int s) {
    s = s < TS ? s : TS - 1;
    it_i = div_small(s, CPL, a.rCPL);
    jj_i = s - it_i * CPL;
    set_task(it_i);
  };
  uint4 qb[D];
  uint32_t sb[D];
  // load the cursor's step into slot d, then advance (stopping at the last step)
  auto issue = [&](int d) {
    qb[d] = load_stream(qp + L * jj_i);
    sb[d] = __builtin_nontemporal_load(sp + L * jj_i);
    if (it_i * CPL + jj_i + 1 < TS && ++jj_i == CPL) {
      jj_i = 0;
      ++it_i;
      set_task(it_i);
    }
  };
  // x -> LDS (rows of K bf16 in 16-byte units, swizzled): ring slot 0 of the
  // first batch, the x loads, the rest of the first batch, then the LDS
  // stores (loads complete in order, so the stores wait for slot 0 and x only)
  constexpr int XMAX = LB > 512 ? 8 : 16;
  uint4 xr[XMAX];
  auto xpos = [](int cu) { return xsw(cu >> 2, cu & 3); };
  int base = wv * D;  // first step of this wave's current batch
  seek(base);
  issue(0);
  x_stage_issue<XC>(xr, a.x, a.M, MT, K, c0 << 2, CRS << 2, a.rUPR, tid, NT);
#pragma unroll
  for (int d = 1; d < D; ++d) issue(d);
  W4A16_STAMP(t_issued);
  const float gv0 = load_f32_vmem(a.g0);
  const float gv1 = FUSED ? load_f32_vmem(a.g1) : 1.0f;
  if (tid == 0) *next_batch = W * D;
  x_stage_store<XC>(xs, xr, a.x, a.M, MT, K, c0 << 2, CRS << 2, a.rUPR, RSU, tid, NT, xpos);
  __syncthreads();
  W4A16_STAMP(t_barrier);
#ifdef W4A16_TRACE
  unsigned long long t_first = 0;
#endif

  while (base < TS) {
    // the next batch: one LDS atomic by lane 0, broadcast to the wave
    int nxt_lane0 = 0;  // read back only after the first step (see below)
    if (lane == 0)
      nxt_lane0 = __hip_atomic_fetch_add(next_batch, D, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    int nxt = 0;
    // compute cursor of the current batch; a run is the batch's steps of one
    // task: its sum stays in registers and is reduced and parked once, in
    // the slot of its first step
    int jj_c = base - div_small(base, CPL, a.rCPL) * CPL;
    int run0 = base;
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      // consume slot d completely, then refill it with step d of the next batch
      const int s = base + d;
      if (s < TS) {
        const uint4 q = qb[d];
        const uint32_t sc = sb[d];
        const int c = p + L * jj_c;
        uint4 xv[MT][4];
        if (L >= 16) {
          // c and p agree in bits 0..3, so the swizzle term is fixed per lane
          const int hp = ((p >> 1) ^ (p >> 2)) & 3;
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int u = 0; u < 4; ++u) xv[m][u] = xs[m * RSU + 4 * c + (u ^ hp)];
        } else {
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int u = 0; u < 4; ++u) xv[m][u] = xs[m * RSU + xsw(c, u)];
        }
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
        for (int m = 0; m < MT; ++m) acc[m] = fmaf(blo[m], s_lo, fmaf(bhi[m], s_hi, acc[m]));
#ifdef W4A16_TRACE
        if (t_first == 0) t_first = wall_clock64();
#endif
        const bool task_end = ++jj_c == CPL;
        if (task_end || d == D - 1 || s + 1 == TS) {
          float* ps = part + (size_t)run0 * V + (r * NSEG + p / GL) * MT;
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const float v = group_allreduce<GL>(acc[m]);
            if ((p % GL) == 0) ps[m] = v;
            acc[m] = 0.0f;
          }
          run0 = s + 1;
        }
        if (task_end) jj_c = 0;
      }
      // the issue cursor moves to the next batch only here, so that the
      // batch counter's latency hides behind the first step's work
      if (d == 0) {
        nxt = __builtin_amdgcn_readfirstlane(nxt_lane0);
        seek(nxt);
      }
      issue(d);
    }
    base = nxt;
  }
  W4A16_STAMP(t_end);

  // ---- workgroup combine: output (row n, m) = its task's step partials ----
  __syncthreads();
  const float ig0 = 1.0f / gv0;
  const float ig1 = FUSED ? 1.0f / gv1 : 1.0f;
  const int nrows = row_hi - row_lo;
  // sum of slot `slot`'s values for activation row m over the task's runs
  // (a run starts at the task's first step and at every batch start), in
  // step order
  auto row_sum = [&](int t, int slot, int m) {
    float v = 0.0f;
    const int s0 = t * CPL;
    const float* pt = part + slot * NSEG * MT + m;
    int s = s0;
    while (s < s0 + CPL) {
#pragma unroll
      for (int g = 0; g < NSEG; ++g) v += pt[(size_t)s * V + g * MT];
      s = (s / D + 1) * D;  // the next batch start (D is a power of two here)
    }
    return v;
  };
  if (EPI == kEpiArgmax) {
    // S == 1 here (the host rejects a K split with this epilogue); x is no
    // longer needed, so its LDS holds the reduction scratch
    float* red = reinterpret_cast<float*>(xs);
    float bv[MT];
    int bi[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      bv[m] = -__builtin_inff();
      bi[m] = kNoIndex;
    }
    for (int n = tid; n < nrows; n += NT) {
      const int t = n / RT, rt = n - t * RT;
#pragma unroll
      for (int m = 0; m < MT; ++m) argmax_take(bv[m], bi[m], row_sum(t, rt, m) * ig0, row_lo + n);
    }
    wg_argmax_rows<MT>(bv, bi, MT, red, W);
    if (tid < MT) {
      float* c = a.cand + ((size_t)rb * a.M + tid) * 2;
      store_coherent(c, bv[0]);
      store_coherent(c + 1, __int_as_float(bi[0]));
    }
    argmax_finish<MT>(a, a.cnt, nwg, red, W);
  } else
  for (int n = tid; n < nrows; n += NT) {
    const int t = n / RT, rt = n - t * RT;
    const int row = row_lo + n;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float v = row_sum(t, rt, m);
      const float u = FUSED ? row_sum(t, rt + G / 2, m) : 0.0f;
      if (S > 1) {
        store_coherent(a.part + ((size_t)ks * a.M + m) * a.N + row, v);
        if (FUSED) store_coherent(a.part + ((size_t)(S + ks) * a.M + m) * a.N + row, u);
      } else if (FUSED) {
        store_y<YC>(a.y, (size_t)m * a.N + row, f32_to_bf16(silu(v * ig0) * (u * ig1)));
      } else {
        store_y<YC>(a.y, (size_t)m * a.N + row, f32_to_bf16(v * ig0));
      }
    }
  }
  if (S > 1) splitk_finish<FUSED, YC>(a, rb, row_lo, row_hi - row_lo, ig0, ig1);
#ifdef W4A16_TRACE
  W4A16_STAMP(t_done);
  W4A16_TRACE_STORE(t_start, t_issued, t_barrier, t_first, t_end, t_done);
#endif
}

// One matmul per launch: workgroup (rb, ks) = (blockIdx.x, blockIdx.y).
template <int MT, int L, int D, int EPI, int LB>
__global__ void __launch_bounds__(LB) k_gemm_valu(MatArgs a) {
  gemm_valu<MT, L, D, EPI, LB, kCoPlain>(a, blockIdx.x, blockIdx.y, gridDim.x);
}

// ---------------------------------------------------------------------------
// Whole-row VALU kernel: M = MT in {1, 2}, K = 1024 * CPL fixed at compile
// time, no K split; plain and gate/up + SwiGLU epilogues.  Launch bound 640
// threads for short rows at M = 1, else 512 (two tasks of CPL loads per lane
// in registers).
//
// A task is two weight rows (fused: a gate row and the same up row): lanes
// 0-31 take the first, lanes 32-63 the second, and at step jj lane p reads
// chunk p + 32*jj of its row (512 contiguous bytes per row per load) and the
// dword of scales that holds the chunk's pair.  Wave w takes tasks w, w + W,
// w + 2W, ... of its row block and holds two in registers: the loads of the
// next task are issued before the current one is computed.  Each task is
// summed in registers over its CPL steps, reduced across its 32 lanes with
// DPP, and written by the wave itself: no LDS partials, no workgroup combine,
// no batch counter.  With K a compile-time constant every per-step address
// is an immediate offset from a per-lane base, for the global loads and the
// LDS reads alike.
//
// Prologue: the x loads, then the first task's weight loads, then the LDS
// stores of x (which wait for x only: loads complete in order), so x's
// latency hides behind the weights'.  A wave's tasks past its last one load
// the first bytes of x instead (cached, never used), so that every load is
// unconditional and the compiler's wait counts stay exact.
//
// Measured with HIP-graph replay on MI355X (weights cycled through 32-64
// copies): square 5120 x 5120 at M = 1 4.82 us against 5.36 us for the
// general VALU kernel; gate/up 2 x 17408 x 5120 17.6 against 18.0 us.
// ---------------------------------------------------------------------------
template <int MT, int CPL, int EPI>
__global__ void __launch_bounds__((MT == 1 && CPL <= 8) ? 640 : 512) k_gemm_rows(MatArgs a) {
  static_assert(EPI != kEpiArgmax, "plain and SwiGLU epilogues only");
  W4A16_STAMP(t_start);
  constexpr bool FUSED = EPI == kEpiSwiglu;
  constexpr int L = 32;                    // lanes per weight row
  constexpr int RT = FUSED ? 1 : 2;        // output rows per task
  constexpr int K = CPL * 1024, CR = K >> 5, RSU = 4 * CR + 1;
  constexpr int XU = MT * CR * 4;          // 16-byte units of x
  constexpr int XMAX = (XU + 255) / 256;   // per thread, for blocks of >= 256 threads
  extern __shared__ uint4 xs[];
  const int W = blockDim.x >> 6, NT = blockDim.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rb = blockIdx.x;
  const int row_lo = rb * a.rq + (rb < a.rr ? rb : a.rr);
  const int row_hi = row_lo + a.rq + (rb < a.rr ? 1 : 0);
  const int ntasks = (row_hi - row_lo + RT - 1) / RT;
  const int p = lane & 31, r = lane >> 5;
  const uint8_t* wq = (FUSED && r) ? a.wq1 : a.wq0;
  const uint8_t* ws = (FUSED && r) ? a.ws1 : a.ws0;
  const uint8_t* xbase = reinterpret_cast<const uint8_t*>(a.x);

  // x rows (contiguous, K bf16 each) into registers
  uint4 xr[XMAX];
  {
    const uint4* xg = reinterpret_cast<const uint4*>(a.x);
#pragma unroll
    for (int i = 0; i < XMAX; ++i) {
      const int u = tid + i * NT;
      xr[i] = make_uint4(0u, 0u, 0u, 0u);
      if (u < XU) xr[i] = xg[u];
    }
  }

  // LDS x: unit q of chunk c of row m at m*RSU + xsw(c, q).  For this lane's
  // chunks c = p + 32*jj the swizzle term depends on p only.
  const int hp = ((p >> 1) ^ (p >> 2)) & 3;
  int xb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) xb[q] = 4 * p + (q ^ hp);
  const int shp = (p & 1) * 16;            // this lane's scale pair within its dword
  float ig0 = 1.0f, ig1 = 1.0f;

  uint4 qa[CPL], qb[CPL];
  uint32_t sa[CPL], sb[CPL];
  auto load_task = [&](uint4 (&q)[CPL], uint32_t (&sc)[CPL], int t) {
    if constexpr (!FUSED) {
      // both rows of the task through one buffer resource each for codes and
      // scales; a task past the wave's last one gets 0 records, so its loads
      // return zeros without touching memory
      const int row0 = row_lo + t * RT;
      const int live = t < ntasks ? (row_hi - row0 < 2 ? row_hi - row0 : 2) : 0;
      const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(wq) + (size_t)(live ? row0 : 0) * (K >> 1), (short)0,
          live * (K >> 1), kBufferWord3);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(ws) + (size_t)(live ? row0 : 0) * (K >> 4), (short)0,
          live * (K >> 4), kBufferWord3);
      const int qo = r * (K >> 1) + p * 16, so = r * (K >> 4) + (p >> 1) * 4;
#pragma unroll
      for (int jj = 0; jj < CPL; ++jj) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rq, qo + 16 * L * jj, 0, kCpolNt);
        q[jj] = make_uint4(v.x, v.y, v.z, v.w);
        sc[jj] = __builtin_amdgcn_raw_buffer_load_b32(rs, so + 2 * L * jj, 0, kCpolNt);
      }
    } else {
      int row = row_lo + t * RT;
      row = row < row_hi ? row : row_hi - 1;
      const bool live = t < ntasks;
      const uint8_t* qr = live ? wq + (size_t)row * (K >> 1) : xbase;
      const uint8_t* sr = live ? ws + (size_t)row * (K >> 4) : xbase;
      const uint4* qp = reinterpret_cast<const uint4*>(qr) + p;
      const uint32_t* sp = reinterpret_cast<const uint32_t*>(sr) + (p >> 1);
#pragma unroll
      for (int jj = 0; jj < CPL; ++jj) {
        q[jj] = load_stream(qp + L * jj);
        sc[jj] = __builtin_nontemporal_load(sp + (L / 2) * jj);
      }
    }
  };
  auto compute = [&](const uint4 (&q)[CPL], const uint32_t (&sc)[CPL], int t) {
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
#pragma unroll
    for (int jj = 0; jj < CPL; ++jj) {
      uint4 xv[MT][4];
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int u = 0; u < 4; ++u) xv[m][u] = xs[xb[u] + m * RSU + 4 * L * jj];
      const uint32_t pair = sc[jj] >> shp;
      const float s_lo = e4m3_to_f32<0>(pair), s_hi = e4m3_to_f32<1>(pair);
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
      W4A16_DOT_WORD(q[jj].x, 0, blo)
      W4A16_DOT_WORD(q[jj].y, 1, blo)
      W4A16_DOT_WORD(q[jj].z, 2, bhi)
      W4A16_DOT_WORD(q[jj].w, 3, bhi)
#undef W4A16_DOT_WORD
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] = fmaf(blo[m], s_lo, fmaf(bhi[m], s_hi, acc[m]));
      // two rows of x per step would otherwise be read for every step at once
      if (MT > 1) __builtin_amdgcn_sched_barrier(0);
    }
    const int row = row_lo + t * RT + (FUSED ? 0 : r);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = group_allreduce<16>(acc[m]);
      v += __shfl_xor(v, 16);                // the row's 32 lanes
      if (FUSED) {
        const float u = __shfl_xor(v, 32);   // the up row's total
        if (lane == 0 && row < row_hi)
          a.y[(size_t)m * a.N + row] = f32_to_bf16(silu(v * ig0) * (u * ig1));
      } else if (p == 0 && row < row_hi) {
        a.y[(size_t)m * a.N + row] = f32_to_bf16(v * ig0);
      }
    }
  };

  int t = wv;
  load_task(qa, sa, t);
#pragma unroll
  for (int i = 0; i < XMAX; ++i) {
    const int u = tid + i * NT;
    if (u < XU) {
      const int m = u / (CR * 4), cu = u - m * (CR * 4);
      xs[m * RSU + xsw(cu >> 2, cu & 3)] = xr[i];
    }
  }
  {
    // g through the scalar cache (constant address space): its wait is the
    // barrier's LDS wait, not a wait for the weight loads
    typedef const __attribute__((address_space(4))) float cfloat;
    ig0 = 1.0f / *reinterpret_cast<cfloat*>(reinterpret_cast<uintptr_t>(a.g0));
    if (FUSED) ig1 = 1.0f / *reinterpret_cast<cfloat*>(reinterpret_cast<uintptr_t>(a.g1));
  }
  W4A16_STAMP(t_issued);
  // workgroup barrier for the LDS stores only (the weight loads stay in flight)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  W4A16_STAMP(t_barrier);
#ifdef W4A16_TRACE
  unsigned long long t_first = 0;
#endif
  // Two tasks per iteration and one exit test.  An exit between the two
  // halves would merge the state "next task's loads pending" into the loop
  // head, where the compiler then waits for every load before issuing the
  // next task's; skipping the second half's arithmetic instead leaves only
  // the (already finished) loads of that half pending there.  The
  // scheduling barriers keep each task's loads ahead of the previous task's
  // arithmetic.
  while (t < ntasks) {
    load_task(qb, sb, t + W);
    __builtin_amdgcn_sched_barrier(0);
    compute(qa, sa, t);
#ifdef W4A16_TRACE
    if (t_first == 0) t_first = wall_clock64();
#endif
    load_task(qa, sa, t + 2 * W);
    __builtin_amdgcn_sched_barrier(0);
    if (t + W < ntasks) compute(qb, sb, t + W);
    t += 2 * W;
  }
#ifdef W4A16_TRACE
  W4A16_STAMP(t_end);
  W4A16_TRACE_STORE(t_start, t_issued, t_barrier, t_first, t_end, t_end);
#endif
}

// ---------------------------------------------------------------------------
// K-column MFMA kernel with x in registers, 3 <= M <= 8, K = 1024 * CPL
// (CPL = 5: the hidden size of the square projections and of gate/up; CPL =
// 17: the down projection's input, in S = 2 K-slices).
//
// The 4x4x4 block product of the MFMA kernel below (block beta = one chunk
// column, its 4 columns = 4 weight rows, its 4 rows = activation rows; P
// passes of 4 activation rows), with the work split over K instead of rows:
// the 2 CPL columns of 16 chunks are shared out one or two to a wave (W
// waves: 2 CPL / 2 of two columns each, or more waves of which the first
// 2 CPL - W own two and the rest one) and every wave walks every row quad of
// the workgroup's row block.  A wave therefore holds its slice of x (its
// columns of M rows) in VGPRs for the whole call, loaded once from memory:
// no per-step LDS reads of x (the MFMA kernel reads 8 bytes of x from LDS
// per weight byte at M = 7).  What crosses waves is one partial sum per
// (quad, weight row, activation row, wave, 16-lane row): the quad's 16 blocks
// are summed in registers (DPP within 16-lane rows) and parked in LDS, and
// after the loop each output adds its 4 W partials in a fixed order.  Fused:
// quad 2i holds gate rows 4i..4i+3, quad 2i+1 the same up rows.  A task is
// two quads; two tasks are in registers, the next one's loads issued before
// the current one is computed (the whole-row kernel's loop).  With S > 1 K-
// slices, workgroup (rb, ks) covers columns ks JT .. ks JT + JT - 1 of row
// block rb and parks its sums in the split-K partials; the row block's last
// workgroup adds the slices in order (splitk_finish).  The ring variant
// (RING) adds the partials every few loop iterations instead of after the
// loop, so that a row block of any size fits the LDS; it also serves the
// argmax epilogue (each thread keeps the best logit it adds, then the
// workgroup's and the grid's candidates are reduced).
// Measured on MI355X (HIP-graph replay, 64 / 32 cycled copies): 5120 x 5120
// at M = 7 in 6.3 us with 6 waves (6.6 with 5, 6.7 with 8) against 7.99 for
// the MFMA kernel; gate/up 2 x 17408 x 5120 at M = 7 in 21.0-21.6 us with 8
// waves (22.5 with 5) against 23.9.
// ---------------------------------------------------------------------------
// Loop iterations (of two tasks) per combine in the ring variant below.
// Measured on the 248 320 x 5120 head (graph replay): M = 5 / 7 / 8 128.2 /
// 136.3 / 137.0 us at 1, 122.7 / 127.1 / 130.0 at 2, 123.3 / 128.5 / 136.5
// at 4, against 139.7 / 143.1 / 144.0 for the MFMA kernel.
constexpr int kXrRingIterations = 2;
template <int M, int CPL, int EPI, int W, int S, bool RING>
__global__ void __launch_bounds__(64 * W) k_gemm_xr(MatArgs a) {
  constexpr bool FUSED = EPI == kEpiSwiglu;
  constexpr bool ARGMAX = EPI == kEpiArgmax;
  static_assert(!ARGMAX || (RING && S == 1), "the argmax epilogue runs on the ring variant");
  static_assert(!RING || S == 1, "the ring variant does not split K");
  constexpr int P = (M + 3) / 4;
  constexpr int K = 1024 * CPL;
  static_assert((2 * CPL) % S == 0, "K-slices of whole columns");
  constexpr int JT = 2 * CPL / S;  // chunk columns of 16 chunks in this K-slice
  constexpr int N2 = JT - W;       // waves 0..N2-1 own two columns, the rest one
  static_assert(W <= JT && JT <= 2 * W, "every wave owns one or two columns");
  // quads per task: 2; 1 for the two-slice down blocks (10 quads: finer tasks
  // keep more of the walk overlapped; measured down M = 5 / 7 / 8 14.9 / 15.5
  // / 15.9 us at 2, 13.9 / 14.6 / 15.1 at 1, while the square and gate/up
  // are 3-4 % slower at 1 and 5-9 % at 3)
  constexpr int G = S > 1 ? 1 : 2;
  // floats per (quad, weight row, activation row): 4 W partials, padded to an
  // odd number of 16-byte units, so that the combine's float4 reads of
  // consecutive activation rows (consecutive threads) spread over the banks
  constexpr int WR = 4 * W + (W % 2 == 0 ? 4 : 0);
  // LDS floats per (quad, weight row), = 4 mod 8: the 16 writer lanes (4 weight
  // rows x 4 lane rows) of a partial then hit 16 distinct banks
  constexpr int JS = M * WR + ((M * WR) % 8 == 0 ? 4 : 0);
  static_assert(M >= 3 && M <= 8, "the K-column kernel serves 3 <= M <= 8");
  // Ring variant: the partials of CI loop iterations (2 G CI quads) are added
  // as soon as every wave has parked them, from two alternating halves of a
  // ring of 4 G CI quads, so that the LDS holds that many quads whatever the
  // block's rows.
  constexpr int CI = kXrRingIterations;
  constexpr int QI = 2 * G * CI;  // quads per combine
  constexpr int RQ = 2 * QI;      // ring slots
  constexpr int RPC = FUSED ? 2 * QI : 4 * QI;  // output rows per combine (fused: QI / 2 pairs)
  static_assert(!RING || RPC * M <= 64 * W, "one thread per output of a combine");
  constexpr int MB = 4 * P;    // activation rows of the argmax candidates
  // 16-byte aligned (x units and partials are read as uint4 / float4), also
  // behind the static LDS of the split-K finish
  extern __shared__ uint4 red_lds[];
  float* const red = reinterpret_cast<float*>(red_lds);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rb = blockIdx.x;
  const int ks = S > 1 ? (int)blockIdx.y : 0;  // K-slice: columns ks JT .. ks JT + JT - 1
  const int row_lo = rb * a.rq + (rb < a.rr ? rb : a.rr);
  const int row_hi = row_lo + a.rq + (rb < a.rr ? 1 : 0);
  const int nrows = row_hi - row_lo;
  const int nq = (nrows + 3) >> 2;
  const int NQ = FUSED ? 2 * nq : nq;
  const int ntasks = (NQ + G - 1) / G;
  const int beta = lane >> 2, j = lane & 3;
  const int shp = (beta & 1) * 16;  // this lane's chunk's scale pair in its scale dword

  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.x), (short)0, M * K * 2, kBufferWord3);
  // partial of (quad v, weight row j, activation row m) from wave wv's 16-lane
  // row rho: red[(4 v + j) JS + m WR + 4 wv + rho]
  float* const park = red + j * JS + 4 * wv + (lane >> 4);
  float gv0 = 1.0f, gv1 = 1.0f;
  W4A16_STAMP(t_start);
#ifdef W4A16_TRACE
  unsigned long long t_issued = 0, t_barrier = 0, t_first = 0, t_end = 0;
#endif

  // ring variant: the outputs of combine i (rows RPC i .. RPC i + RPC - 1 of
  // the block), one per thread; argmax: each thread keeps the best of the
  // logits it has seen
  float abv = -__builtin_inff();
  int abi = kNoIndex;
  auto ring_combine = [&](int i) {
    const int o = tid;
    if (o < RPC * M) {
      const int nl = o / M, m = o - nl * M;
      const int n = RPC * i + nl;
      if (n < nrows) {
        const int vg = FUSED ? 2 * (n >> 2) : (n >> 2);
        const float4* pg =
            reinterpret_cast<const float4*>(red + ((vg & (RQ - 1)) * 4 + (n & 3)) * JS + m * WR);
        float sg = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
          const float4 f = pg[w];
          sg += (f.x + f.y) + (f.z + f.w);
        }
        if (ARGMAX) {
          argmax_take(abv, abi, sg * (1.0f / gv0), row_lo + n);
        } else if (FUSED) {
          const float4* pu =
              reinterpret_cast<const float4*>(red + (((vg + 1) & (RQ - 1)) * 4 + (n & 3)) * JS + m * WR);
          float su = 0.0f;
#pragma unroll
          for (int w = 0; w < W; ++w) {
            const float4 f = pu[w];
            su += (f.x + f.y) + (f.z + f.w);
          }
          a.y[(size_t)m * a.N + row_lo + n] = f32_to_bf16(silu(sg * (1.0f / gv0)) * (su * (1.0f / gv1)));
        } else {
          a.y[(size_t)m * a.N + row_lo + n] = f32_to_bf16(sg * (1.0f / gv0));
        }
      }
    }
  };

  // The wave's work for KJ = 1 or 2 columns (compile-time in each copy).
  auto body = [&](auto kj_count) {
    constexpr int KJ = decltype(kj_count)::value;
    const int c0 = KJ == 2 ? 2 * wv : N2 + wv;  // this wave's first column in the slice
    const int cg = ks * JT + c0;                 // ... in the row
    // x: lane (beta, j) holds activation rows 4 pp + j of chunk beta + 16 c
    // for the wave's columns c = c0 + kj, as 16-byte units u = 0..3.  Loaded
    // as one contiguous 1 KB row span per instruction (lane l: bytes 16 l..,
    // i.e. unit l & 3 of chunk l >> 2 of row 4 pp + u in xv[..][u]) and then
    // transposed within each quad of lanes through LDS (below).  Measured at
    // M = 7 on the square (five waves of two columns): loading each lane's own
    // units directly (16 bytes per lane at a 64-byte stride) 7.11 us per call,
    // contiguous loads with a DPP transpose 6.70, with the LDS transpose 6.53.
    // Rows M..4P-1 are zero without a load.
    uint4 xv[KJ][P][4];
    const int xlane = 16 * 64 * cg + 16 * lane;
#pragma unroll
    for (int kj = 0; kj < KJ; ++kj)
#pragma unroll
      for (int pp = 0; pp < P; ++pp)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (4 * pp + u >= M) {  // a padding row: no load
            xv[kj][pp][u] = make_uint4(0u, 0u, 0u, 0u);
            continue;
          }
          const int off = xlane + ((4 * pp + u) * (K * 2) + 16 * 64 * kj);
          const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
          xv[kj][pp][u] = make_uint4(v.x, v.y, v.z, v.w);
        }
    // weights: one buffer per matrix over this block's rows, so that rows past
    // the block and quads past the last read as zero without touching memory
    const int qrec = nrows * (K >> 1), srec = nrows * (K >> 4);
    const __amdgpu_buffer_rsrc_t rq0 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.wq0) + (size_t)row_lo * (K >> 1), (short)0, qrec, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rs0 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.ws0) + (size_t)row_lo * (K >> 4), (short)0, srec, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rq1 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.wq1) + (size_t)row_lo * (K >> 1), (short)0, qrec, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rs1 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.ws1) + (size_t)row_lo * (K >> 4), (short)0, srec, kBufferWord3);
    auto load_task = [&](uint4 (&q)[G][KJ], uint32_t (&sc)[G][KJ], int t) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int v = t * G + g;
        const bool up = FUSED && (v & 1);
        const int row = 4 * (FUSED ? (v >> 1) : v) + j;
#pragma unroll
        for (int kj = 0; kj < KJ; ++kj) {
          const int c = beta + 16 * (cg + kj);
          const u32x4_t v4 = __builtin_amdgcn_raw_buffer_load_b128(up ? rq1 : rq0, row * (K >> 1) + c * 16,
                                                                   0, kCpolNt);
          q[g][kj] = make_uint4(v4.x, v4.y, v4.z, v4.w);
          sc[g][kj] = __builtin_amdgcn_raw_buffer_load_b32(up ? rs1 : rs0, row * (K >> 4) + (c >> 1) * 4, 0,
                                                           kCpolNt);
        }
      }
    };
    auto compute = [&](const uint4 (&q)[G][KJ], const uint32_t (&sc)[G][KJ], int t) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int v = t * G + g;
        if (v < NQ) {
          float acc[P][4];
#pragma unroll
          for (int pp = 0; pp < P; ++pp)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[pp][r] = 0.0f;
#pragma unroll
          for (int kj = 0; kj < KJ; ++kj) {
            const uint4 qq = q[g][kj];
            const uint32_t pr = sc[g][kj] >> shp;
            const float s_lo = e4m3_to_f32<0>(pr), s_hi = e4m3_to_f32<1>(pr);
            f32x4_t C[P];
            // word wi holds inputs 8wi..8wi+7 of the chunk: two MFMAs of 4 inputs
#define W4A16_XR_WORD(word, wi)                                                           \
  {                                                                                      \
    const i16x4_t b0 = pack4(fp4x2_to_bf16x2<0>(word), fp4x2_to_bf16x2<1>(word));        \
    const i16x4_t b1 = pack4(fp4x2_to_bf16x2<2>(word), fp4x2_to_bf16x2<3>(word));        \
    _Pragma("unroll") for (int pp = 0; pp < P; ++pp) {                                   \
      C[pp] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(                                    \
          pack4(xv[kj][pp][wi].x, xv[kj][pp][wi].y), b0, C[pp], 0, 0, 0);                \
      C[pp] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(                                    \
          pack4(xv[kj][pp][wi].z, xv[kj][pp][wi].w), b1, C[pp], 0, 0, 0);                \
    }                                                                                    \
  }
#pragma unroll
            for (int pp = 0; pp < P; ++pp) C[pp] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            W4A16_XR_WORD(qq.x, 0)
            W4A16_XR_WORD(qq.y, 1)
#pragma unroll
            for (int pp = 0; pp < P; ++pp)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (4 * pp + r < M) acc[pp][r] = fmaf(C[pp][r], s_lo, acc[pp][r]);
#pragma unroll
            for (int pp = 0; pp < P; ++pp) C[pp] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            W4A16_XR_WORD(qq.z, 2)
            W4A16_XR_WORD(qq.w, 3)
#pragma unroll
            for (int pp = 0; pp < P; ++pp)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (4 * pp + r < M) acc[pp][r] = fmaf(C[pp][r], s_hi, acc[pp][r]);
#undef W4A16_XR_WORD
          }
          // the 4 blocks of each 16-lane row (the same weight row j), summed by
          // DPP with every lane active; lanes 16 rho + j then park the sums
          float vv[P][4];
#pragma unroll
          for (int pp = 0; pp < P; ++pp)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (4 * pp + r < M) {
                vv[pp][r] = dpp_add<kDppRor8>(dpp_add<kDppRor4>(acc[pp][r]));
                // keep the DPP adds ahead of the writers' branch (inside it the
                // masked-off lanes would be invalid DPP sources)
                asm volatile("" : "+v"(vv[pp][r]));
              }
          if ((lane & 12) == 0) {
            float* const dst = park + (RING ? (v & (RQ - 1)) : v) * 4 * JS;
#pragma unroll
            for (int pp = 0; pp < P; ++pp)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (4 * pp + r < M) dst[(4 * pp + r) * WR] = vv[pp][r];
          }
        }
      }
    };

    uint4 qa[G][KJ], qb[G][KJ];
    uint32_t sa[G][KJ], sb[G][KJ];
    load_task(qa, sa, 0);
    __builtin_amdgcn_sched_barrier(0);
#ifdef W4A16_TRACE
    t_issued = wall_clock64();
#endif
    // g after the first loads: a scalar load's wait is lgkmcnt(0), which ahead
    // of them would hold back every vector load's address set-up
    typedef const __attribute__((address_space(4))) float cfloat;
    gv0 = *reinterpret_cast<cfloat*>(reinterpret_cast<uintptr_t>(a.g0));
    if (FUSED) gv1 = *reinterpret_cast<cfloat*>(reinterpret_cast<uintptr_t>(a.g1));
    // x units into place, (lane 4 beta + k, unit u) <- (lane 4 beta + u, unit
    // k), through the LDS area of this wave's columns (P x 4 x 64 units per
    // column): unit u' for lane l is stored at [u'][l ^ u'] (a swap within
    // each quad of lanes, so that the 16 lanes of a row write 16 distinct
    // bank groups; the reads stay 16-byte units of one 1 KB span).  The area
    // later holds partial sums of other waves, hence the barrier after every
    // wave has read its own.
    {
      uint4* const xt = reinterpret_cast<uint4*>(red) + c0 * (P * 4 * 64);
#pragma unroll
      for (int kj = 0; kj < KJ; ++kj)
#pragma unroll
        for (int pp = 0; pp < P; ++pp)
#pragma unroll
          for (int u = 0; u < 4; ++u) xt[((kj * P + pp) * 4 + j) * 64 + 4 * beta + (u ^ j)] = xv[kj][pp][u];
#pragma unroll
      for (int kj = 0; kj < KJ; ++kj)
#pragma unroll
        for (int pp = 0; pp < P; ++pp)
#pragma unroll
          for (int u = 0; u < 4; ++u) xv[kj][pp][u] = xt[((kj * P + pp) * 4 + u) * 64 + (lane ^ u)];
      lds_barrier();
    }
#ifdef W4A16_TRACE
    t_barrier = wall_clock64();
#endif
    // two tasks per iteration and one exit test (see the whole-row kernel)
    int t = 0;
    while (t < ntasks) {
      load_task(qb, sb, t + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(qa, sa, t);
#ifdef W4A16_TRACE
      if (t_first == 0) t_first = wall_clock64();
#endif
      load_task(qa, sa, t + 2);
      __builtin_amdgcn_sched_barrier(0);
      if (t + 1 < ntasks) compute(qb, sb, t + 1);
      if constexpr (RING) {
        const int it = t >> 1;
        if (it % CI == CI - 1 || t + 2 >= ntasks) {
          lds_barrier();  // every wave has parked these iterations' quads
          ring_combine(it / CI);
        }
      }
      t += 2;
    }
#ifdef W4A16_TRACE
    t_end = wall_clock64();
#endif
  };
  if constexpr (N2 == W) {
    body(std::integral_constant<int, 2>{});
  } else {
    if (wv < N2)
      body(std::integral_constant<int, 2>{});
    else
      body(std::integral_constant<int, 1>{});
  }

  if constexpr (RING) {
    if constexpr (ARGMAX) {
      lds_barrier();  // the last iteration's partials are read: red is free
      float bv[MB];
      int bi[MB];
#pragma unroll
      for (int mm = 0; mm < MB; ++mm) {
        bv[mm] = -__builtin_inff();
        bi[mm] = kNoIndex;
      }
      if (tid < RPC * M) {
        const int m = tid - (tid / M) * M;
#pragma unroll
        for (int mm = 0; mm < MB; ++mm)
          if (mm == m) {
            bv[mm] = abv;
            bi[mm] = abi;
          }
      }
      wg_argmax_rows<MB>(bv, bi, M, red, W);
      if (tid < M) {
        float* c = a.cand + ((size_t)rb * M + tid) * 2;
        store_coherent(c, bv[0]);
        store_coherent(c + 1, __int_as_float(bi[0]));
      }
      argmax_finish<MB>(a, a.cnt, gridDim.x, red, W);
    }
#ifdef W4A16_TRACE
    W4A16_STAMP(t_done);
    W4A16_TRACE_STORE(t_start, t_issued, t_barrier, t_first, t_end, t_done);
#endif
    return;
  }
  lds_barrier();
  const float ig0 = 1.0f / gv0, ig1 = 1.0f / gv1;
  for (int o = tid; o < nrows * M; o += 64 * W) {
    const int n = o / M, m = o - n * M;
    const int vg = FUSED ? 2 * (n >> 2) : (n >> 2);
    const float4* pg = reinterpret_cast<const float4*>(red + (4 * vg + (n & 3)) * JS + m * WR);
    float sg = 0.0f, su = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float4 f = pg[w];
      sg += (f.x + f.y) + (f.z + f.w);
    }
    if (FUSED) {
      const float4* pu = reinterpret_cast<const float4*>(red + (4 * vg + 4 + (n & 3)) * JS + m * WR);
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float4 f = pu[w];
        su += (f.x + f.y) + (f.z + f.w);
      }
    }
    const size_t i = (size_t)m * a.N + row_lo + n;
    if (S > 1) {
      // this K-slice's sums; the row block's last workgroup adds the slices
      store_coherent(a.part + (size_t)ks * M * a.N + i, sg);
      if (FUSED) store_coherent(a.part + (size_t)(S + ks) * M * a.N + i, su);
    } else if (FUSED) {
      a.y[i] = f32_to_bf16(silu(sg * ig0) * (su * ig1));
    } else {
      a.y[i] = f32_to_bf16(sg * ig0);
    }
  }
  if (S > 1) splitk_finish<FUSED, false>(a, rb, row_lo, nrows, ig0, ig1);
#ifdef W4A16_TRACE
  W4A16_STAMP(t_done);
  W4A16_TRACE_STORE(t_start, t_issued, t_barrier, t_first, t_end, t_done);
#endif
}

// ---------------------------------------------------------------------------
// MFMA kernel, 3 <= M <= 32 (P = ceil(M/4) passes of 4 activation rows; rows
// M..4P-1 are zero).
//
// Uses v_mfma_f32_4x4x4_16b_bf16: 16 independent 4x4x4 products per
// instruction; lane l = 4*beta + j holds B[k=0..3][col j] and A[row j][k] of
// block beta and receives C[row r][col j] in register r.  Here block beta is
// one weight chunk column, col j one of 4 weight rows, row r one activation
// row; each MFMA covers 4 consecutive inputs, which never straddle a 16-input
// scale block, so the E4M3 scale multiplies the fp32 MFMA result of its block
// (4 MFMAs per block, one FMA per result element).
//
// A task is R quads of weight rows (fused: R pairs of gate rows and the same
// pairs of up rows) and takes CPL = ceil(CRS/16) steps.  At step (task, jj)
// lane (beta, j) reads chunk beta + 16*jj of row j of every quad (16 lanes x
// 16 B = 256 contiguous bytes per row per load) and the x slice of activation
// row 4*pp + j from LDS, which then feeds the MFMAs of all R quads.
// ---------------------------------------------------------------------------
template <int P, int R, int D, int EPI, int LB, int CO>
W4A16_DEV void gemm_mfma(const MatArgs& a, int rb, int ks, int nwg) {
  constexpr bool FUSED = EPI == kEpiSwiglu;
  constexpr bool XC = (CO & kCoLoadX) != 0, YC = (CO & kCoStoreY) != 0;
  W4A16_STAMP(t_start);
  extern __shared__ uint4 xs[];
  constexpr int QS = FUSED ? 2 : 4;      // output rows per quad
  constexpr int RT = QS * R;             // output rows per task
  constexpr int NA = R * P * 4;          // accumulators per lane
  constexpr int V = NA * 4;              // values in a segment partial: [acc][j]
  const int W = blockDim.x >> 6, NT = blockDim.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = a.K, S = a.S, CRS = a.CRS;  // CRS: chunks per row in this K-slice
  const int c0 = ks * CRS;
  const int CPL = (CRS + 15) >> 4, RSU = (CRS << 2) + 1;
  const int row_lo = rb * a.rq + (rb < a.rr ? rb : a.rr);
  const int row_hi = row_lo + a.rq + (rb < a.rr ? 1 : 0);
  const int ntasks = (row_hi - row_lo + RT - 1) / RT;
  const StreamSplit split{ntasks * CPL, W, a.rW};
  const int s_begin = split.begin(wv);
  const int T = split.begin(wv + 1) - s_begin;
  const int ft = div_small(s_begin, CPL, a.rCPL), jj0 = s_begin - ft * CPL;  // first task, its first step
  const int beta = lane >> 2, j = lane & 3;
  const int jr = FUSED ? (j & 1) : j;    // row within the quad
  const bool is_up = FUSED && (j >= 2);
  const uint8_t* wq = is_up ? a.wq1 : a.wq0;
  const uint8_t* ws = is_up ? a.ws1 : a.ws0;
  const bool ragged = (CRS & 15) != 0;
  float* scr = reinterpret_cast<float*>(xs + 4 * P * RSU) + wv * (NA * 16);
  float* seg = reinterpret_cast<float*>(xs + 4 * P * RSU) + W * (NA * 16);
  int* tw0 = reinterpret_cast<int*>(seg + W * a.kmax * V);
  int* tw1 = tw0 + W * a.kmax;
  int* wft = tw1 + W * a.kmax;

  const uint4* qp[R];
  const uint16_t* sp[R];
  // s_i: index of the step the next issue loads (among this wave's T steps).
  // Past the last one the ring is still refilled (every wait stays exact) with
  // loads of a cached line (past_line); cb is then 0, so each lane reads its
  // own 16 bytes there.
  const uint4* const q_past = past_line<XC>(a, tid);
  const uint16_t* const s_past = reinterpret_cast<const uint16_t*>(q_past);
  int s_i = 0, it_i = ft, jj_i = jj0, cb = beta;
  auto set_task = [&](int it) {
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      int row = row_lo + it * RT + rr * QS + jr;
      row = row < row_hi ? row : row_hi - 1;
      qp[rr] = reinterpret_cast<const uint4*>(wq + (size_t)row * (size_t)(K >> 1)) + c0;
      sp[rr] = reinterpret_cast<const uint16_t*>(ws + (size_t)row * (size_t)(K >> 4)) + c0;
    }
  };
  set_task(it_i);
  auto go_past = [&]() {
    s_i = T;
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      qp[rr] = q_past;
      sp[rr] = s_past;
    }
    cb = 0;
    jj_i = 0;
  };
  if (T == 0) go_past();
  uint4 qb[D][R];
  uint32_t sb[D][R];
  auto issue = [&](int d) {
    int c = cb + 16 * jj_i;
    c = c < CRS ? c : CRS - 1;
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      qb[d][rr] = load_stream(qp[rr] + c);
      sb[d][rr] = __builtin_nontemporal_load(sp[rr] + c);
    }
    if (s_i >= T) return;  // past the end: stay there
    if (s_i + 1 < T) {
      ++s_i;
      if (++jj_i == CPL) {
        jj_i = 0;
        ++it_i;
        set_task(it_i);
      }
    } else {
      go_past();
    }
  };
  // x -> LDS: rows 0..4P-1 (rows >= M are zero), 16 B pad per row.
  const float gv0 = load_f32_vmem(a.g0);
  const float gv1 = FUSED ? load_f32_vmem(a.g1) : 1.0f;
  if (lane == 0) wft[wv] = T > 0 ? ft : kNoTask;
  const int upr = CRS << 2;  // 16-byte x units per row of the slice
  if ((upr & 63) == 0) {
    // Direct-to-LDS path (every row of the slice is whole 64-unit blocks):
    // the weight prologue first, then one 1 KiB direct-to-LDS load per block
    // of 64 units (a short rolled loop: the launch starts with a cold
    // instruction cache, and a long unrolled staging sequence kept the
    // weight stream waiting), zeros for the padding rows, and one wait for
    // everything before the barrier.
#pragma unroll
    for (int d = 0; d < D; ++d) issue(d);
    W4A16_STAMP(t_issued0);
    const int cpr = upr >> 6;                    // 64-unit blocks per row
    const float rcpr = 64.0f * a.rUPR;           // = fp32(1 / cpr), exactly
    const int nblk = (a.M < 4 * P ? a.M : 4 * P) * cpr;
    const uint4* xg = reinterpret_cast<const uint4*>(a.x) + (c0 << 2) + lane;
    for (int j = wv; j < nblk; j += W) {
      const int m = div_small(j, cpr, rcpr), cb = j - m * cpr;
      __builtin_amdgcn_global_load_lds(
          xg + (size_t)m * (K >> 3) + cb * 64,
          (__attribute__((address_space(3))) void*)(xs + m * RSU + cb * 64), 16, 0,
          XC ? kCpolSc1 : 0);
    }
    for (int u = a.M * RSU + tid; u < 4 * P * RSU; u += NT) xs[u] = make_uint4(0u, 0u, 0u, 0u);
    __builtin_amdgcn_s_waitcnt(0);  // the direct-to-LDS loads have landed
    (void)t_issued0;
  } else {
    // register path: ring slot 0 first (the weight stream starts as early
    // in the cold instruction stream as possible), the x loads, the rest of
    // the prologue, then the LDS stores (loads complete in order, so the
    // stores wait for slot 0 and x only)
    constexpr int XMAX = LB > 512 ? 8 : 16;
    uint4 xr[XMAX];
    auto xpos = [](int cu) { return cu; };
    issue(0);
    x_stage_issue<XC>(xr, a.x, a.M, 4 * P, K, c0 << 2, upr, a.rUPR, tid, NT);
#pragma unroll
    for (int d = 1; d < D; ++d) issue(d);
    x_stage_store<XC>(xs, xr, a.x, a.M, 4 * P, K, c0 << 2, upr, a.rUPR, RSU, tid, NT, xpos);
  }
  // (issue is unconditional: a wave without steps loads its cached line)
  W4A16_STAMP(t_issued);
  __syncthreads();
  W4A16_STAMP(t_barrier);
  // g was the first load: 1/g costs no wait here (after the loop it made the
  // combine wait for every refill still in flight)
  const float ig0 = pin(1.0f / gv0);
  const float ig1 = FUSED ? pin(1.0f / gv1) : 1.0f;
#ifdef W4A16_TRACE
  unsigned long long t_first = 0;
#endif

  float acc[R][P][4];
#pragma unroll
  for (int rr = 0; rr < R; ++rr)
#pragma unroll
    for (int pp = 0; pp < P; ++pp)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[rr][pp][r] = 0.0f;
  int jj_c = jj0, kseg = 0;

  // Segment end: for each accumulator sum the 4 chunk columns inside each
  // 16-lane row with DPP, park the 4 row totals per (accumulator, column j) in
  // the per-wave scratch, then store their sums [acc][j] in segment slot
  // (wv, kseg).  Accumulator index ai = (rr*P + pp)*4 + r = rr*4P + m.
  auto finish_segment = [&](bool task_end) {
    const int row16 = lane >> 4;
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
      for (int pp = 0; pp < P; ++pp)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = acc[rr][pp][r];
          v = dpp_add<kDppRor4>(v);
          v = dpp_add<kDppRor8>(v);
          const int ai = (rr * P + pp) * 4 + r;
          if ((lane & 12) == 0) scr[(ai * 4 + j) * 4 + row16] = v;
          acc[rr][pp][r] = 0.0f;
        }
    wave_lds_sync();
    for (int o = lane; o < V; o += 64) {
      const float4 pv = *reinterpret_cast<const float4*>(&scr[o * 4]);
      seg[(wv * a.kmax + kseg) * V + o] = (pv.x + pv.y) + (pv.z + pv.w);
    }
    if (lane == 0) {
      if (kseg > 0 || jj0 == 0) tw0[ft + kseg] = wv;
      if (task_end) tw1[ft + kseg] = wv;
    }
    ++kseg;
    wave_lds_sync();
  };

  for (int s0 = 0; s0 < T; s0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (s0 + d < T) {
        int c = beta + 16 * jj_c;
        const bool dead = ragged && c >= CRS;  // lane past the end of a ragged slice
        c = dead ? CRS - 1 : c;
        uint4 xv[P][4];
#pragma unroll
        for (int pp = 0; pp < P; ++pp)
#pragma unroll
          for (int u = 0; u < 4; ++u) xv[pp][u] = xs[(4 * pp + j) * RSU + 4 * c + u];
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
          uint4 q = qb[d][rr];
          if (dead) q = make_uint4(0u, 0u, 0u, 0u);
          const uint32_t sc = sb[d][rr];
          const float s_lo = e4m3_to_f32<0>(sc), s_hi = e4m3_to_f32<1>(sc);
          f32x4_t C[P];
          // word wi holds inputs 8wi..8wi+7 of the chunk: two MFMAs of 4 inputs
#define W4A16_MFMA_WORD(word, wi)                                                   \
  {                                                                                 \
    const i16x4_t b0 = pack4(fp4x2_to_bf16x2<0>(word), fp4x2_to_bf16x2<1>(word));   \
    const i16x4_t b1 = pack4(fp4x2_to_bf16x2<2>(word), fp4x2_to_bf16x2<3>(word));   \
    _Pragma("unroll") for (int pp = 0; pp < P; ++pp) {                              \
      C[pp] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(pack4(xv[pp][wi].x, xv[pp][wi].y), \
                                                      b0, C[pp], 0, 0, 0);          \
      C[pp] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(pack4(xv[pp][wi].z, xv[pp][wi].w), \
                                                      b1, C[pp], 0, 0, 0);          \
    }                                                                               \
  }
#pragma unroll
          for (int pp = 0; pp < P; ++pp) C[pp] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
          W4A16_MFMA_WORD(q.x, 0)
          W4A16_MFMA_WORD(q.y, 1)
#pragma unroll
          for (int pp = 0; pp < P; ++pp)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[rr][pp][r] = fmaf(C[pp][r], s_lo, acc[rr][pp][r]);
#pragma unroll
          for (int pp = 0; pp < P; ++pp) C[pp] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
          W4A16_MFMA_WORD(q.z, 2)
          W4A16_MFMA_WORD(q.w, 3)
#pragma unroll
          for (int pp = 0; pp < P; ++pp)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[rr][pp][r] = fmaf(C[pp][r], s_hi, acc[rr][pp][r]);
#undef W4A16_MFMA_WORD
        }
#ifdef W4A16_TRACE
        if (t_first == 0) t_first = wall_clock64();
#endif
        const bool task_end = ++jj_c == CPL;
        if (task_end || s0 + d + 1 == T) finish_segment(task_end);
        if (task_end) jj_c = 0;
      }
      issue(d);
    }
  }
  W4A16_STAMP(t_end);

  // ---- workgroup combine: output (row n, m) = sum of its task's segments --
  lds_barrier();
  const int M = a.M;
  const int nrows = row_hi - row_lo;
  if (EPI == kEpiArgmax && S == 1) {
    // x is no longer needed, so its LDS holds the reduction scratch
    float* red = reinterpret_cast<float*>(xs);
    constexpr int MB = 4 * P;
    float bv[MB];
    int bi[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      bv[m] = -__builtin_inff();
      bi[m] = kNoIndex;
    }
    for (int n = tid; n < nrows; n += NT) {
      const int t = n / RT, rt = n - t * RT;
      const int rr = rt / QS, jo = rt - rr * QS;
      // the logits of weight row n for every activation row m: its task's
      // segment values at (rr * 4P + m) * 4 + jo, added in wave order
      float v[MB];
#pragma unroll
      for (int m = 0; m < MB; ++m) v[m] = 0.0f;
      for (int w = tw0[t]; w <= tw1[t]; ++w) {
        const int k = t - wft[w];
        if (k < 0) continue;  // a wave without steps
        const float* sg = seg + (w * a.kmax + k) * V + rr * (4 * P) * 4 + jo;
#pragma unroll
        for (int m = 0; m < MB; ++m) v[m] += sg[m * 4];
      }
#pragma unroll
      for (int m = 0; m < MB; ++m)
        if (m < M) argmax_take(bv[m], bi[m], v[m] * ig0, row_lo + n);
    }
    wg_argmax_rows<MB>(bv, bi, M, red, W);
    if (tid < M) {
      float* c = a.cand + ((size_t)rb * M + tid) * 2;
      store_coherent(c, bv[0]);
      store_coherent(c + 1, __int_as_float(bi[0]));
    }
    argmax_finish<MB>(a, a.cnt, nwg, red, W);
  } else
  // item o = n * 4P + m (rows m >= M are skipped): a constant divisor.  With
  // a K split every epilogue (argmax too) parks fp32 partials first.
  for (int o = tid; o < nrows * 4 * P; o += NT) {
    const int n = o / (4 * P), m = o - n * (4 * P);
    if (m >= M) continue;
    const int t = n / RT, rt = n - t * RT;
    const int rr = rt / QS, jo = rt - rr * QS;
    const int idx = (rr * (4 * P) + m) * 4 + jo;  // [accumulator][column j]
    const int w0 = tw0[t], w1 = tw1[t];
    float v = 0.0f, u = 0.0f;
    for (int w = w0; w <= w1; ++w) {
      const int k = t - wft[w];
      if (k < 0) continue;  // a wave without steps
      const float* sg = seg + (w * a.kmax + k) * V;
      v += sg[idx];
      if (FUSED) u += sg[idx + 2];
    }
    const int row = row_lo + n;
    if (S > 1) {
      store_coherent(a.part + ((size_t)ks * M + m) * a.N + row, v);
      if (FUSED) store_coherent(a.part + ((size_t)(S + ks) * M + m) * a.N + row, u);
    } else if (FUSED) {
      store_y<YC>(a.y, (size_t)m * a.N + row, f32_to_bf16(silu(v * ig0) * (u * ig1)));
    } else {
      store_y<YC>(a.y, (size_t)m * a.N + row, f32_to_bf16(v * ig0));
    }
  }
  if (S > 1)
    splitk_finish<FUSED, YC, EPI, 4 * P>(a, rb, row_lo, row_hi - row_lo, ig0, ig1,
                                        reinterpret_cast<float*>(xs), W, nwg);
#ifdef W4A16_TRACE
  W4A16_STAMP(t_done);
  W4A16_TRACE_STORE(t_start, t_issued, t_barrier, t_first, t_end, t_done);
#endif
}

template <int P, int R, int D, int EPI, int LB>
__global__ void __launch_bounds__(LB) k_gemm_mfma(MatArgs a) {
  gemm_mfma<P, R, D, EPI, LB, kCoPlain>(a, blockIdx.x, blockIdx.y, gridDim.x);
}

// ---------------------------------------------------------------------------
// Wide kernel, 13 <= M <= 32: one 32 x 32 x 16 bf16 MFMA per 16-input scale
// block, accumulating over the whole K-slice.  An E2M1 value times an E4M3
// scale has at most 6 significant bits, so each weight times its block scale
// is exact in bf16: the weights enter the MFMA already scaled (fp32 products
// packed to bf16 without rounding) and no per-block work waits for an MFMA
// result.  The global scale divides the sum once, in the epilogue.
//
// v_mfma_f32_32x32x16_bf16: lane l holds A[l % 32][8 * (l / 32) + e] and
// B[8 * (l / 32) + e][l % 32] (e = 0..7) and receives C[i][l % 32] in
// register r, i = 8 * (r / 4) + 4 * (l / 32) + r % 4.  Here A is x (rows =
// activation rows; rows >= M are zero), B the scaled weights of 32
// consecutive rows (columns = weight rows).
//
// A wave owns a tile of 32 weight rows over the workgroup's K-slice and walks
// it in steps of 256 inputs: the two lanes of row n read that row's 128 bytes
// of codes (one whole cache line; lane g the 16-byte pieces 2j + g, j = 0..3,
// so each load instruction takes 32 contiguous bytes per row) and its 16
// scale bytes.  Per piece pair j, two cross-half lane swaps leave lane g with
// half g (8 inputs, one dword of codes) of each of blocks 4j..4j+3, which is
// the MFMA's B operand after four E2M1 -> bf16 conversions.  The x slice is
// staged in LDS as [row][k] with a 16-byte pad per row; lane (m, g) reads its
// 8 inputs of a block with one 16-byte LDS read.  A workgroup of W waves owns
// a row block of a.rq tiles (wave w: tiles w, w + W, ...) and K-slice
// blockIdx.y of a.CRS steps (the last slice may be shorter).  With S > 1 the slices' fp32 sums go to the
// split-K partials and the row block's last workgroup adds them in slice
// order (splitk_finish).  Fused gate/up: every tile runs the gate and the up
// rows side by side on the same x reads.
// ---------------------------------------------------------------------------
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
// two E2M1 codes (byte B of w) times the block scale s, as two bf16 in one
// dword: the products are exact in fp32 and in bf16
template <int B>
W4A16_DEV uint32_t scaled_bf16x2(uint32_t w, float s) {
  const f32x2_t v = fp4x2_to_f32x2<B>(w);
  const bf16x2_t r = {(__bf16)(v[0] * s), (__bf16)(v[1] * s)};
  return __builtin_bit_cast(uint32_t, r);
}
// Split-K finish of the wide kernel: as splitk_finish (the row block's last
// workgroup adds the slices in order 0..S-1), but each thread issues the
// loads of G outputs x 8 slices before adding any of them, so that the
// finishing workgroup waits for one far round trip per 8 slices instead of
// one per output.
template <bool FUSED>
W4A16_DEV void wide_finish(const MatArgs& a, int rb, int row_lo, int nrows, float ig0, float ig1) {
  __shared__ int is_last;
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const int before = __hip_atomic_fetch_add(a.cnt + rb, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = before == a.S - 1;
    if (is_last) __hip_atomic_store(a.cnt + rb, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!is_last) return;
  constexpr int G = FUSED ? 4 : 8;  // outputs per thread per pass
  const int S = a.S, NT = blockDim.x, tot = nrows * a.M;
  const size_t MN = (size_t)a.M * a.N;
  const float rn = 1.0f / (float)nrows;
  for (int o0 = threadIdx.x; o0 < tot; o0 += G * NT) {
    size_t idx[G];
    float v[G], u[G];
#pragma unroll
    for (int q = 0; q < G; ++q) {
      const int o = min(o0 + q * NT, tot - 1);  // past the end: repeat a valid output
      const int m = div_small(o, nrows, rn), n = o - m * nrows;
      idx[q] = (size_t)m * a.N + row_lo + n;
      v[q] = 0.0f;
      u[q] = 0.0f;
    }
    for (int s0 = 0; s0 < S; s0 += 8) {
      float t[G][8], tu[G][8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const size_t off = (size_t)min(s0 + j, S - 1) * MN;
#pragma unroll
        for (int q = 0; q < G; ++q) {
          t[q][j] = load_coherent(a.part + off + idx[q]);
          if (FUSED) tu[q][j] = load_coherent(a.part + (size_t)S * MN + off + idx[q]);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (s0 + j < S) {
#pragma unroll
          for (int q = 0; q < G; ++q) {
            v[q] += t[q][j];
            if (FUSED) u[q] += tu[q][j];
          }
        }
    }
#pragma unroll
    for (int q = 0; q < G; ++q)
      if (o0 + q * NT < tot) {
        if (FUSED) a.y[idx[q]] = f32_to_bf16(silu(v[q] * ig0) * (u[q] * ig1));
        else a.y[idx[q]] = f32_to_bf16(v[q] * ig0);
      }
  }
}

template <int MT, int EPI>
__global__ void __launch_bounds__(512) k_gemm_wide(MatArgs a) {
  constexpr bool FUSED = EPI == kEpiSwiglu;
  static_assert(EPI != kEpiArgmax && (MT == 2 || MT == 4), "wide kernel: plain or SwiGLU, 16 or 32 x rows in LDS");
  constexpr int NQ = FUSED ? 2 : 1;  // weight matrices per tile
  constexpr int NR = 4 * MT;         // result registers that can hold rows < M
  extern __shared__ uint4 wide_lds[];
  const int W = blockDim.x >> 6, NT = blockDim.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = a.M, N = a.N, K = a.K;
  const int rb = blockIdx.x, ks = blockIdx.y, S = a.S;
  const int st0 = ks * a.CRS;                                   // first 256-input step of the slice
  const int nst = min(a.CRS, (K >> 8) - st0);                   // steps in the slice (even)
  const int upr = nst << 5;                                     // 16-byte x units per row of the slice
  const int RS = upr + 1;                                       // LDS row stride in units
  const int row_lo = rb * a.rq * 32, row_hi = min(N, row_lo + a.rq * 32);
  const int ntiles = (row_hi - row_lo + 31) >> 5;
  const int nl = lane & 31, g = lane >> 5;

  // x slice -> LDS: 1 KiB direct-to-LDS loads (each row is whole 64-unit
  // pieces: the slice is a multiple of 512 inputs), zeros for rows M..8MT-1
  const float gv0 = load_f32_vmem(a.g0);
  const float gv1 = FUSED ? load_f32_vmem(a.g1) : 1.0f;
  {
    const int ppr = upr >> 6;  // pieces per row
    const uint4* xg = reinterpret_cast<const uint4*>(a.x) + (size_t)st0 * 32 + lane;
    for (int j = wv; j < M * ppr; j += W) {
      const int m = j / ppr, pc = j - m * ppr;
      __builtin_amdgcn_global_load_lds(xg + (size_t)m * (K >> 3) + pc * 64,
                                       (__attribute__((address_space(3))) void*)(wide_lds + m * RS + pc * 64),
                                       16, 0, 0);
    }
    for (int u = M * RS + tid; u < 8 * MT * RS; u += NT) wide_lds[u] = make_uint4(0u, 0u, 0u, 0u);
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
  const float ig0 = 1.0f / gv0, ig1 = FUSED ? 1.0f / gv1 : 1.0f;
  // this lane's A row: lanes 16..31 of a 16-row tile repeat rows 0..15
  const uint4* xa = wide_lds + (MT == 2 ? (lane & 15) : nl) * RS + g;

  for (int ti = wv; ti < ntiles; ti += W) {
    const int r0 = row_lo + ti * 32;
    const int row = min(r0 + nl, row_hi - 1);  // ragged tile: repeat the last row
    const uint4* qp[NQ];
    const uint4* sp[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const uint8_t* wq = q ? a.wq1 : a.wq0;
      const uint8_t* ws = q ? a.ws1 : a.ws0;
      qp[q] = reinterpret_cast<const uint4*>(wq + (size_t)row * (size_t)(K >> 1)) + 8 * st0 + g;
      sp[q] = reinterpret_cast<const uint4*>(ws + (size_t)row * (size_t)(K >> 4)) + st0;
    }
    // two slots of one step each: 4 x 16 bytes of codes (pieces 2j + g of
    // the row's 128 bytes) and the step's 16 scale bytes, per matrix
    uint4 wa[NQ][4], wb2[NQ][4], sa[NQ], sb2[NQ];
    auto load_step = [&](uint4 (&w)[NQ][4], uint4 (&sc)[NQ], int s) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
#pragma unroll
        for (int j = 0; j < 4; ++j) w[q][j] = qp[q][8 * s + 2 * j];
        sc[q] = sp[q][s];
      }
    };
    f32x16_t acc[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[q] = f32x16_t{};
    auto compute_step = [&](uint4 (&w)[NQ][4], uint4 (&sc)[NQ], int s) {
      // an empty asm that "rewrites" the slot's registers: nothing that reads
      // them (the lane swaps, the scale conversions) can be scheduled above
      // it, i.e. above the previous refill, where it would wait for loads
      // still in flight
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        u32x4_t t0 = __builtin_bit_cast(u32x4_t, w[q][0]), t1 = __builtin_bit_cast(u32x4_t, w[q][1]);
        u32x4_t t2 = __builtin_bit_cast(u32x4_t, w[q][2]), t3 = __builtin_bit_cast(u32x4_t, w[q][3]);
        u32x4_t t4 = __builtin_bit_cast(u32x4_t, sc[q]);
        asm volatile("" : "+v"(t0), "+v"(t1), "+v"(t2), "+v"(t3), "+v"(t4));
        w[q][0] = __builtin_bit_cast(uint4, t0);
        w[q][1] = __builtin_bit_cast(uint4, t1);
        w[q][2] = __builtin_bit_cast(uint4, t2);
        w[q][3] = __builtin_bit_cast(uint4, t3);
        sc[q] = __builtin_bit_cast(uint4, t4);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t hq[NQ][4];  // half g of blocks 4j .. 4j+3 of the step
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const auto p0 = __builtin_amdgcn_permlane32_swap(w[q][j].x, w[q][j].y, false, false);
          const auto p1 = __builtin_amdgcn_permlane32_swap(w[q][j].z, w[q][j].w, false, false);
          hq[q][0] = p0[0];
          hq[q][2] = p0[1];
          hq[q][1] = p1[0];
          hq[q][3] = p1[1];
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const bf16x8_t av = __builtin_bit_cast(bf16x8_t, xa[s * 32 + 8 * j + 2 * b]);
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            const uint32_t sw = j == 0 ? sc[q].x : j == 1 ? sc[q].y : j == 2 ? sc[q].z : sc[q].w;
            float scale;
            if (b == 0) scale = e4m3_to_f32<0>(sw);
            else if (b == 1) scale = e4m3_to_f32<1>(sw);
            else if (b == 2) scale = e4m3_to_f32<2>(sw);
            else scale = e4m3_to_f32<3>(sw);
            // the weights times their block scale, exactly (at most 6
            // significant bits): fp32 products, packed to bf16 without rounding
            const uint32_t h = hq[q][b];
            const uint4 bw = make_uint4(scaled_bf16x2<0>(h, scale), scaled_bf16x2<1>(h, scale),
                                        scaled_bf16x2<2>(h, scale), scaled_bf16x2<3>(h, scale));
            acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8_t, bw), acc[q], 0, 0, 0);
          }
        }
      }
    };
    // (the empty asm statements keep the loads in this order and each refill
    // ahead of the next step's work: without them the compiler sinks refills
    // to their first use or reorders the prologue, and the loop then waits
    // for every load in flight)
    load_step(wa, sa, 0);
    asm volatile("" ::: "memory");
    load_step(wb2, sb2, 1);
    asm volatile("" ::: "memory");
    for (int s = 0; s < nst; s += 2) {
      compute_step(wa, sa, s);
      load_step(wa, sa, min(s + 2, nst - 1));
      asm volatile("" ::: "memory");
      compute_step(wb2, sb2, s + 1);
      load_step(wb2, sb2, min(s + 3, nst - 1));
      asm volatile("" ::: "memory");
    }
    const int n = r0 + nl;
    if (n < row_hi) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int m = 8 * (r >> 2) + 4 * g + (r & 3);
        if (m < M) {
          const size_t i = (size_t)m * N + n;
          if (S > 1) {
            store_coherent(a.part + (size_t)ks * M * N + i, acc[0][r]);
            if (FUSED) store_coherent(a.part + (size_t)(S + ks) * M * N + i, acc[NQ - 1][r]);
          } else if (FUSED) {
            a.y[i] = f32_to_bf16(silu(acc[0][r] * ig0) * (acc[NQ - 1][r] * ig1));
          } else {
            a.y[i] = f32_to_bf16(acc[0][r] * ig0);
          }
        }
      }
    }
  }
  if (S > 1) wide_finish<FUSED>(a, rb, row_lo, row_hi - row_lo, ig0, ig1);
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
