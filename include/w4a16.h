/*
 * w4a16.h -- C ABI of libw4a16.so: NVFP4 weight-only (W4A16) matmul for
 * MI355X (gfx950).
 *
 * Weight format (FlashRT, "Qwen3.6-27B NVFP4 on RTX 5090", section 1 "Model
 * dependencies": the compressed-tensors nvfp4-pack-quantized schema):
 *   wq  uint8  [N][K/2]   FP4 E2M1 codes, two per byte.  Byte j of a row
 *                         holds input 2j in its low nibble and input 2j+1 in
 *                         its high nibble (the page says only "two per byte";
 *                         this order is the library's reading).
 *   ws  uint8  [N][K/16]  E4M3 (FN variant: max 448, 0x7F/0xFF NaN) scale of
 *                         the 16 consecutive inputs 16b..16b+15 of the row.
 *   g   fp32   scalar     per-tensor global scale (448 / amax at quantisation).
 *   Element value: W[n][k] = e2m1(code) * e4m3(scale) / g.
 * Activations are bf16 ("A16" of the format name W4A16), passed as their
 * 16-bit patterns (uint16_t).  All arrays are dense and row-major.
 *
 * Shapes: N = out_features, K = in_features (the reduction), M = number of
 * activation rows (tokens): M = 1 is single-token decode, M = 7 a speculative
 * verify block (6 drafts + 1); M up to 32 covers verify trees and batched
 * clients, with each weight read once for all rows.
 *
 * Ownership: every pointer is device memory owned by the caller (any
 * allocator).  The library allocates nothing, frees nothing and keeps no
 * pointer after a call returns.  g is read on the device (no host sync).
 *
 * Semantics: every compute call only enqueues work on `stream` (0 = the
 * default stream) and returns; it never synchronises.  Results for a given
 * input are bitwise identical from run to run.  Calls are re-entrant; two
 * calls that share a workspace must not run concurrently.
 *
 * Errors: a call that returns anything but W4A16_OK has enqueued nothing,
 * except W4A16_ERR_LAUNCH, which reports the HIP launch error.  The library
 * never aborts and never prints.  Unsupported shapes are rejected, not run on
 * a slower path.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W4A16_OK = 0,
  /* null pointer, M/N/K <= 0, or workspace smaller than required */
  W4A16_ERR_INVALID_VALUE = 1,
  /* M > 32, K % 256 != 0, a pointer not aligned as documented, or a shape
   * too large for the kernels (N, K * 2 must fit in 31 bits) */
  W4A16_ERR_UNSUPPORTED = 2,
  /* the HIP launch failed (hipGetLastError after the launch) */
  W4A16_ERR_LAUNCH = 3
} w4a16_status_t;

/* Largest M (activation rows) the matmul entry points accept. */
#define W4A16_MAX_M 32

/*
 * y[M][N] = bf16( x[M][K] * W^T ),  W dequantised from (wq, ws, g) as above,
 * accumulated in fp32, rounded once to bf16 (nearest even).
 *   wq, ws, x : 16-byte aligned;  g : 4-byte aligned;  y : 4-byte aligned.
 *   K % 256 == 0 (keeps every scale row 16-byte aligned).  1 <= M <= 32.
 *   workspace : device scratch of at least w4a16_workspace_size(M, N, K)
 *               bytes, 16-byte aligned (may be NULL when that size is 0).
 *               When the x slice a workgroup needs does not fit in LDS
 *               (M * K large) the reduction is split over K: each K-slice
 *               writes fp32 partial sums here, and the last workgroup of
 *               each row block to finish adds them in a fixed slice order,
 *               in the same kernel.  The first 4096 bytes of such a
 *               workspace hold the arrival counters of the row blocks: they
 *               must be ZERO BEFORE THE FIRST CALL that uses the workspace
 *               (one hipMemset after allocation), and every call leaves them
 *               zero again, so one zero-fill serves any number of calls, of
 *               any shapes, made one after another.  The partial sums after
 *               them need no initialisation.
 *   Calls with 13 <= M <= 32 (gate/up: 17) and K a multiple of 512 run as one launch of
 *   the wide kernel (32 x 32 x 16 MFMA tiles, split-K partials in the
 *   workspace).  Other wide calls (M > 16) whose single launch would split
 *   K very finely run as two launches on `stream`, over activation rows
 *   [0, m1) and [m1, M) (m1 a multiple of 4), one after the other with the
 *   same workspace; w4a16_workspace_size covers the larger of the two.
 * The operation is the "NVFP4 W4A16" matmul of FlashRT, "Qwen3.6-27B NVFP4
 * on RTX 5090", section 1 (weights in the schema above, bf16 activations).
 * Accuracy contract (this library's own target; the pages state no numeric
 * tolerance): |y - y_exact| <= 1e-2 * sum_k |x[m][k] * W[n][k]| + 1e-6 for
 * every (m, n).  On inputs whose fp32 sums are exact (integer x, power-of-two
 * g and scales) y equals y_exact rounded once to bf16.
 */
w4a16_status_t w4a16_gemm(const uint8_t* wq, const uint8_t* ws, const float* g,
                          const uint16_t* x, uint16_t* y, int M, int N, int K,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * w4a16_gemm for callers that cannot allocate device memory (code under graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * operation, kernels and results as w4a16_gemm, without a workspace
 * argument.  Its split-K scratch is a library-owned static device array of
 * W4A16_NOALLOC_SCRATCH_BYTES bytes on each GPU the library runs on, held
 * until the process ends; the call allocates nothing.  Shapes whose
 * w4a16_workspace_size exceeds that array are rejected with
 * W4A16_ERR_UNSUPPORTED (every benchmark shape up to M = 32 fits).  The first
 * call on a device looks the array up and enqueues a clear of its arrival
 * counters on `stream`; every call leaves them zero.  All calls on one GPU
 * share the array: calls that overlap in time on one GPU (different streams
 * or threads) race and their results are undefined; calls made one after
 * another, on any streams, are fine.  Errors as w4a16_gemm; W4A16_ERR_LAUNCH
 * also reports a failed lookup of the array.
 */
#define W4A16_NOALLOC_SCRATCH_BYTES (16u << 20)
w4a16_status_t w4a16_gemm_noalloc(const uint8_t* wq, const uint8_t* ws, const float* g,
                                  const uint16_t* x, uint16_t* y, int M, int N, int K,
                                  hipStream_t stream);

/*
 * Fused MLP input projections with SwiGLU:
 *   a = x * Wg^T,  b = x * Wu^T  (both fp32, each with its own g),
 *   y[M][N] = bf16( silu(a) * b ),  silu(a) = a / (1 + exp(-a)).
 * x is read once for both matrices; gate and up are separate tensors (no
 * concatenated copy is needed).  Same alignment, shape and workspace rules as
 * w4a16_gemm; workspace size from w4a16_workspace_size_gate_up(M, N, K).
 * The gate/up fusion and a SwiGLU kernel appear on the FlashRT page
 * (section 4, MLP gate/up fusion) and the qwen36-fp4 README (kernel list).
 */
w4a16_status_t w4a16_gemm_gate_up_swiglu(const uint8_t* wq_gate, const uint8_t* ws_gate,
                                         const float* g_gate, const uint8_t* wq_up,
                                         const uint8_t* ws_up, const float* g_up,
                                         const uint16_t* x, uint16_t* y, int M, int N, int K,
                                         void* workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/*
 * Head projection with greedy selection: for each activation row m, the row
 * index n of the largest fp32 logit x[m] . W[n] / g (the value that the matmul
 * would round to bf16), ties to the smaller n; a NaN logit is never selected
 * (idx = -1 if every logit of a row is NaN).  idx[m] gets the index and
 * val[m] that logit.  No logits are written.  The qwen36-fp4 README lists
 * greedy sampling among its kernels and an option fusing the lm_head with a
 * greedy argmax that avoids the logits buffer (its "CUDA Runtime Knobs").
 *   idx : int32 [M], val : fp32 [M], both device memory, 4-byte aligned.
 *   Other pointers, alignment and shape rules as w4a16_gemm (1 <= M <= 32).
 *   At 1 <= M <= 2 the shape must not need a K split (the x rows a
 *   workgroup stages must fit in LDS; K = 5120 fits), else
 *   W4A16_ERR_UNSUPPORTED; from M = 3 on a K split is taken when x needs it
 *   (at K = 5120, M > 12): fp32 partial logits go through the workspace and
 *   the last workgroup of each row block forms its candidates.
 *   workspace : at least w4a16_workspace_size_argmax(M, N, K) bytes (never 0
 *               for a supported shape), 16-byte aligned; its first 4096 bytes
 *               must be zero before the first call and are left zero by
 *               every call; the rest needs no initialisation.
 */
w4a16_status_t w4a16_gemm_argmax(const uint8_t* wq, const uint8_t* ws, const float* g,
                                 const uint16_t* x, int32_t* idx, float* val, int M, int N, int K,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace w4a16_gemm_argmax needs (0 = unsupported shape). */
size_t w4a16_workspace_size_argmax(int M, int N, int K);

/*
 * Dequantise to fp32: w[N][K] = e2m1 * e4m3 / g, the product exact and the
 * division IEEE fp32 (correctly rounded), so the result is bit-exact for
 * every finite value; a NaN scale gives NaN.  wq, ws : 16-byte aligned;
 * w : 16-byte aligned; K % 256 == 0.  For tests and debugging.
 */
w4a16_status_t w4a16_dequant(const uint8_t* wq, const uint8_t* ws, const float* g, float* w,
                             int N, int K, hipStream_t stream);

/*
 * NVFP4 encoding of a weight matrix w[N][K] (fp32: w4a16_quantize; bf16 bit
 * patterns: w4a16_quantize_bf16) into the schema above.  The pages give the
 * schema, not the block-scale recipe; the recipe implemented is:
 *   amax = max |w|;  g = fp32(448 / amax)  (g = 1 when amax = 0);
 *   per 16-input block: S = the E4M3FN value nearest to max|w_block| * g / 6
 *   (ties to the even code, saturating at 448); if S = 0 the block's codes
 *   are 0, else each code is the E2M1 value nearest to w * g / S (ties to the
 *   even code, saturating at 6, sign kept, so -0 can occur);
 *   all in fp64 in that order.  Every output byte and g equal the scalar fp64
 *   evaluation of that recipe (bit-exact).
 *   w, wq : 16-byte aligned;  g : one fp32 in device memory, 4-byte aligned;
 *   K % 16 == 0 (the matmul entry points further need K % 256 == 0).
 *   workspace : at least w4a16_quantize_workspace_size(N, K) bytes, 16-byte
 *               aligned, no initialisation needed.
 *   Inputs are expected finite: NaN elements are ignored by the maxima, and an
 *   infinite element makes g = 0 and every code 0.
 * For converting a higher-precision checkpoint at load time: FlashRT (sections
 * 0 and 1) serves checkpoints already in this schema and converts its
 * drafter head to NVFP4 when loading it.
 */
w4a16_status_t w4a16_quantize(const float* w, uint8_t* wq, uint8_t* ws, float* g, int N, int K,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);
w4a16_status_t w4a16_quantize_bf16(const uint16_t* w, uint8_t* wq, uint8_t* ws, float* g, int N,
                                   int K, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/*
 * A decoder layer's MLP block in one call:
 *   h[M][F] = bf16( silu(x * Wg^T) * (x * Wu^T) )   (as w4a16_gemm_gate_up_swiglu)
 *   y[M][H] = bf16( h * Wd^T )                       (as w4a16_gemm)
 * with Wg, Wu : [F][H] and Wd : [H][F] in the schema above (each with its own
 * g), x : bf16 [M][H], y : bf16 [M][H].  Same alignment rules as w4a16_gemm
 * for every matrix; H % 256 == 0 and F % 256 == 0; 1 <= M <= 32.
 * The qwentin README lists a persistent-MLP GEMV among its kernels and sizes
 * grids to one wave of multiprocessors ("How it works", "Performance").
 * By default the block runs as two kernels on `stream`.  With options->launch
 * = W4A16_MLP_ONE_LAUNCH both matmuls run in ONE persistent launch with a
 * device-wide barrier between them, when the two launch plans allow it (same
 * kernel family and block size, and neither phase on the K-column kernel
 * that K = 5120 takes at 3 <= M <= 8; see w4a16_mlp_one_launch) and the
 * stream is not being captured into a graph.  That launch is cooperative: the runtime
 * either makes every workgroup resident at once or refuses it, and a refused
 * launch falls back to the two kernels.  The results are bit-identical
 * either way.
 *   options   : NULL for the defaults, else per-call settings (below); the
 *               library keeps no option state between calls.
 *   workspace : at least w4a16_workspace_size_mlp(M, H, F) bytes (never 0 for
 *               a supported shape), 256-byte aligned.  Its first
 *               W4A16_MLP_H_OFFSET bytes hold counters and barrier words:
 *               they must be ZERO BEFORE THE FIRST CALL and every call leaves
 *               them zero, except the barrier's generation word (the int at
 *               W4A16_MLP_GENERATION_OFFSET), which may hold any value and
 *               changes with every one-launch call.  h is left at byte
 *               offset W4A16_MLP_H_OFFSET (bf16 [M][F]).  The barrier waits
 *               at most options->spin_limit polls per workgroup: if one
 *               stops waiting (only a deliberately tiny limit can make that
 *               happen, since the launch is cooperative), the int at byte
 *               offset W4A16_MLP_TIMEOUT_OFFSET becomes 1 and y of that call
 *               is undefined; the flag stays set until the caller clears it.
 *               Calls that share a workspace must not overlap in time.
 */
#define W4A16_MLP_H_OFFSET 10240
#define W4A16_MLP_GENERATION_OFFSET 9344
#define W4A16_MLP_TIMEOUT_OFFSET 9472
#define W4A16_MLP_TWO_LAUNCHES 0
#define W4A16_MLP_ONE_LAUNCH 1
typedef struct {
  int launch;      /* W4A16_MLP_TWO_LAUNCHES (default) or W4A16_MLP_ONE_LAUNCH */
  int spin_limit;  /* barrier polls before a workgroup stops waiting; < 0 = 2^20 */
} w4a16_mlp_options_t;
w4a16_status_t w4a16_mlp_swiglu(const uint8_t* wq_gate, const uint8_t* ws_gate,
                                const float* g_gate, const uint8_t* wq_up, const uint8_t* ws_up,
                                const float* g_up, const uint8_t* wq_down, const uint8_t* ws_down,
                                const float* g_down, const uint16_t* x, uint16_t* y, int M, int H,
                                int F, void* workspace, size_t workspace_bytes,
                                const w4a16_mlp_options_t* options, hipStream_t stream);

/* Bytes of workspace w4a16_mlp_swiglu needs (0 = unsupported shape). */
size_t w4a16_workspace_size_mlp(int M, int H, int F);

/* 1 if w4a16_mlp_swiglu can run this shape in one launch on the current
 * device (the plans match and the whole grid fits on the device at once), 0
 * if it always takes two, -1 if the shape is unsupported. */
int w4a16_mlp_one_launch(int M, int H, int F);

/* Bytes of workspace w4a16_quantize[_bf16] needs (0 = unsupported shape). */
size_t w4a16_quantize_workspace_size(int N, int K);

/* Bytes of workspace w4a16_gemm needs for this shape (0 = none, or an
 * unsupported shape). */
size_t w4a16_workspace_size(int M, int N, int K);

/* Bytes of workspace w4a16_gemm_gate_up_swiglu needs for this shape. */
size_t w4a16_workspace_size_gate_up(int M, int N, int K);

/* Static English name of a status code (never NULL). */
const char* w4a16_status_string(w4a16_status_t status);

/* ABI version of this header: bumped on any incompatible change. */
#define W4A16_ABI_VERSION 4
int w4a16_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* W4A16_H */
