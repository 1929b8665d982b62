"""Seeded synthetic inputs for the NVFP4 W4A16 matmul (numpy, CPU).

This module is the only thing the CPU oracle (``oracle/``) and the HIP library
(``block_scaled_fp4_w4a16_amd``) have in common: tests and the benchmark draw
inputs here and hand the same bytes to both.  It imports neither of them and
contains none of their arithmetic (no decoding, no matmul); it draws random
numbers and writes them in the checkpoint's storage format.

Workload recipe (shapes from the FlashRT page "Qwen3.6-27B NVFP4 on RTX 5090",
section 1: hidden size 5120; MLP width 17408 and the head width 248320 are the
synthetic shapes of the benchmark configurations):
  * weights  W ~ N(0, 0.02) fp32 from ``numpy.random.default_rng(seed)``,
    stored as NVFP4: E2M1 codes two per byte (low nibble = even input), one
    E4M3 scale per 16 inputs along K, fp32 global scale g = 448/amax;
  * activations x ~ N(0, 1) rounded to bf16 (round to nearest even);
  * "SwiGLU-shaped" activations for the down projection: bf16(a*sigmoid(a)*b)
    with a, b ~ N(0, 1) independent (a heavy-tailed distribution).

Storage encoding used for the weights (the pages give only the schema; this
recipe is the plainest one consistent with g = 448/amax): per 16-block the
scale is the E4M3 value nearest to blockmax*g/6 (ties to even, saturating at
448); each weight's code is the E2M1 value nearest to W*g/scale (ties to the
even code, saturating at 6, sign kept); a block whose scale is 0 gets code 0.
The E4M3 value table comes from torch's float8_e4m3fn type; the E2M1 grid is
the OCP MX element table {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
"""
from __future__ import annotations

import numpy as np

SIGMA_W = 0.02

_E4M3_TABLE = None  # values of codes 0x00..0x7E, from torch's float8_e4m3fn


def _e4m3_table() -> np.ndarray:
    global _E4M3_TABLE
    if _E4M3_TABLE is None:
        import torch
        codes = torch.arange(0, 0x7F, dtype=torch.uint8)
        _E4M3_TABLE = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy().copy()
    return _E4M3_TABLE


def _nearest_even(t: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the grid value nearest to t >= 0 (grid increasing, starting at 0),
    ties to the even index, values past the end saturate to the last index."""
    hi = np.searchsorted(grid, t, side="left")          # first grid value >= t
    hi = np.minimum(hi, grid.size - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = t - grid[lo]
    dhi = grid[hi] - t
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(t >= grid[-1], grid.size - 1, idx)
    return idx.astype(np.int64)


# Decision thresholds between neighbouring E2M1 magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}:
# a magnitude t passes threshold i (moves up one code) when t > mid, or t >= mid
# where the tie goes to the upper (even) code.  Passing all 7 saturates at 6.
_E2M1_MIDS_UP_ON_TIE = (0.75, 1.75, 3.5)     # upper code 2, 4, 6 is even
_E2M1_MIDS_DOWN_ON_TIE = (0.25, 1.25, 2.5, 5.0)  # upper code 1, 3, 5, 7 is odd


def _e2m1_code_magnitude(t: np.ndarray) -> np.ndarray:
    c = np.zeros(t.shape, dtype=np.uint8)
    for m in _E2M1_MIDS_DOWN_ON_TIE:
        c += t > m
    for m in _E2M1_MIDS_UP_ON_TIE:
        c += t >= m
    return c


def encode_nvfp4(w: np.ndarray, rows_per_chunk: int = 1024):
    """Store fp32 W [N][K] in the NVFP4 schema: (wq u8 [N][K/2], ws u8 [N][K/16], g fp32)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    amax = float(np.abs(w).max()) if w.size else 0.0
    g = np.float32(448.0 / amax) if amax > 0 else np.float32(1.0)
    gd = np.float64(g)
    tab = _e4m3_table()
    wq = np.empty((N, K // 2), dtype=np.uint8)
    ws = np.empty((N, K // 16), dtype=np.uint8)
    for r0 in range(0, N, rows_per_chunk):
        r1 = min(N, r0 + rows_per_chunk)
        wc = w[r0:r1].astype(np.float64)                         # [n][K]
        bmax = np.abs(wc).reshape(r1 - r0, K // 16, 16).max(axis=2)
        t = bmax * gd / 6.0
        sc = _nearest_even(np.minimum(t, 448.0), tab).astype(np.uint8)
        sc[t <= 0] = 0
        ws[r0:r1] = sc
        S = tab[sc.astype(np.int64)]
        v = (wc * gd).reshape(r1 - r0, K // 16, 16) / np.where(S > 0, S, 1.0)[:, :, None]
        codes = _e2m1_code_magnitude(np.abs(v)) | (np.signbit(v).astype(np.uint8) << 3)
        codes[S <= 0] = 0
        codes = codes.reshape(r1 - r0, K)
        wq[r0:r1] = codes[:, 0::2] | (codes[:, 1::2] << 4)
    return wq, ws, np.float32(g)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def weights_f32(seed: int, N: int, K: int, sigma: float = SIGMA_W) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.standard_normal((N, K), dtype=np.float32) * np.float32(sigma)


def nvfp4_weights(seed: int, N: int, K: int, sigma: float = SIGMA_W):
    """Seeded N(0, sigma) weights stored as NVFP4: (wq, ws, g)."""
    return encode_nvfp4(weights_f32(seed, N, K, sigma))


def activations(seed: int, M: int, K: int) -> np.ndarray:
    """x ~ N(0, 1) as bf16 bits [M][K]."""
    rng = np.random.default_rng(seed)
    return bf16_bits(rng.standard_normal((M, K), dtype=np.float32))


def swiglu_activations(seed_a: int, seed_b: int, M: int, K: int) -> np.ndarray:
    """Heavy-tailed activations bf16(a*sigmoid(a)*b), a, b ~ N(0,1) iid, as bf16 bits."""
    a = np.random.default_rng(seed_a).standard_normal((M, K)).astype(np.float64)
    b = np.random.default_rng(seed_b).standard_normal((M, K)).astype(np.float64)
    return bf16_bits((a * b / (1.0 + np.exp(-a))).astype(np.float32))


def random_bytes(seed: int, shape) -> np.ndarray:
    """Uniform random bytes (any byte pattern is a legal code/scale input)."""
    return np.random.default_rng(seed).integers(0, 256, size=shape, dtype=np.uint8)


# ---- inputs on which fp32 accumulation is exact --------------------------------
# Scale bytes for exact-arithmetic inputs.  POW2: the E4M3FN codes of 0.5, 1, 2
# and 4 (exponent field 6..9, mantissa 0); MANT: the eight codes with exponent
# field 7, i.e. 1 + m/8 for m = 0..7.  The tests check these values against the
# oracle's decoder; this module only stores bytes.
EXACT_SCALES = {
    "pow2": np.array([0x30, 0x38, 0x40, 0x48], dtype=np.uint8),
    "mant": np.arange(0x38, 0x40, dtype=np.uint8),
}


def exact_weights(seed: int, N: int, K: int, scales: str = "pow2"):
    """Uniformly random code bytes and block scales drawn per (row, block) from
    EXACT_SCALES[scales]: (wq u8 [N][K/2], ws u8 [N][K/16])."""
    rng = np.random.default_rng(seed)
    wq = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    pick = rng.integers(0, EXACT_SCALES[scales].size, size=(N, K // 16))
    return wq, EXACT_SCALES[scales][pick]


def integer_activations(seed: int, M: int, K: int, lo: int = -2, hi: int = 2) -> np.ndarray:
    """x with integer values drawn uniformly from [lo, hi], as bf16 bits [M][K]."""
    rng = np.random.default_rng(seed)
    return bf16_bits(rng.integers(lo, hi + 1, size=(M, K)).astype(np.float32))


# Benchmark configurations: name -> dict(K, N, Ms, seeds, copies)
CONFIGS = {
    "tiny": dict(K=256, N=512, Ms=(1,), seed_w=11, seed_x=12, copies=1),
    "square": dict(K=5120, N=5120, Ms=(1,), seed_w=21, seed_x=22, copies=64),
    "gate_up": dict(K=5120, N=17408, Ms=(1, 7), seed_gate=31, seed_up=32, seed_x=33, copies=32),
    "down": dict(K=17408, N=5120, Ms=(1, 2, 4, 7, 8), seed_w=41, seed_a=42, seed_b=43, copies=32),
}
