"""CPU oracle for the NVFP4 W4A16 matmul (fp64, plain loops in C).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library under ``block_scaled_fp4_w4a16_amd/``: neither side
imports, links or includes the other.  The arithmetic lives in
``nvfp4_oracle.c``; this module only marshals numpy arrays into it.

Follows FlashRT, "Qwen3.6-27B NVFP4 on RTX 5090", section 1 "Model
dependencies" (the nvfp4-pack-quantized tensor schema and w = e2m1*e4m3/g).
Every function is pinned by ``tests/test_oracle_*.py``; none is parity unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libnvfp4_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, strict IEEE: no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    _lib = _bind(_LIB_PATH)
    return _lib


def _bind(path):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int64
    lib.nvfp4_oracle_e2m1.argtypes = [ctypes.c_int]
    lib.nvfp4_oracle_e2m1.restype = ctypes.c_double
    lib.nvfp4_oracle_e4m3.argtypes = [ctypes.c_int]
    lib.nvfp4_oracle_e4m3.restype = ctypes.c_double
    lib.nvfp4_oracle_e4m3_encode.argtypes = [ctypes.c_double]
    lib.nvfp4_oracle_e4m3_encode.restype = ctypes.c_int
    lib.nvfp4_oracle_e2m1_encode.argtypes = [ctypes.c_double]
    lib.nvfp4_oracle_e2m1_encode.restype = ctypes.c_int
    lib.nvfp4_oracle_silu.argtypes = [ctypes.c_double]
    lib.nvfp4_oracle_silu.restype = ctypes.c_double
    lib.nvfp4_oracle_dequant_f64.argtypes = [P, P, ctypes.c_float, I, I, P]
    lib.nvfp4_oracle_dequant_f64.restype = None
    lib.nvfp4_oracle_dequant_f32.argtypes = [P, P, ctypes.c_float, I, I, P]
    lib.nvfp4_oracle_dequant_f32.restype = None
    lib.nvfp4_oracle_gemm.argtypes = [P, P, ctypes.c_float, P, I, I, I, P, P, ctypes.c_int]
    lib.nvfp4_oracle_gemm.restype = None
    lib.nvfp4_oracle_gemm_rows.argtypes = [P, P, ctypes.c_float, P, I, I, P, I, P, P]
    lib.nvfp4_oracle_gemm_rows.restype = None
    lib.nvfp4_oracle_gate_up_swiglu.argtypes = [P, P, ctypes.c_float, P, P, ctypes.c_float, P,
                                                I, I, I, P, P, P, P, P, ctypes.c_int]
    lib.nvfp4_oracle_gate_up_swiglu.restype = None
    lib.nvfp4_oracle_quantize.argtypes = [P, I, I, P, P, P]
    lib.nvfp4_oracle_quantize.restype = None
    lib.nvfp4_oracle_bf16_rne.argtypes = [ctypes.c_double]
    lib.nvfp4_oracle_bf16_rne.restype = ctypes.c_uint16
    lib.nvfp4_oracle_bf16_rne_array.argtypes = [P, I, P]
    lib.nvfp4_oracle_bf16_rne_array.restype = None
    lib.nvfp4_oracle_max_threads.argtypes = []
    lib.nvfp4_oracle_max_threads.restype = ctypes.c_int
    return lib


class use_library:
    """Context manager: route this module's calls to another build of the
    oracle source (the mutation tests load deliberately broken copies)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self._saved = _load()
        _lib = _bind(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self._saved
        return False


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _check_weights(wq, ws, N, K):
    if K % 16 != 0 or K <= 0 or N <= 0:
        raise ValueError(f"oracle needs K a positive multiple of 16 and N > 0, got N={N} K={K}")
    if wq.shape != (N, K // 2) or ws.shape != (N, K // 16):
        raise ValueError(f"weight shapes {wq.shape}, {ws.shape} do not match N={N} K={K}")


# ---- element decoders -------------------------------------------------------

def e2m1(code: int) -> float:
    """Value of a 4-bit E2M1 code (OCP MX element type)."""
    return _load().nvfp4_oracle_e2m1(int(code))


def e4m3(byte: int) -> float:
    """Value of an 8-bit E4M3FN code (NaN for 0x7F / 0xFF)."""
    return _load().nvfp4_oracle_e4m3(int(byte))


def e4m3_encode(t: float) -> int:
    return _load().nvfp4_oracle_e4m3_encode(float(t))


def e2m1_encode(v: float) -> int:
    return _load().nvfp4_oracle_e2m1_encode(float(v))


def silu(v: float) -> float:
    return _load().nvfp4_oracle_silu(float(v))


# ---- dequant / matmul / fused ----------------------------------------------

def dequant_f64(wq, ws, g, N, K) -> np.ndarray:
    wq = _c(wq, np.uint8); ws = _c(ws, np.uint8)
    _check_weights(wq, ws, N, K)
    out = np.empty((N, K), dtype=np.float64)
    _load().nvfp4_oracle_dequant_f64(_ptr(wq), _ptr(ws), float(np.float32(g)), N, K, _ptr(out))
    return out


def dequant_f32(wq, ws, g, N, K) -> np.ndarray:
    wq = _c(wq, np.uint8); ws = _c(ws, np.uint8)
    _check_weights(wq, ws, N, K)
    out = np.empty((N, K), dtype=np.float32)
    _load().nvfp4_oracle_dequant_f32(_ptr(wq), _ptr(ws), float(np.float32(g)), N, K, _ptr(out))
    return out


def gemm(wq, ws, g, x_bf16_bits, M, N, K, nthreads: int = 1):
    """Return (y, a): y[m,n] = sum_k x W^T in fp64, a[m,n] = sum_k |x W|."""
    wq = _c(wq, np.uint8); ws = _c(ws, np.uint8)
    x = _c(x_bf16_bits, np.uint16).reshape(M, K)
    _check_weights(wq, ws, N, K)
    y = np.empty((M, N), dtype=np.float64)
    a = np.empty((M, N), dtype=np.float64)
    _load().nvfp4_oracle_gemm(_ptr(wq), _ptr(ws), float(np.float32(g)), _ptr(x), M, N, K,
                              _ptr(y), _ptr(a), int(nthreads))
    return y, a


def gemm_rows(wq, ws, g, x_bf16_bits, M, K, rows):
    """(y, a) for the listed output rows only: arrays [M][len(rows)]."""
    wq = _c(wq, np.uint8); ws = _c(ws, np.uint8)
    x = _c(x_bf16_bits, np.uint16).reshape(M, K)
    rows = _c(rows, np.int64)
    if wq.ndim != 2 or wq.shape[1] != K // 2 or ws.shape[1] != K // 16:
        raise ValueError("weight shapes do not match K")
    if rows.size and (rows.min() < 0 or rows.max() >= wq.shape[0]):
        raise ValueError("row index out of range")
    y = np.empty((M, rows.size), dtype=np.float64)
    a = np.empty((M, rows.size), dtype=np.float64)
    _load().nvfp4_oracle_gemm_rows(_ptr(wq), _ptr(ws), float(np.float32(g)), _ptr(x), M, K,
                                   _ptr(rows), rows.size, _ptr(y), _ptr(a))
    return y, a


def gate_up_swiglu(wq_g, ws_g, g_g, wq_u, ws_u, g_u, x_bf16_bits, M, N, K, nthreads: int = 1):
    """Return dict with y = silu(gate)*up and gate, up, a_gate, a_up (all fp64 [M][N])."""
    wq_g = _c(wq_g, np.uint8); ws_g = _c(ws_g, np.uint8)
    wq_u = _c(wq_u, np.uint8); ws_u = _c(ws_u, np.uint8)
    _check_weights(wq_g, ws_g, N, K)
    _check_weights(wq_u, ws_u, N, K)
    x = _c(x_bf16_bits, np.uint16).reshape(M, K)
    out = {k: np.empty((M, N), dtype=np.float64) for k in ("y", "gate", "up", "a_gate", "a_up")}
    _load().nvfp4_oracle_gate_up_swiglu(
        _ptr(wq_g), _ptr(ws_g), float(np.float32(g_g)), _ptr(wq_u), _ptr(ws_u),
        float(np.float32(g_u)), _ptr(x), M, N, K, _ptr(out["y"]), _ptr(out["gate"]),
        _ptr(out["up"]), _ptr(out["a_gate"]), _ptr(out["a_up"]), int(nthreads))
    return out


def bf16_rne(v) -> np.ndarray:
    """fp64 values -> bf16 bit patterns (uint16), nearest, ties to even."""
    v = _c(v, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().nvfp4_oracle_bf16_rne_array(_ptr(v), v.size, _ptr(out))
    return out


def mlp_swiglu(gate, up, down, x_bf16_bits, M, H, F, nthreads: int = 1):
    """The MLP block: h = bf16(silu(x Wg^T) * (x Wu^T)) [M][F], then
    y = h Wd^T [M][H] in fp64.  gate, up, down: (wq, ws, g); Wg, Wu are
    [F][H], Wd is [H][F].  Returns dict with y, a (sum |h w|), h (exact
    fp64 silu(gate)*up), h_bits (bf16 of h) and the gate/up dict."""
    r = gate_up_swiglu(*gate, *up, x_bf16_bits, M, F, H, nthreads=nthreads)
    h_bits = bf16_rne(r["y"])
    y, a = gemm(*down, h_bits, M, H, F, nthreads=nthreads)
    return dict(y=y, a=a, h=r["y"], h_bits=h_bits, gate_up=r)


def quantize(w_f32, N, K):
    """NVFP4-encode fp32 W [N][K]: returns (wq u8 [N][K/2], ws u8 [N][K/16], g fp32)."""
    w = _c(w_f32, np.float32).reshape(N, K)
    if K % 16 != 0:
        raise ValueError("K must be a multiple of 16")
    wq = np.empty((N, K // 2), dtype=np.uint8)
    ws = np.empty((N, K // 16), dtype=np.uint8)
    g = np.zeros(1, dtype=np.float32)
    _load().nvfp4_oracle_quantize(_ptr(w), N, K, _ptr(wq), _ptr(ws), _ptr(g))
    return wq, ws, np.float32(g[0])


def max_threads() -> int:
    return int(_load().nvfp4_oracle_max_threads())


# ---- accuracy bounds (the pass criteria parity tests apply) ---------------

def gemm_bound(a):
    """Allowed |y_gpu - y_ref| for the plain matmul: 1e-2 * sum|x w| + 1e-6."""
    return 1e-2 * np.asarray(a) + 1e-6


def mlp_bound(out, down_abs):
    """Allowed |y_gpu - y_ref| for the MLP block.  With B the gate/up bound on
    |h_gpu - h| (h exact), the oracle's h_bits within 2^-9 |h| of h, and the
    matmul bound on the down projection of h_gpu:
        1e-2 * sum_k |h_gpu| |w| + sum_k |w| |h_gpu - h_bits| + 1e-6
     <= sum_k |w_k| * ((1 + 1e-2) B_k + (1e-2 + 2^-9) |h_k|) + 1e-6.
    down_abs: |Wd| in fp64, [H][F]."""
    r = out["gate_up"]
    b = swiglu_bound(r["gate"], r["up"], r["a_gate"], r["a_up"])
    c = (1.0 + 1e-2) * b + (1e-2 + 2.0 ** -9) * np.abs(out["h"])
    return c @ np.asarray(down_abs).T + 1e-6


def swiglu_bound(gate, up, a_gate, a_up):
    """Allowed |y_gpu - y_ref| for silu(gate)*up, propagated to first order from
    the matmul bound E = 1e-2*A + 1e-6 on each pre-activation: |silu'| <= 1.1,
    plus 2^-8 relative for the bf16 output rounding."""
    e_a = gemm_bound(a_gate)
    e_b = gemm_bound(a_up)
    silu_a = gate / (1.0 + np.exp(-gate))
    y = silu_a * up
    core = 1.1 * np.abs(up) * e_a + np.abs(silu_a) * e_b + 1.1 * e_a * e_b
    return core * (1.0 + 2.0 ** -8) + 2.0 ** -8 * np.abs(y) + 1e-6
