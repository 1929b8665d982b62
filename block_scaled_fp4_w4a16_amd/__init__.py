"""NVFP4 (block-scaled FP4) weight-only matmul for MI355X: Python binding.

Thin ctypes layer over ``libw4a16.so`` (hand-written HIP kernels for gfx950,
C ABI declared in ``include/w4a16.h``).  This module only checks tensor
metadata, allocates outputs with torch and passes raw device pointers and the
current HIP stream to the library: every arithmetic step runs in the library's
kernels.  There is no fallback: if the library is not built, importing the
functions raises.

Weight layout (FlashRT, "Qwen3.6-27B NVFP4 on RTX 5090", section 1 "Model
dependencies"): ``wq`` uint8 [N, K/2] packed E2M1 codes (low nibble = even
input), ``ws`` uint8 [N, K/16] E4M3 block scales, ``g`` float32 [1] global
scale; W = e2m1 * e4m3 / g.  Activations ``x`` are bfloat16 [M, K].
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["gemm", "gemm_noalloc", "gemm_gate_up_swiglu", "gemm_argmax", "dequant", "quantize", "workspace_size",
           "workspace_size_argmax",
           "workspace_size_gate_up", "new_workspace", "W4A16Error", "library_path", "lib", "MAX_M"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libw4a16.so")
_lib = None
MAX_M = 32

OK, ERR_INVALID_VALUE, ERR_UNSUPPORTED, ERR_LAUNCH = 0, 1, 2, 3


class W4A16Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class MlpBarrierTimeout(RuntimeError):
    """A one-launch MLP call stopped waiting at its grid barrier: its y is
    undefined (the workspace's time-out flag is set)."""


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded libw4a16.so (ctypes); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run `python -m block_scaled_fp4_w4a16_amd.build`"
                          " (hipcc, gfx950). There is no non-HIP fallback.")
    L = ctypes.CDLL(_LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.w4a16_gemm.argtypes = [P, P, P, P, P, I, I, I, P, Z, P]
    L.w4a16_gemm.restype = I
    L.w4a16_gemm_noalloc.argtypes = [P, P, P, P, P, I, I, I, P]
    L.w4a16_gemm_noalloc.restype = I
    L.w4a16_gemm_gate_up_swiglu.argtypes = [P, P, P, P, P, P, P, P, I, I, I, P, Z, P]
    L.w4a16_gemm_gate_up_swiglu.restype = I
    L.w4a16_dequant.argtypes = [P, P, P, P, I, I, P]
    L.w4a16_dequant.restype = I
    L.w4a16_gemm_argmax.argtypes = [P, P, P, P, P, P, I, I, I, P, Z, P]
    L.w4a16_gemm_argmax.restype = I
    L.w4a16_workspace_size_argmax.argtypes = [I, I, I]
    L.w4a16_workspace_size_argmax.restype = Z
    L.w4a16_quantize.argtypes = [P, P, P, P, I, I, P, Z, P]
    L.w4a16_quantize.restype = I
    L.w4a16_quantize_bf16.argtypes = [P, P, P, P, I, I, P, Z, P]
    L.w4a16_quantize_bf16.restype = I
    L.w4a16_quantize_workspace_size.argtypes = [I, I]
    L.w4a16_quantize_workspace_size.restype = Z
    L.w4a16_workspace_size.argtypes = [I, I, I]
    L.w4a16_workspace_size.restype = Z
    L.w4a16_workspace_size_gate_up.argtypes = [I, I, I]
    L.w4a16_workspace_size_gate_up.restype = Z
    L.w4a16_status_string.argtypes = [I]
    L.w4a16_status_string.restype = ctypes.c_char_p
    L.w4a16_abi_version.argtypes = []
    L.w4a16_abi_version.restype = I
    L.w4a16_mlp_swiglu.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, P, Z,
                                   ctypes.POINTER(MlpOptions), P]
    L.w4a16_mlp_swiglu.restype = I
    L.w4a16_workspace_size_mlp.argtypes = [I, I, I]
    L.w4a16_workspace_size_mlp.restype = Z
    L.w4a16_mlp_one_launch.argtypes = [I, I, I]
    L.w4a16_mlp_one_launch.restype = I
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().w4a16_status_string(int(status)).decode()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(t, name, dtype, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def workspace_size(M: int, N: int, K: int) -> int:
    return int(lib().w4a16_workspace_size(M, N, K))


def workspace_size_gate_up(M: int, N: int, K: int) -> int:
    return int(lib().w4a16_workspace_size_gate_up(M, N, K))


def _weights(wq, ws, g, name):
    _check(wq, f"{name}wq", torch.uint8, 2)
    _check(ws, f"{name}ws", torch.uint8, 2)
    _check(g, f"{name}g", torch.float32, None)
    N, K = wq.shape[0], wq.shape[1] * 2
    if tuple(ws.shape) != (N, K // 16) or g.numel() != 1:
        raise ValueError(f"{name}weights: wq {tuple(wq.shape)}, ws {tuple(ws.shape)}, g {tuple(g.shape)} "
                         "do not form an NVFP4 tensor")
    return N, K


def _workspace(workspace, need, device):
    """The caller's workspace, or a fresh zero-filled one when the shape needs
    one: split-K arrival counters sit at its start and must be zero before the
    first call that uses it (every call leaves them zero again)."""
    if need == 0:
        return workspace, (workspace.numel() * workspace.element_size() if workspace is not None else 0)
    if workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=device)
    _check(workspace, "workspace", workspace.dtype, None)
    return workspace, workspace.numel() * workspace.element_size()


def new_workspace(M: int, N: int, K: int, device, fused: bool = False):
    """A zero-filled workspace for (M, N, K) (at least 16 bytes), reusable by
    any number of calls of that shape made one after another."""
    need = (workspace_size_gate_up if fused else workspace_size)(M, N, K)
    return torch.zeros(max(need, 16), dtype=torch.uint8, device=device)


def gemm(wq, ws, g, x, y=None, workspace=None, stream=None):
    """y[M, N] = bf16(x[M, K] @ W^T) with W the NVFP4 tensor (wq, ws, g)."""
    N, K = _weights(wq, ws, g, "")
    _check(x, "x", torch.bfloat16, 2)
    M = x.shape[0]
    if x.shape[1] != K:
        raise ValueError(f"x has K={x.shape[1]}, weights have K={K}")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check(y, "y", torch.bfloat16, 2)
    if tuple(y.shape) != (M, N):
        raise ValueError(f"y must be ({M}, {N})")
    if workspace is None:
        need = workspace_size(M, N, K) if M <= MAX_M else 0
        workspace, wbytes = _workspace(None, need, x.device)
    else:
        workspace, wbytes = _workspace(workspace, 1, x.device)
    st = lib().w4a16_gemm(_ptr(wq), _ptr(ws), _ptr(g), _ptr(x), _ptr(y), M, N, K,
                          _ptr(workspace), wbytes, _stream(stream))
    if st != OK:
        raise W4A16Error(st, "w4a16_gemm")
    return y


NOALLOC_SCRATCH_BYTES = 16 << 20   # W4A16_NOALLOC_SCRATCH_BYTES


def gemm_noalloc(wq, ws, g, x, y=None, stream=None):
    """gemm without a workspace: the library's own static device scratch holds
    the split-K partials (for callers that cannot allocate).  y must be given
    by such a caller; calls that overlap in time on one GPU race."""
    N, K = _weights(wq, ws, g, "")
    _check(x, "x", torch.bfloat16, 2)
    M = x.shape[0]
    if x.shape[1] != K:
        raise ValueError(f"x has K={x.shape[1]}, weights have K={K}")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check(y, "y", torch.bfloat16, 2)
    if tuple(y.shape) != (M, N):
        raise ValueError(f"y must be ({M}, {N})")
    st = lib().w4a16_gemm_noalloc(_ptr(wq), _ptr(ws), _ptr(g), _ptr(x), _ptr(y), M, N, K,
                                  _stream(stream))
    if st != OK:
        raise W4A16Error(st, "w4a16_gemm_noalloc")
    return y


def gemm_gate_up_swiglu(wq_gate, ws_gate, g_gate, wq_up, ws_up, g_up, x, y=None,
                        workspace=None, stream=None):
    """y[M, N] = bf16(silu(x @ Wg^T) * (x @ Wu^T)), x read once."""
    N, K = _weights(wq_gate, ws_gate, g_gate, "gate ")
    N2, K2 = _weights(wq_up, ws_up, g_up, "up ")
    if (N, K) != (N2, K2):
        raise ValueError("gate and up weights must have the same shape")
    _check(x, "x", torch.bfloat16, 2)
    M = x.shape[0]
    if x.shape[1] != K:
        raise ValueError(f"x has K={x.shape[1]}, weights have K={K}")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check(y, "y", torch.bfloat16, 2)
    if tuple(y.shape) != (M, N):
        raise ValueError(f"y must be ({M}, {N})")
    workspace, wbytes = _workspace(workspace, workspace_size_gate_up(M, N, K) if M <= MAX_M else 0,
                                   x.device)
    st = lib().w4a16_gemm_gate_up_swiglu(_ptr(wq_gate), _ptr(ws_gate), _ptr(g_gate), _ptr(wq_up),
                                         _ptr(ws_up), _ptr(g_up), _ptr(x), _ptr(y), M, N, K,
                                         _ptr(workspace), wbytes, _stream(stream))
    if st != OK:
        raise W4A16Error(st, "w4a16_gemm_gate_up_swiglu")
    return y


# Byte offsets inside the MLP workspace (include/w4a16.h): h (bf16 [M][F]), the
# barrier's generation word (any value) and its time-out flag.
MLP_H_OFFSET = 10240
MLP_GENERATION_OFFSET = 9344
MLP_TIMEOUT_OFFSET = 9472


def workspace_size_mlp(M: int, H: int, F: int) -> int:
    return int(lib().w4a16_workspace_size_mlp(M, H, F))


def mlp_one_launch(M: int, H: int, F: int) -> int:
    """1: the block can run in one persistent launch on the current device
    (when asked to, outside graph capture); 0: always two launches;
    -1: unsupported."""
    return int(lib().w4a16_mlp_one_launch(M, H, F))


MLP_TWO_LAUNCHES, MLP_ONE_LAUNCH = 0, 1


class MlpOptions(ctypes.Structure):
    """w4a16_mlp_options_t: per-call settings of w4a16_mlp_swiglu."""
    _fields_ = [("launch", ctypes.c_int), ("spin_limit", ctypes.c_int)]


def mlp_timed_out(workspace) -> bool:
    """Whether a one-launch call on this workspace stopped waiting at its
    barrier (its y is then undefined).  Reads the flag after the device's
    queued work: synchronises."""
    torch.cuda.synchronize(workspace.device)
    flag = workspace[MLP_TIMEOUT_OFFSET:MLP_TIMEOUT_OFFSET + 4].view(torch.int32).item()
    return flag != 0


def new_workspace_mlp(M: int, H: int, F: int, device):
    """A zero-filled MLP workspace, reusable by calls made one after another."""
    need = workspace_size_mlp(M, H, F)
    if need == 0:
        raise W4A16Error(ERR_UNSUPPORTED, "w4a16_workspace_size_mlp")
    return torch.zeros(need, dtype=torch.uint8, device=device)


def mlp_swiglu(gate, up, down, x, y=None, workspace=None, stream=None, one_launch=False,
               spin_limit=-1, check_barrier=True):
    """y[M, H] = bf16(bf16(silu(x @ Wg^T) * (x @ Wu^T)) @ Wd^T): one MLP block.
    gate, up, down: (wq, ws, g) tuples; Wg, Wu are [F][H], Wd is [H][F].
    one_launch: run both matmuls in one cooperative persistent launch when
    the shape and the stream allow it (bit-identical to two launches);
    spin_limit: the barrier's poll limit (< 0: the library default).
    check_barrier: after a one-launch call on a stream that is not being
    captured, wait for it and raise MlpBarrierTimeout if its barrier timed
    out (leaving the flag set); False skips that synchronisation, and the
    caller reads the flag with mlp_timed_out()."""
    F, H = _weights(*gate, "gate ")
    if _weights(*up, "up ") != (F, H):
        raise ValueError("gate and up weights must have the same shape")
    if _weights(*down, "down ") != (H, F):
        raise ValueError(f"down weights must be [{H}][{F}] (codes [{H}][{F // 2}])")
    _check(x, "x", torch.bfloat16, 2)
    M = x.shape[0]
    if x.shape[1] != H:
        raise ValueError(f"x has K={x.shape[1]}, gate/up weights have K={H}")
    if y is None:
        y = torch.empty((M, H), dtype=torch.bfloat16, device=x.device)
    _check(y, "y", torch.bfloat16, 2)
    if tuple(y.shape) != (M, H):
        raise ValueError(f"y must be ({M}, {H})")
    if workspace is None:
        workspace = new_workspace_mlp(M, H, F, x.device) if M <= MAX_M else None
    else:
        _check(workspace, "workspace", workspace.dtype, None)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    opts = MlpOptions(MLP_ONE_LAUNCH if one_launch else MLP_TWO_LAUNCHES, int(spin_limit))
    st = lib().w4a16_mlp_swiglu(*[_ptr(t) for t in (*gate, *up, *down)], _ptr(x), _ptr(y), M, H, F,
                                _ptr(workspace), wbytes, ctypes.byref(opts), _stream(stream))
    if st != OK:
        raise W4A16Error(st, "w4a16_mlp_swiglu")
    if one_launch and check_barrier and workspace is not None and \
            not torch.cuda.is_current_stream_capturing():
        s = stream if stream is not None else torch.cuda.current_stream(x.device)
        s.synchronize()
        flag = workspace[MLP_TIMEOUT_OFFSET:MLP_TIMEOUT_OFFSET + 4].view(torch.int32).item()
        if flag != 0:
            raise MlpBarrierTimeout("w4a16_mlp_swiglu: the one-launch barrier timed out; y is undefined")
    return y


def workspace_size_argmax(M: int, N: int, K: int) -> int:
    return int(lib().w4a16_workspace_size_argmax(M, N, K))


def gemm_argmax(wq, ws, g, x, idx=None, val=None, workspace=None, stream=None):
    """Greedy selection over the head: (idx int32 [M], val float32 [M]) with
    idx[m] = argmax_n fp32(x[m] . W[n] / g) (ties to the smaller n) and val[m]
    that logit; no logits are materialised."""
    N, K = _weights(wq, ws, g, "")
    _check(x, "x", torch.bfloat16, 2)
    M = x.shape[0]
    if x.shape[1] != K:
        raise ValueError(f"x has K={x.shape[1]}, weights have K={K}")
    idx = torch.empty((M,), dtype=torch.int32, device=x.device) if idx is None else idx
    val = torch.empty((M,), dtype=torch.float32, device=x.device) if val is None else val
    _check(idx, "idx", torch.int32, 1)
    _check(val, "val", torch.float32, 1)
    if idx.numel() != M or val.numel() != M:
        raise ValueError(f"idx and val must have {M} elements")
    need = workspace_size_argmax(M, N, K) if M <= MAX_M else 0
    if workspace is None:
        workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=x.device)
    _check(workspace, "workspace", workspace.dtype, None)
    st = lib().w4a16_gemm_argmax(_ptr(wq), _ptr(ws), _ptr(g), _ptr(x), _ptr(idx), _ptr(val), M, N, K,
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(stream))
    if st != OK:
        raise W4A16Error(st, "w4a16_gemm_argmax")
    return idx, val


def quantize(w, wq=None, ws=None, g=None, workspace=None, stream=None):
    """NVFP4-encode w[N, K] (float32 or bfloat16): returns (wq u8 [N, K/2],
    ws u8 [N, K/16], g float32 [1]), bit-exact to the fp64 recipe."""
    if w.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"w must be float32 or bfloat16, got {w.dtype}")
    _check(w, "w", w.dtype, 2)
    N, K = w.shape
    dev = w.device
    wq = torch.empty((N, K // 2), dtype=torch.uint8, device=dev) if wq is None else wq
    ws = torch.empty((N, K // 16), dtype=torch.uint8, device=dev) if ws is None else ws
    g = torch.empty((1,), dtype=torch.float32, device=dev) if g is None else g
    _check(wq, "wq", torch.uint8, 2)
    _check(ws, "ws", torch.uint8, 2)
    _check(g, "g", torch.float32, None)
    if tuple(wq.shape) != (N, K // 2) or tuple(ws.shape) != (N, K // 16) or g.numel() != 1:
        raise ValueError("wq, ws, g do not match w's shape")
    need = int(lib().w4a16_quantize_workspace_size(N, K))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _check(workspace, "workspace", workspace.dtype, None)
    fn = lib().w4a16_quantize if w.dtype == torch.float32 else lib().w4a16_quantize_bf16
    st = fn(_ptr(w), _ptr(wq), _ptr(ws), _ptr(g), N, K, _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    if st != OK:
        raise W4A16Error(st, "w4a16_quantize")
    return wq, ws, g


def dequant(wq, ws, g, w=None, stream=None):
    """w[N, K] float32 = e2m1 * e4m3 / g (bit-exact)."""
    N, K = _weights(wq, ws, g, "")
    if w is None:
        w = torch.empty((N, K), dtype=torch.float32, device=wq.device)
    _check(w, "w", torch.float32, 2)
    if tuple(w.shape) != (N, K):
        raise ValueError(f"w must be ({N}, {K})")
    st = lib().w4a16_dequant(_ptr(wq), _ptr(ws), _ptr(g), _ptr(w), N, K, _stream(stream))
    if st != OK:
        raise W4A16Error(st, "w4a16_dequant")
    return w
