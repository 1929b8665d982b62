"""The C-ABI library without a GPU: it loads, exports every function that
include/w4a16.h declares, and its argument checks reject bad calls with the
documented status before touching the device."""
import ctypes
import os
import re

import pytest

import block_scaled_fp4_w4a16_amd as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(w4a16_[a-z0-9_]+)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(w4.library_path()):
        from block_scaled_fp4_w4a16_amd import build
        build.build()
    return w4.lib()


def test_header_declares_the_abi():
    names = declared_functions()
    for n in ("w4a16_gemm", "w4a16_gemm_gate_up_swiglu", "w4a16_dequant", "w4a16_workspace_size",
              "w4a16_workspace_size_gate_up", "w4a16_status_string", "w4a16_abi_version",
              "w4a16_mlp_swiglu", "w4a16_workspace_size_mlp", "w4a16_mlp_one_launch"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(w4.library_path())
    for n in declared_functions():
        assert hasattr(raw, n), f"{n} declared in w4a16.h but not exported"


def test_abi_version_and_status_strings(lib):
    assert lib.w4a16_abi_version() == 4
    for st in (0, 1, 2, 3):
        assert len(w4.status_string(st)) > 0
    assert w4.status_string(99) == "unknown status"


P = 0x10000  # a fake, 16-byte aligned "device" address: never dereferenced on these paths


def call_gemm(lib, wq=P, ws=P, g=P, x=P, y=P, M=1, N=64, K=256, work=0, wbytes=0):
    return lib.w4a16_gemm(wq, ws, g, x, y, M, N, K, work, wbytes, None)


def call_fused(lib, wq=P, ws=P, g=P, x=P, y=P, M=1, N=64, K=256, work=0, wbytes=0):
    return lib.w4a16_gemm_gate_up_swiglu(wq, ws, g, wq, ws, g, x, y, M, N, K, work, wbytes, None)


def call_noalloc(lib, wq=P, ws=P, g=P, x=P, y=P, M=1, N=64, K=256, work=0, wbytes=0):
    return lib.w4a16_gemm_noalloc(wq, ws, g, x, y, M, N, K, None)


def test_noalloc_rejects_bad_calls_and_oversize_shapes(lib):
    for arg in ("wq", "ws", "g", "x", "y"):
        assert call_noalloc(lib, **{arg: 0}) == w4.ERR_INVALID_VALUE, arg
    assert call_noalloc(lib, M=0) == w4.ERR_INVALID_VALUE
    assert call_noalloc(lib, M=33) == w4.ERR_UNSUPPORTED
    assert call_noalloc(lib, K=272) == w4.ERR_UNSUPPORTED
    assert call_noalloc(lib, x=P + 8) == w4.ERR_UNSUPPORTED
    # the head at M = 32 needs more split-K scratch than the static array holds
    assert w4.workspace_size(32, 248320, 5120) > w4.NOALLOC_SCRATCH_BYTES
    assert call_noalloc(lib, M=32, N=248320, K=5120) == w4.ERR_UNSUPPORTED
    hdr = open(HEADER).read()
    assert re.search(r"#define W4A16_NOALLOC_SCRATCH_BYTES \(16u << 20\)", hdr)
    assert w4.NOALLOC_SCRATCH_BYTES == 16 << 20
    # every benchmark shape up to M = 32 fits
    for M, N, K in ((32, 5120, 17408), (32, 17408, 5120), (32, 5120, 5120)):
        assert w4.workspace_size(M, N, K) <= w4.NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("call", [call_gemm, call_fused])
def test_null_pointers_rejected(lib, call):
    for arg in ("wq", "ws", "g", "x", "y"):
        assert call(lib, **{arg: 0}) == w4.ERR_INVALID_VALUE, arg


@pytest.mark.parametrize("call", [call_gemm, call_fused])
def test_bad_sizes_rejected(lib, call):
    assert call(lib, M=0) == w4.ERR_INVALID_VALUE
    assert call(lib, N=0) == w4.ERR_INVALID_VALUE
    assert call(lib, K=0) == w4.ERR_INVALID_VALUE
    assert call(lib, M=-3) == w4.ERR_INVALID_VALUE
    assert call(lib, M=33) == w4.ERR_UNSUPPORTED
    assert call(lib, K=272) == w4.ERR_UNSUPPORTED      # multiple of 16 but not of 256
    assert call(lib, K=128) == w4.ERR_UNSUPPORTED


@pytest.mark.parametrize("call", [call_gemm, call_fused])
def test_misaligned_pointers_rejected(lib, call):
    assert call(lib, wq=P + 8) == w4.ERR_UNSUPPORTED
    assert call(lib, ws=P + 4) == w4.ERR_UNSUPPORTED
    assert call(lib, x=P + 2) == w4.ERR_UNSUPPORTED
    assert call(lib, g=P + 2) == w4.ERR_UNSUPPORTED
    assert call(lib, y=P + 2) == w4.ERR_UNSUPPORTED


def test_workspace_sizes(lib):
    # small x: no split, no workspace
    assert w4.workspace_size(1, 5120, 5120) == 0
    assert w4.workspace_size_gate_up(7, 17408, 5120) == 0
    # 8 rows of a 17408-wide x do not fit in LDS: K is split; the workspace
    # holds the row-block arrival counters (a fixed 4096 bytes) and the fp32
    # partials of every slice
    for M, N, K, fused in [(7, 5120, 17408, False), (8, 5120, 17408, False), (8, 512, 17408, True)]:
        size = (w4.workspace_size_gate_up if fused else w4.workspace_size)(M, N, K)
        S, counters = divmod(size - 4096, M * N * 4 * (2 if fused else 1))
        assert S >= 2 and counters == 0, (M, N, K, size)
    assert w4.workspace_size(33, 64, 256) == 0            # unsupported shape: 0
    # the down projection at 3 <= M <= 8 runs the K-column kernel in exactly two
    # K-slices (one workgroup per slice and row block)
    for M in (3, 4, 5, 6, 7, 8):
        assert w4.workspace_size(M, 5120, 17408) == 4096 + 2 * M * 5120 * 4, M
    # the MLP block's workspace holds what either launch plan of each phase needs
    for M in (1, 3, 4, 7, 8, 16):
        assert w4.workspace_size_mlp(M, 5120, 17408) >= (
            w4.MLP_H_OFFSET + M * 17408 * 2 + max(0, w4.workspace_size_gate_up(M, 17408, 5120) - 4096)
            + max(0, w4.workspace_size(M, 5120, 17408) - 4096)), M


def test_wide_kernel_workspace(lib):
    # 13 <= M <= 32 (gate/up: 17) with K a multiple of 512: one launch of the
    # wide kernel, whose split-K partials follow the arrival counters.  At 256
    # CUs the down projection takes 12 K-slices of 1536 inputs at M >= 17
    # (x: 96 KiB of LDS) and 6 of 3072 at M <= 16, gate/up 4 slices (two
    # partial sets each), the square 5 slices.
    assert w4.workspace_size(32, 5120, 17408) == 4096 + 12 * 32 * 5120 * 4
    assert w4.workspace_size(17, 5120, 17408) == 4096 + 12 * 17 * 5120 * 4
    assert w4.workspace_size(16, 5120, 17408) == 4096 + 6 * 16 * 5120 * 4
    assert w4.workspace_size(13, 5120, 17408) == 4096 + 6 * 13 * 5120 * 4
    assert w4.workspace_size_gate_up(32, 17408, 5120) == 4096 + 2 * 4 * 32 * 17408 * 4
    assert w4.workspace_size(32, 5120, 5120) == 4096 + 5 * 32 * 5120 * 4
    # K not a multiple of 512 stays on the 4x4x4 kernel (two launches of rows
    # where its K split would be fine): a different workspace
    assert w4.workspace_size(32, 5120, 17152) != 4096 + 12 * 32 * 5120 * 4


def test_short_workspace_rejected(lib):
    need = w4.workspace_size(8, 5120, 17408)
    assert call_gemm(lib, M=8, N=5120, K=17408, work=P, wbytes=need - 1) == w4.ERR_INVALID_VALUE
    assert call_gemm(lib, M=8, N=5120, K=17408, work=0, wbytes=need) == w4.ERR_INVALID_VALUE
    assert call_gemm(lib, M=8, N=5120, K=17408, work=P + 4, wbytes=need) == w4.ERR_UNSUPPORTED


def test_dequant_argument_checks(lib):
    assert lib.w4a16_dequant(0, P, P, P, 4, 256, None) == w4.ERR_INVALID_VALUE
    assert lib.w4a16_dequant(P, P, P, P, 0, 256, None) == w4.ERR_INVALID_VALUE
    assert lib.w4a16_dequant(P, P, P, P, 4, 272, None) == w4.ERR_UNSUPPORTED
    assert lib.w4a16_dequant(P, P, P, P + 4, 4, 256, None) == w4.ERR_UNSUPPORTED


def test_python_binding_rejects_host_tensors():
    import torch
    wq = torch.zeros((4, 128), dtype=torch.uint8)
    ws = torch.zeros((4, 16), dtype=torch.uint8)
    g = torch.ones(1)
    x = torch.zeros((1, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        w4.gemm(wq, ws, g, x)


def call_quant(lib, w=P, wq=P, ws=P, g=P, N=4, K=32, work=P, wbytes=4096, bf16=False):
    fn = lib.w4a16_quantize_bf16 if bf16 else lib.w4a16_quantize
    return fn(w, wq, ws, g, N, K, work, wbytes, None)


@pytest.mark.parametrize("bf16", [False, True])
def test_quantize_argument_checks(lib, bf16):
    for arg in ("w", "wq", "ws", "g", "work"):
        assert call_quant(lib, bf16=bf16, **{arg: 0}) == w4.ERR_INVALID_VALUE, arg
    assert call_quant(lib, bf16=bf16, N=0) == w4.ERR_INVALID_VALUE
    assert call_quant(lib, bf16=bf16, K=-16) == w4.ERR_INVALID_VALUE
    assert call_quant(lib, bf16=bf16, K=24) == w4.ERR_UNSUPPORTED          # K % 16 != 0
    assert call_quant(lib, bf16=bf16, w=P + 8) == w4.ERR_UNSUPPORTED
    assert call_quant(lib, bf16=bf16, wq=P + 8) == w4.ERR_UNSUPPORTED
    assert call_quant(lib, bf16=bf16, g=P + 2) == w4.ERR_UNSUPPORTED
    assert call_quant(lib, bf16=bf16, wbytes=0) == w4.ERR_INVALID_VALUE   # short workspace


def test_quantize_workspace_size(lib):
    assert lib.w4a16_quantize_workspace_size(5120, 5120) >= 4
    assert lib.w4a16_quantize_workspace_size(5120, 5120) % 256 == 0
    assert lib.w4a16_quantize_workspace_size(3, 24) == 0
    assert lib.w4a16_quantize_workspace_size(0, 32) == 0


def test_argmax_argument_checks(lib):
    def call(wq=P, ws=P, g=P, x=P, idx=P, val=P, M=1, N=64, K=256, work=P, wbytes=1 << 20):
        return lib.w4a16_gemm_argmax(wq, ws, g, x, idx, val, M, N, K, work, wbytes, None)
    for arg in ("wq", "ws", "g", "x", "idx", "val"):
        assert call(**{arg: 0}) == w4.ERR_INVALID_VALUE, arg
    assert call(work=0, wbytes=0) == w4.ERR_INVALID_VALUE     # the workspace is always required
    assert call(idx=P + 2) == w4.ERR_UNSUPPORTED
    assert call(M=33) == w4.ERR_UNSUPPORTED
    # 13 x rows of 5120 need a K split: the workspace then also holds fp32 partial logits
    assert w4.workspace_size_argmax(13, 1000, 5120) >= 4096 + 2 * 13 * 1000 * 4
    assert 4096 < w4.workspace_size_argmax(12, 1000, 5120) < 4096 + 12 * 1000 * 4
    assert w4.workspace_size_argmax(1, 248320, 5120) >= 4096 + 8
    # the head at 3 <= M <= 8 runs the K-column kernel's ring variant, one row
    # block per CU (256 here, without a device): the arrival counter, then one
    # (value, index) candidate per row block and activation row
    for M in range(3, 9):
        assert w4.workspace_size_argmax(M, 248320, 5120) == 4096 + 256 * M * 2 * 4, M
    assert w4.workspace_size_argmax(16, 64, 17408) >= 4096 + 16 * 64 * 4
    assert w4.workspace_size_argmax(2, 64, 65536) == 0         # M <= 2 takes no K split


# ---- MLP block -----------------------------------------------------------------

def call_mlp(lib, ptrs=None, M=1, H=256, F=512, work=P, wbytes=1 << 30, opts=None):
    p = dict(wq_g=P, ws_g=P, g_g=P, wq_u=P, ws_u=P, g_u=P, wq_d=P, ws_d=P, g_d=P, x=P, y=P)
    p.update(ptrs or {})
    return lib.w4a16_mlp_swiglu(*p.values(), M, H, F, work, wbytes,
                                None if opts is None else ctypes.byref(opts), None)


def test_mlp_argument_checks(lib):
    for arg in ("wq_g", "ws_g", "g_g", "wq_u", "ws_u", "g_u", "wq_d", "ws_d", "g_d", "x", "y"):
        assert call_mlp(lib, {arg: 0}) == w4.ERR_INVALID_VALUE, arg
    assert call_mlp(lib, M=0) == w4.ERR_INVALID_VALUE
    assert call_mlp(lib, M=33) == w4.ERR_UNSUPPORTED
    assert call_mlp(lib, H=272) == w4.ERR_UNSUPPORTED
    assert call_mlp(lib, F=400) == w4.ERR_UNSUPPORTED
    for arg, off in (("wq_g", 8), ("ws_u", 4), ("wq_d", 8), ("x", 2), ("g_d", 2), ("y", 2)):
        assert call_mlp(lib, {arg: P + off}) == w4.ERR_UNSUPPORTED, arg
    need = w4.workspace_size_mlp(1, 256, 512)
    assert call_mlp(lib, work=0, wbytes=need) == w4.ERR_INVALID_VALUE        # h lives there
    assert call_mlp(lib, wbytes=need - 1) == w4.ERR_INVALID_VALUE
    assert call_mlp(lib, work=P + 16, wbytes=need) == w4.ERR_UNSUPPORTED     # 256-byte alignment


def test_mlp_workspace_layout(lib):
    # no K split in either phase: counters and barrier words, then h (bf16 [M][F])
    assert w4.workspace_size_mlp(1, 5120, 17408) == w4.MLP_H_OFFSET + 17408 * 2
    assert w4.workspace_size_mlp(3, 256, 512) == w4.MLP_H_OFFSET + 3 * 512 * 2
    # M = 7: the down projection splits K=17408; its fp32 partials follow h
    size = w4.workspace_size_mlp(7, 5120, 17408)
    down = w4.workspace_size(7, 5120, 17408) - 4096
    assert size == w4.MLP_H_OFFSET + ((7 * 17408 * 2 + 255) // 256) * 256 + down
    assert w4.workspace_size_mlp(33, 256, 512) == 0
    assert w4.workspace_size_mlp(1, 272, 512) == 0
    assert w4.MLP_H_OFFSET % 256 == 0
    assert 8192 <= w4.MLP_GENERATION_OFFSET < w4.MLP_TIMEOUT_OFFSET < w4.MLP_H_OFFSET
    hdr = open(HEADER).read()
    for name in ("H_OFFSET", "GENERATION_OFFSET", "TIMEOUT_OFFSET"):
        assert re.search(rf"#define W4A16_MLP_{name} {getattr(w4, 'MLP_' + name)}\b", hdr), name
    assert lib.w4a16_mlp_one_launch(33, 256, 512) == -1


def test_mlp_options_are_per_call_and_checked(lib):
    # an unknown launch mode is rejected before anything is enqueued; there is
    # no process-wide option setter any more
    assert call_mlp(lib, opts=w4.MlpOptions(2, -1)) == w4.ERR_INVALID_VALUE
    assert call_mlp(lib, opts=w4.MlpOptions(-1, -1)) == w4.ERR_INVALID_VALUE
    assert not hasattr(lib, "w4a16_mlp_set_options")
    hdr = open(HEADER).read()
    assert "w4a16_mlp_options_t" in hdr and "set_options" not in hdr
    assert re.search(r"#define W4A16_MLP_TWO_LAUNCHES 0\b", hdr)
    assert re.search(r"#define W4A16_MLP_ONE_LAUNCH 1\b", hdr)


def test_calibration_library_rejects_bad_arguments_without_a_gpu():
    """The benchmark's HBM calibration library (not part of the matmul ABI):
    it loads, exports its one entry point, and rejects bad arguments before
    touching the device."""
    import ctypes
    import os
    path = os.path.join(os.path.dirname(w4.library_path()), "libw4a16_calib.so")
    lib = ctypes.CDLL(path)
    f = lib.w4a16_calib_stream_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p]
    f.restype = ctypes.c_int
    P = 1 << 20                                   # a 16-byte aligned stand-in address
    assert f(0, 1024, P, 1, 64, None) != 0        # null buffer
    assert f(P, 1024, 0, 1, 64, None) != 0        # null sink
    assert f(P, 1000, P, 1, 64, None) != 0        # size not a multiple of 16
    assert f(P + 4, 1024, P, 1, 64, None) != 0    # misaligned buffer
    assert f(P, 1024, P, 0, 64, None) != 0        # empty grid
    assert f(P, 1024, P, 1, 2048, None) != 0      # block above 1024
    assert f(P, 1024, P, 1, 100, None) != 0       # block not whole waves
