"""The no-allocation entry point (w4a16_gemm_noalloc) against w4a16_gemm.

Same operation and kernels; the split-K scratch is the library's static device
array instead of a caller workspace.  On exact-arithmetic inputs both must give
the same bf16 output bit for bit, which is also bf16(exact) (the oracle).  Two
calls in a row, the second with a smaller input, so the second runs on the
scratch the first left behind; both split-K and unsplit shapes.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_w4a16_amd as w4
import oracle
from tests import exact

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _case(seed, M, N, K):
    wq, ws, g, x = exact.exact_gemm_case(seed, M, N, K)
    dx = _dev(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    return (wq, ws, g, x), (_dev(wq), _dev(ws), torch.tensor([float(g)], device="cuda"), dx)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w4.lib()


# (M, N, K) pairs: the first call, then a smaller one
SEQUENCES = [
    ((8, 5120, 17408), (5, 1003, 17408)),     # both split K (the down projection shape, then smaller)
    ((16, 2048, 17408), (2, 640, 17408)),     # split K, then the VALU kernel's split
    ((7, 5120, 5120), (1, 512, 5120)),        # no split, then no split
]


@pytest.mark.parametrize("first,second", SEQUENCES)
def test_noalloc_matches_gemm_two_calls(first, second):
    for i, (M, N, K) in enumerate((first, second)):
        need = w4.workspace_size(M, N, K)
        assert need <= w4.NOALLOC_SCRATCH_BYTES
        host, dev = _case(2000 + 17 * i + M, M, N, K)
        print(f"[noalloc] call {i}: M={M} N={N} K={K} (split-K scratch {need} B)", flush=True)
        y_na = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        w4.gemm_noalloc(*dev, y=y_na)
        y_ws = w4.gemm(*dev)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(y_na), _bits(y_ws)), f"call {i}: noalloc differs from gemm"
        ref, a = oracle.gemm(*host, M, N, K, nthreads=8)
        exact.assert_exact_regime(a, host[2], "pow2")
        exact.assert_bits_exact(_bits(y_na), ref, f"noalloc call {i}")


def test_noalloc_rejects_shapes_beyond_its_scratch():
    M, N, K = 32, 248320, 5120                # the head at M = 32 needs ~127 MB of partials
    assert w4.workspace_size(M, N, K) > w4.NOALLOC_SCRATCH_BYTES
    wq = torch.zeros((N, K // 2), dtype=torch.uint8, device="cuda")
    ws = torch.zeros((N, K // 16), dtype=torch.uint8, device="cuda")
    g = torch.ones(1, device="cuda")
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(w4.W4A16Error) as e:
        w4.gemm_noalloc(wq, ws, g, x)
    assert e.value.status == w4.ERR_UNSUPPORTED


def test_noalloc_under_graph_capture_replays():
    M, N, K = 8, 5120, 17408
    host, dev = _case(2100, M, N, K)
    eager = w4.gemm_noalloc(*dev).clone()
    y = torch.empty_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        w4.gemm_noalloc(*dev, y=y)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        w4.gemm_noalloc(*dev, y=y)
    for _ in range(3):
        y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        _ = (dev[3].float() * 2).sum().item()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16))
