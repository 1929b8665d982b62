"""GPU parity of the HIP library against the CPU oracle (needs an MI355X).

Every call goes through the C ABI (ctypes binding).  Inputs come from the
seeded generator in synth/; expected values come only from oracle/.
Pass criteria:
  * dequant: bit-exact fp32 (NaN positions equal);
  * matmul:  |y - y_ref| <= 1e-2 * sum_k |x w| + 1e-6 for every (m, n);
  * fused:   the first-order propagation of that bound through silu(a)*b
             (oracle.swiglu_bound);
  * closed-form cases (one-hot x with power-of-two g, sign flip, g -> 2g,
    run-to-run, row invariance across M) bit-exact.
"""
import os
import sys

import numpy as np
import pytest
import torch

import block_scaled_fp4_w4a16_amd as w4
import oracle
import synth

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)
_CACHE = {}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w4.lib()
    yield


# ---- host <-> device helpers --------------------------------------------------

def d_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def d_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda().view(
        torch.bfloat16)


def d_g(g):
    return torch.tensor([float(np.float32(g))], dtype=torch.float32, device="cuda")


def h_bf16(t):
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return synth.bf16_to_f32(bits).astype(np.float64)


def weights(seed, N, K):
    key = ("w", seed, N, K)
    if key not in _CACHE:
        _CACHE[key] = synth.nvfp4_weights(seed, N, K)
    return _CACHE[key]


def report_and_check(y, ref, bound, ctx):
    err = np.abs(y - ref)
    ratio = float(np.max(err / bound))
    bad = ~(err <= bound)
    say(f"  {ctx}: max |err|/bound = {ratio:.3e}")
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{ctx}: {int(bad.sum())} outputs outside the bound; first at {tuple(i)}: "
                             f"gpu {y[tuple(i)]!r} ref {ref[tuple(i)]!r} bound {bound[tuple(i)]!r}")


def run_gemm(wq, ws, g, x_bits, M, N, K):
    dwq, dws, dg, dx = d_u8(wq), d_u8(ws), d_g(g), d_bf16(x_bits)
    y = w4.gemm(dwq, dws, dg, dx)
    torch.cuda.synchronize()
    return h_bf16(y)


def check_gemm(wq, ws, g, x_bits, M, N, K, ctx):
    say(f"[gemm] {ctx} M={M} N={N} K={K}")
    y = run_gemm(wq, ws, g, x_bits, M, N, K)
    ref, a = oracle.gemm(wq, ws, g, x_bits, M, N, K, nthreads=NTHREADS)
    report_and_check(y, ref, oracle.gemm_bound(a), ctx)
    return y


def check_fused(wq_g, ws_g, g_g, wq_u, ws_u, g_u, x_bits, M, N, K, ctx):
    say(f"[fused] {ctx} M={M} N={N} K={K}")
    y = w4.gemm_gate_up_swiglu(d_u8(wq_g), d_u8(ws_g), d_g(g_g), d_u8(wq_u), d_u8(ws_u), d_g(g_u),
                               d_bf16(x_bits))
    torch.cuda.synchronize()
    y = h_bf16(y)
    r = oracle.gate_up_swiglu(wq_g, ws_g, g_g, wq_u, ws_u, g_u, x_bits, M, N, K, nthreads=NTHREADS)
    report_and_check(y, r["y"], oracle.swiglu_bound(r["gate"], r["up"], r["a_gate"], r["a_up"]), ctx)
    return y


# ---- dequant: bit-exact -------------------------------------------------------

def _all_codes_all_scales():
    """N = 256 rows x K = 256: row n uses scale byte n in every block; the codes
    of each row run through all 256 (low, high) nibble pairs."""
    N, K = 256, 256
    wq = np.tile(np.arange(256, dtype=np.uint8)[None, :128], (N, 1))
    wq[:, :] = (np.arange(128, dtype=np.uint16)[None, :] * 2 + np.arange(N)[:, None]) % 256
    ws = np.repeat(np.arange(256, dtype=np.uint8)[:, None], K // 16, axis=1)
    return wq.astype(np.uint8), ws, N, K


def assert_bits_equal_f32(gpu, ref, ctx):
    gnan, rnan = np.isnan(gpu), np.isnan(ref)
    assert np.array_equal(gnan, rnan), f"{ctx}: NaN positions differ"
    gb = gpu.view(np.uint32)[~gnan]
    rb = ref.view(np.uint32)[~rnan]
    bad = gb != rb
    assert not bad.any(), f"{ctx}: {int(bad.sum())} values differ in bits"


@pytest.mark.parametrize("g", [1.0, 4071.6726, 448.0 / 0.0873, 2.0 ** -3, 3.0e-5, 1.0e30, 3.0e38])
def test_dequant_every_code_and_scale_bit_exact(g):
    wq, ws, N, K = _all_codes_all_scales()
    say(f"[dequant] all codes x scales, g={g}")
    w = w4.dequant(d_u8(wq), d_u8(ws), d_g(g))
    torch.cuda.synchronize()
    assert_bits_equal_f32(w.cpu().numpy(), oracle.dequant_f32(wq, ws, g, N, K), f"g={g}")


@pytest.mark.parametrize("N,K,seed", [(5120, 5120, 21), (37, 17408, 41), (1, 256, 3)])
def test_dequant_generated_weights_bit_exact(N, K, seed):
    say(f"[dequant] N={N} K={K}")
    wq, ws, g = weights(seed, N, K)
    w = w4.dequant(d_u8(wq), d_u8(ws), d_g(g))
    torch.cuda.synchronize()
    assert_bits_equal_f32(w.cpu().numpy(), oracle.dequant_f32(wq, ws, g, N, K), f"N={N} K={K}")


# ---- the benchmark configurations at full size ------------------------------

def test_tiny_config():
    c = synth.CONFIGS["tiny"]
    wq, ws, g = weights(c["seed_w"], c["N"], c["K"])
    check_gemm(wq, ws, g, synth.activations(c["seed_x"], 1, c["K"]), 1, c["N"], c["K"], "tiny")


@pytest.mark.parametrize("M", [1, 7])
def test_square_config(M):
    """M = 1 is the benchmark's value; M = 7, a verify block on the same
    weights and seeds, is the second figure its line reports."""
    c = synth.CONFIGS["square"]
    wq, ws, g = weights(c["seed_w"], c["N"], c["K"])
    check_gemm(wq, ws, g, synth.activations(c["seed_x"], M, c["K"]), M, c["N"], c["K"], f"square M={M}")


@pytest.mark.parametrize("M", [1, 7])
def test_gate_up_config(M):
    c = synth.CONFIGS["gate_up"]
    N, K = c["N"], c["K"]
    wg = weights(c["seed_gate"], N, K)
    wu = weights(c["seed_up"], N, K)
    check_fused(*wg, *wu, synth.activations(c["seed_x"], M, K), M, N, K, f"gate_up M={M}")


@pytest.mark.parametrize("M", [1, 2, 4, 7, 8])
def test_down_config(M):
    c = synth.CONFIGS["down"]
    N, K = c["N"], c["K"]
    wq, ws, g = weights(c["seed_w"], N, K)
    x = synth.swiglu_activations(c["seed_a"], c["seed_b"], M, K)
    check_gemm(wq, ws, g, x, M, N, K, f"down M={M}")


# ---- every M, ragged shapes, edge cases ---------------------------------------

@pytest.mark.parametrize("M", list(range(1, 33)))
def test_every_m_ragged_n(M):
    N, K = 1003, 1280      # N not a multiple of any row group; K/32 = 40 chunks
    wq, ws, g = weights(100, N, K)
    check_gemm(wq, ws, g, synth.activations(200 + M, M, K), M, N, K, f"ragged M={M}")


@pytest.mark.parametrize("M", [1, 2, 3, 4, 7, 16, 17, 32])
def test_fused_every_family_ragged_n(M):
    N, K = 777, 768
    wg, wu = weights(101, N, K), weights(102, N, K)
    check_fused(*wg, *wu, synth.activations(300 + M, M, K), M, N, K, f"fused ragged M={M}")


@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (16, 1, 256), (3, 2, 256), (5, 3, 512), (16, 5, 256),
                                   (16, 64, 8192), (16, 33, 17408), (2, 7, 33024), (32, 1, 256),
                                   (32, 64, 17408), (20, 33, 5120), (25, 640, 5120)])
def test_small_and_extreme_shapes(M, N, K):
    wq, ws, g = weights(7 + N, N, K)
    check_gemm(wq, ws, g, synth.activations(M * 1000 + N, M, K), M, N, K, "shape")


def test_uniform_random_bytes():
    # any byte pattern is a legal input: random codes and random finite scales
    M, N, K = 7, 300, 2048
    wq = synth.random_bytes(1, (N, K // 2))
    ws = synth.random_bytes(2, (N, K // 16)) & np.uint8(0x77)   # finite, both signs, up to 2^8
    ws |= synth.random_bytes(3, (N, K // 16)) & np.uint8(0x80)
    for MM in (1, 3, M):
        check_gemm(wq, ws, np.float32(1234.5), synth.activations(5, MM, K), MM, N, K, "random bytes")


def test_nan_scale_propagates_to_its_row_only():
    M, N, K = 3, 40, 512
    wq, ws, g = weights(8, N, K)
    ws = ws.copy()
    ws[17, 5] = 0x7F
    for MM in (1, M, 5):
        y = run_gemm(wq, ws, g, synth.activations(9, MM, K), MM, N, K)
        assert np.isnan(y[:, 17]).all()
        assert not np.isnan(np.delete(y, 17, axis=1)).any()


@pytest.mark.parametrize("M", [1, 2, 3, 7, 8, 16, 32])
def test_uniform_random_bytes_at_k5120(M):
    """The K = 5120 kernels (whole-row for M <= 2, K-column for 3 <= M <= 8,
    MFMA for 9 <= M <= 12, wide for 13 <= M <= 32) on every code byte and
    random finite scales of both signs."""
    N, K = 300, 5120
    wq = synth.random_bytes(21, (N, K // 2))
    ws = synth.random_bytes(22, (N, K // 16)) & np.uint8(0x77)
    ws |= synth.random_bytes(23, (N, K // 16)) & np.uint8(0x80)
    check_gemm(wq, ws, np.float32(1234.5), synth.activations(24 + M, M, K), M, N, K, "random bytes K=5120")


@pytest.mark.parametrize("M", [1, 4, 8, 16, 17, 32])
def test_nan_scale_propagates_to_its_row_only_at_k5120(M):
    """A NaN block scale (E4M3 0x7F) in one row reaches that row's outputs
    only, through the K = 5120 kernels' lane, block and wave reductions (the
    wide kernel: one MFMA result column, its K-slice partial and the
    split-K sum)."""
    N, K = 300, 5120
    wq, ws, g = weights(25, N, K)
    ws = ws.copy()
    ws[130, 201] = 0x7F
    y = run_gemm(wq, ws, g, synth.activations(26, M, K), M, N, K)
    assert np.isnan(y[:, 130]).all()
    assert not np.isnan(np.delete(y, 130, axis=1)).any()
    wu, su, gu = weights(27, N, K)
    yf = w4.gemm_gate_up_swiglu(d_u8(wq), d_u8(ws), d_g(g), d_u8(wu), d_u8(su), d_g(gu),
                                d_bf16(synth.activations(26, M, K)))
    yf = h_bf16(yf)
    assert np.isnan(yf[:, 130]).all()
    assert not np.isnan(np.delete(yf, 130, axis=1)).any()


def test_nan_scale_propagates_to_its_row_only_on_the_ring():
    """The same through the K-column kernel's ring variant (110 000 rows at
    M = 5: partials added every two loop iterations): the NaN row lies in the
    middle of a row block's walk."""
    M, N, K = 5, 110000, 5120
    wq = synth.random_bytes(28, (N, K // 2))
    ws = (synth.random_bytes(29, (N, K // 16)) & np.uint8(0x37)) | np.uint8(0x08)   # finite, positive
    ws[70001, 77] = 0x7F
    y = run_gemm(wq, ws, np.float32(512.0), synth.activations(30, M, K), M, N, K)
    assert np.isnan(y[:, 70001]).all()
    assert not np.isnan(np.delete(y, 70001, axis=1)).any()


def test_zero_weights_give_zero():
    for M in (1, 5):
        N, K = 50, 256
        y = run_gemm(np.zeros((N, K // 2), np.uint8), np.zeros((N, K // 16), np.uint8),
                     np.float32(1.0), synth.activations(10, M, K), M, N, K)
        assert not y.any()


# ---- closed-form cases: bit-exact --------------------------------------------

@pytest.mark.parametrize("M", [1, 2, 4, 9])
def test_one_hot_x_with_power_of_two_g_is_exact(M):
    N, K = 96, 1024
    wq, ws, _ = weights(11, N, K)
    g = np.float32(2.0 ** 11)
    w_ref = oracle.dequant_f64(wq, ws, g, N, K)
    ks = [0, 1, 15, 16, 31, 32, 513, 1023, 700][:M]
    x = np.zeros((M, K), np.uint16)
    for m, k in enumerate(ks):
        x[m, k] = 0x3F80
    y = run_gemm(wq, ws, g, x, M, N, K)
    for m, k in enumerate(ks):
        expect = synth.bf16_to_f32(synth.bf16_bits(w_ref[:, k].astype(np.float32))).astype(np.float64)
        assert np.array_equal(expect, w_ref[:, k])        # representable exactly in bf16
        assert np.array_equal(y[m], expect), (m, k)


@pytest.mark.parametrize("M", [1, 3, 7])
def test_sign_flip_negates_and_doubling_g_halves(M):
    N, K = 200, 2048
    wq, ws, g = weights(12, N, K)
    x = synth.activations(13, M, K)
    y = run_gemm(wq, ws, g, x, M, N, K)
    y_neg = run_gemm(wq ^ np.uint8(0x88), ws, g, x, M, N, K)
    y_half = run_gemm(wq, ws, np.float32(2 * g), x, M, N, K)
    assert np.array_equal(y_neg, -y)
    assert np.array_equal(y_half, y / 2)


@pytest.mark.parametrize("M,N,K", [(1, 5120, 5120), (7, 5120, 17408), (7, 17408, 5120)])
def test_run_to_run_bitwise(M, N, K):
    wq, ws, g = weights(14, N, K)
    x = d_bf16(synth.activations(15, M, K))
    dwq, dws, dg = d_u8(wq), d_u8(ws), d_g(g)
    ys = [w4.gemm(dwq, dws, dg, x).view(torch.int16).cpu() for _ in range(3)]
    assert all(torch.equal(ys[0], t) for t in ys[1:])


@pytest.mark.parametrize("family,Ms", [("valu", (1, 2)), ("k-column", (3, 4, 5, 8)),
                                       ("wide", (17, 21, 24, 32)),
                                       ("wide, 16 rows of x", (13, 14, 16))])
def test_rows_do_not_depend_on_m_within_a_kernel_family(family, Ms):
    N, K = 300, 5120
    wq, ws, g = weights(16, N, K)
    xall = synth.activations(17, max(Ms), K)
    outs = [run_gemm(wq, ws, g, xall[:M], M, N, K) for M in Ms]
    for M, y in zip(Ms, outs):
        common = min(Ms)
        assert np.array_equal(y[:common], outs[0][:common]), (family, M)


# ---- boundary behaviour on the device -----------------------------------------

def test_unsupported_shapes_raise():
    wq, ws, g = weights(18, 16, 256)
    with pytest.raises(w4.W4A16Error) as e:
        w4.gemm(d_u8(wq), d_u8(ws), d_g(g), d_bf16(synth.activations(1, 33, 256)))
    assert e.value.status == w4.ERR_UNSUPPORTED


def test_split_k_workspace_is_required_and_used():
    M, N, K = 8, 640, 17408
    assert w4.workspace_size(M, N, K) > 0
    wq, ws, g = weights(19, N, K)
    x = synth.activations(20, M, K)
    lib = w4.lib()
    dwq, dws, dg, dx = d_u8(wq), d_u8(ws), d_g(g), d_bf16(x)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    st = lib.w4a16_gemm(dwq.data_ptr(), dws.data_ptr(), dg.data_ptr(), dx.data_ptr(), y.data_ptr(),
                        M, N, K, None, 0, None)
    assert st == w4.ERR_INVALID_VALUE
    # the arrival counters at the start must be zero; the fp32 partials after
    # them need no initialisation: fill everything past the first 4 KiB (the
    # counter area) with garbage
    size = w4.workspace_size(M, N, K)
    work = torch.zeros((size,), dtype=torch.uint8, device="cuda")
    work[4096:] = 0x7F
    y = w4.gemm(dwq, dws, dg, dx, workspace=work)
    torch.cuda.synchronize()
    ref, a = oracle.gemm(wq, ws, g, x, M, N, K, nthreads=NTHREADS)
    report_and_check(h_bf16(y), ref, oracle.gemm_bound(a), "split-K garbage partials")
    # every call leaves the counters (the first 4096 bytes) zero
    assert int(work[:4096].count_nonzero()) == 0


def test_split_k_workspace_reused_by_many_calls():
    # one zero-fill, then split and unsplit calls of several shapes back to
    # back on one workspace, each checked against the oracle, twice
    work = torch.zeros((1 << 22,), dtype=torch.uint8, device="cuda")
    cases = [(8, 640, 17408, False), (5, 1003, 17408, False), (16, 96, 33024, False),
             (7, 5120, 17408, False), (6, 200, 17408, True), (2, 640, 17408, False),
             (32, 1003, 17408, False), (20, 777, 5120, True), (13, 640, 5120, False)]
    for i, (M, N, K, fused) in enumerate(cases):
        need = (w4.workspace_size_gate_up if fused else w4.workspace_size)(M, N, K)
        assert need <= work.numel()
        wq, ws, g = weights(50 + i, N, K)
        x = synth.activations(60 + i, M, K)
        for rep in range(2):
            if fused:
                y = w4.gemm_gate_up_swiglu(d_u8(wq), d_u8(ws), d_g(g), d_u8(wq), d_u8(ws), d_g(g),
                                           d_bf16(x), workspace=work)
            else:
                y = w4.gemm(d_u8(wq), d_u8(ws), d_g(g), d_bf16(x), workspace=work)
            torch.cuda.synchronize()
            if fused:
                r = oracle.gate_up_swiglu(wq, ws, g, wq, ws, g, x, M, N, K, nthreads=NTHREADS)
                report_and_check(h_bf16(y), r["y"], oracle.swiglu_bound(r["gate"], r["up"], r["a_gate"],
                                                                          r["a_up"]), f"reuse fused {i}")
            else:
                ref, a = oracle.gemm(wq, ws, g, x, M, N, K, nthreads=NTHREADS)
                report_and_check(h_bf16(y), ref, oracle.gemm_bound(a), f"reuse {M}x{N}x{K} #{rep}")
    assert int(work[:4096].count_nonzero()) == 0


def test_graph_capture_replays_match_eager():
    # M = 16 and 32 of the down projection: the wide kernel (split-K partials,
    # arrival counters reset by each call's finishing workgroup)
    cases = [(1, 5120, 5120), (7, 5120, 17408), (16, 5120, 17408), (32, 5120, 17408)]
    for M, N, K in cases:
        wq, ws, g = weights(22, N, K)
        dwq, dws, dg = d_u8(wq), d_u8(ws), d_g(g)
        dx = d_bf16(synth.activations(23, M, K))
        work = w4.new_workspace(M, N, K, "cuda")
        eager = w4.gemm(dwq, dws, dg, dx, workspace=work).clone()
        y = torch.empty_like(eager)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            w4.gemm(dwq, dws, dg, dx, y=y, workspace=work)   # warm up on the capture stream
        torch.cuda.current_stream().wait_stream(s)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            w4.gemm(dwq, dws, dg, dx, y=y, workspace=work)
        for _ in range(3):
            y.zero_()
            graph.replay()
            torch.cuda.synchronize()
            _ = (dx.float() * 2).sum().item()              # unrelated eager work in between
            assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), (M, N, K)
