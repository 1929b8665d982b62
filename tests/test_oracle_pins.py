"""Pins of the CPU oracle against things other than itself (no GPU needed).

Each test fixes the oracle to an external fact: published code tables
(tests/golden/), a library decoder (torch float8_e4m3fn), exact rational
brute force, a hand-worked example, closed forms and invariants.  A plausible
slip in the oracle (swapped nibbles, wrong block index, wrong exponent bias,
dropped sign, g multiplied instead of divided, transposed operands) fails at
least one of them; tests/test_oracle_mutations.py plants such slips to show it.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            c, v = line.split()
            out[int(c, 16)] = float(v)
    return out


E2M1_GOLD = _read_table("e2m1_ocp_mx.txt")


def _torch_e4m3(byte):
    return float(torch.tensor([byte], dtype=torch.uint8).view(torch.float8_e4m3fn).float()[0])


E4M3_TORCH = [_torch_e4m3(b) for b in range(256)]


def _same(a, b):
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


# ---- element decoders -------------------------------------------------------

def test_e2m1_matches_ocp_table():
    assert sorted(E2M1_GOLD) == list(range(16))
    for c in range(16):
        assert _same(oracle.e2m1(c), E2M1_GOLD[c]), c


def test_e4m3_matches_torch_all_codes():
    for b in range(256):
        assert _same(oracle.e4m3(b), E4M3_TORCH[b]), hex(b)


def test_e4m3_matches_ofp8_named_points():
    for b, v in _read_table("e4m3fn_points.txt").items():
        assert _same(oracle.e4m3(b), v), hex(b)
    finite = [oracle.e4m3(b) for b in range(256) if not math.isnan(oracle.e4m3(b))]
    assert max(finite) == 448.0 and min(finite) == -448.0
    assert sum(math.isnan(oracle.e4m3(b)) for b in range(256)) == 2


def test_products_exact_in_fp32_and_bf16():
    # every finite e2m1 * e4m3 product has <= 6 significant bits and lies in
    # [2^-10, 2688]: representable exactly in fp32 and in bf16
    for c in range(16):
        for b in range(256):
            p = oracle.e2m1(c) * oracle.e4m3(b)
            if math.isnan(p):
                continue
            f = np.float32(p)
            assert float(f) == p
            bits = np.array([f], dtype=np.float32).view(np.uint32)[0]
            assert bits & 0xFFFF == 0, (c, b)
            if p != 0:
                assert 2.0 ** -10 <= abs(p) <= 2688.0


# ---- dequantisation ---------------------------------------------------------

def _all_pairs_matrix():
    """N = 256 rows (one per scale byte), K = 32: every code at every position parity."""
    N, K = 256, 32
    codes = np.tile(np.arange(16, dtype=np.uint8), (N, 2))          # [256][32]
    wq = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    ws = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 2, axis=1)
    return wq, ws, codes, N, K


@pytest.mark.parametrize("g", [1.0, 448.0 / 0.0873, 4071.6726, 2.0 ** -3, 3.0e-5, 1.0e6])
def test_dequant_all_codes_and_scales(g):
    wq, ws, codes, N, K = _all_pairs_matrix()
    g32 = np.float32(g)
    w64 = oracle.dequant_f64(wq, ws, g32, N, K)
    w32 = oracle.dequant_f32(wq, ws, g32, N, K)
    for n in range(N):
        s = E4M3_TORCH[n]
        for k in range(K):
            p = E2M1_GOLD[int(codes[n, k])] * s
            ref64 = p / float(g32)
            # fp32 result must be the IEEE fp32 quotient of the two fp32 numbers
            ref32 = np.float32(np.float32(p) / g32) if not math.isnan(p) else np.float32("nan")
            assert _same(w64[n, k], ref64), (n, k)
            assert _same(float(w32[n, k]), float(ref32)), (n, k, g)


def test_dequant_layout_positions():
    # one nonzero code at a time: checks nibble order and block index
    N, K = 3, 64
    for n in range(N):
        for k in range(K):
            wq = np.zeros((N, K // 2), np.uint8)
            ws = np.full((N, K // 16), 0x38, np.uint8)          # scale 1.0 everywhere
            ws[n, k // 16] = 0x40                               # 2.0 on the hot block
            wq[n, k // 2] = 0x5 << (4 * (k % 2))               # code 5 = 3.0
            w = oracle.dequant_f64(wq, ws, np.float32(1.0), N, K)
            expect = np.zeros((N, K))
            expect[n, k] = 6.0
            assert np.array_equal(w, expect), (n, k)


# ---- matmul ------------------------------------------------------------------

def _frac_gemm(wq, ws, g, x_bits, M, N, K):
    """Exact rational y and A from the golden tables (independent of the oracle)."""
    xs = synth.bf16_to_f32(x_bits).reshape(M, K)
    gf = Fraction(float(np.float32(g)))
    y = [[Fraction(0)] * N for _ in range(M)]
    a = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            for k in range(K):
                byte = int(wq[n, k // 2])
                code = (byte >> 4) if k % 2 else (byte & 0xF)
                t = Fraction(float(xs[m, k])) * Fraction(E2M1_GOLD[code]) * \
                    Fraction(E4M3_TORCH[int(ws[n, k // 16])]) / gf
                y[m][n] += t
                a[m][n] += abs(t)
    return y, a


@pytest.mark.parametrize("M,N,K,seed", [(1, 1, 16, 0), (2, 3, 32, 1), (3, 4, 64, 2), (1, 4, 48, 3)])
def test_gemm_bruteforce_exact(M, N, K, seed):
    rng = np.random.default_rng(seed)
    wq = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    ws = rng.integers(0x08, 0x7F, (N, K // 16), dtype=np.uint8)  # finite, normal scales
    ws[:, 0] = 0x03                                             # one subnormal block
    g = np.float32(rng.uniform(0.5, 5000.0))
    x = synth.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    y, a = oracle.gemm(wq, ws, g, x, M, N, K)
    yf, af = _frac_gemm(wq, ws, g, x, M, N, K)
    for m in range(M):
        for n in range(N):
            A = float(af[m][n])
            assert abs(y[m, n] - float(yf[m][n])) <= 1e-12 * A + 1e-300
            assert abs(a[m, n] - A) <= 1e-12 * A


def test_gemm_hand_example():
    vals = {}
    with open(os.path.join(GOLDEN, "nvfp4_hand_example.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                key, *rest = line.split()
                vals[key] = rest
    N, K, M = 2, 32, 1
    wq = np.array([[int(vals["wq_row0"][0], 16)] * 16, [int(vals["wq_row1"][0], 16)] * 16], np.uint8)
    ws = np.array([[int(v, 16) for v in vals["ws_row0"]], [int(v, 16) for v in vals["ws_row1"]]],
                  np.uint8)
    x = np.array([[int(vals["x_first16"][0], 16)] * 16 + [int(vals["x_last16"][0], 16)] * 16],
                 np.uint16)
    g = np.float32(float(vals["g"][0]))
    y, a = oracle.gemm(wq, ws, g, x, M, N, K)
    assert y[0].tolist() == [float(v) for v in vals["y"]]
    assert a[0].tolist() == [float(v) for v in vals["a"]]


def _rand_case(seed, M, N, K):
    rng = np.random.default_rng(seed)
    wq, ws, g = synth.nvfp4_weights(seed, N, K)
    x = synth.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    return wq, ws, g, x


def test_gemm_sign_flip_negates_exactly():
    M, N, K = 2, 7, 96
    wq, ws, g, x = _rand_case(5, M, N, K)
    y, _ = oracle.gemm(wq, ws, g, x, M, N, K)
    y2, _ = oracle.gemm(wq ^ np.uint8(0x88), ws, g, x, M, N, K)
    assert np.array_equal(y2, -y)


def test_gemm_global_scale_halves_exactly():
    M, N, K = 2, 5, 64
    wq, ws, g, x = _rand_case(6, M, N, K)
    y, _ = oracle.gemm(wq, ws, g, x, M, N, K)
    y2, _ = oracle.gemm(wq, ws, np.float32(2 * g), x, M, N, K)
    assert np.array_equal(y2, y / 2)


def test_gemm_one_hot_selects_column():
    # x = e_k picks column k of W (against the separately pinned dequant)
    M, N, K = 1, 6, 64
    wq, ws, g, _ = _rand_case(7, M, N, K)
    w = oracle.dequant_f64(wq, ws, g, N, K)
    for k in (0, 1, 15, 16, 33, 63):
        x = np.zeros((1, K), np.uint16)
        x[0, k] = 0x3F80
        y, a = oracle.gemm(wq, ws, g, x, M, N, K)
        assert np.array_equal(y[0], w[:, k])
        assert np.array_equal(a[0], np.abs(w[:, k]))


def test_gemm_rectangular_is_not_transposed():
    # N != K with distinct rows: y must equal W @ x (via the pinned dequant),
    # and must differ from any transposed reading.
    M, N, K = 3, 5, 32
    wq, ws, g, x = _rand_case(8, M, N, K)
    w = oracle.dequant_f64(wq, ws, g, N, K)
    xf = synth.bf16_to_f32(x).astype(np.float64).reshape(M, K)
    y, a = oracle.gemm(wq, ws, g, x, M, N, K)
    np.testing.assert_allclose(y, xf @ w.T, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(a, np.abs(xf) @ np.abs(w).T, rtol=1e-13, atol=1e-15)


def test_gemm_rows_matches_full():
    M, N, K = 3, 40, 128
    wq, ws, g, x = _rand_case(9, M, N, K)
    y, a = oracle.gemm(wq, ws, g, x, M, N, K)
    rows = np.array([0, 3, 39, 17, 3])
    yr, ar = oracle.gemm_rows(wq, ws, g, x, M, K, rows)
    assert np.array_equal(yr, y[:, rows]) and np.array_equal(ar, a[:, rows])


def test_gemm_threads_do_not_change_results():
    M, N, K = 2, 33, 256
    wq, ws, g, x = _rand_case(10, M, N, K)
    y1, a1 = oracle.gemm(wq, ws, g, x, M, N, K, nthreads=1)
    y4, a4 = oracle.gemm(wq, ws, g, x, M, N, K, nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(a1, a4)


def test_gemm_nan_scale_propagates():
    M, N, K = 1, 2, 32
    wq = np.full((N, K // 2), 0x11, np.uint8)
    ws = np.full((N, K // 16), 0x38, np.uint8)
    ws[1, 1] = 0x7F
    x = np.full((M, K), 0x3F80, np.uint16)
    y, _ = oracle.gemm(wq, ws, np.float32(1.0), x, M, N, K)
    assert y[0, 0] == 16.0 and math.isnan(y[0, 1])


# ---- SwiGLU -----------------------------------------------------------------

def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert oracle.silu(-1.0) == pytest.approx(-1.0 / (1.0 + math.e), rel=1e-15)
    assert oracle.silu(50.0) == pytest.approx(50.0, rel=1e-15)
    assert abs(oracle.silu(-50.0)) < 1e-19
    assert oracle.silu(-1000.0) == 0.0          # exp overflow must give 0, not NaN
    # derivative bound used by the tolerance: max |silu'| < 1.1
    v = np.linspace(-20, 20, 40001)
    d = np.gradient(np.array([oracle.silu(t) for t in v]), v)
    assert d.max() < 1.1 and d.min() > -0.11


def test_gate_up_swiglu_composes_two_matmuls():
    M, N, K = 3, 9, 64
    wq_g, ws_g, g_g, x = _rand_case(11, M, N, K)
    wq_u, ws_u, g_u, _ = _rand_case(12, M, N, K)
    out = oracle.gate_up_swiglu(wq_g, ws_g, g_g, wq_u, ws_u, g_u, x, M, N, K)
    yg, ag = oracle.gemm(wq_g, ws_g, g_g, x, M, N, K)
    yu, au = oracle.gemm(wq_u, ws_u, g_u, x, M, N, K)
    assert np.array_equal(out["gate"], yg) and np.array_equal(out["up"], yu)
    assert np.array_equal(out["a_gate"], ag) and np.array_equal(out["a_up"], au)
    expect = yg / (1.0 + np.exp(-yg)) * yu
    np.testing.assert_allclose(out["y"], expect, rtol=1e-14, atol=1e-300)


def test_swiglu_bound_covers_first_order_perturbation():
    # perturb gate/up by the full matmul bound and check the propagated bound holds
    rng = np.random.default_rng(3)
    gate = rng.standard_normal(10000) * 3
    up = rng.standard_normal(10000) * 3
    ag = np.abs(gate) * 5 + 1
    au = np.abs(up) * 5 + 1
    bound = oracle.swiglu_bound(gate, up, ag, au)
    y = gate / (1 + np.exp(-gate)) * up
    for sa in (-1, 1):
        for sb in (-1, 1):
            g2 = gate + sa * oracle.gemm_bound(ag)
            u2 = up + sb * oracle.gemm_bound(au)
            y2 = g2 / (1 + np.exp(-g2)) * u2
            y2 = synth.bf16_to_f32(synth.bf16_bits(y2.astype(np.float32))).astype(np.float64)
            assert np.all(np.abs(y2 - y) <= bound)


# ---- encoders and quantiser ---------------------------------------------------

def test_e2m1_encode_representable_ties_and_saturation():
    for c in range(16):
        v = E2M1_GOLD[c]
        assert oracle.e2m1_encode(v) == (c if c != 8 else 8)
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for t, c in ties.items():
        assert oracle.e2m1_encode(t) == c
        assert oracle.e2m1_encode(-t) == (8 | c)
    assert oracle.e2m1_encode(6.4) == 7 and oracle.e2m1_encode(1e9) == 7
    assert oracle.e2m1_encode(-0.1) == 8        # rounds to -0, sign kept
    # brute force nearest against the golden grid
    rng = np.random.default_rng(0)
    for v in rng.uniform(-7, 7, 2000):
        c = oracle.e2m1_encode(v)
        d = abs(abs(v) - abs(E2M1_GOLD[c]))
        assert all(d <= abs(abs(v) - E2M1_GOLD[j]) for j in range(8))
        assert (c >> 3) == (1 if v < 0 else 0)


def test_e4m3_encode_matches_torch_cast():
    # torch's fp32 -> float8_e4m3fn cast rounds to nearest even; compare on
    # fp32 inputs in the finite range, including all exact codes and midpoints
    vals = [E4M3_TORCH[b] for b in range(0x7F)]
    mids = [(vals[i] + vals[i + 1]) / 2 for i in range(len(vals) - 1)]
    rng = np.random.default_rng(1)
    rnd = list(np.exp(rng.uniform(np.log(2.0 ** -11), np.log(440.0), 5000)))
    tv = np.array(vals + mids + rnd, dtype=np.float32)
    tc = torch.from_numpy(tv).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for t, c in zip(tv, tc):
        assert oracle.e4m3_encode(float(t)) == int(c), float(t)
    assert oracle.e4m3_encode(448.0) == 0x7E and oracle.e4m3_encode(1e6) == 0x7E
    assert oracle.e4m3_encode(0.0) == 0 and oracle.e4m3_encode(2.0 ** -11) == 0


def test_quantize_global_scale_and_error_bound():
    N, K = 64, 256
    w = synth.weights_f32(123, N, K)
    wq, ws, g = oracle.quantize(w, N, K)
    amax = float(np.abs(w).max())
    assert g == np.float32(448.0 / amax)
    deq = oracle.dequant_f64(wq, ws, g, N, K)
    S = np.array([[E4M3_TORCH[b] for b in row] for row in ws])
    Sx = np.repeat(S, 16, axis=1)
    normal = Sx >= 2.0 ** -6
    err = np.abs(w.astype(np.float64) - deq)
    assert np.all(err[normal] <= (Sx / float(g))[normal])
    # every block scale is the E4M3 value nearest to blockmax*g/6 (checked via torch's cast)
    bmax = np.abs(w).reshape(N, K // 16, 16).max(axis=2).astype(np.float64)
    t = (bmax * float(g) / 6.0).astype(np.float32)
    assert np.array_equal(ws, torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_quantize_exact_round_trip_of_representable_blocks():
    # g forced to 2^5 by one element of magnitude 448/32 = 14 in block 0;
    # every other block is c * S / g with max |c| = 6, so it must come back exactly
    rng = np.random.default_rng(4)
    N, K = 8, 128
    g0 = 32.0
    codes = rng.integers(0, 16, (N, K), dtype=np.uint8)
    codes[:, ::16] = 0x7                                   # max |code| = 6 in every block
    # normal scales with 6*S/g0 < 448/g0, i.e. S <= 72 (code 0x69)
    scales = rng.integers(0x10, 0x6A, (N, K // 16), dtype=np.uint8)
    val = np.array([[E2M1_GOLD[int(c)] for c in row] for row in codes])
    S = np.array([[E4M3_TORCH[int(b)] for b in row] for row in scales])
    w = (val * np.repeat(S, 16, axis=1) / g0).astype(np.float32)
    assert np.array_equal(w.astype(np.float64), val * np.repeat(S, 16, axis=1) / g0)
    w[0, :16] = 0.0
    w[0, 0] = 448.0 / g0                                   # sets amax, hence g
    assert np.abs(w).max() == 448.0 / g0
    wq, ws, g = oracle.quantize(w, N, K)
    assert g == np.float32(g0)
    got_codes = np.empty((N, K), np.uint8)
    got_codes[:, 0::2] = wq & 0xF
    got_codes[:, 1::2] = wq >> 4
    blocks = np.ones((N, K // 16), bool)
    blocks[0, 0] = False
    bm = np.repeat(blocks, 16, axis=1)
    # codes of value 0 may come back as +0 or -0 only if the input was -0; inputs here are +-
    want = np.where((codes & 7) == 0, codes & 8, codes)
    assert np.array_equal(ws[blocks], scales[blocks])
    assert np.array_equal(np.where(bm, got_codes, 0), np.where(bm, want, 0))


def test_quantize_zero_matrix_and_zero_blocks():
    N, K = 2, 32
    w = np.zeros((N, K), np.float32)
    wq, ws, g = oracle.quantize(w, N, K)
    assert g == 1.0 and not wq.any() and not ws.any()
    w[1, 20] = 1.0
    wq, ws, g = oracle.quantize(w, N, K)
    assert g == np.float32(448.0)
    assert ws[0].tolist() == [0, 0] and ws[1, 0] == 0 and ws[1, 1] != 0
    assert not wq[0].any() and not wq[1, :8].any()


def test_synth_encoder_agrees_with_oracle_quantizer():
    # the input generator's storage encoder is a separate implementation;
    # on the benchmark distribution both must produce identical bytes
    for seed, (N, K) in ((21, (64, 512)), (31, (33, 256)), (41, (16, 1024))):
        w = synth.weights_f32(seed, N, K)
        a = synth.encode_nvfp4(w)
        b = oracle.quantize(w, N, K)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


# ---- MLP block: bf16 rounding of h, then the down projection -------------------

def test_bf16_rne_matches_torch_cast():
    # fp32-representable inputs, so torch's fp32 -> bf16 cast (round to nearest
    # even) is a single rounding and serves as the reference
    rng = np.random.default_rng(21)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 20000),
        # exact ties: 1 + (2j+1) 2^-8 lies halfway between two bf16 values
        (1.0 + (2 * np.arange(64) + 1) * 2.0 ** -8).astype(np.float32),
        -(3.0 + (2 * np.arange(64) + 1) * 2.0 ** -7).astype(np.float32),
        # subnormal bf16 range, around the smallest normal, and near overflow
        (np.arange(1, 300) * 2.0 ** -140).astype(np.float32),
        np.float32([2.0 ** -126, 2.0 ** -126 * (1 - 2.0 ** -9), 3.389e38, 3.3962e38, 3.4e38,
                    -3.4e38, 0.0, -0.0]),
    ]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_rne(v.astype(np.float64))
    assert np.array_equal(got, ref)
    assert oracle.bf16_rne(np.array([np.nan]))[0] & 0x7FFF > 0x7F80   # NaN stays NaN


def _py_bf16(v):
    """Nearest bf16 value (ties to even) of a normal-range float, pure Python."""
    if v == 0.0:
        return 0.0
    f, e = math.frexp(abs(v))                     # |v| = f 2^e, f in [0.5, 1)
    r = round(f * 256) / 256                      # round() on an exact binary value: ties to even
    return math.copysign(math.ldexp(r, e), v)


def test_mlp_bruteforce():
    # independent re-derivation on a tiny block: exact rational gate/up from
    # the golden tables, silu in Python floats, h rounded to bf16 in pure
    # Python, then the down projection as exact rationals
    M, H, F = 2, 32, 16
    rng = np.random.default_rng(8)
    def w(n, k, seed):
        r = np.random.default_rng(seed)
        wq = r.integers(0, 256, (n, k // 2), dtype=np.uint8)
        ws = r.integers(0x28, 0x48, (n, k // 16), dtype=np.uint8)
        return wq, ws, np.float32(r.uniform(1.0, 8.0))
    gate, up, down = w(F, H, 1), w(F, H, 2), w(H, F, 3)
    x = synth.bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    out = oracle.mlp_swiglu(gate, up, down, x, M, H, F)
    yg, _ = _frac_gemm(*gate, x, M, F, H)
    yu, _ = _frac_gemm(*up, x, M, F, H)
    h = np.zeros((M, F))
    for m in range(M):
        for n in range(F):
            a, b = float(yg[m][n]), float(yu[m][n])
            h[m, n] = _py_bf16(a / (1.0 + math.exp(-a)) * b)
    hb = synth.bf16_bits(h.astype(np.float32))
    assert np.array_equal(out["h_bits"], hb)
    yd, ad = _frac_gemm(*down, hb, M, H, F)
    for m in range(M):
        for n in range(H):
            A = float(ad[m][n])
            assert abs(out["y"][m, n] - float(yd[m][n])) <= 1e-12 * A + 1e-300
            assert abs(out["a"][m, n] - A) <= 1e-12 * A


def test_mlp_bound_covers_perturbed_h():
    # any h_gpu within the gate/up bound of h, pushed through the down
    # projection with the matmul error at its limit, stays inside mlp_bound
    M, H, F = 3, 64, 48
    rng = np.random.default_rng(4)
    gate, up, down = (synth.nvfp4_weights(s, n, k) for s, n, k in ((31, F, H), (32, F, H), (33, H, F)))
    x = synth.bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    out = oracle.mlp_swiglu(gate, up, down, x, M, H, F)
    wd = oracle.dequant_f64(*down, H, F)
    bound = oracle.mlp_bound(out, np.abs(wd))
    r = out["gate_up"]
    bh = oracle.swiglu_bound(r["gate"], r["up"], r["a_gate"], r["a_up"])
    for sign in (-1.0, 1.0):
        h_gpu = out["h"] + sign * bh * np.sign(wd.sum(axis=0))[None, :]
        y_gpu = h_gpu @ wd.T
        y_gpu += sign * 1e-2 * (np.abs(h_gpu) @ np.abs(wd).T)
        assert np.all(np.abs(y_gpu - out["y"]) <= bound)
