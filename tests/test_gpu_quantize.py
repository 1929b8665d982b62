"""GPU NVFP4 quantiser (w4a16_quantize / w4a16_quantize_bf16) against the
oracle's quantiser: every code byte, scale byte and g must be identical.

Cases: seeded N(0, 0.02) weights of several shapes (ragged block counts);
values spread over 17 decades (subnormal and saturating scales, blocks that
round to scale 0); constructed exact ties for both roundings (g forced to 64
by amax = 7); zeros and negative zeros; a full 5120 x 5120 matrix; bf16 input
(compared with the oracle on the exactly widened values)."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_w4a16_amd as w4
import oracle
import synth

pytestmark = pytest.mark.gpu


def gpu_quantize(w_np, bf16=False):
    if bf16:
        t = torch.from_numpy(np.ascontiguousarray(w_np).view(np.int16)).cuda().view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(w_np, dtype=np.float32)).cuda()
    wq, ws, g = w4.quantize(t)
    torch.cuda.synchronize()
    return wq.cpu().numpy(), ws.cpu().numpy(), np.float32(g.cpu().numpy()[0])


def check_equal(w_f32, ctx, bf16_bits=None):
    N, K = w_f32.shape
    rq, rs, rg = oracle.quantize(w_f32, N, K)
    gq, gs, gg = gpu_quantize(bf16_bits if bf16_bits is not None else w_f32, bf16=bf16_bits is not None)
    assert np.float32(gg).view(np.uint32) == np.float32(rg).view(np.uint32), f"{ctx}: g {gg} vs {rg}"
    bad_s = np.argwhere(gs != rs)
    assert bad_s.size == 0, f"{ctx}: {len(bad_s)} scale bytes differ, first {tuple(bad_s[0])}: {gs[tuple(bad_s[0])]:#x} vs {rs[tuple(bad_s[0])]:#x}"
    bad_q = np.argwhere(gq != rq)
    assert bad_q.size == 0, f"{ctx}: {len(bad_q)} code bytes differ, first {tuple(bad_q[0])}: {gq[tuple(bad_q[0])]:#x} vs {rq[tuple(bad_q[0])]:#x}"


@pytest.mark.parametrize("N,K", [(1, 16), (3, 48), (7, 256), (257, 512), (1003, 1280), (64, 5120)])
def test_normal_weights(N, K):
    check_equal(synth.weights_f32(100 + N, N, K), f"N(0,0.02) {N}x{K}")


def test_full_square_matrix():
    check_equal(synth.weights_f32(21, 5120, 5120), "square 5120x5120")


def test_seventeen_decades():
    rng = np.random.default_rng(7)
    N, K = 96, 1024
    mag = 10.0 ** rng.uniform(-14, 3, size=(N, K))
    w = (np.where(rng.random((N, K)) < 0.5, -1.0, 1.0) * mag).astype(np.float32)
    w[5, 32:48] = 0.0                          # an all-zero block
    w[6, :16] = 1e-30                          # a block whose scale rounds to 0
    check_equal(w, "17 decades")


def test_constructed_ties():
    # amax = 7 -> g = 448/7 = 64 exactly.  Block scales: bmax*64/6 lands exactly
    # on E4M3 midpoints (ties to the even code); codes: w*64/S lands exactly on
    # E2M1 midpoints (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) and on grid values.
    rng = np.random.default_rng(3)
    e4m3 = np.array([oracle.e4m3(c) for c in range(0x7F)])
    N, K = 40, 256
    w = np.zeros((N, K), dtype=np.float64)
    w[0, 0] = 7.0
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 3.0, 6.0, 0.0])
    for n in range(N):
        for j in range(K // 16):
            if n == 0 and j == 0:
                continue
            kind = rng.integers(0, 3)
            # block maxima stay <= 6.75 < amax = 7 (scale codes up to 72 = 0x69)
            if kind == 0:   # scale tie: t = midpoint of two neighbouring E4M3 values
                c = int(rng.integers(1, 0x69))
                t = 0.5 * (e4m3[c] + e4m3[c + 1])
                bmax = t * 6.0 / 64.0
                blk = rng.uniform(-bmax, bmax, 16).astype(np.float32).astype(np.float64)
                blk[rng.integers(0, 16)] = bmax * rng.choice([-1, 1])
            else:           # exact scale S = bmax*64/6 on the grid, codes at midpoints
                c = int(rng.integers(8, 0x6A))
                S = e4m3[c]
                bmax = S * 6.0 / 64.0
                blk = rng.choice(mids, 16) * S / 64.0 * rng.choice([-1, 1], 16)
                blk[rng.integers(0, 16)] = bmax
            w[n, 16 * j:16 * j + 16] = blk
    w32 = w.astype(np.float32)
    assert np.all(w32.astype(np.float64) == w), "construction must be exact in fp32"
    check_equal(w32, "constructed ties")


def test_zeros_and_negative_zeros():
    w = np.zeros((4, 64), dtype=np.float32)
    check_equal(w, "all zero")                 # g = 1, all bytes 0
    w = np.full((4, 64), -0.0, dtype=np.float32)
    w[2, 17] = -3.0
    check_equal(w, "negative zeros")           # -0 codes (8) in the block with a scale


def test_bf16_input():
    rng = np.random.default_rng(11)
    bits = synth.bf16_bits((rng.standard_normal((129, 768)) * 0.02).astype(np.float32))
    check_equal(synth.bf16_to_f32(bits), "bf16", bf16_bits=bits)


def test_quantized_weights_feed_the_matmul():
    # quantise on the GPU, then run the matmul on those bytes: it must match
    # the oracle matmul on the oracle's own encoding (the bytes are identical)
    N, K, M = 640, 1024, 3
    wf = synth.weights_f32(5, N, K)
    wq, ws, g = w4.quantize(torch.from_numpy(wf).cuda())
    x = synth.activations(6, M, K)
    y = w4.gemm(wq, ws, g, torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16))
    torch.cuda.synchronize()
    rq, rs, rg = oracle.quantize(wf, N, K)
    ref, a = oracle.gemm(rq, rs, rg, x, M, N, K)
    got = synth.bf16_to_f32(y.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    assert np.all(np.abs(got - ref) <= oracle.gemm_bound(a))
