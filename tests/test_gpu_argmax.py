"""Head GEMV with fused greedy argmax (w4a16_gemm_argmax) against the oracle.

The kernel's decision is taken on fp32 logits; the oracle's logits are fp64.
Where several rows are within the accuracy bound of the maximum, any of them
is a correct answer, so the check is: the reported logit is within the bound
of the oracle's logit for the reported row, and no row is certainly larger.
Where the oracle's top-1 margin exceeds the bounds, the index must match
exactly.  Ties and NaN handling are checked on constructed inputs whose
arithmetic is exact in fp32 (every product and partial sum representable), so
equal rows give bitwise-equal logits."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_w4a16_amd as w4
import oracle
import synth

pytestmark = pytest.mark.gpu
NTHREADS = 16


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t.view(dtype) if dtype is not None else t


def run(wq, ws, g, x_bits, workspace=None):
    idx, val = w4.gemm_argmax(dev(wq), dev(ws), torch.tensor([g], device="cuda"),
                              dev(x_bits.view(np.int16), torch.bfloat16), workspace=workspace)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), val.cpu().numpy()


def check_valid(idx, val, ref, a, ctx):
    bound = oracle.gemm_bound(a)
    M = ref.shape[0]
    for m in range(M):
        r, b = ref[m], bound[m]
        ok = ~np.isnan(r)
        i = int(idx[m])
        assert 0 <= i < ref.shape[1] and ok[i], f"{ctx} row {m}: index {i}"
        assert abs(val[m] - r[i]) <= b[i], f"{ctx} row {m}: value {val[m]} vs oracle {r[i]} (bound {b[i]})"
        # no row is certainly larger than the chosen one
        lower = np.where(ok, r - b, -np.inf)
        assert r[i] + b[i] >= lower.max(), f"{ctx} row {m}: row {int(lower.argmax())} is certainly larger"
        top = np.argsort(np.where(ok, r, -np.inf))[::-1][:2]
        if r[top[0]] - b[top[0]] > r[top[1]] + b[top[1]]:
            assert i == top[0], f"{ctx} row {m}: clear winner {top[0]}, got {i}"


@pytest.mark.parametrize("M,N,K", [(1, 20000, 5120), (7, 20000, 5120), (3, 1003, 1280), (13, 777, 2048),
                                   (12, 3001, 5120), (32, 515, 1024)])
def test_random_heads(M, N, K):
    wq, ws, g = synth.nvfp4_weights(70 + M, N, K)
    x = synth.activations(80 + M, M, K)
    idx, val = run(wq, ws, g, x)
    ref, a = oracle.gemm(wq, ws, g, x, M, N, K, nthreads=NTHREADS)
    check_valid(idx, val, ref, a, f"random {M}x{N}x{K}")


def exact_case(M, N, K, seed):
    """Codes random, every scale 1.0 (0x38), g = 1, x small integers: all fp32
    sums exact.  Returns weights and x."""
    rng = np.random.default_rng(seed)
    wq = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    ws = np.full((N, K // 16), 0x38, dtype=np.uint8)
    xi = rng.integers(-2, 3, size=(M, K)).astype(np.float32)
    return wq, ws, np.float32(1.0), synth.bf16_bits(xi), xi


def winner_row(xi_row, K):
    """Codes +-6 matching the signs of x: the largest possible logit."""
    codes = np.where(xi_row >= 0, 0x7, 0xF).astype(np.uint8)     # +6 / -6
    return codes[0::2] | (codes[1::2] << 4)


def test_ties_go_to_the_smaller_index():
    M, N, K = 2, 30000, 2048
    wq, ws, g, x, xi = exact_case(M, N, K, 5)
    for m, rows in enumerate([(17, 2049, 29999), (25000, 13000)]):
        w = winner_row(xi[m], K)
        for r in rows:
            wq[r] = w
    idx, val = run(wq, ws, g, x)
    ref, a = oracle.gemm(wq, ws, g, x, M, N, K, nthreads=NTHREADS)
    # exact arithmetic: the GPU logits are the exact ones
    assert idx[0] == 17 and idx[1] == 13000, idx
    assert val[0] == ref[0, 17] and val[1] == ref[1, 13000]


def test_nan_logits_are_never_selected():
    M, N, K = 1, 5000, 1024
    wq, ws, g, x, xi = exact_case(M, N, K, 6)
    wq[100] = winner_row(xi[0], K)
    ws[100, 3] = 0x7F                      # NaN scale: row 100's logit is NaN
    wq[4000] = winner_row(xi[0], K)
    ws[4000, :] = 0x30                     # scale 0.5: the best remaining row
    idx, val = run(wq, ws, g, x)
    ref, a = oracle.gemm(wq, ws, g, x, M, N, K, nthreads=NTHREADS)
    assert np.isnan(ref[0, 100])
    assert idx[0] == 4000 and val[0] == ref[0, 4000]


def test_full_head_shape_and_reused_workspace():
    # the 5120 -> 248320 head at M = 1 and 7; its rows tile an N(0, 0.02)
    # 5120 x 5120 matrix (48.5 copies), so the oracle needs the 5120 distinct
    # rows only.  One workspace serves all calls (its counter is reset by each).
    V, H = 248320, 5120
    wq5, ws5, g = synth.nvfp4_weights(21, H, H)
    reps = (V + H - 1) // H
    wq = np.concatenate([wq5] * reps)[:V]
    ws = np.concatenate([ws5] * reps)[:V]
    work = torch.zeros(w4.workspace_size_argmax(7, V, H), dtype=torch.uint8, device="cuda")
    for M in (1, 7, 1):
        x = synth.activations(90 + M, M, H)
        idx, val = run(wq, ws, g, x, workspace=work)
        ref5, a5 = oracle.gemm(wq5, ws5, g, x, M, H, H, nthreads=NTHREADS)
        ref = np.concatenate([ref5] * reps, axis=1)[:, :V]
        a = np.concatenate([a5] * reps, axis=1)[:, :V]
        check_valid(idx, val, ref, a, f"head M={M}")
    assert int(work[:4096].count_nonzero()) == 0


def test_run_to_run_identical():
    wq, ws, g = synth.nvfp4_weights(77, 9000, 5120)
    x = synth.activations(78, 7, 5120)
    first = run(wq, ws, g, x)
    for _ in range(3):
        again = run(wq, ws, g, x)
        assert np.array_equal(first[0], again[0]) and np.array_equal(first[1].view(np.uint32), again[1].view(np.uint32))


@pytest.mark.parametrize("M,K,N", [(3, 1024, 7000), (5, 1024, 7000), (13, 1024, 7000), (16, 5120, 7000),
                                   (29, 5120, 7000), (3, 5120, 7000), (4, 5120, 7000), (6, 5120, 7000),
                                   (8, 5120, 7000), (8, 5120, 100003)])
def test_ties_and_nan_rows_on_the_mfma_path(M, K, N):
    """M >= 3 runs on MFMA kernels that reduce every activation row side by
    side: at K = 5120 and M <= 8 the K-column kernel's ring variant (each
    thread keeps the best of the logits it adds, then the workgroup and the
    last workgroup reduce), otherwise the general MFMA kernel (at K = 5120 and
    M > 12 after a K split, in the last workgroup of each row block).  Exact
    arithmetic as above: for each activation row m but the last, three weight
    rows hold m's largest possible logit (codes +-6 with x[m]'s signs) and the
    smallest of them must win, with the exact value; the last activation row
    holds a NaN, so all its logits are NaN and its index is -1."""
    wq, ws, g, x, xi = exact_case(M, N, K, 30 + M)
    rng = np.random.default_rng(40 + M)
    planted = rng.choice(N, size=(M - 1, 3), replace=False)
    for m in range(M - 1):
        w = winner_row(xi[m], K)
        for r in planted[m]:
            wq[r] = w
    x = x.copy()
    x[M - 1, 5] = 0x7FC0                      # a bf16 NaN
    idx, val = run(wq, ws, g, x)
    ref, a = oracle.gemm(wq, ws, g, x, M, N, K, nthreads=NTHREADS)
    for m in range(M - 1):
        best = np.flatnonzero(ref[m] == ref[m].max())
        assert set(planted[m]) <= set(best), (M, m)      # the planted rows are maxima
        want = int(best[0])                              # ties: the smallest index
        assert idx[m] == want and val[m] == ref[m, want], (M, m, idx[m], want)
    assert np.isnan(ref[M - 1]).all()
    assert idx[M - 1] == -1, idx[M - 1]
