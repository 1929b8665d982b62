"""The bit-exact parity check is strong where the tolerance is weak (CPU only).

The accuracy bound 1e-2 * sum|x w| is about 0.6 |y| at K = 5120, so a kernel
that drops a 32-input chunk, swaps two blocks' scales or swaps the nibbles of a
byte column in every row would still pass it almost everywhere.  On the
exact-arithmetic inputs of the GPU tests there is one correct bf16 output per
element, and the same slips change most of them.  Here the "kernel output" is
the oracle's own result on perturbed bytes, rounded to bf16: what a GPU kernel
with that slip would return.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import exact

M, N, K = 7, 512, 5120


@pytest.fixture(scope="module")
def case():
    wq, ws, g, x = exact.exact_gemm_case(5, M, N, K)
    y, a = oracle.gemm(wq, ws, g, x, M, N, K, nthreads=4)
    exact.assert_exact_regime(a, g, "pow2")
    return wq, ws, g, x, y, a


def _perturbations(wq, ws):
    c = 37
    drop = wq.copy()
    drop[:, 16 * c:16 * c + 16] = 0                       # chunk c (inputs 32c..32c+31) dropped
    swap = ws.copy()
    swap[:, [2 * c, 2 * c + 1]] = ws[:, [2 * c + 1, 2 * c]]  # the chunk's two block scales swapped
    nib = wq.copy()
    b = nib[:, 100]
    nib[:, 100] = ((b >> 4) | (b << 4)) & 0xFF            # nibbles of byte column 100 swapped
    last = wq.copy()
    last[:, -16:] = 0                                      # the last chunk dropped
    return {"dropped chunk": (drop, ws), "swapped scale pair": (wq, swap),
            "swapped nibbles": (nib, ws), "dropped last chunk": (last, ws)}


def test_exact_check_accepts_the_exact_result(case):
    wq, ws, g, x, y, a = case
    assert not exact.mismatches(exact.expected_bits(y), y).any()


@pytest.mark.parametrize("name", ["dropped chunk", "swapped scale pair", "swapped nibbles",
                                  "dropped last chunk"])
def test_slips_pass_the_tolerance_but_fail_the_exact_check(case, name):
    wq, ws, g, x, y, a = case
    q, s = _perturbations(wq, ws)[name]
    y_slip, _ = oracle.gemm(q, s, g, x, M, N, K, nthreads=4)
    bits = oracle.bf16_rne(y_slip)
    got = exact.f32_of_bf16(bits)
    tol_rejects = int(np.sum(np.abs(got - y) > oracle.gemm_bound(a)))
    exact_rejects = int(exact.mismatches(bits, y).sum())
    assert tol_rejects <= 0.01 * y.size, (name, tol_rejects)
    assert exact_rejects >= 0.25 * y.size, (name, exact_rejects)


def test_exact_regime_guard_rejects_wide_sums():
    # a non-power-of-two g, or sums beyond 2^24 quanta, are refused
    with pytest.raises(AssertionError):
        exact.assert_exact_regime(np.array([1.0]), np.float32(3.0), "pow2")
    with pytest.raises(AssertionError):
        exact.assert_exact_regime(np.array([2.0 ** 23]), np.float32(1.0), "pow2")


def test_scale_sets_decode_to_their_stated_values():
    assert list(exact.scale_values("pow2")) == [0.5, 1.0, 2.0, 4.0]
    assert list(exact.scale_values("mant")) == [1 + m / 8 for m in range(8)]


def test_swiglu_allowed_set_is_one_or_two_neighbouring_values():
    z = np.random.default_rng(3).standard_normal(10000) * 100
    lo, hi = exact.swiglu_allowed(z)
    assert np.all(lo <= hi)
    # at most one bf16 step apart, and the exact rounding is one of them
    assert np.all((lo == hi) | (np.abs(hi - lo) <= np.abs(z) * 2.0 ** -7 * 1.01))
    want = exact.f32_of_bf16(oracle.bf16_rne(z))
    assert np.all((want == lo) | (want == hi))


def test_integer_activations_are_integers_in_range():
    x = exact.f32_of_bf16(synth.integer_activations(1, 3, 512))
    assert np.all(x == np.round(x)) and x.min() == -2 and x.max() == 2
