"""Bit-exact parity checks on exact-arithmetic inputs (shared by GPU and CPU tests).

With integer activations in [-2, 2], power-of-two global scale g and block
scales drawn from a set whose values are all multiples of one quantum, every
product x * e2m1 * scale is a multiple of q = 1/2 * (scale quantum) and every
partial sum any kernel forms is bounded by sum_k |x e2m1 scale| = A * g.  If
A * g < 2^24 q, all those fp32 sums are exact whatever their order, the
division by g is exact, and the kernel's bf16 output must equal the oracle's
fp64 result rounded once to bf16 (nearest even): one correct answer, so any
indexing slip (a dropped chunk, a swapped scale, a wrong nibble) shows.

For silu(gate) * up the pre-activations are exact but the fp32 silu is not:
the fp32 value lies within EPS_SWIGLU relative of the exact one, so the bf16
output must be one of the (at most two) roundings of that interval.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth

# quantum of each scale set's values (all multiples of it)
SCALE_QUANTUM = {"pow2": 0.5, "mant": 0.125}
# relative error allowed for fp32 silu(a) * b with exact a, b: silu's fp32
# evaluation (exp, add, divide) and the product stay within a few units in
# the last place; 2^-18 = 64 ulp leaves a wide margin and is still far below
# the 2^-8 relative granularity of the bf16 result
EPS_SWIGLU = 2.0 ** -18


def scale_values(scales: str) -> np.ndarray:
    """Decoded values of the scale bytes of a set (via the oracle's decoder)."""
    return np.array([oracle.e4m3(int(b)) for b in synth.EXACT_SCALES[scales]])


def assert_exact_regime(a, g, scales: str, ctx: str = ""):
    """Every partial sum is exact in fp32: max A * g < 2^24 * q."""
    q = 0.5 * SCALE_QUANTUM[scales]
    vals = scale_values(scales)
    assert np.all(np.abs(vals / SCALE_QUANTUM[scales] - np.round(vals / SCALE_QUANTUM[scales])) == 0), \
        f"{ctx}: scale set {scales} is not on its quantum"
    gl = float(np.log2(float(g)))
    assert gl == round(gl), f"{ctx}: g = {g} is not a power of two"
    worst = float(np.max(a)) * float(g) if np.size(a) else 0.0
    assert worst < 2.0 ** 24 * q, f"{ctx}: sums up to {worst} exceed the exact fp32 range ({2.0**24*q})"


def f32_of_bf16(bits) -> np.ndarray:
    return synth.bf16_to_f32(np.asarray(bits, dtype=np.uint16)).astype(np.float64)


def expected_bits(y_ref) -> np.ndarray:
    """The one correct bf16 output for an exact fp64 result."""
    return oracle.bf16_rne(y_ref)


def mismatches(y_bits, y_ref) -> np.ndarray:
    """Boolean mask of outputs whose bf16 value differs from bf16(y_ref)
    (NaN positions must agree; -0 equals +0)."""
    got = f32_of_bf16(y_bits)
    want = f32_of_bf16(expected_bits(y_ref))
    both_nan = np.isnan(got) & np.isnan(want)
    return ~((got == want) | both_nan)


def assert_bits_exact(y_bits, y_ref, ctx: str):
    bad = mismatches(y_bits, y_ref)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        got = f32_of_bf16(y_bits)[i]
        want = f32_of_bf16(expected_bits(y_ref))[i]
        raise AssertionError(f"{ctx}: {int(bad.sum())} of {bad.size} outputs differ from bf16(exact); "
                             f"first at {i}: gpu {got!r}, exact {y_ref[i]!r} -> {want!r}")


def swiglu_allowed(z):
    """The bf16 values allowed for silu(gate) * up when its exact value is z:
    the roundings of the ends of [z - EPS|z|, z + EPS|z|] (bf16 rounding is
    monotone, and the interval is narrower than a bf16 step)."""
    z = np.asarray(z, dtype=np.float64)
    lo = f32_of_bf16(oracle.bf16_rne(z - EPS_SWIGLU * np.abs(z)))
    hi = f32_of_bf16(oracle.bf16_rne(z + EPS_SWIGLU * np.abs(z)))
    return lo, hi


def assert_swiglu_exact(y_bits, z, ctx: str):
    got = f32_of_bf16(y_bits)
    lo, hi = swiglu_allowed(z)
    ok = (got == lo) | (got == hi)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{ctx}: {int((~ok).sum())} of {ok.size} outputs are not a rounding of "
                             f"silu(gate)*up; first at {i}: gpu {got[i]!r}, exact {z[i]!r}, "
                             f"allowed {lo[i]!r} / {hi[i]!r}")
    return int(np.count_nonzero(lo != hi))


def exact_gemm_case(seed: int, M: int, N: int, K: int, scales: str = "pow2", gexp: int = 5):
    """(wq, ws, g, x_bits) of an exact-arithmetic case."""
    wq, ws = synth.exact_weights(seed, N, K, scales)
    x = synth.integer_activations(seed + 7919, M, K)
    return wq, ws, np.float32(2.0 ** gexp), x
