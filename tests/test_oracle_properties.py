"""Property pins of the oracle over randomly drawn shapes and magnitudes
(hypothesis, CPU only): the invariants of test_oracle_pins.py must hold for
every draw, not only for the fixed seeds there."""
import numpy as np
from hypothesis import HealthCheck, given, settings, strategies as st

from oracle import w4a4_oracle as O

SET = settings(max_examples=60, deadline=None, derandomize=True, database=None,
               suppress_health_check=[HealthCheck.too_slow])


def _rows(draw, R, K):
    seed = draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    mag = 10.0 ** draw(st.floats(-6, 6))
    y = (rng.standard_normal((R, K)) * mag * rng.lognormal(0, 1.0, (R, 1))).astype(np.float32)
    kind = draw(st.sampled_from(["dense", "one_hot", "zero_row", "outlier"]))
    if kind == "one_hot":
        y[:] = 0
        y[np.arange(R), rng.integers(0, K, R)] = np.float32(mag)
    elif kind == "zero_row":
        y[rng.integers(0, R)] = 0
    elif kind == "outlier":
        y[:, rng.integers(0, K)] *= np.float32(100)
    return y


@st.composite
def operands(draw):
    R = draw(st.integers(1, 12))
    K = 64 * draw(st.integers(1, 6))
    return _rows(draw, R, K)


@SET
@given(operands(), st.sampled_from([7, 127]))
def test_int_quantizer_properties(y, qmax):
    codes, step, v = O.quantize_int(y, qmax)
    nz = step > 0
    assert np.all(codes[~nz] == 0)
    assert np.all(np.abs(codes[nz]).max(axis=1) == qmax)
    dq = O.dequantize_int(codes, step).astype(np.float64)
    assert np.all(np.abs(dq - y) <= step.astype(np.float64)[:, None] * 0.5 * (1 + 1e-5) + 1e-30)
    c2, s2, _ = O.quantize_int(O.dequantize_int(codes, step), qmax)
    assert np.array_equal(c2, codes)


@SET
@given(operands(), st.floats(-3, 3))
def test_nvfp4_quantizer_properties(y, log_gscale):
    amax = np.abs(y).max()
    g = O.nvfp4_tensor_scale(amax * np.float32(10.0 ** log_gscale))   # also saturating (g small) draws
    codes, e, sv, v = O.quantize_nvfp4(y, g)
    assert np.all(e <= 0x7E)
    mag = (codes & 7).reshape(y.shape[0], -1, 16)
    normal = (sv >= 2.0 ** -6) & (sv <= 448.0)
    assert np.all(mag.max(axis=2)[normal] == 7)
    dq = O.dequantize_nvfp4(codes, e, g).astype(np.float32)
    c2, e2, _, _ = O.quantize_nvfp4(dq, g)
    assert np.array_equal(e2, e) and np.array_equal(c2, codes)


@SET
@given(st.integers(1, 6), st.integers(1, 6), st.integers(1, 4), st.integers(0, 2 ** 31 - 1),
       st.sampled_from(["smooth_then_rotate", "rotate_then_smooth"]))
def test_folding_holds_for_random_factors(M, N, kb, seed, order):
    """FoldQuantVLA Proposition 1 for random shapes and smoothing factors."""
    rng = np.random.default_rng(seed)
    K = 64 * kb
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((N, K))
    s = rng.lognormal(0, 1.5, K)
    got = O.transform(x, 1.0 / s, 64, order, np.float64) @ O.transform(w, s, 64, order, np.float64).T
    ref = x @ w.T
    assert np.max(np.abs(got - ref)) <= 1e-11 * np.max(np.abs(x)) * np.max(np.abs(w)) * K


@SET
@given(st.integers(1, 5), st.integers(1, 5), st.integers(1, 3), st.integers(0, 2 ** 31 - 1))
def test_int_gemm_matches_brute_force(M, N, kb, seed):
    rng = np.random.default_rng(seed)
    K = 64 * kb
    a = rng.integers(-128, 128, (M, K))
    w = rng.integers(-128, 128, (N, K))
    acc = O.int_gemm(a, w)
    brute = np.array([[sum(int(a[m, k]) * int(w[n, k]) for k in range(K)) for n in range(N)] for m in range(M)])
    assert np.array_equal(acc, brute)
