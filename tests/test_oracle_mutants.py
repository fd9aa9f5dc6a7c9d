"""Planted mistakes in the oracle are caught by its pins (CPU only).

Each mutant below replaces one oracle function (or constant) with a copy
carrying one plausible slip: a wrong sign, a dropped term or stage, a
transposed or shifted operand, a wrong rounding or tie rule, a wrong
constant.  The test runs every pin of ``tests/test_oracle_pins.py`` against
the mutated oracle and requires at least one to fail.  The mutations live
only in this file and only for the duration of one test; nothing here
touches the HIP path.
"""
import numpy as np
import pytest

import test_oracle_pins as P
from oracle import w4a4_oracle as O

F32 = np.float32
_orig = {name: getattr(O, name) for name in dir(O) if not name.startswith("__")}


def _pin_calls():
    """Every pin of test_oracle_pins with its parametrisations expanded."""
    calls = []
    for name in sorted(dir(P)):
        fn = getattr(P, name)
        if not name.startswith("test_") or not callable(fn):
            continue
        params = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not params:
            calls.append((name, fn, {}))
            continue
        assert len(params) == 1 and "," not in params[0].args[0]
        arg = params[0].args[0]
        for v in params[0].args[1]:
            calls.append((f"{name}[{v}]", fn, {arg: v}))
    return calls


PINS = _pin_calls()


# ----------------------------------------------------------------- mutants
def _fwht(u, block=64, sign=+1, stages=None):
    u = np.array(u, copy=True)
    R, K = u.shape
    h, n = 1, 0
    while h < block and (stages is None or n < stages):
        v = u.reshape(R, K // (2 * h), 2, h)
        a, b = v[:, :, 0, :].copy(), v[:, :, 1, :].copy()
        v[:, :, 0, :] = a + b
        v[:, :, 1, :] = sign * (a - b)
        u = v.reshape(R, K)
        h *= 2
        n += 1
    return u


def _quantize_int(rounding):
    def q(y, qmax):
        y = np.asarray(y, dtype=F32)
        step = (np.abs(y).max(axis=1) / F32(qmax)).astype(F32)
        v = np.zeros_like(y)
        nz = step > 0
        v[nz] = (y[nz] / step[nz, None]).astype(F32)
        return np.clip(rounding(v), -qmax - 1, qmax).astype(np.int8), step, v
    return q


def _nearest_ties_up(mag, grid):
    mag = np.asarray(mag, dtype=np.float64)
    hi = np.clip(np.searchsorted(grid, mag, side="left"), 1, len(grid) - 1)
    lo = hi - 1
    idx = np.where(grid[hi] - mag <= mag - grid[lo], hi, lo)
    idx = np.where(mag >= grid[-1], len(grid) - 1, idx)
    return np.where(mag <= 0, 0, idx).astype(np.int64)


def _e4m3_bias8(code):
    c = np.asarray(code, dtype=np.int64) & 0xFF
    s, e, m = (c >> 7) & 1, (c >> 3) & 0xF, c & 7
    mag = np.where(e == 0, m * 2.0 ** -10, (1.0 + m / 8.0) * np.exp2(e - 8.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(s == 1, -mag, mag)


def _pack_swapped(codes):
    c = (np.asarray(codes).astype(np.int64) & 0xF).astype(np.uint8)
    return (c[..., 1::2] | (c[..., 0::2] << 4)).astype(np.uint8)


def _epilogue_f64(acc, sa, sw):
    return np.asarray(acc, np.float64) * np.asarray(sa, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]


def _gptq_plus(wt, step, u, qmax, perm=None):
    wt = np.asarray(wt, dtype=F32)
    N, K = wt.shape
    perm = np.arange(K) if perm is None else np.asarray(perm)
    W = wt[:, perm].astype(np.float64)
    sf = np.asarray(step, F32).astype(np.float64)
    nz = sf > 0
    Q, E = np.zeros((N, K), np.int64), np.zeros((N, K))
    for t in range(K):
        q = np.zeros(N)
        q[nz] = np.clip(np.rint(W[nz, t] / sf[nz]), -qmax - 1, qmax)
        err = (W[:, t] - q * sf) / u[t, t]
        W[:, t + 1:] += np.outer(err, u[t, t + 1:])          # sign flipped
        Q[:, t], E[:, t] = q, err
    codes = np.empty((N, K), np.int8)
    codes[:, perm] = Q.astype(np.int8)
    return codes, E


def _quantize_int_f64(y, qmax):
    """Step and quotient evaluated in float64 instead of binary32."""
    y = np.asarray(y, dtype=F32)
    step = np.abs(y).max(axis=1).astype(np.float64) / qmax
    v = np.zeros(y.shape)
    nz = step > 0
    v[nz] = y[nz].astype(np.float64) / step[nz, None]
    return np.clip(np.rint(v), -qmax - 1, qmax).astype(np.int8), step.astype(F32), v.astype(F32)


def _nvfp4_with(scale_of):
    """quantize_nvfp4 whose element step comes from scale_of(sv, g) -> (e, S)."""
    def q(y, g):
        y = np.asarray(y, dtype=F32)
        g = F32(g)
        R, K = y.shape
        yb = y.reshape(R, K // 16, 16)
        sv = ((np.abs(yb).max(axis=2) / F32(6)).astype(F32) / g).astype(F32)
        e, S = scale_of(sv, g)
        v = np.zeros_like(yb)
        nz = S > 0
        v[nz] = (yb[nz] / S[nz][:, None]).astype(F32)
        return O.e2m1_encode(v).reshape(R, K).astype(np.uint8), e, sv, v.reshape(R, K)
    return q


def _unrounded_scale(sv, g):
    return O.e4m3_encode(sv), (sv * g).astype(F32)


def _floor_scale(sv, g):
    grid = O.e4m3_value(np.arange(0x7F)).astype(np.float64)
    e = np.clip(np.searchsorted(grid, sv.astype(np.float64), side="right") - 1, 0, 0x7E).astype(np.uint8)
    return e, (O.e4m3_value(e).astype(F32) * g).astype(F32)


def _gptq_with(update):
    """gptq_rows with the feedback step replaced by update(W, err, u, t)."""
    def g(wt, step, u, qmax, perm=None):
        wt = np.asarray(wt, dtype=F32)
        N, K = wt.shape
        perm = np.arange(K) if perm is None else np.asarray(perm)
        W = wt[:, perm].astype(np.float64)
        sf = np.asarray(step, F32).astype(np.float64)
        nz = sf > 0
        Q, E = np.zeros((N, K), np.int64), np.zeros((N, K))
        for t in range(K):
            q = np.zeros(N)
            q[nz] = np.clip(np.rint(W[nz, t] / sf[nz]), -qmax - 1, qmax)
            err = update(W, W[:, t] - q * sf, u, t)
            Q[:, t], E[:, t] = q, err
        codes = np.empty((N, K), np.int8)
        codes[:, perm] = Q.astype(np.int8)
        return codes, E
    return g


def _next_column_only(W, r, u, t):
    err = r / u[t, t]
    if t + 1 < W.shape[1]:
        W[:, t + 1] -= err * u[t, t + 1]
    return err


def _no_pivot_division(W, r, u, t):
    if t + 1 < W.shape[1]:
        W[:, t + 1:] -= np.outer(r, u[t, t + 1:])
    return r



def _gptq_inverse_scatter(wt, step, u, qmax, perm=None):
    """Codes written back with the inverse of the processing order."""
    c, e = _orig["gptq_rows"](wt, step, u, qmax, perm)
    if perm is None:
        return c, e
    perm = np.asarray(perm)
    out = np.empty_like(c)
    out[:, np.argsort(perm)] = c[:, perm]
    return out, e


MUTANTS = {
    # FWHT and the transform
    "butterfly difference sign flipped": {"fwht_blocks": lambda u, block=64: _fwht(u, block, sign=-1)},
    "last butterfly stage dropped": {"fwht_blocks": lambda u, block=64: _fwht(u, block, stages=5)},
    "rotation blocks of 32": {"fwht_blocks": lambda u, block=64: _orig["fwht_blocks"](u, 32)},
    "1/8 normalisation dropped": {"transform": lambda *a, **k: _orig["transform"](*a, **k) * 8},
    "smoothing by the reciprocal factor": {
        "transform": lambda x, scale, *a, **k: _orig["transform"](
            x, None if scale is None else np.divide(1.0, np.asarray(scale, np.float64),
                                                    out=np.zeros(np.shape(scale)), where=np.asarray(scale) != 0),
            *a, **k)},
    "the two transform orders swapped": {
        "transform": lambda x, scale, fwht_block=64, order="smooth_then_rotate", dtype=F32: _orig["transform"](
            x, scale, fwht_block, {"smooth_then_rotate": "rotate_then_smooth",
                                   "rotate_then_smooth": "smooth_then_rotate"}[order], dtype)},
    "smoothing always after the rotation": {
        "transform": lambda x, scale, fwht_block=64, order="smooth_then_rotate", dtype=F32:
            _orig["transform"](x, scale, fwht_block, "rotate_then_smooth", dtype)},
    # integer quantizer
    "truncation instead of round-to-nearest-even": {"quantize_int": _quantize_int(np.trunc)},
    "ties away from zero": {"quantize_int": _quantize_int(lambda v: np.sign(v) * np.floor(np.abs(v) + 0.5))},
    "Q off by one": {"quantize_int": lambda y, qmax: _orig["quantize_int"](y, qmax + 1)},
    "integer step and quotient in float64": {"quantize_int": _quantize_int_f64},
    "integer dequantisation ignores the step": {"dequantize_int": lambda c, s: np.asarray(c).astype(F32)},
    # NVFP4 / E4M3 codecs
    "ties to the larger code": {"_nearest_code": _nearest_ties_up},
    "E4M3 exponent bias 8": {"e4m3_value": _e4m3_bias8},
    "NVFP4 block scale from amax / 4": {"E2M1_MAX": 4.0},
    "NVFP4 element codes from the unrounded block scale": {"quantize_nvfp4": _nvfp4_with(_unrounded_scale)},
    "NVFP4 block scale rounded down": {"quantize_nvfp4": _nvfp4_with(_floor_scale)},
    "FP8 pre-rounding values 0.1% high": {
        "quantize_fp8": lambda y: (lambda c, st, v: (c, st, (v * F32(1.001)).astype(F32)))(*_orig["quantize_fp8"](y))},
    "NVFP4 tensor scale from twice the range": {
        "nvfp4_tensor_scale": lambda amax: F32(_orig["nvfp4_tensor_scale"](amax) / F32(2))},
    "NVFP4 dequantisation applies g twice": {
        "dequantize_nvfp4": lambda c, e, g: _orig["dequantize_nvfp4"](c, e, g) * np.float64(F32(g))},
    "NVFP4 dequantisation ignores g": {
        "dequantize_nvfp4": lambda c, e, g: _orig["dequantize_nvfp4"](c, e, 1.0)},
    "FP8 step amax / 240": {"E4M3_MAX": 240.0},
    # packing
    "nibbles swapped": {"pack_nibbles": _pack_swapped},
    "int4 nibbles not sign-extended": {"int4_from_nibbles": lambda n: np.asarray(n).astype(np.int8)},
    # GEMM and epilogue
    "GEMM drops the first K term": {
        "int_gemm": lambda qa, qw: _orig["int_gemm"](np.asarray(qa)[:, 1:], np.asarray(qw)[:, 1:])},
    "GEMM with the weight rows reversed": {
        "int_gemm": lambda qa, qw: _orig["int_gemm"](qa, np.asarray(qw)[::-1])},
    "FP8 GEMM with unsigned weights": {
        "fp8_gemm": lambda a, w: O.e4m3_value(a) @ np.abs(O.e4m3_value(w)).T},
    "epilogue steps swapped": {"dequant_epilogue": lambda acc, sa, sw: _orig["dequant_epilogue"](acc, sw, sa)},
    "epilogue evaluated in float64": {"dequant_epilogue": _epilogue_f64},
    # branches
    "low-rank branch with L2 transposed": {
        "lowrank_branch": lambda x, l1, lw: (np.asarray(x, np.float64) @ np.asarray(l1, np.float64))
        @ np.asarray(lw, np.float64)},
    "low-rank T rounded to binary32": {
        "lowrank_branch": lambda x, l1, lw: (np.asarray(x, np.float64) @ np.asarray(l1, np.float64)).astype(F32)
        .astype(np.float64) @ np.asarray(lw, np.float64).T},
    "kept-channel index shifted by one": {
        "outlier_branch": lambda x, idx, lw: _orig["outlier_branch"](
            x, (np.asarray(idx) + 1) % np.shape(x)[1], lw)},
    # calibration statistics, GPTQ
    "tensor amax of the raw input": {
        "transformed_amax": lambda x, scale, fwht_block=64, order="smooth_then_rotate":
            F32(np.abs(np.asarray(x, F32)).max()) if np.size(x) else F32(0)},
    "GPTQ feedback sign flipped": {"gptq_rows": _gptq_plus},
    "GPTQ updates only the next column": {"gptq_rows": _gptq_with(_next_column_only)},
    "GPTQ error not divided by the pivot": {"gptq_rows": _gptq_with(_no_pivot_division)},
    "GPTQ codes scattered in the inverse order": {"gptq_rows": _gptq_inverse_scatter},
}


def _run_pins():
    failed = []
    for name, fn, kw in PINS:
        try:
            fn(**kw)
        except Exception:   # an assertion, or an error the slip provokes
            failed.append(name)
    return failed


def test_unmutated_oracle_passes_every_pin():
    assert len(PINS) >= 40
    assert _run_pins() == []


@pytest.mark.parametrize("mutant", list(MUTANTS), ids=list(MUTANTS))
def test_planted_mistake_is_caught(monkeypatch, mutant):
    for attr, repl in MUTANTS[mutant].items():
        assert hasattr(O, attr), attr
        monkeypatch.setattr(O, attr, repl)
    failed = _run_pins()
    print(f"[mutant] {mutant}: caught by {len(failed)} pins, e.g. {failed[:3]}")
    assert failed, f"no pin catches: {mutant}"
