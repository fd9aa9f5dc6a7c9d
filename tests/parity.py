"""Comparison helpers for the GPU-vs-oracle parity tests.

Bars: packed codes (int, E2M1, E4M3) and E4M3 scale bytes equal, where any
mismatch is counted and admissible only if the oracle's pre-rounding value
lies within 1e-6 relative of a rounding boundary; fp32 steps equal; raw int32
accumulators equal; outputs within ``rtol * (|y_ref| + rms(y_ref))``
elementwise (rtol 1e-3 for fp32 output, 1e-2 for bf16).
"""
import numpy as np

from oracle import w4a4_oracle as O

BAND = 1e-6
E2M1_BOUNDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
_E4 = O.e4m3_value(np.arange(0x7F))
E4M3_BOUNDS = (_E4[1:] + _E4[:-1]) / 2


# W4A8 activation storage (a layout of this library, not of the pages): the
# int8 codes of each aligned group of 8 K indices are stored even indices
# first, then odd ones -- the byte order in which packed int4 weight codes
# come apart when widened, so both operands reach the matrix cores in the
# same K order.  The oracle emits logical codes; these convert.
W4A8_GROUP_ORDER = np.array([0, 2, 4, 6, 1, 3, 5, 7])


def pack_w4a8_activations(codes):
    c = np.asarray(codes, dtype=np.int8)
    R, K = c.shape
    assert K % 8 == 0
    return np.ascontiguousarray(c.reshape(R, K // 8, 8)[:, :, W4A8_GROUP_ORDER]).reshape(R, K).view(np.uint8)


def unpack_w4a8_activations(packed):
    p = np.asarray(packed).view(np.int8)
    R, K = p.shape
    out = np.empty((R, K // 8, 8), dtype=np.int8)
    out[:, :, W4A8_GROUP_ORDER] = p.reshape(R, K // 8, 8)
    return out.reshape(R, K)


def near_boundary(v, bounds):
    v = np.abs(np.asarray(v, np.float64))
    d = np.min(np.abs(v[..., None] - bounds), axis=-1)
    return d <= BAND * np.maximum(v, 1e-30)


def near_half_integer(v):
    v = np.asarray(v, np.float64)
    return np.abs(np.abs(v - np.floor(v)) - 0.5) <= BAND * np.maximum(np.abs(v), 1e-30)


def unpack_codes(fmt, packed):
    packed = np.asarray(packed)
    if fmt == "int4":
        return O.int4_from_nibbles(O.unpack_nibbles(packed.view(np.uint8)))
    if fmt == "int8":
        return packed.view(np.int8)
    if fmt == "w4a8":
        return unpack_w4a8_activations(packed)
    if fmt == "fp8":
        return packed.view(np.uint8)
    return O.unpack_nibbles(packed.view(np.uint8))


def check_operand(fmt, gpu_codes, gpu_scales, ref, rows=None, what="operand"):
    """Compare one quantized operand; returns the number of admissible mismatches."""
    codes = unpack_codes(fmt, gpu_codes)
    rc = ref["codes"] if rows is None else ref["codes"][rows]
    rv = ref["v"] if rows is None else ref["v"][rows]
    rs = ref["scales"] if rows is None else ref["scales"][rows]
    if fmt == "nvfp4":
        rc = rc.astype(np.uint8)
        s_bad = np.asarray(gpu_scales).view(np.uint8) != rs
        if s_bad.any():
            sv = ref["sv"] if rows is None else ref["sv"][rows]
            assert near_boundary(sv[s_bad], E4M3_BOUNDS).all(), f"{what}: E4M3 scale mismatch outside band"
            rows_bad = np.repeat(s_bad, 16, axis=1)
        else:
            rows_bad = np.zeros_like(rc, dtype=bool)
        bad = (codes != rc) & ~rows_bad
        if bad.any():
            assert near_boundary(rv[bad], E2M1_BOUNDS).all(), (
                f"{what}: {int(bad.sum())} E2M1 code mismatches outside the band")
        return int(bad.sum()) + int(s_bad.sum())
    assert np.array_equal(np.asarray(gpu_scales, np.float32), rs), f"{what}: fp32 steps differ"
    bad = codes != rc
    if bad.any():
        if fmt == "fp8":   # E4M3 rounding boundaries: midpoints of the magnitude grid
            assert near_boundary(rv[bad], E4M3_BOUNDS).all(), f"{what}: {int(bad.sum())} E4M3 mismatches outside the band"
        else:
            assert near_half_integer(rv[bad]).all(), f"{what}: {int(bad.sum())} code mismatches outside the band"
    return int(bad.sum())


def bf16_round(a):
    """fp32 -> nearest bf16 value (round to nearest even), as fp32."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    u = (u + ((u >> 16) & 1) + np.uint32(0x7FFF)) & np.uint32(0xFFFF0000)
    return u.view(np.float32)


def check_output_exact(y, y_ref_f32, y_dtype):
    """Bit equality of an integer linear's output (no branch) with the
    oracle's fp32-ordered epilogue: fp32 as is, bf16 after one RNE rounding."""
    want = np.asarray(y_ref_f32, np.float32)
    if y_dtype == "bf16":
        want = bf16_round(want)
    got = np.asarray(y, np.float32)
    bad = got.view(np.uint32) != want.view(np.uint32)
    assert not bad.any(), (f"{int(bad.sum())} outputs differ from the fp32-ordered epilogue, "
                           f"first at {np.argwhere(bad)[0].tolist()}")


def check_output(y, y_ref, rtol):
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    assert y.shape == y_ref.shape
    assert np.all(np.isfinite(y))
    rms = np.sqrt(np.mean(y_ref ** 2)) if y_ref.size else 0.0
    err = np.abs(y - y_ref)
    bound = rtol * (np.abs(y_ref) + rms)
    worst = float(np.max(err / np.maximum(bound, 1e-30))) if y.size else 0.0
    assert np.all(err <= bound), f"output outside tolerance: worst err/bound = {worst:.3g}"
    return worst
