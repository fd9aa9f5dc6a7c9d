"""CPU oracle for the W4A4 / W8A8 / NVFP4 quantized linear.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, obviously-correct
statement of what the quantized linear computes.  Only the tests, the smoke
check and the CPU-baseline leg of the benchmark may import it; the product
path never calls it and shares no code with it.

Sources (the pages this restates; no text is quoted):

* FoldQuantVLA, "Key Contributions" 1-2 and the authors' abstract:
  channel scaling, a block Hadamard rotation applied by the fast
  Walsh-Hadamard transform with block size 64, dynamic per-token
  quantization of the transformed activations, and the inverse transform
  folded into every consuming weight (its Proposition 1: the folded graph
  computes the same function in exact arithmetic).  Its overview names the
  per-token / per-channel scale layouts and integer GEMMs; contribution 3
  names INT8 W8A8 projections; contribution 4 names INT4 activations and
  W4A4 projections.
* QuantWAMs sec. 3.1, Eq. 1: the runtime quantizer receives A R S^-1
  (rotation R common to a group, diagonal smoothing S); Eq. 2-3: channel
  energy and the top-K mask; sec. 4.2: NVFP4 W4A4, FP8 W8A8 and a BF16
  bypass for the kept channels.
* LatentQuant abstract: NVFP4 W4A4 and activation quantize-dequantize.
* Q-WAM abstract: a 16-bit low-rank branch plus 4-bit complement, both as
  dense matrix products.
* QuantWAMs sec. 3.3, Eq. 14 and the text after it (the weight distortion
  is governed by the layer's activation second moments Sigma_L, which
  also weight GPTQ's error feedback; per-column scores at most choose the
  order of GPTQ's column sweep, and the Hadamard transform shared by every
  context is folded into W before rounding):
  GPTQ-style rounding of the transformed weights, given the Cholesky
  factor of the damped inverse second-moment matrix (calibration data) and
  a column order.
* QuantWAMs, Experimental Details (quantization configuration) and
  sec. 4.4.3: some denoising steps keep their activations at 8 bits while
  the weights stay at 4 bits (W4A8); sec. 4.2: upgraded layers run FP8
  W8A8 (read here as OCP E4M3 codes with per-token and per-channel steps
  amax/448, like the INT8 sibling).

Readings where the pages are silent (each also listed in the design notes):

* smoothing before rotation (FoldQuantVLA's listing order) is the default;
  rotation before smoothing (QuantWAMs Eq. 1 order) is an option;
* Sylvester-ordered Hadamard, butterfly stages h = 1, 2, 4, 8, 16, 32 in
  that order, then the exact factor 1/8;
* the transform and every quantization decision are evaluated in IEEE
  binary32 with round-to-nearest-even (the precision of the kernels that
  take the same decisions);
* the dequantising epilogue of the integer (and FP8) GEMMs is IEEE binary32
  in a fixed order, y = fp32(fp32(fp32(acc) * step_a) * step_w), so an
  integer linear without a branch has one exact answer; the NVFP4 product
  and the 16-bit branches, whose GPU sums have no fixed order, are
  evaluated in binary64;
* a kept-channel (bypass) branch is defined for smoothing before rotation
  only: it removes the raw channels through s = inv_s = 0;
* symmetric integer quantizers: step = amax/Q with Q = 7 (int4) or 127
  (int8), code = clamp(rne(fp32(y/step)), -Q-1, Q), all-zero rows give
  step 0 and codes 0;
* NVFP4: E2M1 element codes, one OCP E4M3 (bias 7, max 448, saturating)
  scale per 16 consecutive K elements, one fp32 tensor scale g per operand
  (a static calibration constant, g = amax(transformed tensor)/(6*448));
* nibble packing: low nibble holds the even K index.

Every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` (closed forms, invariants, brute force); none
is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
F64 = np.float64

FWHT_BLOCK = 64
INT4_QMAX = 7
INT8_QMAX = 127
E4M3_MAX = 448.0
E2M1_MAX = 6.0
NVFP4_BLOCK = 16


# ----------------------------------------------------------------------------
# Hadamard rotation (FoldQuantVLA contribution 2: FWHT, block 64)
# ----------------------------------------------------------------------------
def hadamard_matrix(n: int = FWHT_BLOCK) -> np.ndarray:
    """Sylvester Hadamard matrix H[i, j] = (-1)^popcount(i & j), as int64."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    parity = np.vectorize(lambda v: bin(int(v)).count("1") & 1)(i & j)
    return np.where(parity == 0, 1, -1).astype(np.int64)


def fwht_blocks(u: np.ndarray, block: int = FWHT_BLOCK) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform of each contiguous
    ``block`` of the last axis.  Butterfly stages h = 1, 2, 4, ..., block/2;
    each pair (j, j+h) becomes (u_j + u_{j+h}, u_j - u_{j+h}), evaluated in
    the dtype of ``u`` (one rounding per add or subtract)."""
    u = np.array(u, copy=True)
    R, K = u.shape
    assert K % block == 0
    h = 1
    while h < block:
        v = u.reshape(R, K // (2 * h), 2, h)
        a = v[:, :, 0, :].copy()
        b = v[:, :, 1, :].copy()
        v[:, :, 0, :] = a + b
        v[:, :, 1, :] = a - b
        u = v.reshape(R, K)
        h *= 2
    return u


def transform(x: np.ndarray, scale, fwht_block: int = FWHT_BLOCK,
              order: str = "smooth_then_rotate", dtype=F32) -> np.ndarray:
    """Quantizer-input transform of each row.

    Activations use ``scale`` = inv_s (QuantWAMs Eq. 1, S^-1); weights use
    ``scale`` = s (the inverse folded into the consuming weight,
    FoldQuantVLA contribution 1).  ``fwht_block`` 0 disables the rotation;
    ``scale`` None disables smoothing.  The normalisation 1/8 = 1/sqrt(64)
    makes the rotation orthogonal.
    """
    x = np.asarray(x).astype(dtype)
    sc = None if scale is None else np.asarray(scale).astype(dtype)
    if order not in ("smooth_then_rotate", "rotate_then_smooth"):
        raise ValueError(order)
    u = x
    if sc is not None and order == "smooth_then_rotate":
        u = u * sc[None, :]
    if fwht_block:
        u = fwht_blocks(u, fwht_block) * dtype(1.0 / np.sqrt(fwht_block))
    if sc is not None and order == "rotate_then_smooth":
        u = u * sc[None, :]
    return u.astype(dtype)


# ----------------------------------------------------------------------------
# Symmetric per-row integer quantizer (per token for activations,
# per output channel for weights; FoldQuantVLA overview and contribution 2)
# ----------------------------------------------------------------------------
def quantize_int(y: np.ndarray, qmax: int):
    """Returns (codes int8 [R,K], step fp32 [R], v fp32 [R,K]).

    step = fp32(amax / qmax); v = fp32(y / step) is the pre-rounding value;
    code = clamp(rne(v), -qmax-1, qmax).  A row whose amax is 0 gets step 0
    and all-zero codes."""
    y = np.asarray(y, dtype=F32)
    amax = np.abs(y).max(axis=1)
    step = (amax / F32(qmax)).astype(F32)
    v = np.zeros_like(y)
    nz = step > 0
    v[nz] = (y[nz] / step[nz, None]).astype(F32)
    codes = np.clip(np.rint(v), -qmax - 1, qmax).astype(np.int8)
    return codes, step, v


def dequantize_int(codes: np.ndarray, step: np.ndarray) -> np.ndarray:
    """Quantize-dequantize partner (LatentQuant abstract): code * step, fp32."""
    return (codes.astype(F32) * step.astype(F32)[:, None]).astype(F32)


# ----------------------------------------------------------------------------
# NVFP4 element and scale codecs
# ----------------------------------------------------------------------------
def e2m1_value(code) -> np.ndarray:
    """E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
    Exponent field 0 is subnormal: m * 0.5."""
    c = np.asarray(code, dtype=np.int64) & 0xF
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e - 1.0))
    return np.where(s == 1, -mag, mag).astype(F64)


def e4m3_value(code) -> np.ndarray:
    """OCP E4M3FN: sign bit 7, exponent bits 6..3 (bias 7), mantissa 2..0.
    Exponent 0 is subnormal (m * 2^-9); 0x7F / 0xFF are NaN."""
    c = np.asarray(code, dtype=np.int64) & 0xFF
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(s == 1, -mag, mag).astype(F64)


def _nearest_code(mag: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index into ascending ``grid`` (grid[i] = value of code i, all finite,
    non-negative) nearest to each non-negative ``mag``; a tie picks the even
    code; values beyond the last grid point saturate to it."""
    mag = np.asarray(mag, dtype=F64)
    hi = np.searchsorted(grid, mag, side="left")
    hi = np.clip(hi, 1, len(grid) - 1)
    lo = hi - 1
    dlo = mag - grid[lo]
    dhi = grid[hi] - mag
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(mag >= grid[-1], len(grid) - 1, idx)
    idx = np.where(mag <= 0, 0, idx)
    return idx.astype(np.int64)


_E2M1_GRID = e2m1_value(np.arange(8))          # 0, .5, 1, 1.5, 2, 3, 4, 6
_E4M3_GRID = e4m3_value(np.arange(0x7F))       # 0 ... 448 (0x7E)


def e2m1_encode(v) -> np.ndarray:
    """Round-to-nearest-even onto E2M1, saturating at 6; zero encodes as +0."""
    v = np.asarray(v, dtype=F64)
    mag_code = _nearest_code(np.abs(v), _E2M1_GRID)
    sign = ((v < 0) & (mag_code != 0)).astype(np.int64)
    return (sign << 3 | mag_code).astype(np.uint8)


def e4m3_encode(v) -> np.ndarray:
    """Round-to-nearest-even onto non-negative E4M3FN, saturating at 448."""
    v = np.asarray(v, dtype=F64)
    assert np.all(v >= 0)
    return _nearest_code(v, _E4M3_GRID).astype(np.uint8)


def e4m3_encode_signed(v) -> np.ndarray:
    """Sign-magnitude E4M3FN code: the magnitude rounded to nearest (ties to
    the even code) onto the grid, saturating at 448; anything that rounds
    to zero encodes +0 (0x00)."""
    v = np.asarray(v, dtype=F64)
    mag_code = _nearest_code(np.abs(v), _E4M3_GRID)
    sign = ((v < 0) & (mag_code != 0)).astype(np.int64)
    return (sign << 7 | mag_code).astype(np.uint8)


def quantize_fp8(y: np.ndarray):
    """FP8 W8A8 quantizer of the rows of y (QuantWAMs sec. 4.2: upgraded
    layers run FP8 W8A8).  The reading: one step per row, as for INT8,
    step = fp32(amax / 448), v = fp32(y / step), code = E4M3(v); an
    all-zero row has step 0 and codes 0.  Returns (codes uint8, step fp32,
    v fp32)."""
    y = np.asarray(y, dtype=F32)
    amax = np.abs(y).max(axis=1)
    step = (amax / F32(E4M3_MAX)).astype(F32)
    v = np.zeros_like(y)
    nz = step > 0
    v[nz] = (y[nz] / step[nz, None]).astype(F32)
    return e4m3_encode_signed(v), step, v


def nvfp4_tensor_scale(amax) -> np.float32:
    """Static per-tensor scale g = fp32(amax / (6 * 448)); 1 if amax is 0."""
    amax = F32(amax)
    if amax == 0:
        return F32(1.0)
    return F32(amax / F32(E2M1_MAX * E4M3_MAX))


def quantize_nvfp4(y: np.ndarray, g):
    """NVFP4 per row and per 16-element block b (LatentQuant; QuantWAMs 4.2).

    sb = fp32(bamax / 6); e = E4M3(fp32(sb / g)); S = fp32(value(e) * g);
    c_k = E2M1(fp32(y_k / S)) (all-zero codes when S = 0).

    Returns (codes uint8 nibbles [R,K], scale bytes uint8 [R,K/16],
    scale pre-rounding values fp32 [R,K/16], element pre-rounding fp32 [R,K]).
    """
    y = np.asarray(y, dtype=F32)
    g = F32(g)
    R, K = y.shape
    assert K % NVFP4_BLOCK == 0
    yb = y.reshape(R, K // NVFP4_BLOCK, NVFP4_BLOCK)
    bamax = np.abs(yb).max(axis=2)
    sb = (bamax / F32(E2M1_MAX)).astype(F32)
    sv = (sb / g).astype(F32)
    e = e4m3_encode(sv)
    S = (e4m3_value(e).astype(F32) * g).astype(F32)
    v = np.zeros_like(yb)
    nz = S > 0
    v[nz] = (yb[nz] / S[nz][:, None]).astype(F32)
    codes = e2m1_encode(v).reshape(R, K)
    return codes, e, sv, v.reshape(R, K)


def dequantize_nvfp4(codes, scale_bytes, g) -> np.ndarray:
    """value(c) * value(e) * g for every element, float64 (exact)."""
    R, K = codes.shape
    sv = e4m3_value(scale_bytes)
    return (e2m1_value(codes).reshape(R, K // NVFP4_BLOCK, NVFP4_BLOCK)
            * sv[:, :, None]).reshape(R, K) * F64(F32(g))


# ----------------------------------------------------------------------------
# Packing (low nibble = even K index; int4 two's complement)
# ----------------------------------------------------------------------------
def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    c = (np.asarray(codes).astype(np.int64) & 0xF).astype(np.uint8)
    assert c.shape[-1] % 2 == 0
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def int4_from_nibbles(n: np.ndarray) -> np.ndarray:
    n = np.asarray(n).astype(np.int64)
    return np.where(n >= 8, n - 16, n).astype(np.int8)


# ----------------------------------------------------------------------------
# GEMM, epilogue, 16-bit branch
# ----------------------------------------------------------------------------
def int_gemm(qa: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k qa[m, k] * qw[n, k], exact.

    Evaluated as a float64 matrix product: every partial sum is an integer of
    magnitude <= 128*128*K < 2^53, so the result is exact in any order."""
    qa = np.asarray(qa, dtype=np.int64)
    qw = np.asarray(qw, dtype=np.int64)
    K = qa.shape[1]
    assert qw.shape[1] == K and 128 * 128 * K < 2 ** 53
    acc = qa.astype(F64) @ qw.astype(F64).T
    acc = acc.astype(np.int64)
    assert np.all(np.abs(acc) < 2 ** 31)
    return acc


def dequant_epilogue(acc, step_a, step_w) -> np.ndarray:
    """Dequantising epilogue in IEEE binary32, one rounding per operation
    (FoldQuantVLA overview: per-token activation steps and per-output-
    channel weight steps applied to the integer GEMM result):
    y = fp32(fp32(fp32(acc) * step_a[m]) * step_w[n]).  The conversion of
    the accumulator rounds to nearest even (exact for |acc| <= 2^24).
    Returns float32."""
    a = np.asarray(acc)
    a = a.astype(F32) if a.dtype != F32 else a
    t = (a * np.asarray(step_a, F32)[:, None]).astype(F32)
    return (t * np.asarray(step_w, F32)[None, :]).astype(F32)


def fp8_gemm(codes_a: np.ndarray, codes_w: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k value(a[m, k]) * value(w[n, k]) over E4M3 codes,
    float64 and exact: every product is a multiple of 2^-18 below 2^18, so
    for K <= 2^16 every partial sum fits 53 bits in any order."""
    assert codes_a.shape[1] <= 1 << 16
    return e4m3_value(codes_a) @ e4m3_value(codes_w).T


def lowrank_branch(x, l1, lw) -> np.ndarray:
    """Q-WAM 16-bit branch: (x L1) L2 with L2 = lw^T, float64."""
    return (np.asarray(x, F64) @ np.asarray(l1, F64)) @ np.asarray(lw, F64).T


def outlier_branch(x, idx, lw) -> np.ndarray:
    """QuantWAMs BF16 bypass: x[:, idx] W[:, idx]^T, float64."""
    return np.asarray(x, F64)[:, np.asarray(idx)] @ np.asarray(lw, F64).T


# ----------------------------------------------------------------------------
# GPTQ-style rounding (pack time)
# ----------------------------------------------------------------------------
def gptq_rows(wt, step, u, qmax: int, perm=None):
    """Round the transformed weight rows ``wt`` (N x K, fp32) column by column
    with error feedback.

    ``step`` holds the per-row steps of the round-to-nearest quantizer (fp32);
    ``u`` (K x K, float64) is the upper Cholesky factor of (Sigma + lambda I)^-1
    with Sigma's rows and columns taken in processing order; ``perm`` is that
    order (natural when None).  Column t of the processing order is rounded
    (nearest, ties to even, clamped) from its current value; its error,
    divided by u[t, t], updates every later column v by -err * u[t, v] (one
    float64 product and one float64 subtraction per element).  Returns
    (codes int8 [N, K] in the original column order, err float64 [N, K] in
    processing order)."""
    wt = np.asarray(wt, dtype=F32)
    N, K = wt.shape
    perm = np.arange(K) if perm is None else np.asarray(perm)
    W = wt[:, perm].astype(F64)
    sf = np.asarray(step, dtype=F32).astype(F64)
    nz = sf > 0
    Q = np.zeros((N, K), dtype=np.int64)
    E = np.zeros((N, K), dtype=F64)
    for t in range(K):
        col = W[:, t]
        q = np.zeros(N, dtype=F64)
        q[nz] = np.clip(np.rint(col[nz] / sf[nz]), -qmax - 1, qmax)
        err = (col - q * sf) / u[t, t]
        if t + 1 < K:
            W[:, t + 1:] -= np.outer(err, u[t, t + 1:])
        Q[:, t] = q
        E[:, t] = err
    codes = np.empty((N, K), dtype=np.int8)
    codes[:, perm] = Q.astype(np.int8)
    return codes, E


# ----------------------------------------------------------------------------
# Whole path
# ----------------------------------------------------------------------------
def quantize_operand(x, scale, fmt: str, fwht_block=FWHT_BLOCK,
                     order="smooth_then_rotate", g=None) -> dict:
    """Transform then quantize the rows of one operand.

    Activations pass inv_s (per-token scales), weights pass s (per-output-
    channel scales): the arithmetic is the same."""
    y = transform(x, scale, fwht_block, order)
    if fmt in ("int4", "int8", "w4a8"):
        # "w4a8": the activation side of W4A8 (int8 codes, Q = 127)
        qmax = INT4_QMAX if fmt == "int4" else INT8_QMAX
        codes, step, v = quantize_int(y, qmax)
        # "w4a8" activations are the int8 codes; any storage order a GEMM
        # prefers is a library layout, not part of the method
        packed = pack_nibbles(codes) if fmt == "int4" else codes.view(np.uint8)
        return {"y": y, "codes": codes, "scales": step, "v": v, "packed": packed}
    if fmt == "fp8":
        codes, step, v = quantize_fp8(y)
        return {"y": y, "codes": codes, "scales": step, "v": v, "packed": codes}
    if fmt == "nvfp4":
        if g is None:
            g = nvfp4_tensor_scale(np.abs(y).max() if y.size else 0.0)
        codes, e, sv, v = quantize_nvfp4(y, g)
        return {"y": y, "codes": codes, "scales": e, "sv": sv, "v": v,
                "packed": pack_nibbles(codes), "g": F32(g)}
    raise ValueError(fmt)


def transformed_amax(x, scale, fwht_block=FWHT_BLOCK, order="smooth_then_rotate"):
    """max |transform(x)| over the whole tensor (fp32): the calibration
    statistic behind the static NVFP4 tensor scale."""
    y = transform(x, scale, fwht_block, order)
    return F32(np.abs(y).max()) if y.size else F32(0)


# Activation and weight formats of each linear: W4A8 is the 8-bit-activation
# step of the QuantWAMs schedule (Experimental Details, quantization
# configuration; sec. 4.4.3), with the same 4-bit weight codes as W4A4; its
# activations are the int8 quantization.
OPERAND_FORMATS = {"int4": ("int4", "int4"), "int8": ("int8", "int8"),
                   "nvfp4": ("nvfp4", "nvfp4"), "w4a8": ("w4a8", "int4"), "fp8": ("fp8", "fp8")}


def linear(case, order="smooth_then_rotate", g_a=None, g_w=None) -> dict:
    """Full quantized linear for a ``workloads.Case``: quantize activations
    and weights, integer (or NVFP4) GEMM, dequant epilogue, 16-bit branch.
    Returns the intermediate codes, scales and accumulators and y (float64)."""
    fb = case.fwht_block
    if case.branch is not None and case.branch["kind"] == "outlier" and order != "smooth_then_rotate":
        # Kept channels leave the quantized path through s = inv_s = 0, which
        # removes the raw channels only when smoothing precedes the rotation;
        # after a rotation the zeros would land on rotated coordinates and the
        # bypass would count the kept channels twice.
        raise ValueError("a kept-channel branch needs smoothing before the rotation")
    fa, fw = OPERAND_FORMATS[case.fmt]
    A = quantize_operand(case.x, case.inv_s, fa, fb, order, g_a)
    W = quantize_operand(case.w, case.s, fw, fb, order, g_w)
    gq = getattr(case, "gptq", None)
    if gq is not None:   # GPTQ rounding of the weights instead of round-to-nearest
        assert fw in ("int4", "int8")
        codes, _ = gptq_rows(W["y"], W["scales"], gq["u"], INT4_QMAX if fw == "int4" else INT8_QMAX,
                             gq["perm"])
        W = dict(W, codes=codes, packed=pack_nibbles(codes) if fw == "int4" else codes.view(np.uint8))
    out = {"a": A, "w": W}
    if case.fmt in ("int4", "int8", "w4a8"):
        acc = int_gemm(A["codes"], W["codes"])
        y = dequant_epilogue(acc, A["scales"], W["scales"])
        out["acc"] = acc
    elif case.fmt == "fp8":
        acc = fp8_gemm(A["codes"], W["codes"])
        y = dequant_epilogue(acc, A["scales"], W["scales"])
        out["acc"] = acc
    else:
        da = dequantize_nvfp4(A["codes"], A["scales"], A["g"])
        dw = dequantize_nvfp4(W["codes"], W["scales"], W["g"])
        y = da @ dw.T
    out["y_main"] = y
    br = case.branch
    if br is not None:
        if br["kind"] == "lowrank":
            y = y + lowrank_branch(case.x, br["l1"], br["lw"])
        elif br["kind"] == "outlier":
            y = y + outlier_branch(case.x, br["idx"], br["lw"])
        else:
            raise ValueError(br["kind"])
    out["y"] = y
    return out
