"""Pins for the CPU oracle (CPU only).

The pages print no worked numeric example for the quantized linear, so each
oracle function is pinned to something other than itself: closed forms,
format definitions (tests/golden/*.txt), invariants of the mechanism and
brute force on tiny inputs.  Each pin is chosen so that a plausible slip
(dropped term, wrong sign, wrong index, transposed operand, wrong tie rule)
fails at least one test.
"""
import os

import numpy as np
import pytest

from oracle import w4a4_oracle as O
from parity import pack_w4a8_activations, unpack_w4a8_activations
from w4a4_post_quantized_channel_amd import workloads as WL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _sections(path):
    out, cur = {}, None
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        if line.startswith("["):
            cur = line.strip("[]").strip()
            out[cur] = []
        else:
            out[cur].append(line.split())
    return out


# --------------------------------------------------------------------- FWHT
def test_hadamard_orthogonal_and_sylvester():
    H = O.hadamard_matrix(64)
    assert np.array_equal(H @ H.T, 64 * np.eye(64, dtype=np.int64))
    assert np.array_equal(H, H.T)
    assert np.all(H[0] == 1) and np.all(H[:, 0] == 1)
    # Sylvester recursion H_2n = [[H, H], [H, -H]]
    h32 = O.hadamard_matrix(32)
    assert np.array_equal(H, np.block([[h32, h32], [h32, -h32]]))


def test_fwht_one_hot_gives_hadamard_rows():
    H = O.hadamard_matrix(64)
    K = 192
    for i in [0, 1, 3, 37, 63, 64, 100, 191]:
        x = np.zeros((1, K))
        x[0, i] = 1.0
        y = O.transform(x, None, 64, dtype=np.float64)[0]
        b, j = divmod(i, 64)
        expect = np.zeros(K)
        expect[64 * b:64 * b + 64] = H[j] / 8.0
        assert np.array_equal(y, expect), i


def test_fwht_matches_dense_product():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((9, 256)).astype(np.float32)
    H = O.hadamard_matrix(64).astype(np.float64) / 8.0
    dense = np.concatenate([x[:, 64 * b:64 * b + 64].astype(np.float64) @ H
                            for b in range(4)], axis=1)
    fast = O.transform(x, None, 64)
    assert fast.dtype == np.float32
    assert np.max(np.abs(fast - dense)) <= 1e-6 * np.max(np.abs(dense))


def test_fwht_is_an_involution_on_small_integers():
    rng = np.random.default_rng(8)
    x = rng.integers(-50, 50, size=(5, 128)).astype(np.float32)
    y = O.transform(O.transform(x, None, 64), None, 64)
    assert np.array_equal(y, x)


def test_fwht_stage_order_matters_only_by_rounding():
    # unnormalised FWHT of integers equals H x exactly
    rng = np.random.default_rng(9)
    x = rng.integers(-9, 9, size=(3, 64)).astype(np.float32)
    H = O.hadamard_matrix(64)
    assert np.array_equal(O.fwht_blocks(x).astype(np.int64), x.astype(np.int64) @ H.T)


@pytest.mark.parametrize("order", ["smooth_then_rotate", "rotate_then_smooth"])
def test_folding_reproduces_float_linear(order):
    # FoldQuantVLA Proposition 1: (X S^-1 R)(W S R)^T = X W^T in exact arithmetic
    c = WL.linear_case(8, 48, 256, seed=11, n_outliers=4, outlier_gain=20.0)
    s64 = c.s.astype(np.float64)
    xa = O.transform(c.x, 1.0 / s64, 64, order, dtype=np.float64)
    wa = O.transform(c.w, s64, 64, order, dtype=np.float64)
    ref = c.x.astype(np.float64) @ c.w.astype(np.float64).T
    got = xa @ wa.T
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_smoothing_is_applied_per_channel_before_rotation():
    # Scaling channel j of x by c and its smoothing factor by 1/c leaves the
    # transformed row unchanged (powers of two keep it exact).
    rng = np.random.default_rng(12)
    x = rng.standard_normal((2, 64)).astype(np.float32)
    inv = np.abs(rng.standard_normal(64)).astype(np.float32) + 0.5
    y0 = O.transform(x, inv, 64)
    x2 = x.copy(); x2[:, 5] *= 4
    inv2 = inv.copy(); inv2[5] /= 4
    assert np.array_equal(O.transform(x2, inv2, 64), y0)
    # with rotation off, smoothing is a plain per-channel product
    assert np.array_equal(O.transform(x, inv, 0), (x * inv).astype(np.float32))


# ------------------------------------------------------------ int quantizer
def test_golden_onehot_fwht_int4():
    g = _sections(os.path.join(GOLDEN, "fwht_int4_onehot.txt"))
    inp = dict((k, v) for k, v in g["input"])
    K, i, val = int(inp["K"]), int(inp["index"]), float(inp["value"])
    x = np.zeros((1, K), np.float32)
    x[0, i] = val
    q = O.quantize_operand(x, None, "int4", 64)
    pattern = [int(v) for v in g["codes_block1_pattern"][0]]
    assert np.all(q["codes"][0, :64] == 0)
    assert np.array_equal(q["codes"][0, 64:], np.tile(pattern, 16))
    assert q["scales"][0] == np.float32(np.float32(0.625) / np.float32(7))
    hexrow = g["packed_row_hex"][0][0]
    assert q["packed"][0].tobytes().hex() == hexrow


def _brute_nearest_int(v, lo, hi):
    cands = np.arange(lo, hi + 1)
    out = []
    for t in np.asarray(v, np.float64).ravel():
        d = np.abs(cands - t)
        best = cands[d == d.min()]
        if len(best) > 1:
            best = best[best % 2 == 0]
        out.append(best[0])
    return np.array(out).reshape(np.shape(v))


@pytest.mark.parametrize("qmax", [7, 127])
def test_int_quantizer_brute_force_rounding(qmax):
    rng = np.random.default_rng(13)
    y = (rng.standard_normal((6, 64)) * rng.uniform(0.01, 50, (6, 1))).astype(np.float32)
    codes, step, v = O.quantize_int(y, qmax)
    assert np.array_equal(codes, _brute_nearest_int(v, -qmax - 1, qmax))
    # exact half-integer pre-rounding values go to the even neighbour
    halves = np.array([[0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 6.5, -7.5]], np.float32)
    assert np.array_equal(_brute_nearest_int(halves, -8, 7), [[0, 2, 2, 0, -2, -2, 6, -8]])
    assert np.array_equal(np.clip(np.rint(halves), -8, 7), [[0, 2, 2, -0, -2, -2, 6, -8]])
    # through the quantizer: a row peaking at qmax has step 1 exactly, so its
    # half-integer entries reach the rounding as exact ties (even neighbour)
    row = np.array([[qmax, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, qmax - 0.5, -(qmax - 0.5)]], np.float32)
    codes, step, v = O.quantize_int(row, qmax)
    assert step[0] == 1 and np.array_equal(v, row)
    even_top = qmax - 1 if (qmax - 1) % 2 == 0 else qmax
    assert codes[0].tolist() == [qmax, 0, 2, 2, 0, -2, -2, even_top, -even_top]


@pytest.mark.parametrize("qmax", [7, 127])
def test_int_quantizer_invariants(qmax):
    rng = np.random.default_rng(14)
    y = (rng.standard_normal((400, 96)) * rng.lognormal(0, 2, (400, 1))).astype(np.float32)
    y[3] = 0.0
    codes, step, v = O.quantize_int(y, qmax)
    # scale definition
    amax = np.abs(y).max(axis=1)
    assert np.array_equal(step, (amax / np.float32(qmax)).astype(np.float32))
    # zero row
    assert step[3] == 0 and np.all(codes[3] == 0)
    nz = step > 0
    # every non-zero row reaches +-qmax and never the (unreachable) -qmax-1
    assert np.all(np.abs(codes[nz]).max(axis=1) == qmax)
    assert codes.min() >= -qmax
    # dequantisation error within half a step
    dq = O.dequantize_int(codes, step).astype(np.float64)
    err = np.abs(dq - y)
    assert np.all(err <= step[:, None].astype(np.float64) * 0.5 * (1 + 1e-5) + 1e-30)
    # quantize-dequantize is idempotent on its own output
    codes2, _, _ = O.quantize_int(O.dequantize_int(codes, step), qmax)
    assert np.array_equal(codes2, codes)


def test_int_quantizer_sign_and_scale_equivariance():
    rng = np.random.default_rng(15)
    y = rng.standard_normal((50, 64)).astype(np.float32)
    c1, s1, _ = O.quantize_int(y, 7)
    c2, s2, _ = O.quantize_int(-y, 7)
    assert np.array_equal(c2, -c1) and np.array_equal(s1, s2)
    c3, s3, _ = O.quantize_int(y * np.float32(4), 7)
    assert np.array_equal(c3, c1) and np.array_equal(s3, s1 * 4)


# ------------------------------------------------------------ NVFP4 codecs
def test_golden_e2m1_and_e4m3_tables():
    g = _sections(os.path.join(GOLDEN, "nvfp4_codec.txt"))
    for code, val in g["e2m1_decode"]:
        got = O.e2m1_value(int(code, 16))
        assert got == float(val) and np.signbit(got) == val.startswith("-")
    for val, code in g["e2m1_encode"]:
        assert int(O.e2m1_encode(float(val))) == int(code, 16), val
    for code, val in g["e4m3_decode"]:
        assert O.e4m3_value(int(code, 16)) == float(val)
    for val, code in g["e4m3_encode"]:
        assert int(O.e4m3_encode(float(val))) == int(code, 16), val
    assert np.isnan(O.e4m3_value(0x7F)) and np.isnan(O.e4m3_value(0xFF))


def test_e4m3_grid_is_the_full_finite_format():
    vals = O.e4m3_value(np.arange(0x7F))
    assert np.all(np.diff(vals) > 0)          # strictly increasing positive codes
    assert vals[0] == 0 and vals[-1] == 448
    # every finite E4M3 value is a 4-significant-bit dyadic number
    for v in vals[1:]:
        m, e = np.frexp(v)
        assert (m * 16) == np.floor(m * 16)


def _brute_nearest_grid(v, values, codes):
    out = []
    for t in np.asarray(v, np.float64).ravel():
        d = np.abs(values - t)
        cand = codes[d == d.min()]
        if len(cand) > 1:
            cand = cand[cand % 2 == 0]
        out.append(cand[0])
    return np.array(out)


def test_e2m1_encode_brute_force():
    rng = np.random.default_rng(16)
    v = np.concatenate([rng.uniform(-8, 8, 3000),
                        np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -6.0])])
    got = O.e2m1_encode(v)
    mag = np.minimum(np.abs(v), 6.0)
    grid = O.e2m1_value(np.arange(8))
    want_mag = _brute_nearest_grid(mag, grid, np.arange(8))
    want = np.where((v < 0) & (want_mag != 0), want_mag | 8, want_mag)
    assert np.array_equal(got, want)


def test_e4m3_encode_brute_force():
    rng = np.random.default_rng(17)
    codes = np.arange(0x7F)
    grid = O.e4m3_value(codes)
    mids = (grid[1:] + grid[:-1]) / 2
    v = np.concatenate([np.exp(rng.uniform(np.log(1e-4), np.log(600), 3000)), mids, grid])
    got = O.e4m3_encode(v)
    want = _brute_nearest_grid(np.minimum(v, 448.0), grid, codes)
    assert np.array_equal(got, want)


def test_nvfp4_quantizer_invariants():
    rng = np.random.default_rng(18)
    y = (rng.standard_normal((64, 256)) * rng.lognormal(0, 1.5, (64, 1))).astype(np.float32)
    y[5, 16:32] = 0.0
    g = O.nvfp4_tensor_scale(np.abs(y).max())
    codes, e, sv, v = O.quantize_nvfp4(y, g)
    assert codes.shape == y.shape and e.shape == (64, 16)
    # zero block -> zero scale and zero codes
    assert e[5, 1] == 0 and np.all(codes[5, 16:32] == 0)
    # the largest block of the tensor maps to the largest finite scale
    assert e.max() == 0x7E
    # g = amax / (6 * 448) puts the tensor's largest element on the top of both
    # grids: scale code 448, element code +-6, and it dequantizes back to
    # +-amax (three binary32 roundings: g, S = 448 g, 6 S)
    i, j = np.unravel_index(np.argmax(np.abs(y)), y.shape)
    assert e[i, j // 16] == 0x7E and (codes[i, j] & 7) == 7
    top = np.float32(6.0) * np.float32(np.float32(448.0) * np.float32(g))
    assert abs(float(top) - float(np.abs(y).max())) <= 4 * np.spacing(np.float32(np.abs(y).max()))
    # blocks whose scale is in the normal E4M3 range reach the largest element code
    mag = codes & 7
    normal = sv >= 2.0 ** -6
    assert np.all(mag.reshape(64, 16, 16).max(axis=2)[normal] == 7)
    # element codes are the nearest E2M1 values of y / S
    S = (O.e4m3_value(e).astype(np.float32) * np.float32(g)).astype(np.float32)
    Sx = np.repeat(S, 16, axis=1)
    ok = Sx > 0
    ratio = np.zeros_like(y)
    ratio[ok] = (y[ok] / Sx[ok]).astype(np.float32)
    assert np.array_equal(codes, O.e2m1_encode(ratio))
    # quantize-dequantize is idempotent for a fixed tensor scale
    dq = O.dequantize_nvfp4(codes, e, g).astype(np.float32)
    codes2, e2, _, _ = O.quantize_nvfp4(dq, g)
    assert np.array_equal(codes2, codes) and np.array_equal(e2, e)


# ----------------------------------------------------------------- packing
def test_packing_layout_and_roundtrip():
    codes = np.array([[1, -2, 7, -8]], np.int8)
    p = O.pack_nibbles(codes)
    assert p.tolist() == [[0xE1, 0x87]]
    rng = np.random.default_rng(19)
    c = rng.integers(-8, 8, size=(7, 64)).astype(np.int8)
    assert np.array_equal(O.int4_from_nibbles(O.unpack_nibbles(O.pack_nibbles(c))), c)


# -------------------------------------------------------------------- GEMM
def test_int_gemm_brute_force_and_closed_forms():
    rng = np.random.default_rng(20)
    for (M, N, K) in [(1, 1, 64), (3, 5, 64), (7, 4, 128)]:
        a = rng.integers(-8, 8, size=(M, K))
        w = rng.integers(-8, 8, size=(N, K))
        acc = O.int_gemm(a, w)
        brute = np.zeros((M, N), np.int64)
        for m in range(M):
            for n in range(N):
                t = 0
                for k in range(K):
                    t += int(a[m, k]) * int(w[n, k])
                brute[m, n] = t
        assert np.array_equal(acc, brute)
    K = 8192
    assert O.int_gemm(np.full((2, K), 7), np.full((3, K), 7)).tolist() == [[49 * K] * 3] * 2
    alt = np.tile([7, -7], K // 2)
    assert np.all(O.int_gemm(np.full((1, K), 7), alt[None]) == 0)
    assert O.int_gemm(np.full((1, K), -128), np.full((1, K), -128))[0, 0] == 16384 * K


def test_dequant_epilogue_orientation():
    acc = np.array([[1, 2, 3], [4, 5, 6]])
    y = O.dequant_epilogue(acc, np.array([10.0, 100.0]), np.array([1.0, 2.0, 4.0]))
    assert y.tolist() == [[10, 40, 120], [400, 1000, 2400]]


def test_dequant_epilogue_is_binary32_in_a_fixed_order():
    """y = fp32(fp32(fp32(acc) * step_a) * step_w).  Pinned by cases whose
    exact value is known and where a rounding step shows:
    * acc = 2^24 + 1 is not a binary32 value; it converts to 2^24 (ties to
      even), so with unit steps y = 2^24 (an exact epilogue gives 2^24 + 1);
    * (1 + 2^-23)^2 = 1 + 2^-22 + 2^-46 rounds to 1 + 2^-22 in binary32;
    * on random data every result is within three binary32 roundings of the
      exact product and some differ from the float64 evaluation."""
    y = O.dequant_epilogue(np.array([[2 ** 24 + 1]], np.int64), np.ones(1), np.ones(1))
    assert y.dtype == np.float32 and y[0, 0] == np.float32(2.0 ** 24)
    a = np.float32(1 + 2.0 ** -23)
    y = O.dequant_epilogue(np.array([[1]]), np.array([a]), np.array([a]))
    assert y[0, 0] == np.float32(1 + 2.0 ** -22)
    # every result lies within three binary32 roundings of the exact product
    rng = np.random.default_rng(30)
    acc = rng.integers(-2 ** 27, 2 ** 27, size=(40, 50))
    sa = rng.lognormal(-8, 2, 40).astype(np.float32)
    sw = rng.lognormal(-4, 2, 50).astype(np.float32)
    y = O.dequant_epilogue(acc, sa, sw).astype(np.float64)
    exact = acc.astype(np.float64) * sa.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]
    assert np.all(np.abs(y - exact) <= 3.0001 * 2.0 ** -24 * np.abs(exact))
    # and it is not the float64 evaluation: some element must differ
    assert np.any(y != exact)


def test_nvfp4_gemm_equals_blockwise_integer_form():
    # y = g_a g_w sum_b value(e_a) value(e_w) sum_{k in b} value(c_a) value(c_w)
    rng = np.random.default_rng(21)
    M, N, K = 3, 4, 64
    ya = rng.standard_normal((M, K)).astype(np.float32)
    yw = rng.standard_normal((N, K)).astype(np.float32)
    ga, gw = O.nvfp4_tensor_scale(np.abs(ya).max()), O.nvfp4_tensor_scale(np.abs(yw).max())
    ca, ea, _, _ = O.quantize_nvfp4(ya, ga)
    cw, ew, _, _ = O.quantize_nvfp4(yw, gw)
    got = O.dequantize_nvfp4(ca, ea, ga) @ O.dequantize_nvfp4(cw, ew, gw).T
    want = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            tot = 0.0
            for b in range(K // 16):
                P = 0
                for k in range(16 * b, 16 * b + 16):
                    P += int(2 * O.e2m1_value(ca[m, k])) * int(2 * O.e2m1_value(cw[n, k]))
                tot += O.e4m3_value(ea[m, b]) * O.e4m3_value(ew[n, b]) * P / 4.0
            want[m, n] = float(ga) * float(gw) * tot
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))


# ------------------------------------------------------------------ branch
def test_branches_brute_force():
    rng = np.random.default_rng(22)
    M, K, N, r = 3, 10, 4, 2
    x = rng.standard_normal((M, K))
    l1 = rng.standard_normal((K, r))
    lw = rng.standard_normal((N, r))
    y = O.lowrank_branch(x, l1, lw)
    for m in range(M):
        for n in range(N):
            t = sum(sum(x[m, k] * l1[k, j] for k in range(K)) * lw[n, j] for j in range(r))
            assert abs(y[m, n] - t) < 1e-12
    idx = np.array([1, 7])
    yo = O.outlier_branch(x, idx, lw)
    for m in range(M):
        for n in range(N):
            assert abs(yo[m, n] - (x[m, 1] * lw[n, 0] + x[m, 7] * lw[n, 1])) < 1e-12
    assert np.all(O.outlier_branch(x, np.zeros(0, int), np.zeros((N, 0))) == 0)


def test_lowrank_case_reconstructs_float_weight():
    c = WL.linear_case(16, 64, 128, seed=23, lowrank=4)
    l1, lw = c.branch["l1"].astype(np.float64), c.branch["lw"].astype(np.float64)
    recon = lw @ l1.T + c.w.astype(np.float64)
    assert np.max(np.abs(recon - c.w_full)) < 1e-6


def test_outlier_case_selects_top_energy_channels():
    c = WL.linear_case(32, 16, 256, seed=24, fmt="nvfp4", n_outliers=8,
                       outlier_gain=30.0, keep_channels=8)
    assert np.array_equal(np.sort(c.branch["idx"]), c.meta["outliers"])
    assert np.all(c.inv_s[c.branch["idx"]] == 0) and np.all(c.s[c.branch["idx"]] == 0)
    # the quantized path carries nothing for the kept channels
    q = O.quantize_operand(c.x, c.inv_s, "nvfp4", 0)
    assert np.all(q["y"][:, c.branch["idx"]] == 0)


def test_transformed_amax_closed_forms():
    """The statistic behind the static NVFP4 tensor scale.  A one-hot row
    v e_i (block b = i // 64, position j = i % 64):
    * smoothing first: u = v s_i e_i, and the rotation spreads it over the
      block as +-v s_i / 8, so the maximum is |v s_i| / 8;
    * rotation first: +-v / 8 over block b, then times s_k, so the maximum
      is |v| / 8 * max_{k in block b} |s_k|.
    An all-zero tensor gives 0.  Powers of two keep every value exact."""
    K = 192
    s = np.exp2(np.arange(K) % 7 - 3).astype(np.float32)
    s[130] = 8.0
    for i, v in [(5, 3.0), (64 + 17, -0.5), (130, 2.0), (191, -6.0)]:
        x = np.zeros((3, K), np.float32)
        x[1, i] = v
        b = i // 64
        got = O.transformed_amax(x, s, 64, "smooth_then_rotate")
        assert got == np.float32(abs(v * s[i]) / 8), i
        got = O.transformed_amax(x, s, 64, "rotate_then_smooth")
        assert got == np.float32(abs(v) / 8 * np.abs(s[64 * b:64 * b + 64]).max()), i
    assert O.transformed_amax(np.zeros((4, 64), np.float32), s[:64]) == 0
    assert O.transformed_amax(np.zeros((0, 64), np.float32), s[:64]) == 0
    # the maximum is over the whole tensor, not a row
    x = np.zeros((4, 128), np.float32)
    x[0, 3], x[3, 70] = 1.0, -16.0
    assert O.transformed_amax(x, None, 64) == np.float32(2.0)


def test_kept_channels_fold_exactly_with_smoothing_first():
    """Kept channels (s = inv_s = 0) plus the bf16 bypass reproduce the float
    linear with those weight columns in bf16, exactly in float64 before
    quantization (FoldQuantVLA Proposition 1 applied to the remaining
    channels), when smoothing precedes the rotation."""
    c = WL.linear_case(16, 40, 256, seed=33, fmt="nvfp4", n_outliers=6, outlier_gain=30.0,
                       keep_channels=6)
    idx = c.branch["idx"]
    s64 = c.s.astype(np.float64)
    inv = np.divide(1.0, s64, out=np.zeros_like(s64), where=s64 != 0)
    xa = O.transform(c.x, inv, 64, "smooth_then_rotate", dtype=np.float64)
    wa = O.transform(c.w, c.s.astype(np.float64), 64, "smooth_then_rotate", dtype=np.float64)
    w_kept = c.w_full.astype(np.float64).copy()
    w_kept[:, idx] = c.branch["lw"]
    want = c.x.astype(np.float64) @ w_kept.T
    got = xa @ wa.T + O.outlier_branch(c.x, idx, c.branch["lw"])
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))
    # the other order cannot express kept channels: the zeros land on rotated
    # coordinates, so the same construction is far off, and the oracle refuses it
    xr = O.transform(c.x, inv, 64, "rotate_then_smooth", dtype=np.float64)
    wr = O.transform(c.w, c.s.astype(np.float64), 64, "rotate_then_smooth", dtype=np.float64)
    bad = xr @ wr.T + O.outlier_branch(c.x, idx, c.branch["lw"])
    assert np.max(np.abs(bad - want)) > 0.1 * np.max(np.abs(want))
    with pytest.raises(ValueError):
        O.linear(c, order="rotate_then_smooth")
    O.linear(c, order="smooth_then_rotate")


# ------------------------------------------------------------- whole path
def test_whole_path_tiny_consistency():
    c = WL.workload("tiny")
    out = O.linear(c)
    A, W = out["a"], out["w"]
    # accumulators from packed codes
    a = O.int4_from_nibbles(O.unpack_nibbles(A["packed"]))
    w = O.int4_from_nibbles(O.unpack_nibbles(W["packed"]))
    assert np.array_equal(O.int_gemm(a, w), out["acc"])
    # quantized product approximates the float linear (sanity, no bound from the pages)
    ref = c.x.astype(np.float64) @ c.w.astype(np.float64).T
    sqnr = 10 * np.log10(np.sum(ref ** 2) / np.sum((out["y"] - ref) ** 2))
    assert sqnr > 10.0
    # rotation + smoothing beat plain per-token int4 on outlier-heavy input
    plain = O.quantize_operand(c.x, None, "int4", 0)
    plainw = O.quantize_operand(c.w, None, "int4", 0)
    yp = O.dequant_epilogue(O.int_gemm(plain["codes"], plainw["codes"]), plain["scales"], plainw["scales"])
    sqnr_plain = 10 * np.log10(np.sum(ref ** 2) / np.sum((yp - ref) ** 2))
    assert sqnr > sqnr_plain


def test_whole_path_nvfp4_and_branch_small():
    c = WL.linear_case(48, 40, 320, seed=25, fmt="nvfp4", n_outliers=8,
                       outlier_gain=30.0, keep_channels=8)
    out = O.linear(c)
    ref = c.x.astype(np.float64) @ c.w_full.astype(np.float64).T
    sqnr = 10 * np.log10(np.sum(ref ** 2) / np.sum((out["y"] - ref) ** 2))
    assert sqnr > 15.0
    # branch contribution is exactly the kept-channel product
    assert np.allclose(out["y"] - out["y_main"],
                       c.x[:, c.branch["idx"]].astype(np.float64) @ c.branch["lw"].astype(np.float64).T)


# ------------------------------------------------------------------- W4A8
def _plain_case(x, w, fmt):
    """A case without smoothing or rotation: the quantizers see x and w."""
    x = np.asarray(x, np.float32)
    w = np.asarray(w, np.float32)
    return WL.Case(name="pin", M=x.shape[0], N=w.shape[0], K=x.shape[1], fmt=fmt,
                   x_dtype="f32", y_dtype="f32", x=x, w=w, s=None, inv_s=None,
                   fwht_block=0, w_full=w)


def test_w4a8_exact_on_grid_values():
    """Integer activations whose rows peak at 127 and integer weights whose
    rows peak at 7 lie on the int8 and int4 grids with step 1, so W4A8 gives
    x w^T exactly.  A 4-bit activation grid, an 8-bit weight grid or a
    transposed product breaks the equality."""
    rng = np.random.default_rng(7)
    M, N, K = 5, 6, 128
    x = rng.integers(-127, 128, size=(M, K))
    x[np.arange(M), rng.integers(0, K, M)] = 127
    w = rng.integers(-7, 8, size=(N, K))
    w[np.arange(N), rng.integers(0, K, N)] = -7
    out = O.linear(_plain_case(x, w, "w4a8"))
    assert np.array_equal(out["a"]["codes"], x)
    assert np.array_equal(out["w"]["codes"], w)
    assert np.all(out["a"]["scales"] == 1) and np.all(out["w"]["scales"] == 1)
    assert np.array_equal(out["acc"], x @ w.T)
    assert np.array_equal(out["y"], (x @ w.T).astype(np.float64))
    # weights go through the nibble packing of the 4-bit format
    assert out["w"]["packed"].shape == (N, K // 2)
    assert out["a"]["packed"].shape == (M, K)
    # the same inputs as W4A4 lose the activation grid
    assert not np.array_equal(O.linear(_plain_case(x, w, "int4"))["y"], out["y"])


def test_w4a8_error_bound_with_transforms():
    """With smoothing and the 64-point rotation (orthonormal, folded into the
    weights), |y - x w^T| <= sum_k (d_a |w^_k| + d_w |a_k|) with half-steps
    d_a = step_a / 2 and d_w = step_w / 2, up to fp32 rounding of the
    transforms; W4A8 error is below W4A4 error on the same layer."""
    c = WL.linear_case(24, 40, 256, seed=31, fmt="w4a8", x_dtype="f32",
                       n_outliers=6, outlier_gain=20.0)
    out = O.linear(c)
    A, W = out["a"], out["w"]
    assert A["codes"].min() >= -128 and np.abs(A["codes"]).max(axis=1).min() == 127
    assert W["codes"].min() >= -8 and np.abs(W["codes"]).max(axis=1).min() == 7
    ref = c.x.astype(np.float64) @ c.w.astype(np.float64).T
    w_hat = W["codes"].astype(np.float64) * W["scales"].astype(np.float64)[:, None]
    a_t = A["y"].astype(np.float64)
    bound = (A["scales"].astype(np.float64)[:, None] / 2 * np.abs(w_hat).sum(axis=1)[None, :]
             + W["scales"].astype(np.float64)[None, :] / 2 * np.abs(a_t).sum(axis=1)[:, None])
    slack = 1e-5 * (np.abs(c.x.astype(np.float64)) @ np.abs(c.w.astype(np.float64)).T)
    err = np.abs(out["y"] - ref)
    assert np.all(err <= bound * (1 + 1e-6) + slack)
    c4 = WL.linear_case(24, 40, 256, seed=31, fmt="int4", x_dtype="f32",
                        n_outliers=6, outlier_gain=20.0)
    err4 = np.abs(O.linear(c4)["y"] - ref)
    assert np.sum(err ** 2) < 0.8 * np.sum(err4 ** 2)


def test_w4a8_activation_layout_example_and_roundtrip():
    """The library's W4A8 activation storage (tests/parity.py converts; the
    oracle itself emits logical int8 codes)."""
    codes = np.arange(16, dtype=np.int8)[None, :] - 8
    packed = pack_w4a8_activations(codes).view(np.int8)[0] + 8
    assert packed.tolist() == [0, 2, 4, 6, 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15]
    rng = np.random.default_rng(3)
    c = rng.integers(-128, 128, size=(7, 192)).astype(np.int8)
    assert np.array_equal(unpack_w4a8_activations(pack_w4a8_activations(c)), c)


def test_w4a8_activation_layout_is_the_int4_unpack_order():
    """Unpacking a packed int4 word d to bytes as (d << 4) & 0xF0F0F0F0 (even
    codes, times 16) then d & 0xF0F0F0F0 (odd codes, times 16) yields the
    codes in exactly the W4A8 activation order."""
    rng = np.random.default_rng(4)
    c = rng.integers(-8, 8, size=(5, 128)).astype(np.int8)
    words = O.pack_nibbles(c).view("<u4")                      # R x K/8 little-endian words
    ev = ((words << np.uint32(4)) & np.uint32(0xF0F0F0F0)).astype("<u4")
    od = (words & np.uint32(0xF0F0F0F0)).astype("<u4")
    seq = np.stack([ev, od], axis=-1).reshape(5, -1).view(np.int8).astype(np.int64) // 16
    assert np.array_equal(seq, pack_w4a8_activations(c).view(np.int8))


# --------------------------------------------------------------------- FP8
def test_e4m3_signed_encode_roundtrip_sign_and_zero():
    codes = np.arange(256)
    finite = (codes & 0x7F) != 0x7F
    enc = O.e4m3_encode_signed(O.e4m3_value(codes[finite]))
    assert np.array_equal(enc, np.where(codes[finite] == 0x80, 0, codes[finite]))   # -0 encodes +0
    rng = np.random.default_rng(8)
    v = rng.uniform(-460.0, 460.0, 4000) * np.exp2(rng.integers(-12, 1, 4000))
    e = O.e4m3_encode_signed(v)
    mag = O.e4m3_encode(np.abs(v))
    assert np.array_equal(e & 0x7F, mag)
    assert np.array_equal(e >> 7, ((v < 0) & (mag != 0)).astype(np.uint8))
    # half the smallest subnormal (2^-10) ties to the even code 0; anything below rounds to +0
    assert O.e4m3_encode_signed(np.array([0.0, -0.0, -2.0 ** -10, 2.0 ** -11, -2.0 ** -11])).tolist() == [0] * 5
    # nearest by brute force over the whole grid, ties to the even code
    grid = O.e4m3_value(np.arange(0x7F))
    for x in np.abs(v[:300]):
        d = np.abs(grid - min(x, 448.0))
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
        assert O.e4m3_encode(np.array([x]))[0] == want


def test_fp8_quantizer_invariants():
    rng = np.random.default_rng(9)
    y = (rng.standard_normal((6, 96)) * np.array([1, 1e3, 1e-4, 1, 7, 0.3])[:, None]).astype(np.float32)
    y[3] = 0
    codes, step, v = O.quantize_fp8(y)
    dq = O.e4m3_value(codes) * step.astype(np.float64)[:, None]
    nz = step > 0
    assert not nz[3] and np.all(codes[3] == 0)
    assert np.all(np.abs(O.e4m3_value(codes[nz])).max(axis=1) == 448.0)
    # E4M3 keeps 3 mantissa bits: half-spacing 2^-4 relative in the normal range,
    # 2^-10 (in units of the step) in the subnormal range
    bound = 2.0 ** -4 * np.abs(y) + 2.0 ** -10 * step.astype(np.float64)[:, None]
    assert np.all(np.abs(dq - y) <= bound * (1 + 1e-6))
    assert np.all((dq == 0) | (np.sign(dq) == np.sign(y)))
    # the pre-rounding value of each row's largest element is 448 up to the
    # two binary32 roundings of the step and the quotient
    imax = np.argmax(np.abs(y), axis=1)
    top = np.abs(v[np.arange(len(y)), imax])[nz]
    assert np.all(np.abs(top.astype(np.float64) - 448.0) <= 2 * 2.0 ** -15)


def test_int_quantizer_decides_in_binary32():
    """The step and the quotient are binary32 values (the precision of the
    kernels), and the code follows from them.  Row [1, 1/2], Q = 7: the exact
    step 1/7 would make 1/2 a tie at 3.5 (code 4); the binary32 step is
    0x3E124925 = 1/7 + 3 / (7 * 2^26), slightly above 1/7, so the exact
    quotient (1/2) / step = 3.49999984... lies below 3.5 and rounds to the
    binary32 value 3.5 - 2^-22, and the code is 3.  Scaling the row by a
    power of two changes nothing; negating it negates the codes."""
    import struct
    step_bits = struct.unpack("<f", struct.pack("<I", 0x3E124925))[0]
    for scale in (1.0, 2.0 ** -6, 2.0 ** 20):
        for sgn in (1.0, -1.0):
            y = np.array([[sgn * scale, sgn * scale / 2]], np.float32)
            codes, step, v = O.quantize_int(y, 7)
            assert step[0] == np.float32(step_bits * scale)
            assert v[0, 1] == np.float32(sgn * (3.5 - 2.0 ** -22))
            assert codes[0].tolist() == [int(sgn * 7), int(sgn * 3)]


def test_fp8_gemm_is_exact():
    """The float64 sum of E4M3 products equals the exact rational sum."""
    from fractions import Fraction
    rng = np.random.default_rng(10)
    ca = rng.integers(0, 256, size=(2, 40)).astype(np.uint8)
    cw = rng.integers(0, 256, size=(3, 40)).astype(np.uint8)
    ca[(ca & 0x7F) == 0x7F] = 0x7E
    cw[(cw & 0x7F) == 0x7F] = 0xFE
    acc = O.fp8_gemm(ca, cw)
    va, vw = O.e4m3_value(ca), O.e4m3_value(cw)
    for m in range(2):
        for n in range(3):
            exact = sum(Fraction(float(va[m, k])) * Fraction(float(vw[n, k])) for k in range(40))
            assert Fraction(float(acc[m, n])) == exact


def test_fp8_linear_exact_on_grid_values():
    """Rows whose values lie on the E4M3 grid and peak at 448 quantize with
    step 1 to themselves, so FP8 W8A8 gives x w^T exactly."""
    rng = np.random.default_rng(11)
    M, N, K = 4, 5, 64

    def grid_rows(R):
        c = rng.integers(0, 0x7F, size=(R, K)) | (rng.integers(0, 2, size=(R, K)) << 7)
        c[np.arange(R), rng.integers(0, K, R)] = 0x7E            # 448 in every row
        return O.e4m3_value(c)

    x, w = grid_rows(M), grid_rows(N)
    out = O.linear(_plain_case(x, w, "fp8"))
    assert np.all(out["a"]["scales"] == 1) and np.all(out["w"]["scales"] == 1)
    assert np.array_equal(O.e4m3_value(out["a"]["codes"]), x)
    assert np.array_equal(out["acc"], x @ w.T)
    # unit steps: the binary32 epilogue is the one rounding of the exact sum
    assert np.array_equal(out["y"], (x @ w.T).astype(np.float32))
    assert out["a"]["packed"].shape == (M, K) and out["a"]["packed"].dtype == np.uint8


# -------------------------------------------------------------------- GPTQ
def _gptq_setup(N=12, K=128, seed=70):
    rng = np.random.default_rng(seed)
    wt = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    wt[3] = 0                                           # an all-zero row
    _, step, _ = O.quantize_int(wt, O.INT4_QMAX)
    cal = WL.gptq_calibration(K, seed + 1)
    return wt, step, cal


def test_gptq_reduces_to_round_to_nearest_without_feedback():
    """With U = I (no correlations) or any diagonal U the error feedback is
    zero, so GPTQ gives the round-to-nearest codes, in any column order."""
    wt, step, _ = _gptq_setup()
    rtn, _, _ = O.quantize_int(wt, O.INT4_QMAX)
    K = wt.shape[1]
    c, _ = O.gptq_rows(wt, step, np.eye(K), O.INT4_QMAX)
    assert np.array_equal(c, rtn)
    perm = np.random.default_rng(5).permutation(K)
    c, _ = O.gptq_rows(wt, step, np.diag(np.linspace(0.5, 2.0, K)), O.INT4_QMAX, perm)
    assert np.array_equal(c, rtn)


def test_gptq_error_identity():
    """The rounding errors satisfy w - q * step = err @ U in processing order
    (each column's error is its own err times U[t, t] plus the feedback it
    received): a wrong sign, index or dropped update breaks it."""
    wt, step, cal = _gptq_setup()
    c, E = O.gptq_rows(wt, step, cal["u"], O.INT4_QMAX, cal["perm"])
    p = cal["perm"]
    lhs = wt[:, p].astype(np.float64) - c[:, p].astype(np.float64) * step.astype(np.float64)[:, None]
    rhs = E @ cal["u"]
    assert np.allclose(lhs, rhs, rtol=0, atol=1e-12 * np.abs(wt).max())
    assert np.all(c[3] == 0)
    assert c.min() >= -8 and c.max() <= 7


def test_gptq_lowers_the_proxy_loss_and_respects_the_order():
    """GPTQ's purpose: sum over rows of d Sigma d^T (d = dequantised - float
    weights) is lower than round-to-nearest's; and running with a column order
    equals running on pre-permuted columns with U for that order."""
    wt, step, cal = _gptq_setup(N=32, K=192, seed=80)
    sig = cal["sigma"]
    c, _ = O.gptq_rows(wt, step, cal["u"], O.INT4_QMAX, cal["perm"])
    rtn, _, _ = O.quantize_int(wt, O.INT4_QMAX)
    def loss(codes):
        d = codes * step.astype(np.float64)[:, None] - wt
        return np.sum((d @ sig) * d)

    assert loss(c) < 0.9 * loss(rtn)
    p = cal["perm"]
    c2, _ = O.gptq_rows(np.ascontiguousarray(wt[:, p]), step, cal["u"], O.INT4_QMAX)
    assert np.array_equal(c2, c[:, p])
