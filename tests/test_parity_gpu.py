"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on
the same seeded inputs.  Needs an MI355X and the built libw4a4.so."""
import zlib

import numpy as np
import pytest

from oracle import w4a4_oracle as O
from w4a4_post_quantized_channel_amd import workloads as WL

from parity import check_operand, check_output, check_output_exact, unpack_codes

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w4a4_post_quantized_channel_amd import ops as _ops   # raises if the library is missing
    return _ops


@pytest.fixture(scope="module")
def pipe(ops):
    from w4a4_post_quantized_channel_amd import pipeline
    return pipeline


def _np(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return WL.from_bf16_bits(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


def _run(pipe, case, order="smooth_then_rotate"):
    layer, t = pipe.build_layer(case, order=order)
    y = layer.forward(t["x"])
    return layer, t, y


def _oracle(case, order="smooth_then_rotate"):
    return O.linear(case, order=order)


def _sides(fmt):
    return O.OPERAND_FORMATS[fmt]


def _raw_linear(ops, fmt, a, sa, w, sw, K, **kw):
    """The linear entry point for ``fmt`` (int4, int8, w4a8, fp8)."""
    if fmt == "int4":
        return ops.w4a4_linear(a, sa, w, sw, K, "int4", **kw)
    fn = {"int8": ops.w8a8_linear, "w4a8": ops.w4a8_linear, "fp8": ops.fp8_linear}[fmt]
    return fn(a, sa, w, sw, K, **kw)


def _random_codes(rng, fmt, R, K):
    if fmt == "int4":
        return rng.integers(0, 256, size=(R, K // 2), dtype=np.uint8)
    return rng.integers(-128, 128, size=(R, K), dtype=np.int8)


def _report(name, **kw):
    print(f"[parity] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


SMALL = [
    # name, M, N, K, fmt, x_dtype, kwargs
    ("int4_ragged", 77, 130, 320, "int4", "bf16", dict(n_outliers=5, outlier_gain=20.0)),
    ("int4_tiles", 160, 256, 512, "int4", "bf16", dict(n_outliers=8, outlier_gain=15.0, row_gain_sigma=0.5)),
    ("int4_f32", 16, 256, 256, "int4", "f32", dict(n_outliers=4, outlier_gain=20.0)),
    ("int8_ragged", 70, 96, 448, "int8", "bf16", dict(n_outliers=6, outlier_gain=15.0)),
    ("int4_lowrank", 90, 200, 384, "int4", "bf16", dict(n_outliers=6, outlier_gain=25.0, lowrank=16)),
    ("nvfp4_outlier", 130, 140, 320, "nvfp4", "bf16", dict(n_outliers=8, outlier_gain=30.0, keep_channels=8)),
    ("nvfp4_plain", 66, 72, 256, "nvfp4", "bf16", dict(n_outliers=4, outlier_gain=10.0)),
    ("int4_single_row", 1, 64, 64, "int4", "bf16", dict()),
    ("int8_lowrank", 33, 48, 192, "int8", "bf16", dict(lowrank=8)),
    # rows longer than 4096: eight waves per row in the integer quantizer (ragged chunks)
    ("int8_long_rows", 5, 40, 4160, "int8", "bf16", dict(n_outliers=6, outlier_gain=20.0)),
    ("int4_long_rows", 3, 24, 8256, "int4", "f32", dict(n_outliers=6, outlier_gain=20.0)),
    # >= 256 rows: the row-per-lane NVFP4 quantizer (ragged last group of 64 rows)
    ("nvfp4_rows", 300, 96, 320, "nvfp4", "bf16", dict(n_outliers=8, outlier_gain=30.0, keep_channels=8)),
    ("nvfp4_rows_f32", 260, 64, 256, "nvfp4", "f32", dict(n_outliers=4, outlier_gain=20.0)),
    # the 256x160 NVFP4 tile (weights widened once per workgroup): ragged M and N,
    # and a last K stage of half length
    ("nvfp4_wide_tile", 2600, 3210, 1088, "nvfp4", "bf16", dict(n_outliers=8, outlier_gain=30.0, keep_channels=16)),
    # shapes the tile model routes to the 128x256 and 128x96 NVFP4 tiles (ragged M, N and K)
    ("nvfp4_tile_128x256", 3100, 1000, 320, "nvfp4", "bf16", dict(n_outliers=8, outlier_gain=30.0)),
    ("nvfp4_tile_128x96", 777, 2600, 320, "nvfp4", "bf16", dict(n_outliers=8, outlier_gain=30.0)),
    # W4A8: int8 activation codes x int4 weight codes
    ("w4a8_ragged", 70, 96, 448, "w4a8", "bf16", dict(n_outliers=6, outlier_gain=15.0)),
    ("w4a8_tiles", 160, 256, 512, "w4a8", "bf16", dict(n_outliers=8, outlier_gain=15.0, row_gain_sigma=0.5)),
    ("w4a8_f32", 16, 256, 256, "w4a8", "f32", dict(n_outliers=4, outlier_gain=20.0)),
    ("w4a8_lowrank", 90, 200, 384, "w4a8", "bf16", dict(n_outliers=6, outlier_gain=25.0, lowrank=16)),
    ("w4a8_outlier", 33, 130, 320, "w4a8", "bf16", dict(n_outliers=8, outlier_gain=30.0, keep_channels=8)),
    ("w4a8_long_rows", 5, 40, 4160, "w4a8", "bf16", dict(n_outliers=6, outlier_gain=20.0)),
    # FP8 (OCP E4M3) W8A8
    ("fp8_ragged", 70, 96, 448, "fp8", "bf16", dict(n_outliers=6, outlier_gain=15.0)),
    ("fp8_tiles", 160, 300, 512, "fp8", "bf16", dict(n_outliers=8, outlier_gain=15.0, row_gain_sigma=0.5)),
    ("fp8_f32", 16, 256, 256, "fp8", "f32", dict(n_outliers=4, outlier_gain=20.0)),
    ("fp8_lowrank", 90, 200, 384, "fp8", "bf16", dict(n_outliers=6, outlier_gain=25.0, lowrank=16)),
    ("fp8_outlier", 33, 130, 320, "fp8", "bf16", dict(n_outliers=8, outlier_gain=30.0, keep_channels=8)),
    ("fp8_long_rows", 5, 40, 4160, "fp8", "bf16", dict(n_outliers=6, outlier_gain=20.0)),
    # the largest K quantize_act accepts (32768): every format, the row kernels,
    # and the row-per-lane NVFP4 quantizer with a ragged last group of rows
    ("int4_max_k", 3, 24, 32768, "int4", "bf16", dict(n_outliers=6, outlier_gain=20.0)),
    ("int8_max_k", 2, 16, 32768, "int8", "f32", dict(n_outliers=6, outlier_gain=20.0)),
    ("w4a8_max_k", 3, 16, 32768, "w4a8", "bf16", dict(n_outliers=6, outlier_gain=20.0)),
    ("fp8_max_k", 3, 16, 32768, "fp8", "bf16", dict(n_outliers=6, outlier_gain=20.0)),
    ("nvfp4_max_k", 5, 16, 32768, "nvfp4", "bf16", dict(n_outliers=6, outlier_gain=20.0, keep_channels=8)),
    ("nvfp4_rows_max_k", 260, 16, 32768, "nvfp4", "bf16", dict(n_outliers=6, outlier_gain=20.0)),
]


@pytest.mark.parametrize("name,M,N,K,fmt,xdt,kw", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("order", ["smooth_then_rotate", "rotate_then_smooth"])
def test_small_cases(ops, pipe, name, M, N, K, fmt, xdt, kw, order):
    case = WL.linear_case(M, N, K, seed=zlib.crc32(name.encode()) % 1000, fmt=fmt, x_dtype=xdt, name=name, **kw)
    _report(name, M=M, N=N, K=K, fmt=fmt, order=order)
    if kw.get("keep_channels") and order != "smooth_then_rotate":
        # kept channels are defined for smoothing first only (s = 0 removes raw
        # channels); both sides refuse the other order before any launch
        with pytest.raises(ValueError):
            _oracle(case, order)
        with pytest.raises(ValueError):
            pipe.build_layer(case, order=order)
        return
    layer, t, y = _run(pipe, case, order)
    ref = _oracle(case, order)
    if fmt == "nvfp4":
        assert np.float32(layer.g_a) == ref["a"]["g"] and np.float32(layer.g_w) == ref["w"]["g"]
    b = layer.buffers(M, t["x"].device)
    fa, fw = _sides(fmt)
    na = check_operand(fa, _np(b["codes"]), _np(b["scales"]), ref["a"], what="activations")
    nw = check_operand(fw, _np(layer.w_codes), _np(layer.w_scales), ref["w"], what="weights")
    rtol = 1e-3 if case.y_dtype == "f32" else 1e-2
    worst = check_output(_np(y), ref["y"], rtol)
    exact = fmt in ("int4", "int8", "w4a8") and case.branch is None and na == 0 and nw == 0
    if exact:   # one exact answer: integer accumulators and the fp32-ordered epilogue
        check_output_exact(_np(y), ref["y_main"], case.y_dtype)
    _report(name, band_mismatch_a=na, band_mismatch_w=nw, worst=f"{worst:.3g}", bit_exact=exact)


@pytest.mark.parametrize("fmt", ["int4", "int8", "w4a8"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (17, 33, 192), (100, 200, 384), (130, 260, 320),
                                   (64, 2048, 2048), (64, 512, 8192), (512, 512, 4096), (300, 100, 64),
                                   (64, 2048, 8192), (40, 4096, 4160), (3, 8200, 2048), (30, 8192, 2048),
                                   (20, 512, 4096), (9, 768, 8192), (50, 640, 8256),
                                   (7, 40, 65536), (100, 72, 65536)])   # the largest K the linears accept
@pytest.mark.parametrize("split", [False, True])
def test_raw_accumulators_exact(ops, fmt, M, N, K, split):
    """Integer GEMM on random codes: bit-exact int32 accumulators (decode kernel with and
    without the split-K workspace, tile kernels)."""
    rng = np.random.default_rng(M * 7 + N * 13 + K)
    fa, fw = _sides(fmt)
    a_b = _random_codes(rng, fa, M, K)
    w_b = _random_codes(rng, fw, N, K)
    ref = O.int_gemm(unpack_codes(fa, a_b), unpack_codes(fw, w_b))
    dev = "cuda"
    a = torch.from_numpy(a_b).to(dev)
    w = torch.from_numpy(w_b).to(dev)
    sa = torch.ones(M, dtype=torch.float32, device=dev)
    sw = torch.ones(N, dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.int32, device=dev)
    ws = ops.make_workspace(M, N, K, fmt) if split else None
    if split and ws is None:
        pytest.skip("shape runs without a workspace")
    _raw_linear(ops, fmt, a, sa, w, sw, K, y=y, workspace=ws)
    got = _np(y).astype(np.int64)
    assert np.array_equal(got, ref)


# Shapes the many-token tile model routes to its 256x160, 128x256 and 128x96
# tiles (the 64x64 tile is covered above); all ragged in M and N, with a
# partial last K stage.
@pytest.mark.parametrize("fmt", ["int4", "int8", "w4a8"])
@pytest.mark.parametrize("M,N,K", [(3100, 2600, 320), (3100, 1000, 320), (777, 2600, 320)])
def test_raw_accumulators_every_tile(ops, fmt, M, N, K):
    """Bit-exact int32 accumulators on random codes through each many-token tile."""
    rng = np.random.default_rng(M * 7 + N * 13 + K + 1)
    fa, fw = _sides(fmt)
    a_b = _random_codes(rng, fa, M, K)
    w_b = _random_codes(rng, fw, N, K)
    ref = O.int_gemm(unpack_codes(fa, a_b), unpack_codes(fw, w_b))
    _report("raw_every_tile", fmt=fmt, M=M, N=N, K=K)
    dev = "cuda"
    a = torch.from_numpy(a_b).to(dev)
    w = torch.from_numpy(w_b).to(dev)
    y = torch.empty((M, N), dtype=torch.int32, device=dev)
    _raw_linear(ops, fmt, a, torch.ones(M, device=dev), w, torch.ones(N, device=dev), K, y=y)
    assert np.array_equal(_np(y).astype(np.int64), ref)


@pytest.mark.parametrize("fmt,val_a,val_w", [("int4", 7, 7), ("int4", -8, -8), ("int4", -8, 7),
                                            ("int8", -128, -128), ("int8", 127, -128),
                                            ("w4a8", -128, -8), ("w4a8", 127, -8), ("w4a8", -128, 7)])
def test_extreme_codes_do_not_overflow(ops, fmt, val_a, val_w):
    M, N, K = 32, 48, 65536
    fa, fw = _sides(fmt)

    def fill(f, R, v):
        if f == "int4":
            return np.full((R, K // 2), (v & 0xF) | ((v & 0xF) << 4), np.uint8)
        return np.full((R, K), v, np.int8)

    a_b, w_b = fill(fa, M, val_a), fill(fw, N, val_w)
    a, w = torch.from_numpy(a_b).cuda(), torch.from_numpy(w_b).cuda()
    ones_m, ones_n = torch.ones(M, device="cuda"), torch.ones(N, device="cuda")
    y = torch.empty((M, N), dtype=torch.int32, device="cuda")
    ws = ops.make_workspace(M, N, K, fmt)
    _raw_linear(ops, fmt, a, ones_m, w, ones_n, K, y=y, workspace=ws)
    assert np.all(_np(y) == val_a * val_w * K)


def _fp8_codes(rng, R, K):
    c = rng.integers(0, 256, size=(R, K), dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] ^= 0x01     # no NaN codes
    return c


@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (17, 33, 192), (64, 2048, 2048), (64, 512, 8192),
                                   (9, 768, 8192), (20, 512, 4096), (130, 260, 320), (300, 100, 64),
                                   (512, 512, 4096), (40, 4096, 4160),
                                   # many tokens: the 128x128 and the 128x256 FP8 tiles
                                   (1030, 3100, 576), (2600, 5200, 320)])
@pytest.mark.parametrize("split", [False, True])
def test_fp8_accumulation(ops, M, N, K, split):
    """FP8 GEMM on random E4M3 codes with unit steps and fp32 output, few-token
    (with and without split K) and many-token kernels.  The fp8 matrix
    instruction adds its products with its own internal precision (measured:
    errors near 2^-15 of sum |products|, above fp32 rounding), so the bar is
    2^-12 of sum |products| per output: a wrong pairing of codes, a dropped
    term or a lost partial tile is of the order of sum |products| itself."""
    rng = np.random.default_rng(M * 5 + N * 3 + K)
    a_b, w_b = _fp8_codes(rng, M, K), _fp8_codes(rng, N, K)
    exact = O.fp8_gemm(a_b, w_b)
    absum = np.abs(O.e4m3_value(a_b)) @ np.abs(O.e4m3_value(w_b)).T
    a, w = torch.from_numpy(a_b).cuda(), torch.from_numpy(w_b).cuda()
    ones_m, ones_n = torch.ones(M, device="cuda"), torch.ones(N, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = ops.make_workspace(M, N, K, "fp8") if split else None
    if split and ws is None:
        pytest.skip("shape runs without a workspace")
    ops.fp8_linear(a, ones_m, w, ones_n, K, y=y, workspace=ws)
    err = np.abs(_np(y).astype(np.float64) - exact)
    _report("fp8_accumulation", M=M, N=N, K=K, split=split, worst_rel=f"{np.max(err / absum):.3g}")
    assert np.all(err <= 2.0 ** -12 * absum)


@pytest.mark.parametrize("val_a,val_w", [(0x7E, 0x7E), (0x7E, 0xFE), (0x01, 0x81)])
def test_fp8_extreme_codes(ops, val_a, val_w):
    """448 x 448 (and the smallest subnormals) over K = 65536: every partial sum
    is exact in fp32, so the result is exact."""
    M, N, K = 32, 48, 65536
    a = torch.full((M, K), val_a, dtype=torch.uint8, device="cuda")
    w = torch.full((N, K), val_w, dtype=torch.uint8, device="cuda")
    ones_m, ones_n = torch.ones(M, device="cuda"), torch.ones(N, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ops.fp8_linear(a, ones_m, w, ones_n, K, y=y, workspace=ops.make_workspace(M, N, K, "fp8"))
    want = float(O.e4m3_value(np.array([val_a]))[0] * O.e4m3_value(np.array([val_w]))[0] * K)
    assert np.all(_np(y) == np.float32(want))


@pytest.mark.parametrize("signed", [False, True])
@pytest.mark.parametrize("M", [20, 127])
def test_nvfp4_every_scale_code(ops, M, signed):
    """Every finite non-negative E4M3 block scale (codes 0..126) through the
    NVFP4 GEMM, on both operands: row m of A uses code m mod 127 for all
    its blocks, row n of W code 7n mod 127.  Divided by the two scale
    values, each output is a dot product of E2M1 codes (a multiple of 1/4),
    so a wrong scale decode shows as a gross error on its own rows.
    signed: odd rows of A and rows n = 1, 2 mod 3 of W carry the sign bit
    as well (codes 128..254, -0 included); the format reads them as the
    negated values, and the GEMM must too."""
    N, K = 160, 2048
    rng = np.random.default_rng(11)
    ca = rng.integers(0, 16, (M, K))
    cw = rng.integers(0, 16, (N, K))
    ea = (np.arange(M) % 127).astype(np.uint8)
    ew = ((7 * np.arange(N)) % 127).astype(np.uint8)
    if signed:
        ea = ea | np.where(np.arange(M) % 2 == 1, 0x80, 0).astype(np.uint8)
        ew = ew | np.where(np.arange(N) % 3 != 0, 0x80, 0).astype(np.uint8)
    sa = np.repeat(ea[:, None], K // 16, axis=1)
    sw = np.repeat(ew[:, None], K // 16, axis=1)
    dot = O.e2m1_value(ca) @ O.e2m1_value(cw).T            # exact in fp64
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ops.w4a4_linear(torch.from_numpy(O.pack_nibbles(ca)).cuda(), torch.from_numpy(sa).cuda(),
                    torch.from_numpy(O.pack_nibbles(cw)).cuda(), torch.from_numpy(sw).cuda(), K, "nvfp4",
                    alpha=1.0, y=y)
    got = _np(y).astype(np.float64)
    va, vw = O.e4m3_value(ea), O.e4m3_value(ew)
    prod = va[:, None] * vw[None, :]
    assert np.all(got[prod == 0] == 0)
    nz = prod != 0
    # fp32 accumulation of exact products: error <= K * 2^-24 of the sum of
    # |terms|; a wrong decode moves the whole row by at least 1/16 of |dot|
    mag = np.abs(O.e2m1_value(ca)) @ np.abs(O.e2m1_value(cw)).T
    err = np.abs(got[nz] / prod[nz] - dot[nz])
    assert np.all(err <= K * 2.0 ** -24 * mag[nz] + 1e-9)


def test_zero_rows_and_saturating_nvfp4(ops, pipe):
    case = WL.linear_case(40, 64, 256, seed=5, fmt="nvfp4", n_outliers=4, outlier_gain=30.0)
    case.x[3] = 0.0
    case.x[17] = 0.0
    t = pipe.case_to_device(case)
    # deliberately small tensor scale: block scales saturate at 448, codes at 6
    y_ref = O.transform(case.x, case.inv_s)
    g = np.float32(O.nvfp4_tensor_scale(np.abs(y_ref).max()) / np.float32(16))
    codes, scales = ops.quantize_act(t["x"], t["inv_s"], "nvfp4", tensor_scale=float(g))
    ref = O.quantize_operand(case.x, case.inv_s, "nvfp4", g=g)
    check_operand("nvfp4", _np(codes), _np(scales), ref)
    assert (ref["scales"] == 0x7E).any() and np.all(_np(scales)[3] == 0) and np.all(_np(codes)[17] == 0)
    c4, s4 = ops.quantize_act(t["x"], t["inv_s"], "int4")
    assert _np(s4)[3] == 0 and np.all(_np(c4)[3] == 0)


def test_transform_amax_matches_oracle(ops, pipe):
    for xdt in ["bf16", "f32"]:
        case = WL.linear_case(123, 16, 640, seed=9, x_dtype=xdt, n_outliers=7, outlier_gain=40.0)
        t = pipe.case_to_device(case)
        for order in ["smooth_then_rotate", "rotate_then_smooth"]:
            got = ops.transform_amax(t["x"], t["inv_s"], order=order)
            assert _np(got)[0] == O.transformed_amax(case.x, case.inv_s, order=order)
            gotw = ops.transform_amax(t["w"], t["s"], order=order)
            assert _np(gotw)[0] == O.transformed_amax(case.w, case.s, order=order)


def test_lowrank_add_standalone(ops, pipe):
    for kind in ["lowrank", "outlier"]:
        kw = dict(lowrank=32) if kind == "lowrank" else dict(keep_channels=16, fmt="nvfp4", n_outliers=16,
                                                            outlier_gain=30.0)
        case = WL.linear_case(75, 150, 256, seed=31, **kw)
        t = pipe.case_to_device(case)
        br = t["branch"]
        for ydt in [torch.float32, torch.bfloat16]:
            y0 = np.random.default_rng(1).standard_normal((75, 150)).astype(np.float32)
            if ydt == torch.bfloat16:
                y0 = WL.bf16_round(y0)
            y = torch.from_numpy(y0).to("cuda", ydt)
            if kind == "lowrank":
                ops.lowrank_add(t["x"], y, br["lw"], l1t=br["l1t"])
                add = O.lowrank_branch(case.x, case.branch["l1"], case.branch["lw"])
            else:
                ops.lowrank_add(t["x"], y, br["lw"], idx=br["idx"])
                add = O.outlier_branch(case.x, case.branch["idx"], case.branch["lw"])
            check_output(_np(y), y0.astype(np.float64) + add, 1e-3 if ydt == torch.float32 else 1e-2)


@pytest.mark.parametrize("M,K,r", [(50, 512, 24), (1, 64, 8), (33, 3072, 40), (130, 4104, 128)])
def test_lowrank_project(ops, pipe, M, K, r):
    """T = x L1 as the bf16 hi/lo pair: ragged rows, a rank that is not a
    multiple of 16, K beyond one round of in-flight steps and not a multiple of 32."""
    case = WL.linear_case(M, 8, K, seed=41 + r, lowrank=r)
    t = pipe.case_to_device(case)
    assert ops.lowrank_width(M, K, r) == 2 * r
    out = _np(ops.lowrank_project(t["x"], l1t=t["branch"]["l1t"]))
    T = case.x.astype(np.float64) @ case.branch["l1"].astype(np.float64)
    assert out.shape == (M, 2 * r)
    recon = out[:, :r].astype(np.float64) + out[:, r:].astype(np.float64)
    assert np.max(np.abs(recon - T)) <= 2.0 ** -15 * np.max(np.abs(T))


@pytest.mark.parametrize("M,K,r,fmt", [(1024, 3072, 32, "int4"), (77, 3072, 32, "int4"), (33, 256, 16, "int8"),
                                       (130, 4096, 16, "w4a8"), (17, 512, 32, "fp8"), (300, 320, 32, "nvfp4"),
                                       (16, 64, 16, "int4"), (1, 1024, 32, "int4"), (2051, 1536, 32, "int4")])
def test_quantize_act_lowrank(ops, pipe, M, K, r, fmt):
    """The fused pass: codes and scales exactly as quantize_act writes them,
    and T = x L1 as the bf16 hi/lo pair within the projection's bound
    (ragged row groups of 4, both ranks the kernel takes, K up to 4096, more
    row groups than workgroups)."""
    case = WL.linear_case(M, 8, K, seed=71 + r + K, fmt=fmt, n_outliers=4, outlier_gain=10.0, lowrank=r)
    t = pipe.case_to_device(case)
    kw = dict(fwht_block=case.fwht_block, tensor_scale=1.0 / 64)
    _report("quantize_act_lowrank", M=M, K=K, r=r, fmt=fmt)
    c0, s0 = ops.quantize_act(t["x"], t["inv_s"], fmt if fmt != "w4a8" else "w4a8", **kw)
    c1, s1, out = ops.quantize_act_lowrank(t["x"], t["inv_s"], t["branch"]["l1t"], fmt, **kw)
    torch.cuda.synchronize()
    assert torch.equal(c0, c1) and torch.equal(s0, s1)
    o = _np(out)
    T = case.x.astype(np.float64) @ case.branch["l1"].astype(np.float64)
    recon = o[:, :r].astype(np.float64) + o[:, r:].astype(np.float64)
    assert np.max(np.abs(recon - T)) <= 2.0 ** -15 * np.max(np.abs(T))
    # the same operand as the separate projection, to its rounding
    ref = _np(ops.lowrank_project(t["x"], l1t=t["branch"]["l1t"]))
    rref = ref[:, :r].astype(np.float64) + ref[:, r:].astype(np.float64)
    assert np.max(np.abs(recon - rref)) <= 2.0 ** -15 * np.max(np.abs(T))


@pytest.mark.slow
@pytest.mark.parametrize("M,K,r,fmt", [(1024, 3072, 32, "int4"), (77, 3072, 32, "int4"), (33, 256, 16, "int8"),
                                        (130, 4096, 16, "w4a8"), (17, 512, 32, "fp8"), (300, 320, 32, "nvfp4"),
                                        (5, 5120, 8, "int4"), (1, 64, 1, "int8"), (2051, 1536, 40, "int4")])
def test_quantize_act_project_matches_the_two_calls(ops, pipe, M, K, r, fmt):
    """quantize_act_project (quantizer and projection workgroups in one
    launch): codes, scales and the hi/lo operand bit-identical to
    quantize_act followed by w4a4_lowrank_project."""
    rng = np.random.default_rng(M + 3 * K + r)
    x = torch.from_numpy(WL.bf16_round(rng.standard_normal((M, K)).astype(np.float32) * 3)).to(torch.bfloat16).cuda()
    inv_s = torch.from_numpy(np.exp2(rng.integers(-2, 3, K)).astype(np.float32)).cuda()
    l1t = torch.from_numpy(WL.bf16_round(rng.standard_normal((r, K)).astype(np.float32) * 0.05)).to(torch.bfloat16).cuda()
    g = 0.01 if fmt == "nvfp4" else 1.0
    c1, s1, t1 = ops.quantize_act_project(x, inv_s, l1t, fmt, tensor_scale=g)
    c0, s0 = ops.quantize_act(x, inv_s, fmt, tensor_scale=g)
    t0 = ops.lowrank_project(x, l1t=l1t)
    torch.cuda.synchronize()
    assert torch.equal(c1, c0) and torch.equal(s1.view(torch.uint8), s0.view(torch.uint8))
    assert torch.equal(t1.view(torch.int16), t0[:, :2 * r].view(torch.int16))
    _report("quantize_act_project", M=M, K=K, r=r, fmt=fmt)


def test_lowrank_layer_one_launch_matches_two_kernels(ops, pipe):
    """The low-rank layer's default call (one launch for quantizer and
    projection) equals the two-kernel call bit for bit."""
    case = WL.workload("lowrank")
    layer, t = pipe.build_layer(case)
    assert layer.launch_lowrank and not layer.has_projection(t["x"].dtype)
    y1 = layer.forward(t["x"]).clone()
    layer.launch_lowrank = False
    assert layer.has_projection(t["x"].dtype)
    y0 = layer.forward(t["x"]).clone()
    assert torch.equal(y1.view(torch.int16), y0.view(torch.int16))


def test_lowrank_fused_end_to_end(ops, pipe):
    """The 1024-token low-rank workload with the single-read quantizer
    (quantize_act_lowrank feeding the fused epilogue): codes exact, output
    within tolerance of the oracle."""
    case = WL.workload("lowrank")
    layer, t = pipe.build_layer(case)
    layer.fuse_lowrank = True
    assert not layer.has_projection()
    y = layer.forward(t["x"])
    ref = _oracle(case)
    b = layer.buffers(case.M, t["x"].device)
    assert check_operand("int4", _np(b["codes"]), _np(b["scales"]), ref["a"], what="activations") == 0
    worst = check_output(_np(y), ref["y"], 1e-2)
    _report("lowrank_fused", worst=f"{worst:.3g}")


def test_lowrank_gather(ops, pipe):
    case = WL.linear_case(50, 8, 512, seed=41, lowrank=24)
    t = pipe.case_to_device(case)
    idx = torch.tensor([0, 5, 511, 100, 7, 8, 9, 300], dtype=torch.int32, device="cuda")
    g = _np(ops.lowrank_project(t["x"], idx=idx))
    assert np.array_equal(g, case.x[:, [0, 5, 511, 100, 7, 8, 9, 300]])


@pytest.mark.parametrize("M,K,fmt,r", [(300, 320, "nvfp4", 64), (260, 256, "nvfp4", 128), (70, 448, "int8", 65),
                                       (5, 4160, "int4", 1), (33, 320, "fp8", 16), (16, 256, "w4a8", 8),
                                       (40, 192, "nvfp4", 24)])
def test_quantize_act_gather(ops, pipe, M, K, fmt, r):
    """The fused gather leaves codes and scales as quantize_act writes them and
    copies x[:, idx] exactly (indices at block edges, repeated, out of range)."""
    case = WL.linear_case(M, 8, K, seed=61 + r, fmt=fmt, n_outliers=4, outlier_gain=10.0)
    t = pipe.case_to_device(case)
    x = t["x"]
    rng = np.random.default_rng(r)
    idx = rng.integers(0, K, size=r)
    special = [0, K - 1, 63, 64, 127, 128, -1, K, 5, 5]
    idx[:min(r, len(special))] = special[:min(r, len(special))]
    idx_t = torch.from_numpy(idx.astype(np.int32)).cuda()
    kw = dict(fwht_block=case.fwht_block, tensor_scale=1.0 / 64)
    c0, s0 = ops.quantize_act(x, t["inv_s"], fmt, **kw)
    c1, s1, xo = ops.quantize_act_gather(x, t["inv_s"], idx_t, fmt, **kw)
    torch.cuda.synchronize()
    assert torch.equal(c0, c1) and torch.equal(s0, s1)
    xb = case.x_bits
    want = np.where((idx >= 0) & (idx < K), xb[:, np.clip(idx, 0, K - 1)], 0).astype(np.uint16)
    assert np.array_equal(xo.view(torch.int16).cpu().numpy().view(np.uint16), want)


@pytest.mark.parametrize("N,K,fmt,use_perm", [(64, 256, "int4", True), (130, 320, "int4", True),
                                              (48, 1024, "int4", False), (70, 448, "int8", True),
                                              (300, 192, "int4", True)])
def test_pack_weights_gptq(ops, pipe, N, K, fmt, use_perm):
    """GPTQ-style rounding on the GPU: codes and steps bit-exact against the
    oracle's sequential float64 evaluation (with a zero row, ragged N)."""
    case = WL.linear_case(8, N, K, seed=90 + N, fmt=fmt, n_outliers=4, outlier_gain=10.0, gptq=True)
    case.w[5] = 0
    if not use_perm:
        case.gptq["perm"] = np.arange(K, dtype=np.int32)
        sp = case.gptq["sigma"] + 0.01 * np.mean(np.diag(case.gptq["sigma"])) * np.eye(K)
        case.gptq["u"] = np.ascontiguousarray(np.linalg.cholesky(np.linalg.inv(sp)).T)
    t = pipe.case_to_device(case)
    ref = O.quantize_operand(case.w, case.s, fmt, case.fwht_block)
    qmax = O.INT4_QMAX if fmt == "int4" else O.INT8_QMAX
    codes_ref, _ = O.gptq_rows(ref["y"], ref["scales"], case.gptq["u"], qmax, case.gptq["perm"])
    import time
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    codes, scales = ops.pack_weights_gptq(t["w"], t["s"], t["gptq"]["u"], t["gptq"]["perm"], fmt,
                                          fwht_block=case.fwht_block)
    torch.cuda.synchronize()
    _report("gptq", N=N, K=K, fmt=fmt, ms=f"{(time.perf_counter() - t0) * 1e3:.2f}",
            changed_vs_rtn=f"{np.mean(codes_ref != ref['codes']):.3f}")
    assert np.array_equal(_np(scales), ref["scales"])
    assert np.array_equal(unpack_codes(fmt, _np(codes)), codes_ref)


@pytest.mark.slow
def test_pack_weights_gptq_full_size(ops, pipe):
    """GPTQ rounding at a workload's size: the 3072x3072 int4 residual weight
    of the 1024-token low-rank case.  Steps are compared on every row; codes
    on 128 sampled rows (GPTQ treats rows independently, so the oracle can
    run the sampled rows alone), bit-exact."""
    case = WL.workload("lowrank")
    cal = WL.gptq_calibration(case.K, 3 + 7)
    t = pipe.case_to_device(case)
    u = torch.from_numpy(np.ascontiguousarray(cal["u"])).cuda()
    perm = torch.from_numpy(cal["perm"].astype(np.int32)).cuda()
    codes, scales = ops.pack_weights_gptq(t["w"], t["s"], u, perm, "int4", fwht_block=case.fwht_block)
    ref = O.quantize_operand(case.w, case.s, "int4", case.fwht_block)
    rows = np.sort(np.random.default_rng(12).choice(case.N, 128, replace=False))
    codes_ref, _ = O.gptq_rows(ref["y"][rows], ref["scales"][rows], cal["u"], O.INT4_QMAX, cal["perm"])
    got = unpack_codes("int4", _np(codes))
    _report("gptq_full", N=case.N, K=case.K, rows=len(rows),
            changed_vs_rtn=f"{np.mean(codes_ref != ref['codes'][rows]):.3f}")
    assert np.array_equal(_np(scales), ref["scales"])
    assert np.array_equal(got[rows], codes_ref)
    assert np.mean(codes_ref != ref["codes"][rows]) > 0.05    # the feedback did change codes


def test_gptq_linear_end_to_end(ops, pipe):
    """A W4A4 layer packed with GPTQ rounding: output within tolerance of the
    oracle's GPTQ linear."""
    case = WL.linear_case(40, 96, 256, seed=95, fmt="int4", n_outliers=4, outlier_gain=15.0, gptq=True)
    layer, t, y = _run(pipe, case)
    ref = _oracle(case)
    nw = check_operand("int4", _np(layer.w_codes), _np(layer.w_scales), ref["w"], what="weights")
    assert nw == 0
    check_output(_np(y), ref["y"], 1e-2)


def test_determinism_and_side_stream(ops, pipe):
    case = WL.linear_case(64, 2048, 2048, seed=51, n_outliers=16, outlier_gain=15.0)
    layer, t = pipe.build_layer(case)
    y1 = layer.forward(t["x"]).clone()
    layer_nows, _ = pipe.build_layer(case, use_workspace=False)
    y0 = layer_nows.forward(t["x"]).clone()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))   # split-K changes nothing
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y2 = layer.forward(t["x"], stream=s).clone()
    s.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_graph_capture_replays_match_eager(ops, pipe):
    """The whole per-call path captured in a HIP graph: every replay (with
    eager work and synchronisations in between) equals the eager result."""
    for name in ["decode_w4a4", "lowrank"]:
        case = WL.workload(name)
        layer, t = pipe.build_layer(case)
        y_eager = layer.forward(t["x"]).clone()
        out = torch.empty_like(y_eager)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            layer.forward(t["x"], out=out)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer.forward(t["x"], out=out)
        for rep in range(4):
            out.fill_(0)
            layer.forward(t["x"] * 0)          # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), y_eager.view(torch.int16)), (name, rep)


def test_nvfp4_quantizer_long_row_stride(ops, pipe):
    """Many NVFP4 rows whose row stride puts 64 rows beyond 31-bit offsets
    (ldx = 2^24 + 64 bf16 elements, an 8.6 GB view): the launcher takes the
    row kernels, and codes and scales match the oracle on the K real
    columns of every row."""
    M, K, ldx = 260, 256, (1 << 24) + 64
    case = WL.linear_case(M, 16, K, seed=97, fmt="nvfp4", n_outliers=4, outlier_gain=20.0)
    t = pipe.case_to_device(case)
    big = torch.zeros((M, ldx), dtype=torch.bfloat16, device="cuda")
    big[:, :K] = t["x"]
    x = big[:, :K]
    assert x.stride(0) == ldx
    g = float(O.nvfp4_tensor_scale(O.transformed_amax(case.x, case.inv_s)))
    codes, scales = ops.quantize_act(x, t["inv_s"], "nvfp4", tensor_scale=g)
    ref = O.quantize_operand(case.x, case.inv_s, "nvfp4", g=np.float32(g))
    n = check_operand("nvfp4", _np(codes), _np(scales), ref, what="activations")
    assert n == 0
    del big, x
    torch.cuda.empty_cache()


def test_empty_batch_is_noop(ops):
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    codes, scales = ops.quantize_act(x, None, "int4")
    assert codes.shape == (0, 64)
    y = ops.w4a4_linear(codes, scales, torch.zeros((8, 64), dtype=torch.uint8, device="cuda"),
                        torch.ones(8, device="cuda"), 128)
    assert y.shape == (0, 8)


@pytest.mark.slow
@pytest.mark.parametrize("name", WL.WORKLOADS)
def test_full_workloads(ops, pipe, name):
    """Full-size workloads in the launch configuration the benchmark times."""
    case = WL.workload(name)
    _report(name, M=case.M, N=case.N, K=case.K, fmt=case.fmt)
    layer, t, y = _run(pipe, case)
    ref = _oracle(case)
    b = layer.buffers(case.M, t["x"].device)
    fa, fw = _sides(case.fmt)
    na = check_operand(fa, _np(b["codes"]), _np(b["scales"]), ref["a"], what="activations")
    nw = check_operand(fw, _np(layer.w_codes), _np(layer.w_scales), ref["w"], what="weights")
    worst = check_output(_np(y), ref["y"], 1e-3 if case.y_dtype == "f32" else 1e-2)
    exact = case.fmt in ("int4", "int8", "w4a8") and case.branch is None and na == 0 and nw == 0
    if exact:   # e.g. the 16x256x256 fp32 case: the output itself is bit-exact
        check_output_exact(_np(y), ref["y_main"], case.y_dtype)
    if case.fmt in ("int4", "int8", "w4a8"):
        yi = torch.empty((case.M, case.N), dtype=torch.int32, device="cuda")
        _raw_linear(ops, case.fmt, b["codes"], b["scales"], layer.w_codes, layer.w_scales, case.K,
                    y=yi, workspace=b["ws"])
        acc = O.int_gemm(unpack_codes(fa, _np(b["codes"])), unpack_codes(fw, _np(layer.w_codes)))
        assert np.array_equal(_np(yi).astype(np.int64), acc)
    _report(name, band_mismatch_a=na, band_mismatch_w=nw, worst=f"{worst:.3g}", bit_exact=exact)
