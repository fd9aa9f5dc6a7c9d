"""The allocation-free linear (w4a4_linear_noalloc) against the linear entry
points given a workspace, through the C ABI: same kernels, so the int32
accumulators and the outputs are bit-identical.  Two calls in a row share
the library's static split-K buffer, the second with a smaller input."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w4a4_post_quantized_channel_amd import ops as _ops
    return _ops


def _codes(rng, fmt, R, K, side):
    if fmt == "nvfp4":
        return (torch.from_numpy(rng.integers(0, 256, (R, K // 2), dtype=np.uint8)).cuda(),
                torch.from_numpy(rng.integers(0x30, 0x40, (R, K // 16), dtype=np.uint8)).cuda())
    if fmt == "int4" or (fmt == "w4a8" and side == "w"):
        c = torch.from_numpy(rng.integers(0, 256, (R, K // 2), dtype=np.uint8)).cuda()
    elif fmt == "fp8":
        b = rng.integers(0, 256, (R, K), dtype=np.uint8)
        b[(b & 0x7F) == 0x7F] ^= 1
        c = torch.from_numpy(b).cuda()
    else:
        c = torch.from_numpy(rng.integers(-128, 128, (R, K), dtype=np.int8)).cuda()
    return c, torch.from_numpy(rng.uniform(0.5, 2.0, R).astype(np.float32)).cuda()


def _with_workspace(ops, fmt, a, sa, w, sw, K, y):
    ws = ops.make_workspace(a.shape[0], w.shape[0], K, fmt)
    if fmt in ("int4", "nvfp4"):
        return ops.w4a4_linear(a, sa, w, sw, K, fmt, y=y, workspace=ws, alpha=0.75)
    fn = {"int8": ops.w8a8_linear, "w4a8": ops.w4a8_linear, "fp8": ops.fp8_linear}[fmt]
    return fn(a, sa, w, sw, K, y=y, workspace=ws, alpha=0.75)


# first call larger, second smaller; both few-token shapes split K
CALLS = [(64, 512, 8192), (20, 512, 4096)]


@pytest.mark.parametrize("fmt", ["int4", "int8", "w4a8", "fp8", "nvfp4"])
@pytest.mark.parametrize("y_kind", ["bf16", "i32"])
def test_noalloc_matches_workspace_entry_point(ops, fmt, y_kind):
    if y_kind == "i32" and fmt in ("fp8", "nvfp4"):
        pytest.skip("raw accumulators exist for the integer formats only")
    ydt = torch.int32 if y_kind == "i32" else torch.bfloat16
    rng = np.random.default_rng(77)
    calls = CALLS if fmt != "nvfp4" else [(300, 256, 1024), (80, 128, 512)]
    for M, N, K in calls:
        if fmt != "nvfp4":
            p = ops.linear_plan(M, N, K, fmt, True)
            assert p["family"] == "decode_split" and ops.workspace_size(M, N, K, fmt) <= 4 << 20
        a, sa = _codes(rng, fmt, M, K, "a")
        w, sw = _codes(rng, fmt, N, K, "w")
        print(f"[noalloc] fmt={fmt} y={y_kind} M={M} N={N} K={K}", flush=True)
        want = _with_workspace(ops, fmt, a, sa, w, sw, K, torch.empty((M, N), dtype=ydt, device="cuda"))
        got = torch.full((M, N), 7, dtype=ydt, device="cuda")
        ops.linear_noalloc(a, sa, w, sw, K, fmt, y=got, alpha=0.75)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16 if ydt == torch.bfloat16 else torch.int32),
                           want.view(torch.int16 if ydt == torch.bfloat16 else torch.int32)), (fmt, M, N, K)


def test_noalloc_on_a_side_stream_and_many_tokens(ops):
    """Ordered calls on another stream, and a many-token shape (no split, no scratch)."""
    rng = np.random.default_rng(5)
    s = torch.cuda.Stream()
    for M, N, K in [(64, 512, 8192), (300, 640, 512)]:
        a, sa = _codes(rng, "int8", M, K, "a")
        w, sw = _codes(rng, "int8", N, K, "w")
        want = _with_workspace(ops, "int8", a, sa, w, sw, K, torch.empty((M, N), dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        got = torch.empty((M, N), dtype=torch.int32, device="cuda")
        with torch.cuda.stream(s):
            ops.linear_noalloc(a, sa, w, sw, K, "int8", y=got, alpha=0.75, stream=s)
        s.synchronize()
        assert torch.equal(got, want)
