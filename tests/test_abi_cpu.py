"""C-ABI library checks that need no GPU: the library loads, exports every
symbol the header declares, and rejects bad arguments before any launch
(so these calls never touch a device)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a4.h")
LIBPATH = os.path.join(ROOT, "w4a4_post_quantized_channel_amd", "libw4a4.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIBPATH), reason="libw4a4.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^(?:int|int64_t|size_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)


@pytest.fixture(scope="module")
def ops():
    from w4a4_post_quantized_channel_amd import ops as _ops
    return _ops


def test_header_declares_the_five_entry_points():
    names = declared_functions()
    for n in ["quantize_act", "pack_weights", "w4a4_linear", "w8a8_linear", "w4a8_linear", "fp8_linear",
              "lowrank_add"]:
        assert n in names


def test_library_exports_every_declared_symbol(ops):
    names = declared_functions()
    assert len(names) >= 10
    lib = ctypes.CDLL(LIBPATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(ops.EXPORTS)
    assert ops.LIB.w4a4_abi_version() == 3


def test_lowrank_width_host_query(ops):
    L = ops.LIB
    # gather: |r| columns; projection: the hi/lo pair, 2r columns
    assert L.w4a4_lowrank_width(1024, 3072, -64) == 64
    assert L.w4a4_lowrank_width(4096, 5120, 32) == 64
    assert L.w4a4_lowrank_width(1024, 3072, 32) == 64
    assert L.w4a4_lowrank_width(50, 64, 8) == 16


def test_status_strings(ops):
    for code, text in [(0, "ok"), (-1, "invalid argument"), (-2, "unsupported shape"),
                       (-3, "misaligned"), (-4, "unsupported format"), (-5, "workspace"),
                       (-6, "launch")]:
        assert text in ops.LIB.w4a4_status_string(code).decode()


FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: every call below is rejected
FAKE2 = ctypes.c_void_p(0x20000)
MISAL = ctypes.c_void_p(0x10008)


def _q(ops, fmt=0, fwht=64, order=0, g=1.0):
    return ctypes.byref(ops.QDesc(fmt, fwht, order, g))


def test_quantize_act_rejects_bad_arguments(ops):
    L = ops.LIB
    assert L.quantize_act(FAKE, 1, 4, 128, 128, None, None, FAKE2, FAKE2, None) == -1      # q NULL
    assert L.quantize_act(FAKE, 1, -1, 128, 128, None, _q(ops), FAKE2, FAKE2, None) == -1  # M < 0
    assert L.quantize_act(FAKE, 1, 4, 0, 128, None, _q(ops), FAKE2, FAKE2, None) == -1     # K == 0
    assert L.quantize_act(FAKE, 1, 4, 96, 96, None, _q(ops), FAKE2, FAKE2, None) == -2     # K % 64 with FWHT
    assert L.quantize_act(FAKE, 1, 4, 40, 40, None, _q(ops, fwht=0), FAKE2, FAKE2, None) == -2  # K % 16
    assert L.quantize_act(FAKE, 1, 4, 128, 64, None, _q(ops), FAKE2, FAKE2, None) == -1    # ldx < K
    assert L.quantize_act(MISAL, 1, 4, 128, 128, None, _q(ops), FAKE2, FAKE2, None) == -3  # x misaligned
    assert L.quantize_act(FAKE, 1, 4, 128, 132, None, _q(ops), FAKE2, FAKE2, None) == -3   # row stride
    assert L.quantize_act(FAKE, 7, 4, 128, 128, None, _q(ops), FAKE2, FAKE2, None) == -4   # dtype
    assert L.quantize_act(FAKE, 1, 4, 128, 128, None, _q(ops, fmt=9), FAKE2, FAKE2, None) == -4
    assert L.quantize_act(FAKE, 1, 4, 128, 128, None, _q(ops, fwht=32), FAKE2, FAKE2, None) == -4
    assert L.quantize_act(FAKE, 1, 4, 128, 128, None, _q(ops, order=5), FAKE2, FAKE2, None) == -4
    assert L.quantize_act(FAKE, 1, 4, 128, 128, None, _q(ops, fmt=2, g=0.0), FAKE2, FAKE2, None) == -1
    assert L.quantize_act(FAKE, 1, 4, 128, 128, None, _q(ops, fmt=2, g=float("inf")), FAKE2, FAKE2, None) == -1
    assert L.quantize_act(None, 1, 4, 128, 128, None, _q(ops), FAKE2, FAKE2, None) == -1
    assert L.quantize_act(FAKE, 1, 4, 128, 128, None, _q(ops), None, FAKE2, None) == -1
    assert L.quantize_act(FAKE, 1, 4, 128, 128, None, _q(ops), MISAL, FAKE2, None) == -3
    assert L.quantize_act(FAKE, 1, 4, 1 << 20, 1 << 20, None, _q(ops), FAKE2, FAKE2, None) == -2
    assert "quantize_act" in L.w4a4_last_error().decode()
    # M == 0 is a valid no-op (no pointers needed)
    assert L.quantize_act(None, 1, 0, 128, 128, None, _q(ops), None, None, None) == 0
    assert L.pack_weights(FAKE, 0, 4, 96, 96, None, _q(ops), FAKE2, FAKE2, None) == -2
    # W4A8: activations only (int8 in the W4A8 layout); weights are packed as INT4
    assert L.pack_weights(FAKE, 1, 4, 128, 128, None, _q(ops, fmt=3), FAKE2, FAKE2, None) == -4
    assert L.quantize_act(FAKE, 1, 4, 96, 96, None, _q(ops, fmt=3), FAKE2, FAKE2, None) == -2
    assert L.quantize_act(None, 1, 0, 128, 128, None, _q(ops, fmt=3), None, None, None) == 0
    assert L.quantize_act(None, 1, 0, 128, 128, None, _q(ops, fmt=4), None, None, None) == 0
    assert L.pack_weights(FAKE, 1, 4, 96, 96, None, _q(ops, fmt=4), FAKE2, FAKE2, None) == -2
    assert L.quantize_act(FAKE, 1, 4, 128, 128, None, _q(ops, fmt=5), FAKE2, FAKE2, None) == -4


def _lin(ops, fn="w4a4_linear", M=8, N=8, K=128, fmt=0, alpha=1.0, br=None, y=FAKE, ydt=1, ldy=None,
         ws=None, wsb=0, a=FAKE, sa=FAKE, w=FAKE, sw=FAKE):
    ldy = N if ldy is None else ldy
    brp = None if br is None else ctypes.byref(br)
    if fn in ("w8a8_linear", "w4a8_linear", "fp8_linear"):
        return getattr(ops.LIB, fn)(a, sa, w, sw, M, N, K, alpha, brp, y, ydt, ldy, ws, wsb, None)
    return ops.LIB.w4a4_linear(a, sa, w, sw, M, N, K, fmt, alpha, brp, y, ydt, ldy, ws, wsb, None)


def test_linear_rejects_bad_arguments(ops):
    assert _lin(ops, K=96) == -2
    assert _lin(ops, K=0) == -1
    assert _lin(ops, M=-1) == -1
    assert _lin(ops, K=1 << 20) == -2
    assert _lin(ops, M=(1 << 28) + 1) == -2       # per-row scales take 32-bit offsets
    assert _lin(ops, fn="w8a8_linear", M=(1 << 28) + 1) == -2
    assert _lin(ops, fmt=1) == -4                 # int8 codes go through w8a8_linear
    assert _lin(ops, fmt=3) == -4                 # int8 x int4 goes through w4a8_linear
    assert _lin(ops, fn="w4a8_linear", K=96) == -2
    assert _lin(ops, fn="w4a8_linear", a=MISAL) == -3
    assert _lin(ops, fn="w4a8_linear", ydt=5) == -4
    assert _lin(ops, fmt=4) == -4                 # FP8 codes go through fp8_linear
    assert _lin(ops, fn="fp8_linear", ydt=2) == -4   # no raw accumulators for FP8
    assert _lin(ops, fn="fp8_linear", K=96) == -2
    assert _lin(ops, fn="fp8_linear", w=MISAL) == -3
    assert _lin(ops, fn="fp8_linear", M=0, a=None, sa=None, y=None) == 0
    assert _lin(ops, fmt=2, ydt=2) == -4          # raw accumulators only for integer formats
    assert _lin(ops, ydt=5) == -4
    assert _lin(ops, ldy=4) == -1
    assert _lin(ops, alpha=float("nan")) == -1
    assert _lin(ops, a=None) == -1
    assert _lin(ops, a=MISAL) == -3
    assert _lin(ops, fn="w8a8_linear", w=MISAL) == -3
    br = ops.BranchDesc(1, 12, 12, 0, 0x10000, 16, 0x20000, 16)
    assert _lin(ops, br=br) == -1                 # r not a multiple of 8
    br = ops.BranchDesc(1, 16, 24, 0, 0x10000, 32, 0x20000, 16)
    assert _lin(ops, br=br) == -1                 # ra neither r nor 2r
    br = ops.BranchDesc(1, 16, 32, 0, 0x10008, 32, 0x20000, 16)
    assert _lin(ops, br=br) == -3                 # misaligned branch operand
    br = ops.BranchDesc(3, 16, 16, 0, 0x10000, 16, 0x20000, 16)
    assert _lin(ops, br=br) == -4
    br = ops.BranchDesc(1, 16, 16, 0, 0x10000, 16, 0x20000, 16)
    assert _lin(ops, br=br, ydt=2) == -4          # no raw accumulators with a branch
    # workspace present but smaller than the split-K plan needs
    M, N, K = 64, 512, 8192
    need = ops.LIB.w4a4_workspace_size(M, N, K, 1)
    assert need > 0
    assert _lin(ops, fn="w8a8_linear", M=M, N=N, K=K, ws=FAKE2, wsb=need - 1) == -5
    need = ops.LIB.w4a4_workspace_size(M, N, K, 3)
    assert need > 0
    assert _lin(ops, fn="w4a8_linear", M=M, N=N, K=K, ws=FAKE2, wsb=need - 1) == -5
    assert _lin(ops, fn="w4a8_linear", M=0, a=None, sa=None, y=None) == 0
    # empty problems are valid no-ops
    assert _lin(ops, M=0, a=None, sa=None, y=None) == 0
    assert _lin(ops, N=0, a=None, sa=None, w=None, sw=None, y=None) == 0


def test_workspace_sizes(ops):
    L = ops.LIB
    assert L.w4a4_workspace_size(4096, 5120, 5120, 2) == 0        # NVFP4: no split-K
    assert L.w4a4_workspace_size(512, 16384, 2048, 0) == 0        # many tokens: tile kernel
    assert L.w4a4_workspace_size(64, 512, 8192, 1) > 0            # few tokens, few channels, long K: split-K
    assert L.w4a4_workspace_size(9, 768, 8192, 0) > 0
    assert L.w4a4_workspace_size(64, 2048, 8192, 1) == 0          # 256 workgroups unsplit: no split
    assert L.w4a4_workspace_size(64, 2048, 2048, 0) == 0
    assert L.w4a4_workspace_size(9, 768, 8192, 3) > 0             # W4A8 decode splits like INT4
    assert L.w4a4_workspace_size(64, 2048, 8192, 3) == 0
    assert L.w4a4_workspace_size(512, 5120, 5120, 3) == 0         # many tokens: tile kernel
    assert L.w4a4_workspace_size(9, 768, 8192, 4) > 0             # FP8 decode splits like INT8
    assert L.w4a4_workspace_size(64, 512, 8192, 4) == L.w4a4_workspace_size(64, 512, 8192, 1)
    assert L.w4a4_workspace_size(9, 768, 8192, 5) == 0            # unknown format
    assert L.w4a4_workspace_size(64, 256, 1024, 0) == 0           # small weight: no split
    assert L.w4a4_workspace_size(16, 256, 256, 0) == 0            # a single K split
    assert L.w4a4_workspace_size(0, 2048, 2048, 0) == 0


def test_quantize_act_gather_rejects_bad_arguments(ops):
    L = ops.LIB
    g = lambda dt=1, M=4, r=8, ldo=8, idx=FAKE, xo=FAKE2, q=None: L.quantize_act_gather(
        FAKE, dt, M, 128, 128, None, q or _q(ops), FAKE2, FAKE2, idx, r, xo, ldo, None)
    assert g(dt=0) == -4                        # x must be bf16
    assert g(r=0) == -1 and g(r=129, ldo=129) == -1
    assert g(ldo=4) == -1
    assert g(idx=None) == -1 and g(xo=None) == -1
    assert g(xo=ctypes.c_void_p(0x20001)) == -3
    assert g(q=_q(ops, fmt=9)) == -4
    assert g(M=0, idx=None, xo=None) == 0       # empty batch


def test_pack_weights_gptq_rejects_bad_arguments(ops):
    L = ops.LIB
    need = L.w4a4_gptq_workspace_size(64, 256)
    assert need >= 64 * 256 * (4 + 8 + 1)
    WS = ctypes.c_void_p(0x100000)
    g = lambda K=256, fmt=0, u=FAKE, ws=WS, wsb=need, perm=None: L.pack_weights_gptq(
        FAKE, 1, 64, K, K, None, _q(ops, fmt=fmt), u, perm, FAKE2, FAKE2, ws, wsb, None)
    assert g(fmt=2) == -4 and g(fmt=4) == -4     # INT4 / INT8 only
    assert g(K=96) == -2                         # K % 64 with the rotation
    assert g(u=None) == -1
    assert g(u=ctypes.c_void_p(0x10004)) == -3
    assert g(perm=ctypes.c_void_p(0x10002)) == -3
    assert g(ws=None) == -5 and g(wsb=need - 1) == -5
    assert g(ws=ctypes.c_void_p(0x100080)) == -3
    assert L.w4a4_gptq_workspace_size(0, 256) == 0


def test_lowrank_rejects_bad_arguments(ops):
    L = ops.LIB
    B = 1   # W4A4_DT_BF16
    # both or neither of l1 / idx
    assert L.lowrank_add(FAKE, B, 4, 64, 64, FAKE, FAKE, FAKE, 8, 8, 16, FAKE2, 1, 16, None) == -1
    assert L.lowrank_add(FAKE, B, 4, 64, 64, None, None, FAKE, 8, 8, 16, FAKE2, 1, 16, None) == -1
    assert L.lowrank_add(FAKE, B, 4, 64, 64, FAKE, None, FAKE, 8, 0, 16, FAKE2, 1, 16, None) == -1    # r
    assert L.lowrank_add(FAKE, B, 4, 64, 64, FAKE, None, FAKE, 8, 200, 16, FAKE2, 1, 16, None) == -1  # r max
    assert L.lowrank_add(FAKE, B, 4, 60, 60, FAKE, None, FAKE, 8, 8, 16, FAKE2, 1, 16, None) == -2    # K % 8
    assert L.lowrank_add(MISAL, B, 4, 64, 64, FAKE, None, FAKE, 8, 8, 16, FAKE2, 1, 16, None) == -3
    assert L.lowrank_add(FAKE, B, 4, 64, 64, FAKE, None, FAKE, 8, 8, 16, FAKE2, 2, 16, None) == -4    # y dtype
    assert L.lowrank_add(FAKE, B, 4, 64, 64, FAKE, None, FAKE, 4, 8, 16, FAKE2, 1, 16, None) == -1    # ldlw
    assert L.w4a4_lowrank_project(FAKE, B, 4, 64, 64, FAKE, None, 8, FAKE2, 8, None) == -1           # ldo < 2r
    assert L.w4a4_lowrank_project(FAKE, B, 4, 64, 1 << 27, FAKE, None, 8, FAKE2, 16, None) == -2     # ldx too large
    assert L.w4a4_transform_amax(FAKE, 1, 4, 96, 96, None, _q(ops), FAKE2, None) == -2
    assert L.w4a4_transform_amax(FAKE, 1, 4, 128, 128, None, _q(ops), None, None) == -1


@pytest.mark.parametrize("dt", [0, 2, 7])   # F32, I32, unknown
def test_branch_calls_reject_non_bf16_activations(ops, dt):
    """The branch kernels read bf16; any other x dtype is refused before a launch
    (an fp32 tensor must not come back as silent garbage with status OK)."""
    L = ops.LIB
    assert L.lowrank_add(FAKE, dt, 4, 64, 64, FAKE, None, FAKE, 8, 8, 16, FAKE2, 1, 16, None) == -4
    assert L.lowrank_add(FAKE, dt, 4, 64, 64, None, FAKE, FAKE, 8, 8, 16, FAKE2, 0, 16, None) == -4
    assert L.w4a4_lowrank_project(FAKE, dt, 4, 64, 64, FAKE, None, 8, FAKE2, 16, None) == -4
    assert L.w4a4_lowrank_project(FAKE, dt, 4, 64, 64, None, FAKE, 8, FAKE2, 16, None) == -4
    assert b"BF16" in L.w4a4_last_error()


def test_gather_rejects_rotation_before_smoothing(ops):
    """Kept channels are removed by zero smoothing factors, which only removes
    raw channels when smoothing comes first."""
    L = ops.LIB
    st = L.quantize_act_gather(FAKE, 1, 4, 128, 128, None, _q(ops, order=1), FAKE2, FAKE2, FAKE, 8, FAKE2, 8, None)
    assert st == -4 and b"smoothing before the rotation" in L.w4a4_last_error()


def test_linear_plan_names_a_kernel_for_every_supported_shape(ops):
    """The host-side plan is what the linear entry points launch: every
    format at a grid of shapes (the workloads' and ragged ones) has a kernel,
    and the tile-shape dispatcher refuses (instead of silently launching
    nothing) any combination without one."""
    shapes = [(1, 1, 64), (16, 256, 256), (64, 2048, 2048), (64, 2048, 8192), (65, 2048, 2048),
              (512, 16384, 2048), (512, 2048, 8192), (1024, 3072, 3072), (4096, 5120, 5120),
              (3100, 2600, 320), (777, 2600, 320), (3100, 1000, 320), (300, 100, 64), (2600, 3210, 1088)]
    for fmt in ["int4", "int8", "nvfp4", "w4a8", "fp8"]:
        for (M, N, K) in shapes:
            for ws in (False, True):
                p = ops.linear_plan(M, N, K, fmt, ws)
                if M <= 64 and fmt != "nvfp4":
                    assert p["family"] in ("decode", "decode_split")
                    assert (p["splits"] > 1) == (p["family"] == "decode_split")
                    assert p["splits"] == 1 or (ws and ops.workspace_size(M, N, K, fmt) > 0)
                else:
                    assert p["family"] in ("tile", "nvfp4_shared") and p["splits"] == 1
                    assert p["family"] != "nvfp4_shared" or fmt == "nvfp4"
                    assert p["tile"] in [(256, 160), (128, 256), (128, 96), (64, 64), (128, 128)]
                    assert p["tile"] != (256, 160) or fmt in ("int4", "int8", "nvfp4")
                    assert p["tile"] != (128, 128) or fmt == "fp8"
    out = (ctypes.c_int32 * 4)()
    L = ops.LIB
    assert L.w4a4_linear_plan(64, 64, 100, 0, 0, out) == -2           # K % 64
    assert L.w4a4_linear_plan(64, 64, 128, 9, 0, out) == -4           # unknown format
    assert L.w4a4_linear_plan(0, 64, 128, 0, 0, out) == -1
    assert L.w4a4_linear_plan(64, 64, 128, 0, 0, None) == -1


def test_split_plans_fit_the_static_buffer(ops):
    """w4a4_linear_noalloc keeps split-K partials in a 4 MiB static buffer per
    GPU: no few-token plan needs more (at most 256 partial tiles of 64 x 64
    int32), so its size check never refuses a shape the linear entry points
    accept."""
    worst = 0
    for M in [1, 7, 16, 17, 32, 33, 48, 63, 64]:
        for N in [16, 48, 64, 100, 256, 512, 768, 1000, 2048, 4096]:
            for K in [64, 1024, 4096, 8192, 8256, 30016, 65536]:
                for fmt in [0, 1, 3, 4]:
                    worst = max(worst, ops.LIB.w4a4_workspace_size(M, N, K, fmt))
    assert 0 < worst <= 4 << 20
    args = [FAKE, FAKE, FAKE, FAKE, 4, 8, 128]
    assert ops.LIB.w4a4_linear_noalloc(*args, 9, 1.0, None, FAKE2, 1, 8, None) == -4     # unknown format
    assert ops.LIB.w4a4_linear_noalloc(*args[:6], 100, 0, 1.0, None, FAKE2, 1, 8, None) == -2   # K % 64
    assert ops.LIB.w4a4_linear_noalloc(*args, 0, 1.0, None, FAKE2, 1, 4, None) == -1     # ldy < N


def test_quantize_act_lowrank_rejects_bad_arguments(ops):
    L = ops.LIB
    g = lambda dt=1, M=4, K=128, r=32, ldo=64, l1=FAKE, out=FAKE2, q=None: L.quantize_act_lowrank(
        FAKE, dt, M, K, K, None, q or _q(ops), FAKE2, FAKE2, l1, r, out, ldo, None)
    assert g(dt=0) == -4                          # x must be bf16
    assert g(r=8) == -1 and g(r=24) == -1 and g(r=64, ldo=128) == -1
    assert g(ldo=63) == -1                        # hi and lo need 2r columns
    assert g(K=96 + 64) == -2                     # K % 64
    assert g(K=4096 + 64, r=16) == -2             # the staged row fits LDS up to K = 4096
    assert g(l1=None) == -1 and g(out=None) == -1
    assert g(l1=ctypes.c_void_p(0x10008)) == -3
    assert g(q=_q(ops, fmt=9)) == -4
    assert g(M=0, l1=None, out=None) == 0         # empty batch


def test_quantize_act_project_rejects_bad_arguments(ops):
    L = ops.LIB
    g = lambda dt=1, M=4, K=128, r=32, ldo=64, l1=FAKE, out=FAKE2, q=None: L.quantize_act_project(
        FAKE, dt, M, K, K, None, q or _q(ops), FAKE2, FAKE2, l1, r, out, ldo, None)
    assert g(dt=0) == -4                          # x must be bf16
    assert g(r=0) == -1 and g(r=129, ldo=258) == -1
    assert g(ldo=63) == -1                        # hi and lo need 2r columns
    assert g(K=96 + 64 + 8) == -2                 # K % 16
    assert g(K=5120 + 64) == -2                   # one wave per row: K <= 5120
    assert g(l1=None) == -1 and g(out=None) == -1
    assert g(l1=ctypes.c_void_p(0x10008)) == -3
    assert g(q=_q(ops, fmt=9)) == -4
    assert g(M=0, out=None) == 0                  # empty batch
