"""Python binding of the C ABI in ``include/w4a4.h`` (ctypes).

Argument marshalling only: every step of the quantized linear runs in the
HIP kernels of ``libw4a4.so``.  PyTorch supplies device memory and the HIP
stream.  If the library is missing this module raises at import: there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a4.so")

FMT_INT4, FMT_INT8, FMT_NVFP4, FMT_W4A8, FMT_FP8 = 0, 1, 2, 3, 4
DT_F32, DT_BF16, DT_I32 = 0, 1, 2
ORDER_SMOOTH_THEN_ROTATE, ORDER_ROTATE_THEN_SMOOTH = 0, 1
BRANCH_NONE, BRANCH_BF16 = 0, 1
# w4a8: quantize_act writes W4A8-layout int8 activations; the weights are int4
FMTS = {"int4": FMT_INT4, "int8": FMT_INT8, "nvfp4": FMT_NVFP4, "w4a8": FMT_W4A8, "fp8": FMT_FP8}
ORDERS = {"smooth_then_rotate": ORDER_SMOOTH_THEN_ROTATE,
          "rotate_then_smooth": ORDER_ROTATE_THEN_SMOOTH}
ABI_VERSION = 3
MAX_BRANCH = 128   # W4A4_MAX_BRANCH: largest branch width (rank or kept channels)

EXPORTS = ["quantize_act", "quantize_act_gather", "quantize_act_lowrank", "quantize_act_project", "pack_weights", "pack_weights_gptq", "w4a4_gptq_workspace_size", "w4a4_linear", "w4a4_linear_noalloc", "w8a8_linear", "w4a8_linear", "fp8_linear", "lowrank_add",
           "w4a4_lowrank_project", "w4a4_lowrank_width", "w4a4_transform_amax", "w4a4_linear_plan",
           "w4a4_workspace_size", "w4a4_status_string",
           "w4a4_last_error", "w4a4_abi_version"]


class QDesc(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("fwht_block", ctypes.c_int32),
                ("order", ctypes.c_int32), ("tensor_scale", ctypes.c_float)]


class BranchDesc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("r", ctypes.c_int32), ("ra", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("a", ctypes.c_void_p), ("lda", ctypes.c_int64),
                ("b", ctypes.c_void_p), ("ldb", ctypes.c_int64)]


class W4A4Error(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} not built: run __graft_entry__.build() or "
                          f"python -m w4a4_post_quantized_channel_amd.build")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    qd, br = ctypes.POINTER(QDesc), ctypes.POINTER(BranchDesc)
    sig = {
        "quantize_act": [vp, i32, i64, i64, i64, vp, qd, vp, vp, vp],
        "quantize_act_gather": [vp, i32, i64, i64, i64, vp, qd, vp, vp, vp, i64, vp, i64, vp],
        "quantize_act_lowrank": [vp, i32, i64, i64, i64, vp, qd, vp, vp, vp, i64, vp, i64, vp],
        "quantize_act_project": [vp, i32, i64, i64, i64, vp, qd, vp, vp, vp, i64, vp, i64, vp],
        "pack_weights": [vp, i32, i64, i64, i64, vp, qd, vp, vp, vp],
        "pack_weights_gptq": [vp, i32, i64, i64, i64, vp, qd, vp, vp, vp, vp, vp, sz, vp],
        "w4a4_gptq_workspace_size": [i64, i64],
        "w4a4_linear": [vp, vp, vp, vp, i64, i64, i64, i32, f32, br, vp, i32, i64, vp, sz, vp],
        "w4a4_linear_noalloc": [vp, vp, vp, vp, i64, i64, i64, i32, f32, br, vp, i32, i64, vp],
        "w8a8_linear": [vp, vp, vp, vp, i64, i64, i64, f32, br, vp, i32, i64, vp, sz, vp],
        "w4a8_linear": [vp, vp, vp, vp, i64, i64, i64, f32, br, vp, i32, i64, vp, sz, vp],
        "fp8_linear": [vp, vp, vp, vp, i64, i64, i64, f32, br, vp, i32, i64, vp, sz, vp],
        "w4a4_workspace_size": [i64, i64, i64, i32],
        "lowrank_add": [vp, i32, i64, i64, i64, vp, vp, vp, i64, i64, i64, vp, i32, i64, vp],
        "w4a4_lowrank_project": [vp, i32, i64, i64, i64, vp, vp, i64, vp, i64, vp],
        "w4a4_linear_plan": [i64, i64, i64, i32, i32, ctypes.POINTER(ctypes.c_int32)],
        "w4a4_lowrank_width": [i64, i64, i64],
        "w4a4_transform_amax": [vp, i32, i64, i64, i64, vp, qd, vp, vp],
        "w4a4_status_string": [ctypes.c_int],
        "w4a4_last_error": [],
        "w4a4_abi_version": [],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.w4a4_workspace_size.restype = ctypes.c_size_t
    lib.w4a4_gptq_workspace_size.restype = ctypes.c_size_t
    lib.w4a4_lowrank_width.restype = ctypes.c_int64
    lib.w4a4_status_string.restype = ctypes.c_char_p
    lib.w4a4_last_error.restype = ctypes.c_char_p
    if lib.w4a4_abi_version() != ABI_VERSION:
        raise ImportError("libw4a4.so ABI version mismatch")
    return lib


LIB = load_library()


def _check(fn: str, status: int):
    if status != 0:
        raise W4A4Error(fn, status, LIB.w4a4_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DT_BF16
    if t.dtype == torch.float32:
        return DT_F32
    if t.dtype == torch.int32:
        return DT_I32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _rowmajor(t: torch.Tensor):
    assert t.dim() == 2 and t.stride(1) == 1, "expect a 2-D row-major tensor"
    return t.shape[0], t.shape[1], t.stride(0)


def qdesc(fmt, fwht_block: int = 64, order="smooth_then_rotate", tensor_scale: float = 1.0) -> QDesc:
    f = FMTS[fmt] if isinstance(fmt, str) else int(fmt)
    o = ORDERS[order] if isinstance(order, str) else int(order)
    return QDesc(f, int(fwht_block), o, float(tensor_scale))


def code_shapes(fmt: str, R: int, K: int):
    """(codes shape, codes dtype, scales shape, scales dtype) of a packed operand."""
    if fmt == "int4":
        return (R, K // 2), torch.uint8, (R,), torch.float32
    if fmt in ("int8", "w4a8"):   # w4a8: activation side, int8 in the W4A8 layout
        return (R, K), torch.int8, (R,), torch.float32
    if fmt == "fp8":              # OCP E4M3 codes
        return (R, K), torch.uint8, (R,), torch.float32
    if fmt == "nvfp4":
        return (R, K // 2), torch.uint8, (R, K // 16), torch.uint8
    raise ValueError(fmt)


def _alloc_codes(fmt, R, K, device):
    cs, cd, ss, sd = code_shapes(fmt, R, K)
    return torch.empty(cs, dtype=cd, device=device), torch.empty(ss, dtype=sd, device=device)


def quantize_act(x: torch.Tensor, inv_smooth: Optional[torch.Tensor], fmt: str = "int4", *,
                 fwht_block: int = 64, order="smooth_then_rotate", tensor_scale: float = 1.0,
                 codes=None, scales=None, stream=None, M: Optional[int] = None):
    """Per-token quantization of the transformed activations (see include/w4a4.h)."""
    R, K, ld = _rowmajor(x)
    if M is not None:
        R = M
    if codes is None:
        codes, scales = _alloc_codes(fmt, R, K, x.device)
    q = qdesc(fmt, fwht_block, order, tensor_scale)
    _check("quantize_act", LIB.quantize_act(_ptr(x), _dtype_code(x), R, K, ld, _ptr(inv_smooth),
                                            ctypes.byref(q), _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def pack_weights_gptq(w: torch.Tensor, smooth: Optional[torch.Tensor], u: torch.Tensor,
                      perm: Optional[torch.Tensor] = None, fmt: str = "int4", *, fwht_block: int = 64,
                      order="smooth_then_rotate", codes=None, scales=None, workspace=None, stream=None):
    """pack_weights with GPTQ-style rounding (u: float64 K x K upper factor, perm: int32[K] or None)."""
    R, K, ld = _rowmajor(w)
    if codes is None:
        codes, scales = _alloc_codes(fmt, R, K, w.device)
    if workspace is None:
        workspace = torch.empty(int(LIB.w4a4_gptq_workspace_size(R, K)), dtype=torch.uint8, device=w.device)
    assert u.dtype == torch.float64 and u.is_contiguous()
    q = qdesc(fmt, fwht_block, order)
    _check("pack_weights_gptq", LIB.pack_weights_gptq(
        _ptr(w), _dtype_code(w), R, K, ld, _ptr(smooth), ctypes.byref(q), _ptr(u), _ptr(perm), _ptr(codes),
        _ptr(scales), _ptr(workspace), workspace.numel(), _stream(stream)))
    return codes, scales


def quantize_act_gather(x: torch.Tensor, inv_smooth: Optional[torch.Tensor], idx: torch.Tensor,
                        fmt: str = "int4", *, fwht_block: int = 64, order="smooth_then_rotate",
                        tensor_scale: float = 1.0, codes=None, scales=None, xo=None, stream=None):
    """quantize_act plus the kept-channel operand xo = x[:, idx] from the same pass."""
    R, K, ld = _rowmajor(x)
    r = idx.shape[0]
    if codes is None:
        codes, scales = _alloc_codes(fmt, R, K, x.device)
    if xo is None:
        xo = torch.empty((R, r), dtype=torch.bfloat16, device=x.device)
    q = qdesc(fmt, fwht_block, order, tensor_scale)
    _check("quantize_act_gather",
           LIB.quantize_act_gather(_ptr(x), _dtype_code(x), R, K, ld, _ptr(inv_smooth), ctypes.byref(q),
                                   _ptr(codes), _ptr(scales), _ptr(idx), r, _ptr(xo), xo.stride(0),
                                   _stream(stream)))
    return codes, scales, xo


def lowrank_fusable(x: torch.Tensor, l1t: torch.Tensor) -> bool:
    """Whether quantize_act_lowrank takes this activation / rank (see the header)."""
    r, K = l1t.shape
    return x.dtype == torch.bfloat16 and K % 64 == 0 and K <= 4096 and r in (16, 32)


def quantize_act_lowrank(x: torch.Tensor, inv_smooth: Optional[torch.Tensor], l1t: torch.Tensor,
                         fmt: str = "int4", *, fwht_block: int = 64, order="smooth_then_rotate",
                         tensor_scale: float = 1.0, codes=None, scales=None, out=None, stream=None):
    """quantize_act plus the low-rank operand [bf16(x L1) | residual] from the same pass."""
    R, K, ld = _rowmajor(x)
    r = l1t.shape[0]
    if codes is None:
        codes, scales = _alloc_codes(fmt, R, K, x.device)
    if out is None:
        out = torch.empty((R, 2 * r), dtype=torch.bfloat16, device=x.device)
    q = qdesc(fmt, fwht_block, order, tensor_scale)
    _check("quantize_act_lowrank",
           LIB.quantize_act_lowrank(_ptr(x), _dtype_code(x), R, K, ld, _ptr(inv_smooth), ctypes.byref(q),
                                    _ptr(codes), _ptr(scales), _ptr(l1t), r, _ptr(out), out.stride(0),
                                    _stream(stream)))
    return codes, scales, out


def project_fusable(x: torch.Tensor, l1t: torch.Tensor) -> bool:
    """Whether quantize_act_project takes this activation / rank (see the header)."""
    r, K = l1t.shape
    return x.dtype == torch.bfloat16 and K % 16 == 0 and K <= 5120 and 1 <= r <= MAX_BRANCH


def quantize_act_project(x: torch.Tensor, inv_smooth: Optional[torch.Tensor], l1t: torch.Tensor,
                         fmt: str = "int4", *, fwht_block: int = 64, order="smooth_then_rotate",
                         tensor_scale: float = 1.0, codes=None, scales=None, out=None, stream=None):
    """quantize_act and lowrank_project (low-rank form) in one launch."""
    R, K, ld = _rowmajor(x)
    r = l1t.shape[0]
    if codes is None:
        codes, scales = _alloc_codes(fmt, R, K, x.device)
    if out is None:
        out = torch.empty((R, 2 * r), dtype=torch.bfloat16, device=x.device)
    q = qdesc(fmt, fwht_block, order, tensor_scale)
    _check("quantize_act_project",
           LIB.quantize_act_project(_ptr(x), _dtype_code(x), R, K, ld, _ptr(inv_smooth), ctypes.byref(q),
                                    _ptr(codes), _ptr(scales), _ptr(l1t), r, _ptr(out), out.stride(0),
                                    _stream(stream)))
    return codes, scales, out


def pack_weights(w: torch.Tensor, smooth: Optional[torch.Tensor], fmt: str = "int4", *,
                 fwht_block: int = 64, order="smooth_then_rotate", tensor_scale: float = 1.0,
                 codes=None, scales=None, stream=None):
    """Per-output-channel quantization of W S R (inverse transform folded in)."""
    R, K, ld = _rowmajor(w)
    if codes is None:
        codes, scales = _alloc_codes(fmt, R, K, w.device)
    q = qdesc(fmt, fwht_block, order, tensor_scale)
    _check("pack_weights", LIB.pack_weights(_ptr(w), _dtype_code(w), R, K, ld, _ptr(smooth),
                                            ctypes.byref(q), _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def transform_amax(x: torch.Tensor, scale: Optional[torch.Tensor], *, fwht_block: int = 64,
                   order="smooth_then_rotate", out=None, stream=None) -> torch.Tensor:
    R, K, ld = _rowmajor(x)
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    q = qdesc("int4", fwht_block, order, 1.0)
    _check("w4a4_transform_amax", LIB.w4a4_transform_amax(_ptr(x), _dtype_code(x), R, K, ld, _ptr(scale),
                                                          ctypes.byref(q), _ptr(out), _stream(stream)))
    return out


def branch_desc(a: Optional[torch.Tensor], b: Optional[torch.Tensor], r: Optional[int] = None) -> BranchDesc:
    """Fused-branch descriptor: a is bf16 M x ra (ra = r, or 2 P r from lowrank_project), b is bf16 N x r."""
    if a is None:
        return BranchDesc(BRANCH_NONE, 0, 0, 0, None, 0, None, 0)
    r = b.shape[1] if r is None else r
    return BranchDesc(BRANCH_BF16, r, a.shape[1], 0, a.data_ptr(), a.stride(0), b.data_ptr(), b.stride(0))


PLAN_FAMILIES = {1: "decode", 2: "decode_split", 3: "tile", 4: "nvfp4_shared"}


def linear_plan(M: int, N: int, K: int, fmt: str, with_workspace: bool = True) -> dict:
    """The kernel the linear entry point runs for this shape (host query)."""
    out = (ctypes.c_int32 * 4)()
    _check("w4a4_linear_plan", LIB.w4a4_linear_plan(M, N, K, FMTS[fmt], int(with_workspace), out))
    return {"family": PLAN_FAMILIES[out[0]], "tile": (out[1], out[2]), "splits": out[3]}


def workspace_size(M: int, N: int, K: int, fmt: str) -> int:
    return int(LIB.w4a4_workspace_size(M, N, K, FMTS[fmt]))


def make_workspace(M: int, N: int, K: int, fmt: str, device="cuda") -> Optional[torch.Tensor]:
    n = workspace_size(M, N, K, fmt)
    return None if n == 0 else torch.empty(n, dtype=torch.uint8, device=device)


def _linear(fn: str, fmt: str, a_codes, a_scales, w_codes, w_scales, K: int, *, alpha=1.0,
            branch: Optional[BranchDesc] = None, y=None, y_dtype=torch.bfloat16, workspace=None,
            stream=None, M: Optional[int] = None):
    M = a_codes.shape[0] if M is None else M
    N = w_codes.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=y_dtype, device=a_codes.device)
    br = branch if branch is not None else branch_desc(None, None)
    args = (_ptr(a_codes), _ptr(a_scales), _ptr(w_codes), _ptr(w_scales), M, N, K)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    tail = (ctypes.byref(br), _ptr(y), _dtype_code(y), y.stride(0), _ptr(workspace), ws_bytes, _stream(stream))
    if fn in ("w8a8_linear", "w4a8_linear", "fp8_linear"):
        st = getattr(LIB, fn)(*args, float(alpha), *tail)
    else:
        st = LIB.w4a4_linear(*args, FMTS[fmt], float(alpha), *tail)
    _check(fn, st)
    return y


def w4a4_linear(a_codes, a_scales, w_codes, w_scales, K: int, fmt: str = "int4", **kw):
    """y = alpha * dequant(A . W^T) (+ fused bf16 branch); fmt int4 or nvfp4."""
    return _linear("w4a4_linear", fmt, a_codes, a_scales, w_codes, w_scales, K, **kw)


def linear_noalloc(a_codes, a_scales, w_codes, w_scales, K: int, fmt: str = "int4", *, alpha=1.0,
                   branch: Optional[BranchDesc] = None, y=None, y_dtype=torch.bfloat16, stream=None,
                   M: Optional[int] = None):
    """The linear of ``fmt`` with split-K partials in the library's static
    per-GPU buffer (no workspace, no allocation inside the call; ``y`` must
    be given by callers that cannot allocate)."""
    M = a_codes.shape[0] if M is None else M
    N = w_codes.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=y_dtype, device=a_codes.device)
    br = branch if branch is not None else branch_desc(None, None)
    _check("w4a4_linear_noalloc", LIB.w4a4_linear_noalloc(
        _ptr(a_codes), _ptr(a_scales), _ptr(w_codes), _ptr(w_scales), M, N, K, FMTS[fmt], float(alpha),
        ctypes.byref(br), _ptr(y), _dtype_code(y), y.stride(0), _stream(stream)))
    return y


def w8a8_linear(a_codes, a_scales, w_codes, w_scales, K: int, **kw):
    """INT8 W8A8 sibling of w4a4_linear."""
    return _linear("w8a8_linear", "int8", a_codes, a_scales, w_codes, w_scales, K, **kw)


def w4a8_linear(a_codes, a_scales, w_codes, w_scales, K: int, **kw):
    """INT8 activation codes x packed INT4 weight codes (W4A8)."""
    return _linear("w4a8_linear", "w4a8", a_codes, a_scales, w_codes, w_scales, K, **kw)


def fp8_linear(a_codes, a_scales, w_codes, w_scales, K: int, **kw):
    """FP8 (OCP E4M3) W8A8, fp32 accumulation."""
    return _linear("fp8_linear", "fp8", a_codes, a_scales, w_codes, w_scales, K, **kw)


def _check_branch_inputs(x, l1t, idx, lw=None):
    if x.dtype != torch.bfloat16:
        raise TypeError("the 16-bit branch takes bf16 activations")
    if l1t is not None and (l1t.dtype != torch.bfloat16 or not l1t.is_contiguous()
                            or l1t.shape[1] != x.shape[1]):
        raise TypeError("l1t must be a contiguous bf16 r x K tensor (L1 transposed)")
    if idx is not None and idx.dtype != torch.int32:
        raise TypeError("idx must be int32")
    if lw is not None and lw.dtype != torch.bfloat16:
        raise TypeError("lw must be bf16")


def lowrank_add(x: torch.Tensor, y: torch.Tensor, lw: torch.Tensor, *, l1t: Optional[torch.Tensor] = None,
                idx: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y += (x L1) lw^T  or  y += x[:, idx] lw^T, in place (l1t = L1 transposed, r x K)."""
    _check_branch_inputs(x, l1t, idx, lw)
    M, K, ldx = _rowmajor(x)
    N, r = lw.shape
    _check("lowrank_add", LIB.lowrank_add(_ptr(x), _dtype_code(x), M, K, ldx, _ptr(l1t), _ptr(idx), _ptr(lw),
                                          lw.stride(0), r, N, _ptr(y), _dtype_code(y), y.stride(0), _stream(stream)))
    return y


def lowrank_width(M: int, K: int, r: int) -> int:
    """Columns lowrank_project needs in its output: 2 P r for a rank-r
    projection (r > 0; the result is the first 2r), or |r| for a gather of
    |r| kept channels (r < 0)."""
    return int(LIB.w4a4_lowrank_width(M, K, r))


def lowrank_project(x: torch.Tensor, *, l1t: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                    out=None, stream=None) -> torch.Tensor:
    """The fused branch's ``a`` operand: [hi | lo] bf16 halves of x L1 (a view of
    the first 2r columns of ``out``), or x[:, idx]."""
    _check_branch_inputs(x, l1t, idx)
    M, K, ldx = _rowmajor(x)
    r = l1t.shape[0] if l1t is not None else idx.shape[0]
    width = lowrank_width(M, K, r if l1t is not None else -r)
    if out is None:
        out = torch.empty((M, width), dtype=torch.bfloat16, device=x.device)
    _check("w4a4_lowrank_project", LIB.w4a4_lowrank_project(_ptr(x), _dtype_code(x), M, K, ldx, _ptr(l1t), _ptr(idx),
                                                            r, _ptr(out), out.stride(0), _stream(stream)))
    return out[:, :2 * r] if l1t is not None else out
