"""A quantized linear layer assembled from the C-ABI calls.

``QuantizedLinear`` packs a float weight once (``pack_weights``: smoothing
and the block-64 rotation folded into the weight, FoldQuantVLA contribution
1) and then runs, per call, ``quantize_act`` -> [``w4a4_lowrank_project``]
-> ``w4a4_linear`` / ``w8a8_linear`` with the 16-bit branch fused into the
GEMM epilogue.  Everything runs in the HIP library; this file only holds
buffers and argument plumbing.
"""
from __future__ import annotations

import copy
from typing import Optional

import numpy as np
import torch

from . import ops

E2M1_TIMES_E4M3_MAX = np.float32(6.0 * 448.0)


def nvfp4_scale_from_amax(amax: float) -> float:
    """Static NVFP4 tensor scale g = fp32(amax / (6 * 448)); 1 when amax is 0."""
    a = np.float32(amax)
    return float(np.float32(1.0) if a == 0 else np.float32(a / E2M1_TIMES_E4M3_MAX))


class QuantizedLinear:
    """y = x W^T computed as the quantized path (int4 / int8 / nvfp4).

    w        N x K float weight (the part the quantized path carries), device.
    s        K smoothing factors (weights multiplied by s, activations by
             inv_s), device fp32, or None.
    inv_s    K factors for the activations (fp32(1/s)), device, or None.
    branch   None, {"kind": "lowrank", "l1t": r x K bf16 (L1 transposed), "lw": N x r bf16}
             or {"kind": "outlier", "idx": int32[r], "lw": N x r bf16}.
    """

    def __init__(self, w: torch.Tensor, s: Optional[torch.Tensor], inv_s: Optional[torch.Tensor],
                 fmt: str = "int4", *, fwht_block: int = 64, order: str = "smooth_then_rotate",
                 branch: Optional[dict] = None, y_dtype=torch.bfloat16, use_workspace: bool = True,
                 gptq: Optional[dict] = None, stream=None):
        if branch is not None and branch["kind"] == "outlier" and order != "smooth_then_rotate":
            # kept channels leave the quantized path through s = inv_s = 0,
            # which removes raw channels only when smoothing comes first
            raise ValueError("a kept-channel branch needs order='smooth_then_rotate'")
        self.fmt, self.fwht_block, self.order = fmt, fwht_block, order
        # W4A8 (the 8-bit-activation denoising steps) keeps 4-bit weight codes;
        # its activations are int8 codes in the W4A8 layout
        self.a_fmt, w_fmt = {"w4a8": ("w4a8", "int4")}.get(fmt, (fmt, fmt))
        self.use_workspace = use_workspace
        self.N, self.K = w.shape
        self.inv_s = inv_s
        self.y_dtype = y_dtype
        self.branch = branch
        self.g_w = 1.0
        if fmt == "nvfp4":
            amax = ops.transform_amax(w, s, fwht_block=fwht_block, order=order, stream=stream)
            self.g_w = nvfp4_scale_from_amax(float(amax.item()))
        if gptq is not None:   # GPTQ-style rounding: {"u": float64 K x K, "perm": int32[K] or None}
            self.w_codes, self.w_scales = ops.pack_weights_gptq(w, s, gptq["u"], gptq.get("perm"), w_fmt,
                                                                fwht_block=fwht_block, order=order, stream=stream)
        else:
            self.w_codes, self.w_scales = ops.pack_weights(w, s, w_fmt, fwht_block=fwht_block, order=order,
                                                           tensor_scale=self.g_w, stream=stream)
        self.g_a = 1.0
        self._bufs = {}
        # Low-rank branch operand T = x L1:
        # * launch_lowrank (default): quantizer and projection workgroups in
        #   one launch (quantize_act_project), outputs identical to the two
        #   calls;
        # * fuse_lowrank: from the quantizer's own pass over x
        #   (quantize_act_lowrank), which reads x once but measured slower on
        #   MI355X (every CU holding rows must stream all of L1);
        # * neither: quantize_act, then w4a4_lowrank_project.
        self.fuse_lowrank = False
        self.launch_lowrank = True

    # NVFP4 activations use a static per-tensor scale from calibration data
    # (statistics after both transforms, QuantWAMs sec. 4.2).
    def calibrate(self, x_cal: torch.Tensor, stream=None) -> float:
        if self.fmt == "nvfp4":
            amax = ops.transform_amax(x_cal, self.inv_s, fwht_block=self.fwht_block, order=self.order,
                                      stream=stream)
            self.g_a = nvfp4_scale_from_amax(float(amax.item()))
        return self.g_a

    @property
    def alpha(self) -> float:
        if self.fmt == "nvfp4":
            return float(np.float32(self.g_a) * np.float32(self.g_w))
        return 1.0

    def buffers(self, M: int, device):
        b = self._bufs.get(M)
        if b is None:
            codes, scales = ops._alloc_codes(self.a_fmt, M, self.K, device)
            br_a = None
            if self.branch is not None:
                r = self.branch["lw"].shape[1]
                width = ops.lowrank_width(M, self.K, r if self.branch["kind"] == "lowrank" else -r)
                br_a = torch.empty((M, width), dtype=torch.bfloat16, device=device)
            y = torch.empty((M, self.N), dtype=self.y_dtype, device=device)
            ws = ops.make_workspace(M, self.N, self.K, self.fmt, device=device) if self.use_workspace else None
            b = {"codes": codes, "scales": scales, "br_a": br_a, "y": y, "ws": ws}
            self._bufs[M] = b
        return b

    def quantize(self, x: torch.Tensor, stream=None):
        """quantize_act into this layer's M-row buffers; with kept channels
        (bf16 x) the same pass also writes the bypass operand."""
        b = self.buffers(x.shape[0], x.device)
        if self.branch is not None and self.branch["kind"] == "lowrank" and self.fuse_lowrank and \
                ops.lowrank_fusable(x, self.branch["l1t"]):
            # one pass over x: codes, scales and the low-rank operand x L1
            ops.quantize_act_lowrank(x, self.inv_s, self.branch["l1t"], self.a_fmt, fwht_block=self.fwht_block,
                                     order=self.order, tensor_scale=self.g_a, codes=b["codes"],
                                     scales=b["scales"], out=b["br_a"], stream=stream)
        elif self._one_launch_lowrank(x):
            # quantizer and projection workgroups side by side in one launch
            ops.quantize_act_project(x, self.inv_s, self.branch["l1t"], self.a_fmt, fwht_block=self.fwht_block,
                                     order=self.order, tensor_scale=self.g_a, codes=b["codes"],
                                     scales=b["scales"], out=b["br_a"], stream=stream)
        elif self.branch is not None and self.branch["kind"] == "outlier" and x.dtype == torch.bfloat16:
            ops.quantize_act_gather(x, self.inv_s, self.branch["idx"], self.a_fmt, fwht_block=self.fwht_block,
                                    order=self.order, tensor_scale=self.g_a, codes=b["codes"],
                                    scales=b["scales"], xo=b["br_a"], stream=stream)
        else:
            ops.quantize_act(x, self.inv_s, self.a_fmt, fwht_block=self.fwht_block, order=self.order,
                             tensor_scale=self.g_a, codes=b["codes"], scales=b["scales"], stream=stream)

    def _one_launch_lowrank(self, x) -> bool:
        return (self.branch is not None and self.branch["kind"] == "lowrank" and self.launch_lowrank and
                not (self.fuse_lowrank and ops.lowrank_fusable(x, self.branch["l1t"])) and
                ops.project_fusable(x, self.branch["l1t"]))

    def has_projection(self, x_dtype=torch.bfloat16) -> bool:
        """Whether the branch operand needs its own kernel (w4a4_lowrank_project)."""
        if self.branch is None:
            return False
        if self.branch["kind"] == "lowrank":
            xe = torch.empty(0, dtype=x_dtype)
            if self.fuse_lowrank and ops.lowrank_fusable(xe, self.branch["l1t"]):
                return False
            return not self._one_launch_lowrank(xe)
        return x_dtype != torch.bfloat16

    def project(self, x: torch.Tensor, stream=None):
        """The branch operand when the quantizer pass does not write it."""
        if not self.has_projection(x.dtype):
            return
        b = self.buffers(x.shape[0], x.device)
        if self.branch["kind"] == "lowrank":
            ops.lowrank_project(x, l1t=self.branch["l1t"], out=b["br_a"], stream=stream)
        else:
            ops.lowrank_project(x, idx=self.branch["idx"], out=b["br_a"], stream=stream)

    def gemm(self, M: int, device, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """The linear on the quantized activations in the M-row buffers, with
        the branch fused into its epilogue."""
        b = self.buffers(M, device)
        bd = None if self.branch is None else ops.branch_desc(self.branch_operand(M, device), self.branch["lw"])
        y = b["y"] if out is None else out
        if self.fmt in ("int8", "w4a8", "fp8"):
            fn = {"int8": ops.w8a8_linear, "w4a8": ops.w4a8_linear, "fp8": ops.fp8_linear}[self.fmt]
            return fn(b["codes"], b["scales"], self.w_codes, self.w_scales, self.K,
                      branch=bd, y=y, workspace=b["ws"], stream=stream)
        return ops.w4a4_linear(b["codes"], b["scales"], self.w_codes, self.w_scales, self.K, self.fmt,
                               alpha=self.alpha, branch=bd, y=y, workspace=b["ws"], stream=stream)

    def forward(self, x: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        self.quantize(x, stream)
        self.project(x, stream)
        return self.gemm(x.shape[0], x.device, out, stream)

    def replica(self) -> "QuantizedLinear":
        """A layer with the same configuration and its own device copies of the
        packed weights and branch operands (and its own buffers)."""
        r = copy.copy(self)
        r.w_codes, r.w_scales = self.w_codes.clone(), self.w_scales.clone()
        if self.branch is not None:
            r.branch = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in self.branch.items()}
        r._bufs = {}
        return r

    __call__ = forward

    def branch_operand(self, M: int, device):
        """The branch ``a`` operand inside the M-row buffers (after forward)."""
        b = self.buffers(M, device)
        if self.branch is None:
            return None
        r = self.branch["lw"].shape[1]
        return b["br_a"][:, :2 * r] if self.branch["kind"] == "lowrank" else b["br_a"]


def case_to_device(case, device="cuda"):
    """Upload a ``workloads.Case`` (numpy) as device tensors."""
    from .workloads import bf16_bits

    def bf16(a):
        return torch.from_numpy(bf16_bits(np.ascontiguousarray(a)).view(np.int16)).view(torch.bfloat16).to(device)

    t = {}
    t["x"] = bf16(case.x) if case.x_dtype == "bf16" else torch.from_numpy(case.x).to(device)
    t["w"] = torch.from_numpy(np.ascontiguousarray(case.w)).to(device)
    t["s"] = None if case.s is None else torch.from_numpy(case.s).to(device)
    t["inv_s"] = None if case.inv_s is None else torch.from_numpy(case.inv_s).to(device)
    br = None
    if case.branch is not None:
        br = {"kind": case.branch["kind"], "lw": bf16(case.branch["lw"])}
        if case.branch["kind"] == "lowrank":
            br["l1t"] = bf16(np.ascontiguousarray(case.branch["l1"].T))
        else:
            br["idx"] = torch.from_numpy(case.branch["idx"].astype(np.int32)).to(device)
    t["branch"] = br
    t["gptq"] = None
    if getattr(case, "gptq", None) is not None:
        t["gptq"] = {"u": torch.from_numpy(np.ascontiguousarray(case.gptq["u"])).to(device),
                     "perm": torch.from_numpy(case.gptq["perm"].astype(np.int32)).to(device)}
    return t


def build_layer(case, device="cuda", order="smooth_then_rotate", calibrate=True, use_workspace=True) -> tuple:
    """QuantizedLinear + device inputs for a ``workloads.Case``."""
    t = case_to_device(case, device)
    y_dtype = torch.float32 if case.y_dtype == "f32" else torch.bfloat16
    layer = QuantizedLinear(t["w"], t["s"], t["inv_s"], case.fmt, fwht_block=case.fwht_block, order=order,
                            branch=t["branch"], y_dtype=y_dtype, use_workspace=use_workspace, gptq=t["gptq"])
    if calibrate:
        layer.calibrate(t["x"])
    return layer, t
