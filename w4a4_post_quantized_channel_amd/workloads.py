"""Seeded synthetic inputs for the W4A4 quantized-linear path.

This module only *draws and shapes data*: it holds none of the quantized
path's arithmetic (no rotation, no quantizer, no GEMM).  Both the HIP path
and the CPU oracle take their inputs from here and from nowhere else.

What it builds, per workload (all NumPy, PCG64 ``default_rng(seed)``):

* ``x``   activations, M x K, fp32 values (bf16-representable for bf16 cases);
* ``w``   the weight matrix that the quantized path consumes, N x K;
* ``s`` / ``inv_s``  per-channel smoothing factors (calibration data, the
  SmoothQuant-style migration the QuantWAMs page names in its related-work
  section and applies as the diagonal S of its runtime-quantizer equation,
  Eq. 1).  The pages give no formula; the workload recipe uses
  s_j = sqrt(amax_x(j) / amax_w(j)) evaluated in float64;
* an optional 16-bit branch: a rank-r factor pair (Q-WAM abstract,
  "Action-Subspace Protection") or a set of kept outlier channels
  (QuantWAMs sec. 3.1 top-K mask, sec. 4.2 BF16 exception path).

Shapes and value laws follow the five workload descriptions (tiny
16x256x256 case, batch-1 64-token action-expert step, 512-token backbone
prefill, 1024-token low-rank-protected linear, 4096-token video-latent
projection).  The pages measure on robot benchmarks and model checkpoints
that are not available; these seeded draws stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "Case", "linear_case", "workload", "WORKLOADS", "bf16_round", "bf16_bits",
    "from_bf16_bits",
]


# ----------------------------------------------------------------------------
# bf16 storage helpers (a storage format, not part of the method)
# ----------------------------------------------------------------------------
def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even.  Finite input only."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32 values (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value (kept as fp32)."""
    return from_bf16_bits(bf16_bits(a))


# ----------------------------------------------------------------------------
# A single linear-layer case
# ----------------------------------------------------------------------------
@dataclass
class Case:
    name: str
    M: int
    N: int
    K: int
    fmt: str                 # "int4" | "int8" | "nvfp4" | "w4a8" (int8 x, int4 w) | "fp8"
    x_dtype: str             # "bf16" | "f32"
    y_dtype: str             # "bf16" | "f32"
    x: np.ndarray            # M x K fp32 values
    w: np.ndarray            # N x K fp32 (matrix the quantized path consumes)
    s: Optional[np.ndarray]  # K fp32 smoothing (weights are multiplied by s)
    inv_s: Optional[np.ndarray]  # K fp32, fp32(1/s) (activations multiplied)
    fwht_block: int = 64
    branch: Optional[dict] = None   # {"kind": "lowrank", "l1": KxR, "lw": NxR}
                                    # {"kind": "outlier", "idx": int32[R], "lw": NxR}
    w_full: Optional[np.ndarray] = None  # float weight the whole layer approximates
    meta: dict = field(default_factory=dict)
    gptq: Optional[dict] = None   # {"u": K x K float64 upper factor, "perm": int32[K], "sigma": K x K}

    @property
    def x_bits(self) -> np.ndarray:
        assert self.x_dtype == "bf16"
        return bf16_bits(self.x)


def gptq_calibration(K: int, seed: int, rows: int = 256, damp: float = 0.01) -> dict:
    """Synthetic GPTQ calibration in the quantizer's (transformed) space.

    Sigma = A^T A / rows for A = Z (I + 0.3 G / sqrt(K)) D with Z, G standard
    normal and D a log-normal per-channel gain (sigma 0.5): correlated
    channels of unequal energy, standing in for the layer's activation
    second moments.  Processing order: diag(Sigma) descending (stable).
    u is the upper Cholesky factor of (Sigma_pp + damp * mean(diag) * I)^-1,
    Sigma_pp being Sigma in that order, so that the inverse equals u^T u.
    All float64."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((rows, K))
    g = rng.standard_normal((K, K))
    d = rng.lognormal(0.0, 0.5, size=K)
    a = (z @ (np.eye(K) + 0.3 * g / np.sqrt(K))) * d[None, :]
    sigma = a.T @ a / rows
    perm = np.argsort(-np.diag(sigma), kind="stable").astype(np.int32)
    sp = sigma[np.ix_(perm, perm)]
    sp = sp + damp * np.mean(np.diag(sp)) * np.eye(K)
    lower = np.linalg.cholesky(np.linalg.inv(sp))
    return {"u": np.ascontiguousarray(lower.T), "perm": perm, "sigma": sigma}


def _outliers(rng, K, n):
    if n <= 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(rng.choice(K, size=n, replace=False))


def smoothing_factors(x: np.ndarray, w: np.ndarray, zero_channels=None):
    """Calibration recipe s_j = sqrt(amax_x(j)/amax_w(j)) in float64.

    s = 1 where either absolute maximum is zero.  Channels listed in
    ``zero_channels`` (kept in 16 bit elsewhere) get s = inv_s = 0 so that
    the quantized path carries nothing for them.  inv_s = fp32(1/fp32(s)).
    """
    ax = np.abs(x.astype(np.float64)).max(axis=0)
    aw = np.abs(w.astype(np.float64)).max(axis=0)
    ok = (ax > 0) & (aw > 0)
    s64 = np.ones_like(ax)
    s64[ok] = np.sqrt(ax[ok] / aw[ok])
    s = s64.astype(np.float32)
    inv_s = (np.float32(1.0) / s).astype(np.float32)
    if zero_channels is not None and len(zero_channels):
        s[zero_channels] = 0.0
        inv_s[zero_channels] = 0.0
    return s, inv_s


def linear_case(M: int, N: int, K: int, *, seed: int, fmt: str = "int4",
                x_dtype: str = "bf16", y_dtype: Optional[str] = None,
                n_outliers: int = 0, outlier_gain: float = 1.0,
                row_gain_sigma: float = 0.0, w_std: float = 0.02,
                smooth: bool = True, fwht_block: int = 64,
                lowrank: int = 0, lowrank_std: float = 0.05,
                keep_channels: int = 0, name: str = "case",
                x_override: Optional[np.ndarray] = None, gptq: bool = False) -> Case:
    """Draw one seeded linear case.

    Draw order (fixed): X, outlier channel indices, per-row gains, W, U, V, R0.
    ``keep_channels`` > 0 selects the top-energy raw channels of X (sum of
    squares in float64, ties to the lower index) for the bf16 outlier branch.
    ``lowrank`` > 0 builds W = U V^T + R0 and keeps the bf16 rank-r factors as
    the branch, quantizing the residual W - L1 L2.  ``gptq`` attaches the
    synthetic GPTQ calibration of ``gptq_calibration(K, seed + 7)``.
    """
    if y_dtype is None:
        y_dtype = "f32" if x_dtype == "f32" else "bf16"
    rng = np.random.default_rng(seed)
    if x_override is None:
        x = rng.standard_normal((M, K), dtype=np.float32)
    else:
        x = np.array(x_override, dtype=np.float32)
        assert x.shape == (M, K)
    idx = _outliers(rng, K, n_outliers)
    if row_gain_sigma > 0:
        g = rng.lognormal(mean=0.0, sigma=row_gain_sigma, size=(M, 1)).astype(np.float32)
        x = x * g
    if len(idx):
        x[:, idx] *= np.float32(outlier_gain)
    if x_dtype == "bf16":
        x = bf16_round(x)
    else:
        x = x.astype(np.float32)

    branch = None
    if lowrank > 0:
        u = (rng.standard_normal((N, lowrank)) * lowrank_std).astype(np.float32)
        v = (rng.standard_normal((K, lowrank)) * lowrank_std).astype(np.float32)
        r0 = (rng.standard_normal((N, K)) * w_std).astype(np.float32)
        w_full = (u.astype(np.float64) @ v.astype(np.float64).T + r0).astype(np.float32)
        l1 = bf16_round(v)          # K x r
        lw = bf16_round(u)          # N x r  (= L2 transposed)
        w = (w_full.astype(np.float64) - lw.astype(np.float64) @ l1.astype(np.float64).T
             ).astype(np.float32)
        branch = {"kind": "lowrank", "l1": l1, "lw": lw}
    else:
        w_full = (rng.standard_normal((N, K)) * w_std).astype(np.float32)
        w = w_full

    zero = None
    if keep_channels > 0:
        energy = np.square(x.astype(np.float64)).sum(axis=0)
        order = np.argsort(-energy, kind="stable")
        keep = np.sort(order[:keep_channels]).astype(np.int32)
        lw = bf16_round(w_full[:, keep])      # N x r, bf16 values
        branch = {"kind": "outlier", "idx": keep, "lw": lw}
        zero = keep

    if smooth:
        s, inv_s = smoothing_factors(x, w, zero)
    elif zero is not None:
        s = np.ones(K, np.float32); inv_s = np.ones(K, np.float32)
        s[zero] = 0; inv_s[zero] = 0
    else:
        s = inv_s = None
    return Case(name=name, M=M, N=N, K=K, fmt=fmt, x_dtype=x_dtype, y_dtype=y_dtype,
                x=x, w=w, s=s, inv_s=inv_s, fwht_block=fwht_block, branch=branch,
                w_full=w_full, meta={"seed": seed, "outliers": idx},
                gptq=gptq_calibration(K, seed + 7) if gptq else None)


def _silu(v):
    return v / (1.0 + np.exp(-v))


def workload(name: str) -> Case:
    """The named workloads at their full sizes."""
    if name == "tiny":          # 16x256x256, fp32 X, int4, smoothing + FWHT-64, seed 0
        return linear_case(16, 256, 256, seed=0, fmt="int4", x_dtype="f32",
                           n_outliers=4, outlier_gain=20.0, name=name)
    if name == "decode_w4a4":   # batch-1 action-expert step, projection (a)
        return linear_case(64, 2048, 2048, seed=1, fmt="int4", n_outliers=16,
                           outlier_gain=15.0, name=name)
    if name == "decode_w8a8":   # batch-1 action-expert step, down projection (b)
        return linear_case(64, 2048, 8192, seed=101, fmt="int8", n_outliers=16,
                           outlier_gain=15.0, name=name)
    if name == "prefill_gate_up":
        return linear_case(512, 16384, 2048, seed=2, fmt="int4", n_outliers=32,
                           outlier_gain=20.0, row_gain_sigma=0.5, name=name)
    if name == "prefill_down":
        # Down-projection input: SwiGLU of the float gate/up projection of the
        # prefill activations (rows 0..8191 gate, 8192..16383 up), rounded to bf16.
        gu = workload("prefill_gate_up")
        h = gu.x.astype(np.float32) @ gu.w_full.T.astype(np.float32)
        x2 = bf16_round((_silu(h[:, :8192].astype(np.float64)) * h[:, 8192:]).astype(np.float32))
        return linear_case(512, 2048, 8192, seed=202, fmt="int4", x_override=x2,
                           name=name)
    if name == "lowrank":
        return linear_case(1024, 3072, 3072, seed=3, fmt="int4", n_outliers=48,
                           outlier_gain=25.0, lowrank=32, name=name)
    if name == "video_nvfp4":
        return linear_case(4096, 5120, 5120, seed=4, fmt="nvfp4", n_outliers=64,
                           outlier_gain=30.0, keep_channels=64, name=name)
    # W4A8: the 8-bit-activation denoising steps (QuantWAMs, Experimental
    # Details, quantization configuration; sec. 4.4.3) on the same shapes
    if name == "decode_w4a8":   # protected batch-1 action step, projection (a)
        return linear_case(64, 2048, 2048, seed=11, fmt="w4a8", n_outliers=16,
                           outlier_gain=15.0, name=name)
    if name == "decode_w4a8_down":   # protected batch-1 action step, 4-bit-weight down projection
        return linear_case(64, 2048, 8192, seed=111, fmt="w4a8", n_outliers=16,
                           outlier_gain=15.0, name=name)
    if name == "video_w4a8":    # protected video-denoising step, integer codes
        return linear_case(4096, 5120, 5120, seed=44, fmt="w4a8", n_outliers=64,
                           outlier_gain=30.0, keep_channels=64, name=name)
    # FP8 W8A8 for upgraded layers (QuantWAMs sec. 4.2), on the shapes of
    # the batch-1 down projection and the video projection
    if name == "decode_fp8":
        return linear_case(64, 2048, 8192, seed=121, fmt="fp8", n_outliers=16,
                           outlier_gain=15.0, name=name)
    if name == "video_fp8":
        return linear_case(4096, 5120, 5120, seed=45, fmt="fp8", n_outliers=64,
                           outlier_gain=30.0, keep_channels=64, name=name)
    raise KeyError(name)


WORKLOADS = ["tiny", "decode_w4a4", "decode_w8a8", "prefill_gate_up", "prefill_down",
             "lowrank", "video_nvfp4", "decode_w4a8", "decode_w4a8_down", "video_w4a8",
             "decode_fp8", "video_fp8"]
