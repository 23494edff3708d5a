"""Seeded synthetic inputs for the W8A8 INT8 fused-MoE layer.

This module is shared by the CPU oracle side and the GPU side and holds none
of the method's arithmetic: it only draws inputs (activations, gate logits,
unquantized fp32 expert weights) from the counter-based generator defined in
``synth_core.h``.  Host fills (``libsynth_host.so``, gcc) and device fills
(``libsynth_dev.so``, hipcc) are bit-identical, so a test can draw a tensor on
the GPU and the same tensor, or any slice of it, on the CPU.

Workloads.  The pages measure a whole DeepSeek-R1 model under SGLang on A100s
(PR #3888 "Performance" and "Reproduce" sections; the jiqizhixin article,
"INT8 quantized model inference throughput" section).  Those runs need trained
weights and datasets, so the five configurations below stand in for them with
synthetic tensors of the DeepSeek-V3 MoE layer's shapes (hidden 7168, expert
intermediate 2048, 256 routed experts, top-8, 8 groups / top-4 groups,
routed scaling 2.5) plus one tiny case.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))

STREAM_X = 1
STREAM_X_OUTLIER = 2
STREAM_LOGITS = 3
STREAM_W13 = 4
STREAM_W2 = 5
STREAM_PERM = 6
STREAM_MISC = 7

DTYPE_F32 = 0
DTYPE_BF16 = 1

OUTLIER_THRESHOLD = 42949672  # floor(0.01 * 2**32): 1% of elements


@dataclass(frozen=True)
class MoEConfig:
    """One synthetic workload (shapes, routing rule and value distributions)."""

    name: str
    index: int
    T: int
    H: int
    I: int
    E: int
    k: int
    route: str  # "softmax" or "sigmoid"
    n_group: int
    topk_group: int
    routed_scaling: float
    renormalize: bool
    x_dtype: int
    x_sigma: float
    outlier_threshold: int
    outlier_mult: float
    w_sigma: float
    scale_mode: str  # "channel", "block" (INT8, 128x128), "fp8" (E4M3, 128x128) or "w4a8" (int4, FP8 acts)
    zipf_s: Optional[float] = None
    zipf_beta: Optional[float] = None
    note: str = field(default="", compare=False)

    @property
    def seed(self) -> int:
        return self.index + 1

    @property
    def P(self) -> int:
        return self.T * self.k


_DSV3 = dict(H=7168, I=2048, E=256, k=8, route="sigmoid", n_group=8, topk_group=4,
             routed_scaling=2.5, renormalize=True, x_dtype=DTYPE_BF16, x_sigma=1.0,
             outlier_threshold=OUTLIER_THRESHOLD, outlier_mult=20.0, w_sigma=0.006)

CONFIGS = {
    "tiny": MoEConfig(
        name="tiny", index=0, T=16, H=256, I=128, E=8, k=2, route="softmax", n_group=1,
        topk_group=1, routed_scaling=1.0, renormalize=True, x_dtype=DTYPE_F32, x_sigma=1.0,
        outlier_threshold=0, outlier_mult=1.0, w_sigma=0.02, scale_mode="channel",
        note="T=16, hidden 256, intermediate 128, 8 experts, softmax top-2"),
    "decode": MoEConfig(name="decode", index=1, T=128, scale_mode="channel",
                        note="DeepSeek-V3 MoE layer, decode batch T=128", **_DSV3),
    "prefill": MoEConfig(name="prefill", index=2, T=8192, scale_mode="channel",
                         note="DeepSeek-V3 MoE layer, prefill batch T=8192", **_DSV3),
    # zipf_beta is calibrated by oracle/calibrate_zipf.py so that the 8 most
    # popular experts take ~40% of the 32768 assignments.
    "skew": MoEConfig(name="skew", index=3, T=4096, scale_mode="channel", zipf_s=1.2,
                      zipf_beta=0.580934, note="DeepSeek-V3 shapes, Zipf(1.2)-skewed expert load, T=4096",
                      **_DSV3),
    # The same seeded logits with a stronger bias, calibrated (oracle/calibrate_zipf.py) so that at
    # least 30 of the 256 experts receive no assignment: empty experts, their zero tiles and
    # offsets at the DeepSeek-V3 shapes.
    "skew-empty": MoEConfig(name="skew-empty", index=3, T=4096, scale_mode="channel", zipf_s=1.2,
                            zipf_beta=0.774107, note="DeepSeek-V3 shapes, Zipf(1.2)-skewed expert load with ~30 "
                                                 "empty experts, T=4096", **_DSV3),
    "block": MoEConfig(name="block", index=4, T=2048, scale_mode="block",
                       note="DeepSeek-V3 shapes, 128x128 block-wise INT8, T=2048", **_DSV3),
}

CONFIG_ORDER = ["tiny", "decode", "prefill", "skew", "skew-empty", "block"]


# --------------------------------------------------------------------------- libraries

_host = None
_dev = None


def _load_host():
    global _host
    if _host is None:
        path = os.path.join(_HERE, "libsynth_host.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        lib = ctypes.CDLL(path)
        i64, u64, u32, f32, vp = (ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32,
                                  ctypes.c_float, ctypes.c_void_p)
        lib.synth_fill_normal_f32.argtypes = [vp, i64, u64, u64, i64, f32]
        lib.synth_fill_logits_f32.argtypes = [vp, i64, i64, u64, vp, i64]
        lib.synth_fill_activation.argtypes = [vp, ctypes.c_int32, i64, i64, u64, f32, u32, f32, i64]
        lib.synth_permutation.argtypes = [vp, i64, u64]
        lib.synth_words.argtypes = [vp, i64, u64, u64, i64]
        lib.synth_splitmix64.argtypes = [vp, i64, u64]
        lib.synth_splitmix64.restype = None
        for fn in (lib.synth_fill_normal_f32, lib.synth_fill_logits_f32, lib.synth_fill_activation,
                   lib.synth_permutation, lib.synth_words):
            fn.restype = None
        _host = lib
    return _host


def _load_dev():
    global _dev
    if _dev is None:
        path = os.path.join(_HERE, "libsynth_dev.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        lib = ctypes.CDLL(path)
        i64, u64, u32, f32, vp = (ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32,
                                  ctypes.c_float, ctypes.c_void_p)
        lib.synth_dev_fill_normal_f32.argtypes = [vp, i64, u64, u64, i64, f32, vp]
        lib.synth_dev_fill_logits_f32.argtypes = [vp, i64, i64, u64, vp, i64, vp]
        lib.synth_dev_fill_activation.argtypes = [vp, ctypes.c_int32, i64, i64, u64, f32, u32, f32,
                                                  i64, vp]
        for fn in (lib.synth_dev_fill_normal_f32, lib.synth_dev_fill_logits_f32,
                   lib.synth_dev_fill_activation):
            fn.restype = ctypes.c_int
        _dev = lib
    return _dev


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# --------------------------------------------------------------------------- host draws

def words(n: int, seed: int, stream: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load_host().synth_words(_ptr(out), n, seed, stream, start)
    return out


def splitmix64(n: int, state: int) -> np.ndarray:
    """The raw SplitMix64 sequence from a given state (generator self-check)."""
    out = np.empty(n, dtype=np.uint64)
    _load_host().synth_splitmix64(_ptr(out), n, state)
    return out


def normal(n: int, seed: int, stream: int, start: int = 0, sigma: float = 1.0) -> np.ndarray:
    """sigma * N(0,1) draws start .. start+n-1 of one stream (fp32)."""
    out = np.empty(n, dtype=np.float32)
    _load_host().synth_fill_normal_f32(_ptr(out), n, seed, stream, start, sigma)
    return out


def permutation(n: int, seed: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load_host().synth_permutation(_ptr(out), n, seed)
    return out


def zipf_bias(cfg: MoEConfig, beta: Optional[float] = None) -> Optional[np.ndarray]:
    """Per-expert logit bias beta * (-s * ln rank_e); ranks 1..E from a seeded permutation."""
    if cfg.zipf_s is None:
        return None
    beta = cfg.zipf_beta if beta is None else beta
    perm = permutation(cfg.E, cfg.seed)
    bias = np.empty(cfg.E, dtype=np.float64)
    for r in range(cfg.E):
        bias[perm[r]] = beta * (-cfg.zipf_s * math.log(r + 1))
    return bias.astype(np.float32)


def logits(cfg: MoEConfig, rows: Optional[slice] = None, beta: Optional[float] = None) -> np.ndarray:
    """Gate logits [T, E] fp32: N(0,1), plus the Zipf bias for the skewed workload."""
    r0, r1 = (0, cfg.T) if rows is None else (rows.start, rows.stop)
    bias = zipf_bias(cfg, beta)
    out = np.empty((r1 - r0, cfg.E), dtype=np.float32)
    _load_host().synth_fill_logits_f32(_ptr(out), r1 - r0, cfg.E, cfg.seed,
                                       None if bias is None else _ptr(bias), r0)
    return out


def activations(cfg: MoEConfig, rows: Optional[slice] = None) -> np.ndarray:
    """Activations [T, H]: fp32 array, or uint16 bf16 bits for bf16 workloads."""
    r0, r1 = (0, cfg.T) if rows is None else (rows.start, rows.stop)
    dt = np.uint16 if cfg.x_dtype == DTYPE_BF16 else np.float32
    out = np.empty((r1 - r0, cfg.H), dtype=dt)
    _load_host().synth_fill_activation(_ptr(out), cfg.x_dtype, r1 - r0, cfg.H, cfg.seed, cfg.x_sigma,
                                       cfg.outlier_threshold, cfg.outlier_mult, r0)
    return out


def w13_f32(cfg: MoEConfig, expert: int) -> np.ndarray:
    """Unquantized gate+up weights of one expert, [2I, H] fp32 (rows [0,I) gate, [I,2I) up)."""
    n = 2 * cfg.I * cfg.H
    return normal(n, cfg.seed, STREAM_W13, expert * n, cfg.w_sigma).reshape(2 * cfg.I, cfg.H)


def w2_f32(cfg: MoEConfig, expert: int) -> np.ndarray:
    """Unquantized down weights of one expert, [H, I] fp32."""
    n = cfg.H * cfg.I
    return normal(n, cfg.seed, STREAM_W2, expert * n, cfg.w_sigma).reshape(cfg.H, cfg.I)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------- device draws

def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed with status {rc}")


def dev_normal(out_ptr: int, n: int, seed: int, stream: int, start: int, sigma: float, hip_stream: int):
    _check(_load_dev().synth_dev_fill_normal_f32(out_ptr, n, seed, stream, start, sigma, hip_stream),
           "synth_dev_fill_normal_f32")


def dev_logits(out_ptr: int, cfg: MoEConfig, bias_ptr: Optional[int], hip_stream: int, T: Optional[int] = None,
               row_start: int = 0):
    T = cfg.T if T is None else T
    _check(_load_dev().synth_dev_fill_logits_f32(out_ptr, T, cfg.E, cfg.seed, bias_ptr, row_start,
                                                 hip_stream), "synth_dev_fill_logits_f32")


def dev_activations(out_ptr: int, cfg: MoEConfig, hip_stream: int, T: Optional[int] = None, row_start: int = 0):
    T = cfg.T if T is None else T
    _check(_load_dev().synth_dev_fill_activation(out_ptr, cfg.x_dtype, T, cfg.H, cfg.seed, cfg.x_sigma,
                                                 cfg.outlier_threshold, cfg.outlier_mult, row_start,
                                                 hip_stream), "synth_dev_fill_activation")


def int8_matrix(rows: int, cols: int, seed: int, start: int = 0) -> np.ndarray:
    """Uniform int8 in [-127, 127] (for raw GEMM inputs), from the MISC stream."""
    w = words(rows * cols, seed, STREAM_MISC, start)
    return ((w % np.uint64(255)).astype(np.int16) - 127).astype(np.int8).reshape(rows, cols)


def positive_scales(n: int, seed: int, lo: float, hi: float, start: int = 0) -> np.ndarray:
    """Uniform fp32 scales in [lo, hi) (for raw GEMM inputs), from the MISC stream."""
    w = words(n, seed + 7919, STREAM_MISC, start)
    u = (w >> np.uint64(40)).astype(np.float64) / float(1 << 24)
    return (lo + (hi - lo) * u).astype(np.float32)
