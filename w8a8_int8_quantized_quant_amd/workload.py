"""Device-resident synthetic MoE layers for tests and benchmarks.

Draws a workload's inputs directly in HBM with the seeded generator (``synth``,
device fills bit-identical to its host fills) and quantizes the expert weights
with this library's own quantization entry point: one scale per output channel
(rows of each expert's [N, K] weight), or one per 128 x 128 block.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

import synth

from . import (SCALE_BLOCK128, SCALE_CHANNEL, SCALE_FP8_BLOCK128, SCALE_W4A8, SCORE_SIGMOID, SCORE_SOFTMAX,
               w8a8_fp8_quant_blocks, w8a8_moe_forward, w8a8_moe_workspace_bytes, w8a8_quant_blocks,
               w8a8_w4a8_quant_weights)


@dataclass
class DeviceLayer:
    cfg: synth.MoEConfig
    x: torch.Tensor            # [T, H] bf16 or fp32
    logits: torch.Tensor       # [T, E] fp32
    w13: torch.Tensor          # [E, 2I, H] int8 (uint8 FP8 codes for "fp8")
    w13_scale: torch.Tensor    # [E, 2I] or [E, 2I/128, H/128]
    w2: torch.Tensor           # [E, H, I] int8 (uint8 FP8 codes for "fp8")
    w2_scale: torch.Tensor     # [E, H] or [E, H/128, I/128]

    @property
    def scale_mode(self) -> int:
        return {"block": SCALE_BLOCK128, "fp8": SCALE_FP8_BLOCK128, "w4a8": SCALE_W4A8}.get(self.cfg.scale_mode,
                                                                                           SCALE_CHANNEL)

    @property
    def score_fn(self) -> int:
        return SCORE_SOFTMAX if self.cfg.route == "softmax" else SCORE_SIGMOID


def _quantize_experts(cfg, stream_tag: int, E: int, N: int, K: int, block: bool, device, chunk_bytes: int,
                      fp8: bool = False, w4: bool = False):
    """Draw [E, N, K] fp32 weights chunk by chunk and quantize them into int8 (FP8 codes, packed int4)
    + scales."""
    q = torch.empty((E, N, K // 2 if w4 else K), dtype=torch.uint8 if (fp8 or w4) else torch.int8, device=device)
    if w4:
        scale = torch.empty((E, N, K // 128), dtype=torch.float32, device=device)
    else:
        scale = torch.empty((E, N // 128, K // 128) if block else (E, N), dtype=torch.float32, device=device)
    per_expert = N * K
    chunk = max(1, min(E, chunk_bytes // (4 * per_expert)))
    scratch = torch.empty(chunk * per_expert, dtype=torch.float32, device=device)
    hs = torch.cuda.current_stream(device).cuda_stream
    for e0 in range(0, E, chunk):
        c = min(chunk, E - e0)
        buf = scratch[: c * per_expert]
        synth.dev_normal(buf.data_ptr(), c * per_expert, cfg.seed, stream_tag, e0 * per_expert, cfg.w_sigma, hs)
        mat = buf.view(c * N, K)
        if w4:
            w8a8_w4a8_quant_weights(mat, q[e0:e0 + c].view(c * N, K // 2), scale[e0:e0 + c].view(c * N, K // 128))
        elif fp8:
            w8a8_fp8_quant_blocks(mat, 128, 128, q[e0:e0 + c].view(c * N, K),
                                  scale[e0:e0 + c].view(c * N // 128, K // 128))
        elif block:
            w8a8_quant_blocks(mat, 128, 128, q[e0:e0 + c].view(c * N, K), scale[e0:e0 + c].view(c * N // 128, K // 128))
        else:
            w8a8_quant_blocks(mat, 1, K, q[e0:e0 + c].view(c * N, K), scale[e0:e0 + c].view(c * N, 1))
    del scratch
    return q, scale


def make_layer(cfg: synth.MoEConfig, device="cuda", T: Optional[int] = None,
               chunk_bytes: int = 2 << 30) -> DeviceLayer:
    """All inputs of one synthetic workload, resident on `device`."""
    T = cfg.T if T is None else T
    hs = torch.cuda.current_stream(device).cuda_stream
    xdt = torch.bfloat16 if cfg.x_dtype == synth.DTYPE_BF16 else torch.float32
    x = torch.empty((T, cfg.H), dtype=xdt, device=device)
    synth.dev_activations(x.data_ptr(), cfg, hs, T=T)
    logits = torch.empty((T, cfg.E), dtype=torch.float32, device=device)
    bias = synth.zipf_bias(cfg)
    bias_t = None if bias is None else torch.from_numpy(bias).to(device)
    synth.dev_logits(logits.data_ptr(), cfg, None if bias_t is None else bias_t.data_ptr(), hs, T=T)
    fp8, w4 = cfg.scale_mode == "fp8", cfg.scale_mode == "w4a8"
    block = cfg.scale_mode == "block" or fp8
    w13, w13_s = _quantize_experts(cfg, synth.STREAM_W13, cfg.E, 2 * cfg.I, cfg.H, block, device, chunk_bytes, fp8,
                                   w4)
    w2, w2_s = _quantize_experts(cfg, synth.STREAM_W2, cfg.E, cfg.H, cfg.I, block, device, chunk_bytes, fp8, w4)
    torch.cuda.synchronize(device)
    return DeviceLayer(cfg, x, logits, w13, w13_s, w2, w2_s)


def forward_workspace(layer: DeviceLayer, block_m: int = 0) -> torch.Tensor:
    c = layer.cfg
    nbytes = w8a8_moe_workspace_bytes(layer.x.shape[0], c.k, c.E, c.H, c.I, block_m, layer.scale_mode)
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=layer.x.device)


def forward(layer: DeviceLayer, out: torch.Tensor, ws: torch.Tensor, block_m: int = 0, topk_ids=None,
            topk_weights=None, stream=None) -> None:
    """One pass of the whole layer (route, quantize, align, both grouped GEMMs, combine)."""
    c = layer.cfg
    w8a8_moe_forward(layer.x, layer.logits, layer.w13, layer.w13_scale, layer.w2, layer.w2_scale, out, ws, k=c.k,
                     score_fn=layer.score_fn, n_group=c.n_group, topk_group=c.topk_group,
                     renormalize=c.renormalize, routed_scaling=c.routed_scaling, scale_mode=layer.scale_mode,
                     block_m=block_m, topk_ids=topk_ids, topk_weights=topk_weights, stream=stream)
