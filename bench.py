"""Benchmark of the W8A8 INT8 fused-MoE layer on one MI355X.

One step = one pass of the whole layer over one batch of synthetic input:
top-k routing, per-token activation quantization, align by expert, the grouped
INT8 gate+up GEMM with SiLU and requantization, the grouped INT8 down GEMM with
the top-k weighted combine.  Inputs (activations, gate logits, int8 expert
weights and scales) are resident in HBM before timing starts.

Prints one JSON line.  value = tokens/s of the DeepSeek-V3 decode layer
(T=128, hidden 7168, intermediate 2048, 256 experts, top-8); the same line
carries the T=8192 prefill layer's figures under "prefill", the tiny (T=16), skewed
(T=4096), block-wise (T=2048, INT8 and FP8) layers and the FP8 / W4A8 variants of the decode
and block-wise workloads under "configs", the dense W8A8 linear
under "linear", the roofline of the
dominant kernel (the gate+up GEMM, weight-streaming and so HBM-bound at T=128),
the device's measured read / copy / INT8-MFMA rates under "peaks_measured", and
the CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + int8 TOPS at T=128/8192; % of INT8 MFMA or HBM peak"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0    # MI355X dense INT8 MFMA
FP8_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="decode",
                    help="decode (the headline), prefill, tiny, skew, skew-empty, block, fp8-block, fp8-decode, "
                         "w4a8-decode or w4a8-block")
    ap.add_argument("--no-prefill", action="store_true", help="skip the T=8192 prefill figures")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=128, help="tokens in the CPU oracle sample")
    ap.add_argument("--no-configs", action="store_true", help="skip the tiny / skew / block workloads")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak probes")
    ap.add_argument("--linear-only", action="store_true",
                    help="only time the dense W8A8 linear shapes and print their figures (profiling)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy kernel 3 times (counter calibration)")
    return ap.parse_args()


def copy_probe():
    """A plain copy of known size: 1 GiB read + 1 GiB written per launch, for scaling HBM counters."""
    import torch

    a = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": a.numel() * 4, "copy_probe_bytes_written": b.numel() * 4}))


class Stages:
    """Device buffers and the stage-by-stage calls of one layer pass (all on torch's current stream)."""

    def __init__(self, layer, block_m=0):
        import torch

        import w8a8_int8_quantized_quant_amd as w8

        self.w8 = w8
        self.L = layer
        c = layer.cfg
        T = layer.x.shape[0]
        self.T = T
        self.w4 = c.scale_mode == "w4a8"
        self.fp8 = c.scale_mode == "fp8" or self.w4  # FP8 activations and intermediate
        self.block = c.scale_mode == "block" or self.fp8
        self.bm = block_m or w8.w8a8_moe_pick_block_m(T, c.k, c.E)
        dev = layer.x.device
        R = w8.w8a8_moe_max_rows(T, c.k, c.E, self.bm)
        i32, f32 = torch.int32, torch.float32
        self.ids = torch.empty((T, c.k), dtype=i32, device=dev)
        self.tw = torch.empty((T, c.k), dtype=f32, device=dev)
        code = torch.uint8 if self.fp8 else torch.int8
        self.a_q = torch.empty((T, c.H), dtype=code, device=dev)
        self.a_s = torch.empty((T, c.H // 128) if self.block else (T,), dtype=f32, device=dev)
        self.counts = torch.empty(c.E, dtype=i32, device=dev)
        self.offsets = torch.empty(c.E + 1, dtype=i32, device=dev)
        self.padded = torch.empty(c.E + 1, dtype=i32, device=dev)
        self.sorted = torch.empty(max(R, 1), dtype=i32, device=dev)
        self.tile_expert = torch.empty(max(R // self.bm, 1), dtype=i32, device=dev)
        self.num_tiles = torch.empty(1, dtype=i32, device=dev)
        self.h_q = torch.empty((max(R, 1), c.I), dtype=code, device=dev)
        self.h_s = torch.empty((max(R, 1), c.I // 128) if self.block else (max(R, 1),), dtype=f32, device=dev)
        self.out = torch.empty((T, c.H), dtype=f32, device=dev)
        mode = (w8.SCALE_W4A8 if self.w4 else w8.SCALE_FP8_BLOCK128 if self.fp8 else w8.SCALE_BLOCK128 if self.block
                else w8.SCALE_CHANNEL)
        self.ws_align = torch.empty(max(w8.moe_align_workspace_bytes(T, c.k, c.E), 256), dtype=torch.uint8, device=dev)
        gws = max(w8.w8a8_w13_workspace_bytes(T, c.k, c.E, c.H, c.I, self.bm, mode),
                  w8.w8a8_w2_workspace_bytes(T, c.k, c.E, c.H, c.I, self.bm, mode))
        self.ws_gemm = torch.empty(gws, dtype=torch.uint8, device=dev)

    def route(self):
        c = self.L.cfg
        self.w8.moe_topk_route(self.L.logits, c.k, self.L.score_fn, c.n_group, c.topk_group, c.renormalize,
                               c.routed_scaling, None, self.ids, self.tw)

    def quant(self):
        if self.fp8:
            self.w8.w8a8_fp8_quant_blocks(self.L.x, 1, 128, self.a_q, self.a_s)
        else:
            self.w8.w8a8_quant_per_token(self.L.x, 128 if self.block else 0, self.a_q, self.a_s)

    def align(self):
        self.w8.moe_align_by_expert(self.ids, self.L.cfg.E, self.bm, self.counts, self.offsets, self.padded,
                                    self.sorted, self.tile_expert, self.num_tiles, self.ws_align)

    def w13(self):
        fn = (self.w8.w8a8_w4a8_grouped_gemm_w13_silu if self.w4 else self.w8.w8a8_fp8_grouped_gemm_w13_silu
              if self.fp8 else self.w8.w8a8_block_grouped_gemm_w13_silu if self.block
              else self.w8.w8a8_grouped_gemm_w13_silu)
        fn(self.a_q, self.a_s, self.L.w13, self.L.w13_scale, self.sorted, self.padded, self.tile_expert,
           self.num_tiles, self.T, self.L.cfg.k, self.bm, self.h_q, self.h_s, self.ws_gemm)

    def w2(self):
        fn = (self.w8.w8a8_w4a8_grouped_gemm_w2_combine if self.w4 else self.w8.w8a8_fp8_grouped_gemm_w2_combine
              if self.fp8 else self.w8.w8a8_block_grouped_gemm_w2_combine if self.block
              else self.w8.w8a8_grouped_gemm_w2_combine)
        fn(self.h_q, self.h_s, self.L.w2, self.L.w2_scale, self.sorted, self.padded, self.tile_expert,
           self.num_tiles, self.tw, self.T, self.L.cfg.k, self.bm, self.out, self.ws_gemm)

    NAMES = ("route", "quant", "align", "w13", "w2")

    def step(self, events=None):
        for i, name in enumerate(self.NAMES):
            if events is not None:
                events[i].record()
            getattr(self, name)()
        if events is not None:
            events[len(self.NAMES)].record()


VARIANTS = {  # name: (workload it re-quantizes, scale mode, description)
    "fp8-block": ("block", "fp8", "DeepSeek-V3 shapes, 128x128 block-wise FP8 (E4M3), T=2048"),
    "fp8-decode": ("decode", "fp8", "DeepSeek-V3 MoE layer, decode batch T=128, 128x128 block-wise FP8 (E4M3)"),
    "w4a8-decode": ("decode", "w4a8", "DeepSeek-V3 MoE layer, decode batch T=128, W4A8 (int4 weights, FP8 "
                                      "activations)"),
    "w4a8-block": ("block", "w4a8", "DeepSeek-V3 shapes, W4A8 (int4 weights, FP8 activations), T=2048"),
}


def config_of(name):
    """A workload by name: the five base workloads, or a variant that re-quantizes one of them
    (same shapes, same draws) in FP8 or W4A8."""
    import dataclasses

    import synth

    if name in VARIANTS:
        base, mode, note = VARIANTS[name]
        return dataclasses.replace(synth.CONFIGS[base], name=name, scale_mode=mode, note=note)
    return synth.CONFIGS[name]


def measure_graph(st, steps, warmup):
    """The same step captured once into a HIP graph (the five stages' kernels, no host work) and
    replayed: wall time per replay, synchronised on both sides."""
    import torch

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        st.step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        st.step()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    del g
    return (t1 - t0) * 1000.0 / steps


def measure(layer, steps, warmup):
    """Whole-step wall time (synchronised on both sides) and per-stage event times."""
    import torch

    st = Stages(layer)
    for _ in range(warmup):
        st.step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(Stages.NAMES) + 1)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        st.step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stage_ms = {name: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps for j, name in enumerate(Stages.NAMES)}
    counts = st.counts.cpu().numpy()
    return (t1 - t0) * 1000.0 / steps, stage_ms, st, counts


def layer_figures(cfg, T, ms, counts):
    P = T * cfg.k
    ops = 2.0 * P * (2 * cfg.I * cfg.H + cfg.H * cfg.I)
    active = int((counts > 0).sum())
    w4 = cfg.scale_mode == "w4a8"
    blk = cfg.scale_mode in ("block", "fp8", "w4a8")
    nsh = cfg.I // 128 if blk else 1
    nsw13 = (2 * cfg.I * (cfg.H // 128) if w4 else (2 * cfg.I // 128) * (cfg.H // 128)) if blk else 2 * cfg.I
    nsw2 = (cfg.H * (cfg.I // 128) if w4 else (cfg.H // 128) * (cfg.I // 128)) if blk else cfg.H
    nsa = cfg.H // 128 if blk else 1
    wdiv = 2 if w4 else 1  # int4: two weights per byte
    w_bytes = active * ((2 * cfg.I * cfg.H + cfg.H * cfg.I) // wdiv + 4 * (nsw13 + nsw2))
    x_bytes = T * cfg.H * (2 if cfg.x_dtype else 4)
    other = (T * cfg.E * 4 + x_bytes + 2 * (T * cfg.H + 4 * T * nsa) + 2 * (P * cfg.I + 4 * P * nsh)
             + T * cfg.H * 4 + P * 8)
    total_bytes = w_bytes + other
    return dict(tokens_per_s=T / (ms / 1000.0), ms_per_step=ms, int8_tops=ops / (ms / 1000.0) / 1e12,
                frac_int8_peak=ops / (ms / 1000.0) / 1e12 / INT8_PEAK_TOPS, hbm_gbs=total_bytes / (ms / 1000.0) / 1e9,
                frac_hbm_peak=total_bytes / (ms / 1000.0) / 1e9 / HBM_PEAK_GBS, active_experts=active,
                algorithmic_bytes=total_bytes, algorithmic_ops=ops)


def w13_algorithmic_bytes(cfg, T, counts):
    """Bytes the gate+up GEMM stage must move: int8 weights and scales of the active experts,
    the int8 token rows and their scales, and the int8 intermediate with its scales."""
    P = T * cfg.k
    active = int((counts > 0).sum())
    w4 = cfg.scale_mode == "w4a8"
    blk = cfg.scale_mode in ("block", "fp8", "w4a8")
    nsw = (2 * cfg.I * (cfg.H // 128) if w4 else (2 * cfg.I // 128) * (cfg.H // 128)) if blk else 2 * cfg.I
    nsa = cfg.H // 128 if blk else 1
    nsh = cfg.I // 128 if blk else 1
    return active * (2 * cfg.I * cfg.H // (2 if w4 else 1) + 4 * nsw) + T * (cfg.H + 4 * nsa) + P * (cfg.I + 4 * nsh)


def w13_algorithmic_ops(cfg, T):
    """INT8 multiply-add operations of the gate+up GEMM on the real (token, expert) pairs."""
    return 2 * T * cfg.k * 2 * cfg.I * cfg.H


def engine_name(cfg, T):
    """The GEMM engine the library picks for this workload (include/w8a8moe.h, w8a8_moe_engine)."""
    import w8a8_int8_quantized_quant_amd as w8

    mode = {"block": w8.SCALE_BLOCK128, "fp8": w8.SCALE_FP8_BLOCK128, "w4a8": w8.SCALE_W4A8}.get(cfg.scale_mode,
                                                                                               w8.SCALE_CHANNEL)
    e = w8.w8a8_moe_engine(T, cfg.k, cfg.E, cfg.H, cfg.I, w8.w8a8_moe_pick_block_m(T, cfg.k, cfg.E), mode)
    return {w8.ENGINE_STAGED: "staged", w8.ENGINE_DMA: "dma", w8.ENGINE_RING: "ring",
            w8.ENGINE_STREAM: "stream"}.get(e, "none")


def measured_peaks():
    """Rates of the probe kernels (include/w8a8probe.h) on this device: a 4 GiB non-temporal read
    stream, a 2 GiB non-temporal copy, and INT8 MFMA loops on pseudo-random operands with each of
    the two instruction shapes (the larger rate is the measured INT8 ceiling)."""
    import ctypes

    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "w8a8_int8_quantized_quant_amd", "libw8a8probe.so"))
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.w8a8_probe_read.argtypes = [vp, i64, vp, vp]
    lib.w8a8_probe_copy.argtypes = [vp, vp, i64, vp]
    lib.w8a8_probe_mfma_i8.argtypes = [i64, i32, i32, vp, vp]
    lib.w8a8_probe_mfma_i8_ops.argtypes = [i64, i32]
    for f in (lib.w8a8_probe_read, lib.w8a8_probe_copy, lib.w8a8_probe_mfma_i8):
        f.restype = i32
    lib.w8a8_probe_mfma_i8_ops.restype = i64
    stream = torch.cuda.current_stream()
    hs = stream.cuda_stream

    def timed(fn, reps=5):
        for _ in range(2):
            if fn() != 0:
                raise RuntimeError("probe launch failed")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps / 1000.0

    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    t_read = timed(lambda: lib.w8a8_probe_read(buf.data_ptr(), nbytes, sink.data_ptr(), hs))
    half = nbytes // 2
    t_copy = timed(lambda: lib.w8a8_probe_copy(buf.data_ptr(), buf.data_ptr() + half, half, hs))
    del buf
    torch.cuda.empty_cache()
    iters, wgs = 4096, 1024
    ops = lib.w8a8_probe_mfma_i8_ops(iters, wgs)
    tops = {}
    for shape in (16, 32):
        t = timed(lambda: lib.w8a8_probe_mfma_i8(iters, wgs, shape, sink.data_ptr(), hs))
        tops[shape] = round(ops / t / 1e12, 1)
    return {"hbm_read_gbs": round(nbytes / t_read / 1e9, 1), "hbm_copy_gbs": round(2 * half / t_copy / 1e9, 1),
            "int8_mfma_tops": max(tops.values()), "int8_mfma_16x16x64_tops": tops[16],
            "int8_mfma_32x32x32_tops": tops[32],
            "note": "probe kernels of libw8a8probe.so: non-temporal 16-byte read stream over 4 GiB; "
                    "non-temporal copy of 2 GiB (read + written bytes); independent INT8 MFMA chains "
                    "on pseudo-random operands, 4 workgroups of 4 wavefronts per CU, either 8 chains of "
                    "v_mfma_i32_16x16x64_i8 (the layer's GEMMs) or 4 of v_mfma_i32_32x32x32_i8 per "
                    "wavefront; int8_mfma_tops is the larger"}


def linear_figures(steps, warmup):
    """The dense W8A8 linear (w8a8_linear) on DeepSeek-V3's attention output projection (N = 7168,
    K = 16384) at 128 and 8192 tokens, seeded uniform int8 operands; hipBLASLt's int8 GEMM
    (torch._int_mm, int32 out, no dequantization) on the same operands as a reference point."""
    import torch

    import w8a8_int8_quantized_quant_amd as w8

    out = {}
    g = torch.Generator(device="cuda")
    g.manual_seed(16384)
    stream = torch.cuda.current_stream()
    for name, M, N, K in (("decode", 128, 7168, 16384), ("prefill", 8192, 7168, 16384)):
        a_q = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda", generator=g)
        w = torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda", generator=g)
        a_s = torch.rand(M, device="cuda", generator=g) * 1e-2 + 1e-3
        w_s = torch.rand(N, device="cuda", generator=g) * 1e-2 + 1e-3
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(w8.w8a8_linear_workspace_bytes(M, N, K), 256), dtype=torch.uint8, device="cuda")

        def timed(fn):
            for _ in range(warmup):
                fn()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(steps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / steps

        ms = timed(lambda: w8.w8a8_linear(a_q, a_s, w, w_s, y, ws))
        wt = w.t()
        ref_ms = timed(lambda: torch._int_mm(a_q, wt))
        ops = 2.0 * M * N * K
        nbytes = M * K + N * K + 4 * (M + N) + 4 * M * N
        out[name] = {"M": M, "N": N, "K": K, "ms": round(ms, 4), "int8_tops": round(ops / ms / 1e9, 1),
                     "frac_int8_peak": round(ops / ms / 1e9 / INT8_PEAK_TOPS, 4),
                     "hbm_gbs": round(nbytes / ms / 1e6, 1), "frac_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
                     "hipblaslt_int_mm_ms": round(ref_ms, 4)}
        del a_q, w, y, ws, wt
    torch.cuda.empty_cache()
    return out


def measured_traffic(workload):
    """HBM bytes per launch of the roofline kernel from the committed rocprofv3 counter summary, or
    None once the kernel source has changed since the counters were taken (the summary records the
    SHA-256 of gemm.hip it was measured with)."""
    import hashlib

    summary = os.path.join(ROOT, "profiles", "moe_layer_hbm_counters.txt")
    src = os.path.join(ROOT, "w8a8_int8_quantized_quant_amd", "csrc", "gemm.hip")
    try:
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        for line in open(summary):
            f = line.split()
            if len(f) == 4 and f[0] == "bench-traffic" and f[1] == workload:
                fields = dict(x.split("=", 1) for x in f[2:])
                if fields.get("gemm_sha256") == sha:
                    return int(fields["bytes"])
    except (OSError, ValueError, KeyError):
        return None
    return None


def cpu_baseline(cfg, ntok):
    """The CPU oracle, unchanged, on the first `ntok` tokens of the workload: routing from
    the logits, then the dense per-token layer.  Oracle-side expert weights are drawn by the
    shared generator's device fill (bit-identical to its host fill) and quantized by the
    oracle before the clock starts."""
    import numpy as np
    import torch

    import oracle
    import synth

    lg = synth.logits(cfg, slice(0, ntok))
    x = oracle.activations_f32(cfg, slice(0, ntok))
    ids, _ = oracle.route_cfg(cfg, lg)
    experts = np.unique(ids)
    w13q, w13s, w2q, w2s = [None] * cfg.E, [None] * cfg.E, [None] * cfg.E, [None] * cfg.E
    hs = torch.cuda.current_stream().cuda_stream
    buf = torch.empty(2 * cfg.I * cfg.H, dtype=torch.float32, device="cuda")
    fp8, w4 = cfg.scale_mode == "fp8", cfg.scale_mode == "w4a8"

    def quant(w):
        if w4:
            return oracle.w4_quant(w)
        return oracle.fp8_quant_blocks(w, 128, 128) if fp8 else oracle.quant_weight(w, cfg.scale_mode)

    for e in experts:
        n13, n2 = 2 * cfg.I * cfg.H, cfg.H * cfg.I
        synth.dev_normal(buf.data_ptr(), n13, cfg.seed, synth.STREAM_W13, int(e) * n13, cfg.w_sigma, hs)
        w13q[e], w13s[e] = quant(buf[:n13].cpu().numpy().reshape(2 * cfg.I, cfg.H))
        synth.dev_normal(buf.data_ptr(), n2, cfg.seed, synth.STREAM_W2, int(e) * n2, cfg.w_sigma, hs)
        w2q[e], w2s[e] = quant(buf[:n2].cpu().numpy().reshape(cfg.H, cfg.I))
    del buf
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    t0 = time.perf_counter()
    ids, tw = oracle.route_cfg(cfg, lg)
    if w4:
        oracle.w4_moe_tokens(x, ids, tw, w13q, w13s, w2q, w2s, I=cfg.I)
    elif fp8:
        oracle.fp8_moe_tokens(x, ids, tw, w13q, w13s, w2q, w2s, I=cfg.I)
    else:
        oracle.moe_tokens(x, ids, tw, w13q, w13s, w2q, w2s, I=cfg.I, block=cfg.scale_mode == "block")
    dt = time.perf_counter() - t0
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), model)
    except OSError:
        pass
    return {"value": ntok / dt, "unit": "tokens/s", "cores": min(threads, ntok), "kind": "oracle", "cpu_model": model,
            "sample": f"first {ntok} of the {cfg.T} tokens of the same layer (routing + dense per-token "
                      f"quantized MoE over {len(experts)} experts, OpenMP over tokens), {dt:.2f} s wall, "
                      f"host has {os.cpu_count()} logical CPUs"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the layer runs unsharded on a "
              f"single MI355X.", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    if args.linear_only:
        print(json.dumps({"linear": linear_figures(args.steps, args.warmup)}), flush=True)
        return
    import torch

    import synth
    from w8a8_int8_quantized_quant_amd import workload

    cfg = config_of(args.config)
    print(f"[bench] drawing {cfg.note}", file=sys.stderr, flush=True)
    layer = workload.make_layer(cfg)
    ms, stage_ms, st, counts = measure(layer, args.steps, args.warmup)
    fig = layer_figures(cfg, cfg.T, ms, counts)
    print(f"[bench] {cfg.name}: {ms:.3f} ms/step, stages {stage_ms}", file=sys.stderr, flush=True)
    graph_ms = measure_graph(st, args.steps, args.warmup)
    print(f"[bench] {cfg.name}: {graph_ms:.3f} ms/step replayed from a HIP graph", file=sys.stderr, flush=True)
    w13_bytes = w13_algorithmic_bytes(cfg, cfg.T, counts)
    achieved = w13_bytes / (stage_ms["w13"] / 1000.0) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic("decode-w13-stage") if args.config == "decode" else None,
                "kernel": "gate+up grouped GEMM stage (w8a8_grouped_gemm_w13_silu)",
                "kernel_ms": round(stage_ms["w13"], 4), "algorithmic_bytes": w13_bytes}
    del st, layer
    torch.cuda.empty_cache()

    prefill = None
    if not args.no_prefill and args.config == "decode":
        pc = synth.CONFIGS["prefill"]
        print(f"[bench] drawing {pc.note}", file=sys.stderr, flush=True)
        pl = workload.make_layer(pc)
        pms, pstage, pst, pcounts = measure(pl, max(3, args.steps // 4), args.warmup)
        pf = layer_figures(pc, pc.T, pms, pcounts)
        print(f"[bench] prefill: {pms:.3f} ms/step, stages {pstage}", file=sys.stderr, flush=True)
        w13_ops = w13_algorithmic_ops(pc, pc.T)
        w13_tops = w13_ops / (pstage["w13"] / 1000.0) / 1e12
        prefill = {"T": pc.T, "ms_per_step": round(pms, 4), "tokens_per_s": round(pf["tokens_per_s"], 1),
                   "int8_tops": round(pf["int8_tops"], 2), "frac_int8_peak": round(pf["frac_int8_peak"], 4),
                   "hbm_gbs": round(pf["hbm_gbs"], 1), "stage_ms": {k: round(v, 4) for k, v in pstage.items()},
                   "engine": engine_name(pc, pc.T),
                   "roofline": {"bound": "mfma", "achieved": round(w13_tops, 1), "peak": INT8_PEAK_TOPS,
                                "unit": "TOPS", "frac": round(w13_tops / INT8_PEAK_TOPS, 4),
                                "traffic": measured_traffic("prefill-w13-stage"),
                                "kernel": "gate+up grouped GEMM stage (w8a8_grouped_gemm_w13_silu)",
                                "kernel_ms": round(pstage["w13"], 4), "algorithmic_ops": w13_ops,
                                "algorithmic_bytes": w13_algorithmic_bytes(pc, pc.T, pcounts)}}
        del pst, pl
        torch.cuda.empty_cache()

    configs = None
    if not args.no_configs and args.config == "decode":
        configs = {}
        for name in ("tiny", "skew", "skew-empty", "block", "fp8-block", "fp8-decode", "w4a8-decode", "w4a8-block"):
            oc = config_of(name)
            print(f"[bench] drawing {oc.note}", file=sys.stderr, flush=True)
            ol = workload.make_layer(oc)
            oms, ostage, ost, ocounts = measure(ol, max(3, args.steps // 2), args.warmup)
            of = layer_figures(oc, oc.T, oms, ocounts)
            print(f"[bench] {name}: {oms:.3f} ms/step, stages {ostage}", file=sys.stderr, flush=True)
            entry = {"T": oc.T, "ms_per_step": round(oms, 4), "tokens_per_s": round(of["tokens_per_s"], 1),
                     "int8_tops": round(of["int8_tops"], 3), "frac_int8_peak": round(of["frac_int8_peak"], 4),
                     "hbm_gbs": round(of["hbm_gbs"], 1), "frac_hbm_peak": round(of["frac_hbm_peak"], 4),
                     "active_experts": of["active_experts"], "scale": oc.scale_mode, "engine": engine_name(oc, oc.T),
                     "stage_ms": {k: round(v, 4) for k, v in ostage.items()}}
            if oc.scale_mode in ("fp8", "w4a8"):  # the same operation count on the FP8 MFMA
                for key in ("int8_tops", "frac_int8_peak"):
                    del entry[key]
                entry["fp8_tflops"] = round(of["int8_tops"], 3)
                entry["frac_fp8_peak"] = round(of["int8_tops"] / FP8_PEAK_TFLOPS, 4)
            if name in ("skew", "skew-empty"):
                import numpy as np

                c = np.sort(ocounts)[::-1]
                entry["top8_share"] = round(float(c[:8].sum() / max(c.sum(), 1)), 4)
                entry["empty_experts"] = int((ocounts == 0).sum())
            configs[name] = entry
            del ost, ol
            torch.cuda.empty_cache()

    linear = None
    if not args.no_configs and args.config == "decode":
        print("[bench] dense W8A8 linear", file=sys.stderr, flush=True)
        linear = linear_figures(max(5, args.steps // 2), args.warmup)
        print(f"[bench] linear: {linear}", file=sys.stderr, flush=True)

    peaks = None
    if not args.no_peaks:
        print("[bench] measured peaks (probe kernels)", file=sys.stderr, flush=True)
        peaks = measured_peaks()
        roofline["frac_of_measured_read"] = round(achieved / peaks["hbm_read_gbs"], 4)
        if prefill is not None:
            prefill["frac_of_measured_mfma"] = round(prefill["int8_tops"] / peaks["int8_mfma_tops"], 4)
            prefill["roofline"]["frac_of_measured_mfma"] = round(prefill["roofline"]["achieved"]
                                                                 / peaks["int8_mfma_tops"], 4)
        for entry in (linear or {}).values():
            entry["frac_of_measured_mfma"] = round(entry["int8_tops"] / peaks["int8_mfma_tops"], 4)
            entry["frac_of_measured_read"] = round(entry["hbm_gbs"] / peaks["hbm_read_gbs"], 4)
        for entry in (configs or {}).values():
            if "int8_tops" in entry:
                entry["frac_of_measured_mfma"] = round(entry["int8_tops"] / peaks["int8_mfma_tops"], 4)
            entry["frac_of_measured_read"] = round(entry["hbm_gbs"] / peaks["hbm_read_gbs"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        print(f"[bench] CPU oracle baseline on {args.cpu_tokens} tokens", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, min(args.cpu_tokens, cfg.T))

    line = {
        "metric": METRIC, "value": round(fig["tokens_per_s"], 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": {"fp8": "fp8", "w4a8": "int4xfp8"}.get(cfg.scale_mode, "int8"), "data": "synthetic",
        "config": {"workload": f"{cfg.note}: hidden {cfg.H}, intermediate {cfg.I}, {cfg.E} experts, top-{cfg.k}, "
                               + {"fp8": "128x128 block-wise FP8 (E4M3)",
                                  "w4a8": "W4A8 (int4 weights, FP8 activations)"}.get(
                                      cfg.scale_mode, f"{cfg.scale_mode}-wise W8A8 INT8"), "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E,
                   "k": cfg.k, "scale": cfg.scale_mode, "active_experts": fig["active_experts"]},
        "int8_tops": round(fig["int8_tops"], 3), "frac_int8_peak": round(fig["frac_int8_peak"], 4),
        "hbm_gbs": round(fig["hbm_gbs"], 1), "frac_hbm_peak": round(fig["frac_hbm_peak"], 4),
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "graph": {"ms_per_step": round(graph_ms, 4), "tokens_per_s": round(cfg.T / (graph_ms / 1000.0), 1),
                  "note": "the same step captured once into a HIP graph and replayed (value: eager launches)"},
        "roofline": roofline, "prefill": prefill, "configs": configs, "linear": linear, "peaks_measured": peaks,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
