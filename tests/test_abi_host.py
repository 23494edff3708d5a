"""Host-side checks of the C ABI: the library loads without a GPU, exports every
symbol the header declares, and rejects invalid calls before touching HIP."""
import os
import re

import numpy as np
import pytest

import oracle
import w8a8_int8_quantized_quant_amd as w8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w8a8moe.h")

OK, INV, SHAPE, WS, DT = (w8.W8A8_OK, w8.W8A8_INVALID_ARGUMENT, w8.W8A8_UNSUPPORTED_SHAPE,
                          w8.W8A8_WORKSPACE_TOO_SMALL, w8.W8A8_UNSUPPORTED_DTYPE)
P16 = 1 << 20  # a fake, 256-byte aligned device address: these calls must fail validation first


def header_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = header_functions()
    assert len(names) >= 17
    L = w8.lib()
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    assert sorted(w8.EXPORTS) == names


def test_probe_library_exports_its_header_and_validates():
    """The benchmark's measured-peak probes (libw8a8probe.so): every declared symbol exported,
    invalid arguments rejected without a GPU, and the MFMA op count of a launch."""
    import ctypes

    names = header_functions(os.path.join(ROOT, "include", "w8a8probe.h"))
    assert names == ["w8a8_probe_copy", "w8a8_probe_mfma_f8_block", "w8a8_probe_mfma_i8", "w8a8_probe_mfma_i8_ops",
                     "w8a8_probe_read"]
    L = ctypes.CDLL(os.path.join(ROOT, "w8a8_int8_quantized_quant_amd", "libw8a8probe.so"))
    for n in names:
        assert hasattr(L, n), n
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.w8a8_probe_read.argtypes = [vp, i64, vp, vp]
    L.w8a8_probe_copy.argtypes = [vp, vp, i64, vp]
    L.w8a8_probe_mfma_i8.argtypes = [i64, i32, i32, vp, vp]
    L.w8a8_probe_mfma_i8_ops.argtypes = [i64, i32]
    L.w8a8_probe_mfma_i8_ops.restype = i64
    assert L.w8a8_probe_read(None, 1024, P16, None) == 1
    assert L.w8a8_probe_read(P16, 1000, P16, None) == 1
    assert L.w8a8_probe_copy(P16, P16, 0, None) == 1
    assert L.w8a8_probe_mfma_i8(0, 8, 16, P16, None) == 1
    assert L.w8a8_probe_mfma_i8(1, 8, 16, None, None) == 1
    assert L.w8a8_probe_mfma_i8(1, 8, 24, P16, None) == 1
    L.w8a8_probe_mfma_f8_block.argtypes = [vp, vp, vp, i32, vp]
    assert L.w8a8_probe_mfma_f8_block(P16, P16, None, 1, None) == 1
    assert L.w8a8_probe_mfma_f8_block(P16, P16, P16, 0, None) == 1
    # 2 workgroups x 4 wavefronts x 3 rounds x 8 MFMAs x (16*16*64 multiply-adds x 2)
    assert L.w8a8_probe_mfma_i8_ops(3, 2) == 2 * 4 * 3 * 8 * 2 * 16 * 16 * 64


def test_linear_validation():
    """w8a8_linear rejects bad calls on the host: sizes, shapes outside the engine, a short
    workspace, missing pointers."""
    L = w8.lib()
    ws = w8.w8a8_linear_workspace_bytes(1000, 256, 256)
    assert ws >= 256 and w8.w8a8_linear_workspace_bytes(0, 256, 256) >= 256
    assert w8.w8a8_linear_workspace_bytes(4, 576, 256) == 0  # unsupported shape
    # few rows: K slices, their int32 partials in the workspace (128 x 7168 outputs, K = 16384)
    assert w8.w8a8_linear_workspace_bytes(128, 7168, 16384) >= 2 * 4 * 128 * 7168
    call = lambda M, N, K, wsb=ws, a=P16, w=P16, out=P16: L.w8a8_linear(a, P16, w, P16, M, N, K, out, P16, wsb, None)
    assert call(-1, 256, 256) == INV
    assert call(4, 576, 256) == SHAPE  # N not a multiple of 256
    assert call(4, 256, 384) == SHAPE  # K not a multiple of 256
    assert call(4, 256, 0) == SHAPE
    assert call(1 << 17, 256, 1 << 16) == SHAPE  # M*K beyond 32-bit offsets
    assert call(1000, 256, 256, wsb=ws - 1) == WS
    assert call(128, 7168, 16384, wsb=ws) == WS  # needs room for its K-slice partials
    assert call(4, 256, 256, a=None) == INV
    assert call(4, 256, 256, w=P16 + 4) == INV  # weights not 16-byte aligned
    assert call(0, 256, 256, a=None, w=None, out=None) == OK  # no rows: nothing to do


def test_status_strings():
    assert w8.status_string(0) == "W8A8_OK"
    assert w8.status_string(3) == "W8A8_WORKSPACE_TOO_SMALL"
    assert w8.status_string(99) == "W8A8_UNKNOWN_STATUS"


def test_quant_validation():
    L = w8.lib()
    assert L.w8a8_quant_per_token(None, 0, 4, 128, 0, P16, P16, None) == INV
    assert L.w8a8_quant_per_token(P16, 7, 4, 128, 0, P16, P16, None) == DT
    assert L.w8a8_quant_per_token(P16, 0, 4, 100, 64, P16, P16, None) == SHAPE
    assert L.w8a8_quant_per_token(P16, 0, -1, 128, 0, P16, P16, None) == INV
    assert L.w8a8_quant_per_token(P16, 0, 0, 128, 0, P16, P16, None) == OK  # no rows: no-op
    assert L.w8a8_quant_blocks(P16, 1, 4, 128, 0, 128, P16, P16, None) == INV
    assert L.w8a8_quant_blocks(P16 + 2, 0, 4, 128, 1, 128, P16, P16, None) == INV  # misaligned fp32


def test_route_validation():
    L = w8.lib()
    args = lambda T, E, k, fn, ng, tg, bias=None, ids=P16: (P16, T, E, k, fn, ng, tg, 1, 1.0, bias, ids, P16, None)
    assert L.moe_topk_route(*args(4, 8, 9, 0, 1, 1)) == SHAPE            # k > E
    assert L.moe_topk_route(*args(4, 0, 1, 0, 1, 1)) == SHAPE            # no experts
    assert L.moe_topk_route(*args(4, 2048, 8, 1, 8, 4)) == SHAPE         # E > 1024
    assert L.moe_topk_route(*args(4, 256, 8, 1, 7, 4)) == SHAPE          # groups do not divide E
    assert L.moe_topk_route(*args(4, 256, 8, 0, 8, 4)) == INV            # grouped softmax
    assert L.moe_topk_route(*args(4, 256, 64, 1, 8, 1)) == SHAPE         # k > topk_group * group size
    assert L.moe_topk_route(*args(4, 256, 8, 1, 8, 9)) == SHAPE          # topk_group > n_group
    assert L.moe_topk_route(*args(4, 256, 8, 2, 8, 4)) == INV            # unknown score function
    assert L.moe_topk_route(*args(4, 256, 8, 1, 8, 4, ids=P16 + 2)) == INV
    assert L.moe_topk_route(*args(0, 256, 8, 1, 8, 4)) == OK             # no tokens: no-op


def test_align_validation():
    L = w8.lib()
    need = w8.moe_align_workspace_bytes(128, 8, 256)
    assert need > 0
    a = lambda T, k, E, bm, ws, n: (P16, T, k, E, bm, P16, P16, P16, P16, P16, P16, ws, n, None)
    assert L.moe_align_by_expert(*a(128, 8, 256, 48, P16, need)) == SHAPE
    assert L.moe_align_by_expert(*a(128, 8, 256, 16, P16, need - 1)) == WS
    assert L.moe_align_by_expert(*a(128, 8, 2000, 16, P16, need)) == SHAPE
    assert L.moe_align_by_expert(*a(128, 300, 256, 16, P16, need)) == SHAPE   # k > E
    assert L.moe_align_by_expert(*a(128, 8, 256, 16, P16 + 4, need)) == INV  # ws not 256-aligned
    assert L.moe_align_by_expert(P16, 1 << 28, 8, 256, 16, P16, P16, P16, P16, P16, P16, P16, 1 << 40,
                                 None) == SHAPE  # too many pairs


def test_noalloc_align_validation():
    """The allocation-free align rejects, before any HIP call, pair counts whose align scratch
    exceeds its fixed 4 MiB, and the same invalid arguments as the workspace align."""
    L = w8.lib()
    assert w8.moe_align_noalloc_scratch_bytes() == 4 << 20
    na = lambda T, k, E, bm: (P16, T, k, E, bm, P16, P16, P16, P16, P16, P16, None)
    assert w8.moe_align_workspace_bytes(131072, 8, 256) > 4 << 20
    assert L.moe_align_by_expert_noalloc(*na(131072, 8, 256, 16)) == SHAPE   # 1M pairs
    assert L.moe_align_by_expert_noalloc(*na(60000, 16, 1024, 16)) == SHAPE  # E = 1024: 8 bytes a pair
    assert L.moe_align_by_expert_noalloc(*na(128, 8, 256, 24)) == SHAPE
    assert L.moe_align_by_expert_noalloc(*na(128, 300, 256, 16)) == SHAPE
    assert L.moe_align_by_expert_noalloc(*na(-1, 8, 256, 16)) == INV
    bad = list(na(128, 8, 256, 16))
    bad[5] = P16 + 2  # counts not 4-byte aligned
    assert L.moe_align_by_expert_noalloc(*bad) == INV


def test_gemm_validation():
    L = w8.lib()
    ineed = w8.w8a8_grouped_gemm_i32_workspace_bytes(True, 256, 256, 16, 2, 8, 16)
    assert ineed > 0
    g = lambda gather, N, K, bm, out=P16, ws_bytes=ineed: (P16, gather, P16, N, K, P16, P16, P16, P16, 16, 2, 8, bm,
                                                          out, P16, ws_bytes, None)
    assert L.w8a8_grouped_gemm_i32(*g(1, 100, 256, 16)) == SHAPE
    assert L.w8a8_grouped_gemm_i32(*g(1, 256, 200, 16)) == SHAPE
    assert L.w8a8_grouped_gemm_i32(*g(1, 258, 256, 16)) == SHAPE  # odd I = N / 2
    assert L.w8a8_grouped_gemm_i32(*g(2, 256, 256, 16)) == INV
    assert L.w8a8_grouped_gemm_i32(*g(1, 256, 256, 24)) == SHAPE
    assert L.w8a8_grouped_gemm_i32(*g(1, 256, 256, 16, out=P16 + 4)) == INV
    assert L.w8a8_grouped_gemm_i32(*g(1, 256, 256, 16, ws_bytes=ineed - 1)) == WS
    assert w8.w8a8_grouped_gemm_i32_workspace_bytes(True, 100, 256, 16, 2, 8, 16) == 0
    T, k, E, H, I, bm = 16, 2, 8, 256, 128, 16
    need = w8.w8a8_w13_workspace_bytes(T, k, E, H, I, bm)
    w13 = lambda H_, a_q=P16, ws_bytes=need, T_=T: (a_q, P16, P16, P16, P16, P16, P16, P16, T_, k, E, H_, I, bm,
                                                     P16, P16, P16, ws_bytes, None)
    assert L.w8a8_grouped_gemm_w13_silu(*w13(100)) == SHAPE
    assert L.w8a8_grouped_gemm_w13_silu(*w13(H, ws_bytes=need - 1)) == WS
    assert L.w8a8_grouped_gemm_w13_silu(*w13(H, a_q=None)) == INV
    assert L.w8a8_grouped_gemm_w13_silu(*w13(H, T_=0)) == OK
    need2 = w8.w8a8_w2_workspace_bytes(T, k, E, H, I, bm)
    w2 = lambda ws_bytes=need2, tw=P16: (P16, P16, P16, P16, P16, P16, P16, P16, tw, T, k, E, H, I, bm, P16, P16,
                                         ws_bytes, None)
    assert L.w8a8_grouped_gemm_w2_combine(*w2(ws_bytes=need2 - 1)) == WS
    assert L.w8a8_grouped_gemm_w2_combine(*w2(tw=None)) == INV
    assert L.w8a8_block_grouped_gemm_w2_combine(*w2(ws_bytes=0)) == WS


def test_forward_validation():
    L = w8.lib()
    import ctypes

    assert L.w8a8_moe_forward(None, P16, 1 << 30, None) == INV

    def args(**kw):
        base = dict(x=P16, x_dtype=1, router_logits=P16, w13=P16, w13_scale=P16, w2=P16, w2_scale=P16,
                    correction_bias=None, out=P16, topk_ids=None, topk_weights=None, T=128, H=7168, I=2048,
                    E=256, k=8, score_fn=1, n_group=8, topk_group=4, renormalize=1, routed_scaling=2.5,
                    scale_mode=0, block_m=0)
        base.update(kw)
        return ctypes.byref(w8.MoEArgs(**base))

    need = w8.w8a8_moe_workspace_bytes(128, 8, 256, 7168, 2048)
    assert L.w8a8_moe_forward(args(), P16, need - 1, None) == WS
    assert L.w8a8_moe_forward(args(scale_mode=5), P16, need, None) == INV
    assert L.w8a8_moe_forward(args(x_dtype=3), P16, need, None) == DT
    assert L.w8a8_moe_forward(args(H=7000), P16, need, None) == SHAPE
    assert L.w8a8_moe_forward(args(block_m=8), P16, need, None) == SHAPE
    assert L.w8a8_moe_forward(args(n_group=3), P16, need, None) == SHAPE
    assert L.w8a8_moe_forward(args(T=0), P16, need, None) == OK


def test_engine_choice():
    """The GEMM engine follows the average rows per expert (decode: staged; skewed and block-wise
    mid-size batches: ring; prefill: DMA; W4A8 decode: streaming); invalid shapes give -1."""
    H, I, E, k = 7168, 2048, 256, 8
    assert w8.w8a8_moe_engine(128, k, E, H, I, 16, w8.SCALE_CHANNEL) == w8.ENGINE_STAGED
    assert w8.w8a8_moe_engine(8192, k, E, H, I, 128, w8.SCALE_CHANNEL) == w8.ENGINE_DMA
    assert w8.w8a8_moe_engine(4096, k, E, H, I, 128, w8.SCALE_CHANNEL) == w8.ENGINE_RING
    assert w8.w8a8_moe_engine(2048, k, E, H, I, 64, w8.SCALE_BLOCK128) == w8.ENGINE_RING
    assert w8.w8a8_moe_engine(2048, k, E, H, I, 64, w8.SCALE_FP8_BLOCK128) == w8.ENGINE_RING
    assert w8.w8a8_moe_engine(128, k, E, H, I, 16, w8.SCALE_W4A8) == w8.ENGINE_STREAM
    assert w8.w8a8_moe_engine(16, 2, 8, 256, 128, 16, w8.SCALE_CHANNEL) == w8.ENGINE_STAGED
    assert w8.w8a8_moe_engine(128, k, E, 7000, I, 16, w8.SCALE_CHANNEL) == -1
    assert w8.w8a8_moe_engine(128, k, E, H, I, 24, w8.SCALE_CHANNEL) == -1
    assert w8.w8a8_moe_engine(128, k, E, H, I, 16, 7) == -1


def test_engine_choice_keeps_grids_launchable():
    """A dispatch counts its work-items in 32 bits, so a work-list engine takes a shape only while
    its (row tile, N-tile) items stay within 2^20 workgroups; past that the staged engine, which
    launches in pieces, runs the layer.  Here H = 65536, I = 256, E = 64, k = 32: 65535 tokens make
    (ceil(P / 320) + E) * (H / 256) = 6618 * 256 items (over 2^20), half of them 3341 * 256 (under)."""
    H, I, E, k = 65536, 256, 64, 32
    assert (-(-32768 * k // 320) + E) * (H // 256) <= 1 << 20 < (-(-65535 * k // 320) + E) * (H // 256)
    assert w8.w8a8_moe_engine(32768, k, E, H, I, 128, w8.SCALE_CHANNEL) == w8.ENGINE_DMA
    assert w8.w8a8_moe_engine(65535, k, E, H, I, 128, w8.SCALE_CHANNEL) == w8.ENGINE_STAGED
    # 2^24 + 4096 tokens of a 256-wide layer (more than 2^32 activation elements): staged
    assert w8.w8a8_moe_engine((1 << 24) + 4096, 2, 8, 256, 256, 128, w8.SCALE_CHANNEL) == w8.ENGINE_STAGED


def test_launch_size_limits():
    """Shapes whose one grid would pass 2^20 workgroups are rejected before any HIP call: the dense
    linear's output tiles, and a quantization block row that would not fit one launch."""
    L = w8.lib()
    assert w8.w8a8_linear_workspace_bytes(1 << 20, 1 << 16, 256) >= 256  # 3277 * 256 tiles
    assert w8.w8a8_linear_workspace_bytes(1 << 20, 1 << 19, 256) == 0    # 3277 * 2048 tiles
    assert L.w8a8_linear(P16, P16, P16, P16, 1 << 20, 1 << 19, 256, P16, P16, 1 << 30, None) == SHAPE
    # 2^21 + 1 column blocks of 1 x 1 in a row; then 2^20 of them (accepted, but rows = 0 is a no-op)
    assert L.w8a8_quant_blocks(P16, 0, 2, (1 << 21) + 1, 2, 1, P16, P16, None) == SHAPE
    assert L.w8a8_quant_per_token(P16, 0, 2, (1 << 21) + 2, 2, P16, P16, None) == SHAPE
    assert L.w8a8_quant_blocks(P16, 0, 0, 1 << 20, 2, 1, P16, P16, None) == OK
    assert L.w8a8_w4a8_quant_weights(P16, 0, 2, 128 * ((1 << 20) + 1), P16, P16, None) == SHAPE


def test_size_queries():
    assert w8.w8a8_moe_max_rows(128, 8, 256, 16) == (1024 + 256 * 15) // 16 * 16
    assert w8.w8a8_moe_max_rows(1, 8, 256, 128) == (8 + 8 * 127) // 128 * 128
    assert w8.w8a8_moe_max_rows(0, 8, 256, 16) == 0
    assert w8.w8a8_moe_max_rows(4, 8, 256, 24) == -1
    assert w8.w8a8_moe_pick_block_m(128, 8, 256) == 16
    assert w8.w8a8_moe_pick_block_m(8192, 8, 256) == 128
    assert w8.w8a8_moe_workspace_bytes(0, 8, 256, 7168, 2048) > 0
    assert w8.w8a8_w13_workspace_bytes(16, 2, 8, 100, 128, 16) == 0


@pytest.mark.parametrize("bm", [16, 32, 64, 128])
def test_max_rows_bounds_every_padding(bm):
    """The row capacity bounds the padded total for any routing, including the worst case
    where every non-empty expert ends one row into a new tile."""
    rng = np.random.default_rng(bm)
    for T, k, E in [(128, 8, 256), (5, 8, 256), (1000, 2, 8), (3, 1, 1), (40, 8, 16)]:
        for trial in range(4):
            if trial == 0:
                ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
            elif trial == 1:  # as many experts as possible with count = 1 (mod bm)
                ids = (np.arange(T * k) % E).reshape(T, k) if k <= E else None
                if ids is not None and T * k >= E:
                    ids = np.stack([(np.arange(k) + t * k) % E for t in range(T)])
            elif trial == 2:
                ids = np.zeros((T, k), np.int64) + np.arange(k)
            else:
                ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
            ids = np.ascontiguousarray(ids, dtype=np.int32)
            al = oracle.align(ids, E, bm)
            assert al["padded_offsets"][-1] <= w8.w8a8_moe_max_rows(T, k, E, bm)
