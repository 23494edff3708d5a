"""Python binding of libw8a8moe.so, the gfx950 W8A8 INT8 fused-MoE layer.

Argument marshalling only: every function here forwards to the C entry point of
the same name declared in ``include/w8a8moe.h``; all computation runs in the
HIP kernels behind it.  PyTorch provides device memory and the current stream.
A missing library is an error (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw8a8moe.so")

W8A8_OK = 0
W8A8_INVALID_ARGUMENT = 1
W8A8_UNSUPPORTED_SHAPE = 2
W8A8_WORKSPACE_TOO_SMALL = 3
W8A8_UNSUPPORTED_DTYPE = 4
W8A8_HIP_ERROR = 5

DTYPE_F32 = 0
DTYPE_BF16 = 1
SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1
SCALE_CHANNEL = 0
SCALE_BLOCK128 = 1
SCALE_FP8_BLOCK128 = 2
SCALE_W4A8 = 3

# Every symbol the C header declares (checked by the CPU test suite).
EXPORTS = (
    "w8a8_status_string", "w8a8_quant_per_token", "w8a8_quant_blocks", "moe_topk_route", "w8a8_moe_max_rows",
    "moe_align_workspace_bytes", "moe_align_by_expert", "moe_align_by_expert_noalloc",
    "moe_align_noalloc_scratch_bytes", "w8a8_grouped_gemm_i32",
    "w8a8_grouped_gemm_i32_workspace_bytes", "w8a8_moe_engine", "w8a8_w13_workspace_bytes",
    "w8a8_grouped_gemm_w13_silu", "w8a8_w2_workspace_bytes", "w8a8_grouped_gemm_w2_combine",
    "w8a8_block_grouped_gemm_w13_silu", "w8a8_block_grouped_gemm_w2_combine", "w8a8_moe_pick_block_m",
    "w8a8_moe_workspace_bytes", "w8a8_moe_forward", "w8a8_linear_workspace_bytes", "w8a8_linear",
    "w8a8_fp8_quant_blocks", "w8a8_fp8_grouped_gemm_w13_silu", "w8a8_fp8_grouped_gemm_w2_combine",
    "w8a8_w4a8_quant_weights", "w8a8_w4a8_grouped_gemm_w13_silu", "w8a8_w4a8_grouped_gemm_w2_combine",
)


class W8A8Error(RuntimeError):
    def __init__(self, name: str, status: int):
        super().__init__(f"{name} returned {status_string(status)} ({status})")
        self.status = status


class MoEArgs(ctypes.Structure):
    """struct w8a8_moe_args."""

    _fields_ = [
        ("x", ctypes.c_void_p), ("x_dtype", ctypes.c_int32), ("router_logits", ctypes.c_void_p),
        ("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p), ("w2", ctypes.c_void_p),
        ("w2_scale", ctypes.c_void_p), ("correction_bias", ctypes.c_void_p), ("out", ctypes.c_void_p),
        ("topk_ids", ctypes.c_void_p), ("topk_weights", ctypes.c_void_p), ("T", ctypes.c_int64),
        ("H", ctypes.c_int64), ("I", ctypes.c_int64), ("E", ctypes.c_int64), ("k", ctypes.c_int64),
        ("score_fn", ctypes.c_int32), ("n_group", ctypes.c_int64), ("topk_group", ctypes.c_int64),
        ("renormalize", ctypes.c_int32), ("routed_scaling", ctypes.c_float), ("scale_mode", ctypes.c_int32),
        ("block_m", ctypes.c_int64),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        sig = {
            "w8a8_status_string": (ctypes.c_char_p, [i32]),
            "w8a8_quant_per_token": (i32, [vp, i32, i64, i64, i64, vp, vp, vp]),
            "w8a8_quant_blocks": (i32, [vp, i32, i64, i64, i64, i64, vp, vp, vp]),
            "moe_topk_route": (i32, [vp, i64, i64, i64, i32, i64, i64, i32, f32, vp, vp, vp, vp]),
            "w8a8_moe_max_rows": (i64, [i64, i64, i64, i64]),
            "moe_align_workspace_bytes": (sz, [i64, i64, i64]),
            "moe_align_by_expert": (i32, [vp, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "moe_align_by_expert_noalloc": (i32, [vp, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp]),
            "moe_align_noalloc_scratch_bytes": (sz, []),
            "w8a8_grouped_gemm_i32": (i32, [vp, i32, vp, i64, i64, vp, vp, vp, vp, i64, i64, i64, i64, vp, vp, sz,
                                            vp]),
            "w8a8_grouped_gemm_i32_workspace_bytes": (sz, [i32, i64, i64, i64, i64, i64, i64]),
            "w8a8_moe_engine": (i32, [i64, i64, i64, i64, i64, i64, i32]),
            "w8a8_w13_workspace_bytes": (sz, [i64, i64, i64, i64, i64, i64, i32]),
            "w8a8_w2_workspace_bytes": (sz, [i64, i64, i64, i64, i64, i64, i32]),
            "w8a8_grouped_gemm_w13_silu": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, vp, vp,
                                                 vp, sz, vp]),
            "w8a8_block_grouped_gemm_w13_silu": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                                       vp, vp, vp, sz, vp]),
            "w8a8_grouped_gemm_w2_combine": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                                   vp, vp, sz, vp]),
            "w8a8_block_grouped_gemm_w2_combine": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                                         i64, vp, vp, sz, vp]),
            "w8a8_moe_pick_block_m": (i64, [i64, i64, i64]),
            "w8a8_moe_workspace_bytes": (sz, [i64, i64, i64, i64, i64, i64, i32]),
            "w8a8_moe_forward": (i32, [ctypes.POINTER(MoEArgs), vp, sz, vp]),
            "w8a8_linear_workspace_bytes": (sz, [i64, i64, i64]),
            "w8a8_linear": (i32, [vp, vp, vp, vp, i64, i64, i64, vp, vp, sz, vp]),
            "w8a8_fp8_quant_blocks": (i32, [vp, i32, i64, i64, i64, i64, vp, vp, vp]),
            "w8a8_w4a8_quant_weights": (i32, [vp, i32, i64, i64, vp, vp, vp]),
            "w8a8_w4a8_grouped_gemm_w13_silu": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                                      vp, vp, vp, sz, vp]),
            "w8a8_w4a8_grouped_gemm_w2_combine": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                                        i64, vp, vp, sz, vp]),
            "w8a8_fp8_grouped_gemm_w13_silu": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                                     vp, vp, vp, sz, vp]),
            "w8a8_fp8_grouped_gemm_w2_combine": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                                       i64, vp, vp, sz, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().w8a8_status_string(status).decode()


# --------------------------------------------------------------------------- marshalling helpers

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to the W8A8 MoE library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    return -1


def _call(name: str, *args) -> None:
    st = getattr(lib(), name)(*args)
    if st != W8A8_OK:
        raise W8A8Error(name, st)


# --------------------------------------------------------------------------- entry points

def w8a8_quant_per_token(x, group: int, q, scale, stream=None) -> None:
    rows, cols = x.shape
    _call("w8a8_quant_per_token", _ptr(x), _dtype_code(x), rows, cols, group, _ptr(q), _ptr(scale), _stream(stream))


def w8a8_quant_blocks(x, block_rows: int, block_cols: int, q, scale, stream=None) -> None:
    rows, cols = x.shape
    _call("w8a8_quant_blocks", _ptr(x), _dtype_code(x), rows, cols, block_rows, block_cols, _ptr(q), _ptr(scale),
          _stream(stream))


def w8a8_fp8_quant_blocks(x, block_rows: int, block_cols: int, q, scale, stream=None) -> None:
    """FP8 (E4M3) codes (uint8 q) with one scale per block_rows x block_cols block."""
    rows, cols = x.shape
    _call("w8a8_fp8_quant_blocks", _ptr(x), _dtype_code(x), rows, cols, block_rows, block_cols, _ptr(q), _ptr(scale),
          _stream(stream))


def w8a8_w4a8_quant_weights(x, q, scale, stream=None) -> None:
    """Packed int4 weights (uint8 q [rows, cols/2]) with one scale per (row, 128 columns)."""
    rows, cols = x.shape
    _call("w8a8_w4a8_quant_weights", _ptr(x), _dtype_code(x), rows, cols, _ptr(q), _ptr(scale), _stream(stream))


def moe_topk_route(logits, k: int, score_fn: int, n_group: int, topk_group: int, renormalize: bool,
                   routed_scaling: float, correction_bias, topk_ids, topk_weights, stream=None) -> None:
    T, E = logits.shape
    _call("moe_topk_route", _ptr(logits), T, E, k, score_fn, n_group, topk_group, int(renormalize), routed_scaling,
          _ptr(correction_bias), _ptr(topk_ids), _ptr(topk_weights), _stream(stream))


def w8a8_moe_max_rows(T: int, k: int, E: int, block_m: int) -> int:
    return lib().w8a8_moe_max_rows(T, k, E, block_m)


def moe_align_workspace_bytes(T: int, k: int, E: int) -> int:
    return lib().moe_align_workspace_bytes(T, k, E)


def moe_align_by_expert(topk_ids, E: int, block_m: int, expert_counts, expert_offsets, padded_offsets,
                        sorted_pair_ids, tile_expert, num_tiles, ws, stream=None) -> None:
    T, k = topk_ids.shape
    _call("moe_align_by_expert", _ptr(topk_ids), T, k, E, block_m, _ptr(expert_counts), _ptr(expert_offsets),
          _ptr(padded_offsets), _ptr(sorted_pair_ids), _ptr(tile_expert), _ptr(num_tiles), _ptr(ws),
          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))


def moe_align_by_expert_noalloc(topk_ids, E: int, block_m: int, expert_counts, expert_offsets, padded_offsets,
                                sorted_pair_ids, tile_expert, num_tiles, stream=None) -> None:
    """moe_align_by_expert without a workspace (the library's own 4 MiB device scratch)."""
    T, k = topk_ids.shape
    _call("moe_align_by_expert_noalloc", _ptr(topk_ids), T, k, E, block_m, _ptr(expert_counts), _ptr(expert_offsets),
          _ptr(padded_offsets), _ptr(sorted_pair_ids), _ptr(tile_expert), _ptr(num_tiles), _stream(stream))


def moe_align_noalloc_scratch_bytes() -> int:
    return lib().moe_align_noalloc_scratch_bytes()


def w8a8_grouped_gemm_i32_workspace_bytes(gather: bool, N: int, K: int, T: int, k: int, E: int, block_m: int) -> int:
    return lib().w8a8_grouped_gemm_i32_workspace_bytes(int(gather), N, K, T, k, E, block_m)


def w8a8_grouped_gemm_i32(a, gather: bool, w, sorted_pair_ids, padded_offsets, tile_expert, num_tiles, T: int, k: int,
                          block_m: int, out, ws, stream=None) -> None:
    E, N, K = w.shape
    _call("w8a8_grouped_gemm_i32", _ptr(a), int(gather), _ptr(w), N, K, _ptr(sorted_pair_ids), _ptr(padded_offsets),
          _ptr(tile_expert), _ptr(num_tiles), T, k, E, block_m, _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream))


ENGINE_STAGED = 0
ENGINE_DMA = 1
ENGINE_RING = 2
ENGINE_STREAM = 3


def w8a8_moe_engine(T: int, k: int, E: int, H: int, I: int, block_m: int, scale_mode: int = SCALE_CHANNEL) -> int:
    """GEMM engine of a layer of this shape (ENGINE_*), -1 for an invalid shape."""
    return lib().w8a8_moe_engine(T, k, E, H, I, block_m, scale_mode)


def w8a8_w13_workspace_bytes(T, k, E, H, I, block_m, scale_mode=SCALE_CHANNEL) -> int:
    return lib().w8a8_w13_workspace_bytes(T, k, E, H, I, block_m, scale_mode)


def w8a8_w2_workspace_bytes(T, k, E, H, I, block_m, scale_mode=SCALE_CHANNEL) -> int:
    return lib().w8a8_w2_workspace_bytes(T, k, E, H, I, block_m, scale_mode)


def _nbytes(ws) -> int:
    return 0 if ws is None else ws.numel() * ws.element_size()


def _w13(name, a_q, a_scale, w13, w13_scale, sorted_pair_ids, padded_offsets, tile_expert, num_tiles, T, k,
         block_m, h_q, h_scale, ws, stream):
    E, N2, H = w13.shape
    _call(name, _ptr(a_q), _ptr(a_scale), _ptr(w13), _ptr(w13_scale), _ptr(sorted_pair_ids), _ptr(padded_offsets),
          _ptr(tile_expert), _ptr(num_tiles), T, k, E, H, N2 // 2, block_m, _ptr(h_q), _ptr(h_scale), _ptr(ws),
          _nbytes(ws), _stream(stream))


def _w2(name, h_q, h_scale, w2, w2_scale, sorted_pair_ids, padded_offsets, tile_expert, num_tiles, topk_weights,
        T, k, block_m, out, ws, stream):
    E, H, I = w2.shape
    _call(name, _ptr(h_q), _ptr(h_scale), _ptr(w2), _ptr(w2_scale), _ptr(sorted_pair_ids), _ptr(padded_offsets),
          _ptr(tile_expert), _ptr(num_tiles), _ptr(topk_weights), T, k, E, H, I, block_m, _ptr(out), _ptr(ws),
          _nbytes(ws), _stream(stream))


def w8a8_grouped_gemm_w13_silu(a_q, a_scale, w13, w13_scale, sorted_pair_ids, padded_offsets, tile_expert,
                               num_tiles, T, k, block_m, h_q, h_scale, ws, stream=None) -> None:
    _w13("w8a8_grouped_gemm_w13_silu", a_q, a_scale, w13, w13_scale, sorted_pair_ids, padded_offsets, tile_expert,
         num_tiles, T, k, block_m, h_q, h_scale, ws, stream)


def w8a8_block_grouped_gemm_w13_silu(a_q, a_scale, w13, w13_scale, sorted_pair_ids, padded_offsets, tile_expert,
                                     num_tiles, T, k, block_m, h_q, h_scale, ws, stream=None) -> None:
    _w13("w8a8_block_grouped_gemm_w13_silu", a_q, a_scale, w13, w13_scale, sorted_pair_ids, padded_offsets,
         tile_expert, num_tiles, T, k, block_m, h_q, h_scale, ws, stream)


def w8a8_grouped_gemm_w2_combine(h_q, h_scale, w2, w2_scale, sorted_pair_ids, padded_offsets, tile_expert,
                                 num_tiles, topk_weights, T, k, block_m, out, ws, stream=None) -> None:
    _w2("w8a8_grouped_gemm_w2_combine", h_q, h_scale, w2, w2_scale, sorted_pair_ids, padded_offsets, tile_expert,
        num_tiles, topk_weights, T, k, block_m, out, ws, stream)


def w8a8_block_grouped_gemm_w2_combine(h_q, h_scale, w2, w2_scale, sorted_pair_ids, padded_offsets, tile_expert,
                                       num_tiles, topk_weights, T, k, block_m, out, ws, stream=None) -> None:
    _w2("w8a8_block_grouped_gemm_w2_combine", h_q, h_scale, w2, w2_scale, sorted_pair_ids, padded_offsets,
        tile_expert, num_tiles, topk_weights, T, k, block_m, out, ws, stream)


def w8a8_fp8_grouped_gemm_w13_silu(a_q, a_scale, w13, w13_scale, sorted_pair_ids, padded_offsets, tile_expert,
                                   num_tiles, T, k, block_m, h_q, h_scale, ws, stream=None) -> None:
    _w13("w8a8_fp8_grouped_gemm_w13_silu", a_q, a_scale, w13, w13_scale, sorted_pair_ids, padded_offsets,
         tile_expert, num_tiles, T, k, block_m, h_q, h_scale, ws, stream)


def w8a8_fp8_grouped_gemm_w2_combine(h_q, h_scale, w2, w2_scale, sorted_pair_ids, padded_offsets, tile_expert,
                                     num_tiles, topk_weights, T, k, block_m, out, ws, stream=None) -> None:
    _w2("w8a8_fp8_grouped_gemm_w2_combine", h_q, h_scale, w2, w2_scale, sorted_pair_ids, padded_offsets,
        tile_expert, num_tiles, topk_weights, T, k, block_m, out, ws, stream)


def _w13_w4(a_q, a_scale, w13, w13_scale, sorted_pair_ids, padded_offsets, tile_expert, num_tiles, T, k, block_m,
            h_q, h_scale, ws, stream):
    E, N2, Hh = w13.shape  # packed: H/2 bytes per row
    _call("w8a8_w4a8_grouped_gemm_w13_silu", _ptr(a_q), _ptr(a_scale), _ptr(w13), _ptr(w13_scale),
          _ptr(sorted_pair_ids), _ptr(padded_offsets), _ptr(tile_expert), _ptr(num_tiles), T, k, E, 2 * Hh, N2 // 2,
          block_m, _ptr(h_q), _ptr(h_scale), _ptr(ws), _nbytes(ws), _stream(stream))


def w8a8_w4a8_grouped_gemm_w13_silu(a_q, a_scale, w13, w13_scale, sorted_pair_ids, padded_offsets, tile_expert,
                                    num_tiles, T, k, block_m, h_q, h_scale, ws, stream=None) -> None:
    """w13: packed int4 [E, 2I, H/2] (uint8)."""
    _w13_w4(a_q, a_scale, w13, w13_scale, sorted_pair_ids, padded_offsets, tile_expert, num_tiles, T, k, block_m,
            h_q, h_scale, ws, stream)


def w8a8_w4a8_grouped_gemm_w2_combine(h_q, h_scale, w2, w2_scale, sorted_pair_ids, padded_offsets, tile_expert,
                                      num_tiles, topk_weights, T, k, block_m, out, ws, stream=None) -> None:
    """w2: packed int4 [E, H, I/2] (uint8)."""
    E, H, Ih = w2.shape
    _call("w8a8_w4a8_grouped_gemm_w2_combine", _ptr(h_q), _ptr(h_scale), _ptr(w2), _ptr(w2_scale),
          _ptr(sorted_pair_ids), _ptr(padded_offsets), _ptr(tile_expert), _ptr(num_tiles), _ptr(topk_weights), T, k,
          E, H, 2 * Ih, block_m, _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream))


def w8a8_linear_workspace_bytes(M: int, N: int, K: int) -> int:
    return lib().w8a8_linear_workspace_bytes(M, N, K)


def w8a8_linear(a_q, a_scale, w, w_scale, out, ws, stream=None) -> None:
    """out[M, N] fp32 = ((float)(a_q . w) * a_scale[m]) * w_scale[n]; a_q [M, K] int8, w [N, K] int8."""
    M, K = a_q.shape
    N = w.shape[0]
    _call("w8a8_linear", _ptr(a_q), _ptr(a_scale), _ptr(w), _ptr(w_scale), M, N, K, _ptr(out), _ptr(ws),
          _nbytes(ws), _stream(stream))


def w8a8_moe_pick_block_m(T: int, k: int, E: int) -> int:
    return lib().w8a8_moe_pick_block_m(T, k, E)


def w8a8_moe_workspace_bytes(T, k, E, H, I, block_m=0, scale_mode=SCALE_CHANNEL) -> int:
    return lib().w8a8_moe_workspace_bytes(T, k, E, H, I, block_m, scale_mode)


def w8a8_moe_forward(x, router_logits, w13, w13_scale, w2, w2_scale, out, ws, *, k: int, score_fn: int,
                     n_group: int = 1, topk_group: int = 1, renormalize: bool = True, routed_scaling: float = 1.0,
                     correction_bias=None, scale_mode: int = SCALE_CHANNEL, block_m: int = 0, topk_ids=None,
                     topk_weights=None, stream=None) -> None:
    T, H = x.shape
    E, N2, _ = w13.shape
    args = MoEArgs(x=_ptr(x), x_dtype=_dtype_code(x), router_logits=_ptr(router_logits), w13=_ptr(w13),
                   w13_scale=_ptr(w13_scale), w2=_ptr(w2), w2_scale=_ptr(w2_scale),
                   correction_bias=_ptr(correction_bias), out=_ptr(out), topk_ids=_ptr(topk_ids),
                   topk_weights=_ptr(topk_weights), T=T, H=H, I=N2 // 2, E=E, k=k, score_fn=score_fn,
                   n_group=n_group, topk_group=topk_group, renormalize=int(renormalize),
                   routed_scaling=routed_scaling, scale_mode=scale_mode, block_m=block_m)
    _call("w8a8_moe_forward", ctypes.byref(args), _ptr(ws), _nbytes(ws), _stream(stream))
