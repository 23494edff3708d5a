"""CPU oracle of the W8A8 INT8 fused-MoE layer (numpy front end of liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``__graft_entry__.smoke()``
and by the benchmark's CPU-baseline leg, never by the product path.  It shares
no code with the HIP path; the two meet only through the seeded input
generator in ``synth/``.

What each function computes, and the passage it follows, is documented in
``oracle.c``.  Parity pins: the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` check these functions against closed forms,
hand-worked values, brute force and invariants that the pages and the
mathematics fix.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Iterable, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

SOFTMAX = 0
SIGMOID = 1


def _load():
    global _lib
    if _lib is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        lib = ctypes.CDLL(path)
        i64, i32, f32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
        lib.oracle_quant_blocks.argtypes = [vp, i64, i64, i64, i64, vp, vp]
        lib.oracle_route.argtypes = [vp, i64, i64, i64, i32, i64, i64, i32, f32, vp, vp, vp]
        lib.oracle_align.argtypes = [vp, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp]
        lib.oracle_grouped_gemm_i32.argtypes = [vp, i64, i32, vp, i64, vp, vp, i64, i64, i64, vp, i64, vp]
        lib.oracle_w13_silu.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp, i64,
                                        vp, vp]
        lib.oracle_w2_combine.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, vp, i64, i64, i64, i64, i32,
                                          vp, i64, vp]
        lib.oracle_moe_tokens.argtypes = [vp, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, i32, vp]
        lib.oracle_linear.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, i64, vp]
        lib.oracle_fp8_decode.argtypes = [vp, i64, vp]
        lib.oracle_fp8_encode.argtypes = [vp, i64, vp]
        lib.oracle_fp8_quant_blocks.argtypes = [vp, i64, i64, i64, i64, vp, vp]
        lib.oracle_fp8_w13_silu.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, i64, vp, vp]
        lib.oracle_fp8_w2_combine.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, vp, i64, i64, i64, i64, vp, i64,
                                              vp]
        lib.oracle_fp8_moe_tokens.argtypes = [vp, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp]
        lib.oracle_w4_unpack.argtypes = [vp, i64, i64, vp]
        lib.oracle_w4_quant.argtypes = [vp, i64, i64, vp, vp]
        lib.oracle_w4_w13_silu.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, i64, vp, vp]
        lib.oracle_w4_w2_combine.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, vp, i64, i64, i64, i64, vp, i64, vp]
        lib.oracle_w4_moe_tokens.argtypes = [vp, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp]
        for name in ("oracle_w4_unpack", "oracle_w4_quant", "oracle_w4_w13_silu", "oracle_w4_w2_combine",
                     "oracle_w4_moe_tokens"):
            getattr(lib, name).restype = None
        for name in ("oracle_quant_blocks", "oracle_route", "oracle_align", "oracle_grouped_gemm_i32",
                     "oracle_w13_silu", "oracle_w2_combine", "oracle_moe_tokens", "oracle_linear",
                     "oracle_fp8_decode", "oracle_fp8_encode", "oracle_fp8_quant_blocks", "oracle_fp8_w13_silu",
                     "oracle_fp8_w2_combine", "oracle_fp8_moe_tokens"):
            getattr(lib, name).restype = None
        _lib = lib
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _ptr_array(arrs: Sequence[Optional[np.ndarray]]):
    """ctypes array of per-expert pointers (NULL where an expert is not materialised)."""
    out = (ctypes.c_void_p * len(arrs))()
    for i, a in enumerate(arrs):
        out[i] = None if a is None else a.ctypes.data
    return out


def _experts(w, dtype) -> List[Optional[np.ndarray]]:
    """Accepts a dense [E, ...] array or a per-expert list (None = absent)."""
    if isinstance(w, np.ndarray):
        return [_c(w[e], dtype) for e in range(w.shape[0])]
    return [None if x is None else _c(x, dtype) for x in w]


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------- quantization

def quant_blocks(x: np.ndarray, br: int, bc: int):
    """Symmetric INT8, one scale per br x bc block: returns (q int8 [rows, cols], s fp32 [nbr, nbc])."""
    x = _c(x, np.float32)
    rows, cols = x.shape
    q = np.empty((rows, cols), dtype=np.int8)
    s = np.empty(((rows + br - 1) // br, (cols + bc - 1) // bc), dtype=np.float32)
    if rows and cols:
        _load().oracle_quant_blocks(_p(x), rows, cols, br, bc, _p(q), _p(s))
    return q, s


def quant_per_token(x: np.ndarray, group: int = 0):
    """Online activation quantization: per token (group=0) -> s [rows]; per token-group -> s [rows, cols/group]."""
    x = _c(x, np.float32)
    rows, cols = x.shape
    q, s = quant_blocks(x, 1, cols if group == 0 else group)
    return q, (s.reshape(rows) if group == 0 else s)


def quant_weight(w: np.ndarray, mode: str):
    """Offline weight quantization of one expert [N, K]: per output channel -> s [N];
    128x128 blocks -> s [N/128, K/128]."""
    if mode == "channel":
        q, s = quant_blocks(w, 1, w.shape[1])
        return q, s.reshape(w.shape[0])
    q, s = quant_blocks(w, 128, 128)
    return q, s


# --------------------------------------------------------------------------- routing

def route(logits: np.ndarray, k: int, score_fn: int, n_group: int = 1, topk_group: int = 1,
          renormalize: bool = True, routed_scaling: float = 1.0, bias: Optional[np.ndarray] = None):
    lg = _c(logits, np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    b = None if bias is None else _c(bias, np.float32)
    if T:
        _load().oracle_route(_p(lg), T, E, k, score_fn, n_group, topk_group, int(renormalize),
                             routed_scaling, _p(b), _p(ids), _p(w))
    return ids, w


def route_cfg(cfg, logits: np.ndarray):
    """Routing rule of a synthetic workload (the Zipf skew lives in the logits, not in a bias)."""
    fn = SOFTMAX if cfg.route == "softmax" else SIGMOID
    return route(logits, cfg.k, fn, cfg.n_group, cfg.topk_group, cfg.renormalize, cfg.routed_scaling)


# --------------------------------------------------------------------------- align

def max_rows(P: int, E: int, block_m: int) -> int:
    return P + E * (block_m - 1)


def align(ids: np.ndarray, E: int, block_m: int) -> Dict[str, np.ndarray]:
    ids = _c(ids, np.int32)
    T, k = ids.shape
    P = T * k
    R = max_rows(P, E, block_m)
    out = dict(counts=np.empty(E, np.int32), offsets=np.empty(E + 1, np.int32),
               padded_offsets=np.empty(E + 1, np.int32), sorted_pair_ids=np.full(max(R, 1), -1, np.int32),
               tile_expert=np.full(max(R // block_m, 1), -1, np.int32), num_tiles=np.zeros(1, np.int32))
    _load().oracle_align(_p(ids), T, k, E, block_m, _p(out["counts"]), _p(out["offsets"]),
                         _p(out["padded_offsets"]), _p(out["sorted_pair_ids"]), _p(out["tile_expert"]),
                         _p(out["num_tiles"]))
    return out


# --------------------------------------------------------------------------- grouped stages

def _rows(rows: Optional[Iterable[int]], num_tiles: int, block_m: int):
    if rows is None:
        return None, num_tiles * block_m
    r = np.ascontiguousarray(np.fromiter(rows, dtype=np.int64))
    return r, len(r)


def grouped_gemm_i32(a: np.ndarray, gather: bool, w, al: Dict[str, np.ndarray], block_m: int, P: int, k: int,
                     rows: Optional[Iterable[int]] = None) -> np.ndarray:
    """Raw int32 accumulators per sorted row ([num_tiles*block_m, N]; rows not computed stay 0)."""
    a = _c(a, np.int8)
    ws = _experts(w, np.int8)
    N = next(x.shape[0] for x in ws if x is not None)
    K = a.shape[1]
    nt = int(al["num_tiles"][0])
    r, nr = _rows(rows, nt, block_m)
    out = np.zeros((nt * block_m, N), dtype=np.int32)
    _load().oracle_grouped_gemm_i32(_p(a), K, int(gather), _ptr_array(ws), N, _p(al["sorted_pair_ids"]),
                                    _p(al["tile_expert"]), block_m, P, k, _p(r), nr, _p(out))
    return out


def w13_silu(a_q: np.ndarray, a_s: np.ndarray, w13, w13_s, al: Dict[str, np.ndarray], block_m: int, T: int,
             k: int, H: int, I: int, block: bool, rows: Optional[Iterable[int]] = None):
    """Sorted-row intermediate: h_q [R, I] int8 and h_s [R] (channel) or [R, I/128] (block)."""
    a_q = _c(a_q, np.int8)
    a_s = _c(a_s, np.float32)
    wq = _experts(w13, np.int8)
    wsc = _experts(w13_s, np.float32)
    nt = int(al["num_tiles"][0])
    R = nt * block_m
    r, nr = _rows(rows, nt, block_m)
    h_q = np.zeros((R, I), dtype=np.int8)
    h_s = np.zeros((R, I // 128) if block else (R,), dtype=np.float32)
    _load().oracle_w13_silu(_p(a_q), _p(a_s), _ptr_array(wq), _ptr_array(wsc), _p(al["sorted_pair_ids"]),
                            _p(al["tile_expert"]), block_m, T, k, H, I, int(block), _p(r), nr, _p(h_q),
                            _p(h_s))
    return h_q, h_s


def w2_combine(h_q: np.ndarray, h_s: np.ndarray, w2, w2_s, al: Dict[str, np.ndarray], block_m: int,
               topk_weights: np.ndarray, T: int, k: int, H: int, I: int, block: bool,
               tokens: Optional[Iterable[int]] = None) -> np.ndarray:
    """Combined output rows: [T, H], or [len(tokens), H] for the listed tokens."""
    h_q = _c(h_q, np.int8)
    h_s = _c(h_s, np.float32)
    wq = _experts(w2, np.int8)
    wsc = _experts(w2_s, np.float32)
    tw = _c(topk_weights, np.float32)
    tk = None if tokens is None else np.ascontiguousarray(np.fromiter(tokens, dtype=np.int64))
    ntok = T if tk is None else len(tk)
    out = np.empty((ntok, H), dtype=np.float32)
    _load().oracle_w2_combine(_p(h_q), _p(h_s), _ptr_array(wq), _ptr_array(wsc), _p(al["sorted_pair_ids"]),
                              _p(al["tile_expert"]), int(al["num_tiles"][0]), block_m, _p(tw), T, k, H, I,
                              int(block), _p(tk), ntok, _p(out))
    return out


def linear(a_q: np.ndarray, a_s: np.ndarray, w: np.ndarray, w_s: np.ndarray,
           rows: Optional[Iterable[int]] = None) -> np.ndarray:
    """Dense W8A8 linear: out [M, N] fp32 = ((float)(a_q . w) * a_s[m]) * w_s[n]; with `rows`, only
    those rows are computed (the others are zero)."""
    a_q = _c(a_q, np.int8)
    w = _c(w, np.int8)
    a_s = _c(a_s, np.float32)
    w_s = _c(w_s, np.float32)
    M, K = a_q.shape
    N = w.shape[0]
    assert w.shape[1] == K and a_s.shape == (M,) and w_s.shape == (N,)
    out = np.zeros((M, N), dtype=np.float32)
    r = None if rows is None else _c(np.asarray(list(rows), dtype=np.int64), np.int64)
    _load().oracle_linear(_p(a_q), _p(a_s), _p(w), _p(w_s), M, N, K, None if r is None else _p(r),
                          0 if r is None else len(r), _p(out))
    return out


def moe_tokens(x: np.ndarray, ids: np.ndarray, topk_weights: np.ndarray, w13, w13_s, w2, w2_s,
               I: int, block: bool) -> np.ndarray:
    """Dense per-token reference of the whole layer for the given token rows (fp32 x)."""
    x = _c(x, np.float32)
    ntok, H = x.shape
    ids = _c(ids, np.int32)
    k = ids.shape[1]
    tw = _c(topk_weights, np.float32)
    out = np.empty((ntok, H), dtype=np.float32)
    _load().oracle_moe_tokens(_p(x), ntok, H, I, k, _p(ids), _p(tw), _ptr_array(_experts(w13, np.int8)),
                              _ptr_array(_experts(w13_s, np.float32)), _ptr_array(_experts(w2, np.int8)),
                              _ptr_array(_experts(w2_s, np.float32)), int(block), _p(out))
    return out


# --------------------------------------------------------------------------- FP8 (E4M3) block-wise path

def fp8_decode(codes: np.ndarray) -> np.ndarray:
    """Values of E4M3 codes (uint8) as fp32 (exact)."""
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, dtype=np.float32)
    if c.size:
        _load().oracle_fp8_decode(_p(c), c.size, _p(out))
    return out


def fp8_encode(x: np.ndarray) -> np.ndarray:
    """E4M3 codes nearest to fp32 values (clamped to +-448, ties to even, zero keeps the sign)."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    if x.size:
        _load().oracle_fp8_encode(_p(x), x.size, _p(out))
    return out


def fp8_quant_blocks(x: np.ndarray, br: int, bc: int):
    """FP8 E4M3, one scale per br x bc block: (codes uint8 [rows, cols], s fp32 [nbr, nbc])."""
    x = _c(x, np.float32)
    rows, cols = x.shape
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty(((rows + br - 1) // br, (cols + bc - 1) // bc), dtype=np.float32)
    if rows and cols:
        _load().oracle_fp8_quant_blocks(_p(x), rows, cols, br, bc, _p(q), _p(s))
    return q, s


def fp8_w13_silu(a_q: np.ndarray, a_s: np.ndarray, w13, w13_s, al: Dict[str, np.ndarray], block_m: int, T: int,
                 k: int, H: int, I: int, rows: Optional[Iterable[int]] = None):
    """FP8 sorted-row intermediate: h_q [R, I] codes and h_s [R, I/128]."""
    a_q = _c(a_q, np.uint8)
    a_s = _c(a_s, np.float32)
    nt = int(al["num_tiles"][0])
    R = nt * block_m
    r, nr = _rows(rows, nt, block_m)
    h_q = np.zeros((R, I), dtype=np.uint8)
    h_s = np.zeros((R, I // 128), dtype=np.float32)
    _load().oracle_fp8_w13_silu(_p(a_q), _p(a_s), _ptr_array(_experts(w13, np.uint8)),
                                _ptr_array(_experts(w13_s, np.float32)), _p(al["sorted_pair_ids"]),
                                _p(al["tile_expert"]), block_m, T, k, H, I, _p(r), nr, _p(h_q), _p(h_s))
    return h_q, h_s


def fp8_w2_combine(h_q: np.ndarray, h_s: np.ndarray, w2, w2_s, al: Dict[str, np.ndarray], block_m: int,
                   topk_weights: np.ndarray, T: int, k: int, H: int, I: int,
                   tokens: Optional[Iterable[int]] = None) -> np.ndarray:
    """FP8 second GEMM + combine: [T, H], or [len(tokens), H] for the listed tokens."""
    h_q = _c(h_q, np.uint8)
    h_s = _c(h_s, np.float32)
    tw = _c(topk_weights, np.float32)
    tk = None if tokens is None else np.ascontiguousarray(np.fromiter(tokens, dtype=np.int64))
    ntok = T if tk is None else len(tk)
    out = np.empty((ntok, H), dtype=np.float32)
    _load().oracle_fp8_w2_combine(_p(h_q), _p(h_s), _ptr_array(_experts(w2, np.uint8)),
                                  _ptr_array(_experts(w2_s, np.float32)), _p(al["sorted_pair_ids"]),
                                  _p(al["tile_expert"]), int(al["num_tiles"][0]), block_m, _p(tw), T, k, H, I,
                                  _p(tk), ntok, _p(out))
    return out


def fp8_moe_tokens(x: np.ndarray, ids: np.ndarray, topk_weights: np.ndarray, w13, w13_s, w2, w2_s,
                   I: int) -> np.ndarray:
    """Dense per-token reference of the whole FP8 layer for the given token rows (fp32 x)."""
    x = _c(x, np.float32)
    ntok, H = x.shape
    ids = _c(ids, np.int32)
    k = ids.shape[1]
    tw = _c(topk_weights, np.float32)
    out = np.empty((ntok, H), dtype=np.float32)
    _load().oracle_fp8_moe_tokens(_p(x), ntok, H, I, k, _p(ids), _p(tw), _ptr_array(_experts(w13, np.uint8)),
                                  _ptr_array(_experts(w13_s, np.float32)), _ptr_array(_experts(w2, np.uint8)),
                                  _ptr_array(_experts(w2_s, np.float32)), _p(out))
    return out


def fp8_abs(codes: np.ndarray) -> np.ndarray:
    """Codes of the magnitudes (sign bit cleared): feeding these and |scales| through the same
    functions gives the sums of absolute terms that bound rounding differences."""
    return np.asarray(codes, dtype=np.uint8) & np.uint8(0x7F)


# --------------------------------------------------------------------------- W4A8 path (int4 weights, FP8 activations)

def w4_quant(x: np.ndarray):
    """Int4 weights, one scale per (row, 128 columns): (packed uint8 [rows, cols/2], s fp32 [rows, cols/128])."""
    x = _c(x, np.float32)
    rows, cols = x.shape
    q = np.empty((rows, cols // 2), dtype=np.uint8)
    s = np.empty((rows, cols // 128), dtype=np.float32)
    if rows and cols:
        _load().oracle_w4_quant(_p(x), rows, cols, _p(q), _p(s))
    return q, s


def w4_unpack(packed: np.ndarray) -> np.ndarray:
    """Integer values [rows, 2 * bytes] of packed int4 rows."""
    q = _c(packed, np.uint8)
    rows, nb = q.shape
    out = np.empty((rows, 2 * nb), dtype=np.int8)
    if q.size:
        _load().oracle_w4_unpack(_p(q), rows, 2 * nb, _p(out))
    return out


def w4_w13_silu(a_q: np.ndarray, a_s: np.ndarray, w13, w13_s, al: Dict[str, np.ndarray], block_m: int, T: int,
                k: int, H: int, I: int, rows: Optional[Iterable[int]] = None):
    """W4A8 sorted-row intermediate: h_q [R, I] FP8 codes and h_s [R, I/128]."""
    a_q = _c(a_q, np.uint8)
    a_s = _c(a_s, np.float32)
    nt = int(al["num_tiles"][0])
    R = nt * block_m
    r, nr = _rows(rows, nt, block_m)
    h_q = np.zeros((R, I), dtype=np.uint8)
    h_s = np.zeros((R, I // 128), dtype=np.float32)
    _load().oracle_w4_w13_silu(_p(a_q), _p(a_s), _ptr_array(_experts(w13, np.uint8)),
                               _ptr_array(_experts(w13_s, np.float32)), _p(al["sorted_pair_ids"]),
                               _p(al["tile_expert"]), block_m, T, k, H, I, _p(r), nr, _p(h_q), _p(h_s))
    return h_q, h_s


def w4_w2_combine(h_q: np.ndarray, h_s: np.ndarray, w2, w2_s, al: Dict[str, np.ndarray], block_m: int,
                  topk_weights: np.ndarray, T: int, k: int, H: int, I: int,
                  tokens: Optional[Iterable[int]] = None) -> np.ndarray:
    """W4A8 second GEMM + combine: [T, H], or [len(tokens), H] for the listed tokens."""
    h_q = _c(h_q, np.uint8)
    h_s = _c(h_s, np.float32)
    tw = _c(topk_weights, np.float32)
    tk = None if tokens is None else np.ascontiguousarray(np.fromiter(tokens, dtype=np.int64))
    ntok = T if tk is None else len(tk)
    out = np.empty((ntok, H), dtype=np.float32)
    _load().oracle_w4_w2_combine(_p(h_q), _p(h_s), _ptr_array(_experts(w2, np.uint8)),
                                 _ptr_array(_experts(w2_s, np.float32)), _p(al["sorted_pair_ids"]),
                                 _p(al["tile_expert"]), int(al["num_tiles"][0]), block_m, _p(tw), T, k, H, I,
                                 _p(tk), ntok, _p(out))
    return out


def w4_moe_tokens(x: np.ndarray, ids: np.ndarray, topk_weights: np.ndarray, w13, w13_s, w2, w2_s,
                  I: int) -> np.ndarray:
    """Dense per-token reference of the whole W4A8 layer for the given token rows (fp32 x)."""
    x = _c(x, np.float32)
    ntok, H = x.shape
    ids = _c(ids, np.int32)
    k = ids.shape[1]
    tw = _c(topk_weights, np.float32)
    out = np.empty((ntok, H), dtype=np.float32)
    _load().oracle_w4_moe_tokens(_p(x), ntok, H, I, k, _p(ids), _p(tw), _ptr_array(_experts(w13, np.uint8)),
                                 _ptr_array(_experts(w13_s, np.float32)), _ptr_array(_experts(w2, np.uint8)),
                                 _ptr_array(_experts(w2_s, np.float32)), _p(out))
    return out


def w4_abs(packed: np.ndarray) -> np.ndarray:
    """Packed int4 rows of the magnitudes (sign bits cleared)."""
    return np.asarray(packed, dtype=np.uint8) & np.uint8(0x77)


# --------------------------------------------------------------------------- layer construction

def expert_weights(cfg, experts: Iterable[int]):
    """Oracle-side quantized weights of the listed experts of a synthetic workload, drawn
    from the shared generator and quantized here.  Returns per-expert lists (None for
    experts not listed): w13_q [2I,H], w13_s, w2_q [H,I], w2_s."""
    import synth

    mode = cfg.scale_mode
    E = cfg.E
    w13_q: List[Optional[np.ndarray]] = [None] * E
    w13_s: List[Optional[np.ndarray]] = [None] * E
    w2_q: List[Optional[np.ndarray]] = [None] * E
    w2_s: List[Optional[np.ndarray]] = [None] * E
    for e in sorted(set(int(x) for x in experts)):
        if mode == "w4a8":
            w13_q[e], w13_s[e] = w4_quant(synth.w13_f32(cfg, e))
            w2_q[e], w2_s[e] = w4_quant(synth.w2_f32(cfg, e))
            continue
        if mode == "fp8":
            w13_q[e], w13_s[e] = fp8_quant_blocks(synth.w13_f32(cfg, e), 128, 128)
            w2_q[e], w2_s[e] = fp8_quant_blocks(synth.w2_f32(cfg, e), 128, 128)
            continue
        w13_q[e], w13_s[e] = quant_weight(synth.w13_f32(cfg, e), mode)
        w2_q[e], w2_s[e] = quant_weight(synth.w2_f32(cfg, e), mode)
    return w13_q, w13_s, w2_q, w2_s


def activations_f32(cfg, rows: Optional[slice] = None) -> np.ndarray:
    import synth

    x = synth.activations(cfg, rows)
    return bf16_to_f32(x) if x.dtype == np.uint16 else x
