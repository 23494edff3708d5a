"""Pins of the CPU oracle's FP8 (E4M3) block-wise path.

Source: SGLang PR #8273 (cutlass_moe_fp8: per-block FP8 weights, per-token-group FP8
activations, a block-scaled grouped GEMM).  The pages name the scheme only; the format is
the OCP E4M3 format, so its pins are facts of that format (hand-worked code values, and
PyTorch's own float8_e4m3fn conversion as an independent implementation), and the GEMM
pins are exact special cases (integer-valued codes, where the FP8 path must equal the
pinned INT8 block-wise path bit for bit), the exact fp64 result within the rounding bound,
and invariants of the pipeline.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

U = 2.0 ** -24  # fp32 unit roundoff


def small_cfg(name="fp8-small", index=50, T=48, H=512, I=256, E=16, k=4, route="sigmoid", n_group=4,
              topk_group=2, scaling=2.5, x_dtype=synth.DTYPE_BF16, w_sigma=0.006):
    return synth.MoEConfig(name=name, index=index, T=T, H=H, I=I, E=E, k=k, route=route, n_group=n_group,
                           topk_group=topk_group, routed_scaling=scaling, renormalize=True, x_dtype=x_dtype,
                           x_sigma=1.0, outlier_threshold=synth.OUTLIER_THRESHOLD, outlier_mult=20.0,
                           w_sigma=w_sigma, scale_mode="fp8")


def torch_e4m3(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).float().numpy()


# ---------------------------------------------------------------- the format

def test_fp8_decode_hand_worked_values():
    v = oracle.fp8_decode(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x3F, 0x40, 0x7E, 0xB8, 0xFE], dtype=np.uint8))
    # subnormals m/8 * 2^-6, normals (1 + m/8) * 2^(e-7), largest finite 448 = 1.75 * 2^8
    assert list(v) == [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.875, 2.0, 448.0, -1.0, -448.0]
    assert np.signbit(oracle.fp8_decode(np.array([0x80], dtype=np.uint8))[0])


def test_fp8_decode_matches_torch_on_every_finite_code():
    c = np.arange(256, dtype=np.uint8)
    finite = (c & 0x7F) != 0x7F
    assert np.array_equal(oracle.fp8_decode(c)[finite], torch_e4m3(c)[finite])
    # values are strictly increasing in the code over the non-negative half
    v = oracle.fp8_decode(c[:0x7F])
    assert np.all(np.diff(v) > 0)


def test_fp8_encode_ties_neighbours_saturation_sign():
    c = np.arange(0x7E, dtype=np.uint8)
    lo, hi = oracle.fp8_decode(c), oracle.fp8_decode(c + 1)
    mid = ((lo.astype(np.float64) + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo.astype(np.float64) + hi) / 2)  # midpoints are fp32 values
    even = np.where(c % 2 == 0, c, c + 1).astype(np.uint8)
    assert np.array_equal(oracle.fp8_encode(mid), even)
    assert np.array_equal(oracle.fp8_encode(np.nextafter(mid, np.float32(np.inf))), c + 1)
    assert np.array_equal(oracle.fp8_encode(np.nextafter(mid, np.float32(0))), c)
    assert np.array_equal(oracle.fp8_encode(-mid), even | 0x80)
    assert np.array_equal(oracle.fp8_encode(lo), c)  # exact values map to themselves
    big = np.array([448.0, 449.0, 464.0, 500.0, 1e6, 3e38], dtype=np.float32)
    assert np.all(oracle.fp8_encode(big) == 0x7E) and np.all(oracle.fp8_encode(-big) == 0xFE)
    tiny = np.array([1e-30, 2.0 ** -11, 2.0 ** -10], dtype=np.float32)  # 2^-10 is the tie between 0 and 2^-9
    assert list(oracle.fp8_encode(tiny)) == [0x00, 0x00, 0x00]
    assert list(oracle.fp8_encode(-tiny)) == [0x80, 0x80, 0x80]
    assert oracle.fp8_encode(np.array([np.float32(2.0 ** -10) * np.float32(1.0000001)]))[0] == 0x01


def test_fp8_encode_matches_torch():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(100000) * 60, rng.standard_normal(20000) * 1e-3,
                        rng.uniform(-448, 448, 20000)]).astype(np.float32)
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.fp8_encode(x), ref)


# ---------------------------------------------------------------- the quantization rule

@pytest.mark.parametrize("br,bc", [(1, 128), (128, 128), (1, 384)])
def test_fp8_quant_rule(br, bc):
    x = synth.normal(300 * 384, 7, 0, sigma=3.0).astype(np.float32).reshape(300, 384)
    x[5, :128] = 0.0
    q, s = oracle.fp8_quant_blocks(x, br, bc)
    nbr, nbc = s.shape
    for bi in range(nbr):
        for bj in range(nbc):
            blk = x[bi * br:(bi + 1) * br, bj * bc:(bj + 1) * bc]
            qb = q[bi * br:(bi + 1) * br, bj * bc:(bj + 1) * bc]
            amax = np.abs(blk).max()
            assert s[bi, bj] == max(np.float32(amax) / np.float32(448.0), np.float32(1e-8))
            if amax == 0:
                assert np.all((qb & 0x7F) == 0)
                continue
            # the largest magnitude lands on +-448
            i = np.unravel_index(np.abs(blk).argmax(), blk.shape)
            assert qb[i] & 0x7F == 0x7E
            # round-trip error: half a step of a 3-bit mantissa, or half the subnormal step
            err = np.abs(oracle.fp8_decode(qb).astype(np.float64) * s[bi, bj] - blk)
            bound = np.maximum(2.0 ** -4 * np.abs(blk), 2.0 ** -10 * s[bi, bj]) * (1 + 1e-6)
            assert np.all(err <= bound)


# ---------------------------------------------------------------- the block-scaled GEMMs

def integer_codes(shape, seed):
    """FP8 codes of integers in [-16, 16] (all exact in E4M3), and the same integers as int8."""
    v = np.random.default_rng(seed).integers(-16, 17, size=shape).astype(np.int8)
    c = oracle.fp8_encode(v.astype(np.float32))
    assert np.array_equal(oracle.fp8_decode(c), v.astype(np.float32))
    return c, v


def routing(T, E, k, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    tw = rng.uniform(0.1, 1.0, size=(T, k)).astype(np.float32)
    return ids, tw


def test_fp8_second_gemm_equals_int8_block_path_on_integer_codes():
    """With integer-valued codes every K-block sum is an exact integer on both paths, so the FP8
    path must reproduce the (pinned) INT8 block-wise second GEMM + combine bit for bit."""
    T, E, k, H, I, bm = 40, 6, 2, 256, 384, 16
    ids, tw = routing(T, E, k, 3)
    al = oracle.align(ids, E, bm)
    R = int(al["num_tiles"][0]) * bm
    hc, hv = integer_codes((R, I), 11)
    h_s = synth.positive_scales(R * (I // 128), 4, 1e-3, 3e-2).reshape(R, I // 128)
    w2c, w2v, w2s = [], [], []
    for e in range(E):
        c, v = integer_codes((H, I), 20 + e)
        w2c.append(c)
        w2v.append(v)
        w2s.append(synth.positive_scales((H // 128) * (I // 128), 30 + e, 1e-3, 3e-2).reshape(H // 128, I // 128))
    got = oracle.fp8_w2_combine(hc, h_s, w2c, w2s, al, bm, tw, T, k, H, I)
    ref = oracle.w2_combine(hv, h_s, w2v, w2s, al, bm, tw, T, k, H, I, True)
    assert np.array_equal(got, ref)
    # a swapped scale-block index (a plausible layout mistake) breaks it
    bad = oracle.fp8_w2_combine(hc, h_s, w2c, [s.T.copy() if s.shape[0] == s.shape[1] else s[::-1].copy()
                                                for s in w2s], al, bm, tw, T, k, H, I)
    assert not np.array_equal(bad, ref)


def fp8_w13_fp64(a_c, a_s, w_c, w_s, I):
    """SiLU(gate) * up of one token row against one expert in fp64 from the decoded values."""
    a = oracle.fp8_decode(a_c).astype(np.float64) * np.repeat(a_s.astype(np.float64), 128)
    wf = oracle.fp8_decode(w_c).astype(np.float64) * np.repeat(np.repeat(w_s.astype(np.float64), 128, 0), 128, 1)
    gu = wf @ a
    g, u = gu[:I], gu[I:]
    return g / (1 + np.exp(-g)) * u


def test_fp8_first_gemm_within_rounding_of_fp64():
    cfg = small_cfg()
    x = oracle.activations_f32(cfg)
    ids, _ = oracle.route_cfg(cfg, synth.logits(cfg))
    w = oracle.expert_weights(cfg, range(cfg.E))
    a_c, a_s = oracle.fp8_quant_blocks(x, 1, 128)
    bm = 16
    al = oracle.align(ids, cfg.E, bm)
    h_q, h_s = oracle.fp8_w13_silu(a_c, a_s, w[0], w[1], al, bm, cfg.T, cfg.k, cfg.H, cfg.I)
    P = cfg.T * cfg.k
    checked = 0
    for r in range(int(al["num_tiles"][0]) * bm):
        p = al["sorted_pair_ids"][r]
        if p >= P:
            continue
        e = al["tile_expert"][r // bm]
        hf = fp8_w13_fp64(a_c[p // cfg.k], a_s[p // cfg.k], w[0][e], w[1][e], cfg.I).reshape(-1, 128)
        amax = np.abs(hf).max(1)
        assert np.all(np.abs(h_s[r] - amax / 448) <= 1e-5 * amax / 448)
        deq = oracle.fp8_decode(h_q[r]).astype(np.float64).reshape(-1, 128) * h_s[r][:, None]
        bound = np.maximum(2.0 ** -4 * np.abs(hf), 2.0 ** -10 * h_s[r][:, None]) + 1e-5 * amax[:, None]
        assert np.all(np.abs(deq - hf) <= bound)
        checked += 1
    assert checked == P


def test_fp8_sorted_pipeline_equals_dense_loop():
    cfg = small_cfg()
    x = oracle.activations_f32(cfg)
    ids, tw = oracle.route_cfg(cfg, synth.logits(cfg))
    w = oracle.expert_weights(cfg, range(cfg.E))
    a_c, a_s = oracle.fp8_quant_blocks(x, 1, 128)
    bm = 32
    al = oracle.align(ids, cfg.E, bm)
    h_q, h_s = oracle.fp8_w13_silu(a_c, a_s, w[0], w[1], al, bm, cfg.T, cfg.k, cfg.H, cfg.I)
    out = oracle.fp8_w2_combine(h_q, h_s, w[2], w[3], al, bm, tw, cfg.T, cfg.k, cfg.H, cfg.I)
    dense = oracle.fp8_moe_tokens(x, ids, tw, *w, I=cfg.I)
    assert np.array_equal(out, dense)


def test_fp8_layer_tracks_fp64_layer():
    cfg = small_cfg(T=16, H=256, I=128, E=8, k=2, route="softmax", n_group=1, topk_group=1, scaling=1.0,
                    x_dtype=synth.DTYPE_F32, w_sigma=0.02)
    x = oracle.activations_f32(cfg)
    ids, tw = oracle.route_cfg(cfg, synth.logits(cfg))
    w = oracle.expert_weights(cfg, range(cfg.E))
    out = oracle.fp8_moe_tokens(x, ids, tw, *w, I=cfg.I)
    ref = np.zeros((cfg.T, cfg.H))
    for t in range(cfg.T):
        for j in range(cfg.k):
            e = ids[t, j]
            gu = synth.w13_f32(cfg, e).astype(np.float64) @ x[t].astype(np.float64)
            g, u = gu[: cfg.I], gu[cfg.I:]
            ref[t] += float(tw[t, j]) * (synth.w2_f32(cfg, e).astype(np.float64) @ (g / (1 + np.exp(-g)) * u))
    cos = (out.astype(np.float64) * ref).sum() / np.linalg.norm(out) / np.linalg.norm(ref)
    assert cos >= 0.99, cos
