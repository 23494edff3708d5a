"""Pins of the CPU oracle's W4A8 path (int4 weights, FP8 activations).

Source: SGLang PR #8311 (w4a8 DeepSeek-R1; its layer enables the path with a w4afp8 flag).  The
pages name the scheme only; the int4 format, its packing and the per-(row, 128) weight scales are
readings.  Pins: hand-packed bytes, the quantization rule, the W4A8 second GEMM equal bit for bit
to the (pinned) INT8 block-wise oracle when both see the same integers and the weight scales are
constant over each 128 x 128 block, the first GEMM within rounding of fp64, sorted == dense, and
the layer tracking the unquantized fp64 layer.
"""
import numpy as np
import pytest

import oracle
import synth


def small_cfg(name="w4-small", index=70, T=48, H=512, I=256, E=16, k=4, route="sigmoid", n_group=4,
              topk_group=2, scaling=2.5, x_dtype=synth.DTYPE_BF16, w_sigma=0.006):
    return synth.MoEConfig(name=name, index=index, T=T, H=H, I=I, E=E, k=k, route=route, n_group=n_group,
                           topk_group=topk_group, routed_scaling=scaling, renormalize=True, x_dtype=x_dtype,
                           x_sigma=1.0, outlier_threshold=synth.OUTLIER_THRESHOLD, outlier_mult=20.0,
                           w_sigma=w_sigma, scale_mode="w4a8")


def test_w4_packing_hand_worked():
    # one row of 128 values: 0..7, then -1..-7 and 0, then zeros; the group's max |w| = 7 -> scale 1
    x = np.zeros((1, 128), dtype=np.float32)
    x[0, :8] = [0, 1, 2, 3, 4, 5, 6, 7]
    x[0, 8:16] = [-1, -2, -3, -4, -5, -6, -7, 0]
    q, s = oracle.w4_quant(x)
    assert s[0, 0] == 1.0
    # byte b of an 8-value group: value b in the low nibble, value 4+b in the high nibble;
    # nibble = sign (bit 3) | magnitude
    assert list(q[0, :4]) == [0x40, 0x51, 0x62, 0x73]
    assert list(q[0, 4:8]) == [0xD9, 0xEA, 0xFB, 0x0C]
    assert np.all(q[0, 8:] == 0)
    assert np.array_equal(oracle.w4_unpack(q)[0], x[0].astype(np.int8))


@pytest.mark.parametrize("sigma", [0.02, 3.0])
def test_w4_quant_rule(sigma):
    x = synth.normal(64 * 512, 12, 0, sigma=sigma).astype(np.float32).reshape(64, 512)
    x[3, 128:256] = 0.0
    q, s = oracle.w4_quant(x)
    v = oracle.w4_unpack(q).astype(np.float64)
    assert v.min() >= -7 and v.max() <= 7
    g = np.abs(x).reshape(64, 4, 128).max(-1)
    assert np.array_equal(s, np.maximum(g / np.float32(7.0), np.float32(1e-8)).astype(np.float32))
    deq = v * np.repeat(s.astype(np.float64), 128, 1)
    assert np.all(np.abs(deq - x) <= 0.5 * np.repeat(s.astype(np.float64), 128, 1) * (1 + 1e-6))
    # the largest magnitude of each non-zero group lands on +-7
    big = np.abs(v).reshape(64, 4, 128).max(-1)
    assert np.all(big[g > 0] == 7) and np.all(big[g == 0] == 0)


def routing(T, E, k, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    tw = rng.uniform(0.1, 1.0, size=(T, k)).astype(np.float32)
    return ids, tw


def test_w4_second_gemm_equals_int8_block_path():
    """Integer weights in [-7, 7] with per-row-group scales that are constant over each 128 x 128
    block, and integer-valued FP8 intermediates: every K-block sum is the same exact integer on
    both paths, so the W4A8 oracle must reproduce the INT8 block-wise oracle bit for bit."""
    T, E, k, H, I, bm = 40, 6, 2, 256, 384, 16
    ids, tw = routing(T, E, k, 5)
    al = oracle.align(ids, E, bm)
    R = int(al["num_tiles"][0]) * bm
    rng = np.random.default_rng(9)
    hv = rng.integers(-16, 17, size=(R, I)).astype(np.int8)
    hc = oracle.fp8_encode(hv.astype(np.float32))
    h_s = synth.positive_scales(R * (I // 128), 6, 1e-3, 3e-2).reshape(R, I // 128)
    w4q, w4s, w8q, w8s = [], [], [], []
    for e in range(E):
        wv = rng.integers(-7, 8, size=(H, I)).astype(np.float32)
        q, s = oracle.w4_quant(wv)  # every group's max |w| is 7 here, so scale 1 and q = the integers
        assert np.all(s == 1.0) and np.array_equal(oracle.w4_unpack(q), wv.astype(np.int8))
        blk = synth.positive_scales((H // 128) * (I // 128), 40 + e, 1e-3, 3e-2).reshape(H // 128, I // 128)
        w4q.append(q)
        w4s.append(np.repeat(blk, 128, 0).copy())  # [H, I/128]: per row group, constant over 128 rows
        w8q.append(wv.astype(np.int8))
        w8s.append(blk)
    got = oracle.w4_w2_combine(hc, h_s, w4q, w4s, al, bm, tw, T, k, H, I)
    ref = oracle.w2_combine(hv, h_s, w8q, w8s, al, bm, tw, T, k, H, I, True)
    assert np.array_equal(got, ref)
    # scales of the wrong row (a plausible indexing mistake) break it
    bad = oracle.w4_w2_combine(hc, h_s, w4q, [np.roll(s, 1, 0) for s in w4s], al, bm, tw, T, k, H, I)
    assert not np.array_equal(bad, ref)


def test_w4_first_gemm_within_rounding_of_fp64():
    cfg = small_cfg()
    x = oracle.activations_f32(cfg)
    ids, _ = oracle.route_cfg(cfg, synth.logits(cfg))
    w = oracle.expert_weights(cfg, range(cfg.E))
    a_c, a_s = oracle.fp8_quant_blocks(x, 1, 128)
    bm = 16
    al = oracle.align(ids, cfg.E, bm)
    h_q, h_s = oracle.w4_w13_silu(a_c, a_s, w[0], w[1], al, bm, cfg.T, cfg.k, cfg.H, cfg.I)
    P = cfg.T * cfg.k
    checked = 0
    for r in range(int(al["num_tiles"][0]) * bm):
        p = al["sorted_pair_ids"][r]
        if p >= P:
            continue
        e = al["tile_expert"][r // bm]
        a = oracle.fp8_decode(a_c[p // cfg.k]).astype(np.float64) * np.repeat(a_s[p // cfg.k].astype(np.float64), 128)
        wf = oracle.w4_unpack(w[0][e]).astype(np.float64) * np.repeat(w[1][e].astype(np.float64), 128, 1)
        gu = wf @ a
        g, u = gu[:cfg.I], gu[cfg.I:]
        hf = (g / (1 + np.exp(-g)) * u).reshape(-1, 128)
        amax = np.abs(hf).max(1)
        assert np.all(np.abs(h_s[r] - amax / 448) <= 1e-5 * amax / 448)
        deq = oracle.fp8_decode(h_q[r]).astype(np.float64).reshape(-1, 128) * h_s[r][:, None]
        bound = np.maximum(2.0 ** -4 * np.abs(hf), 2.0 ** -10 * h_s[r][:, None]) + 1e-5 * amax[:, None]
        assert np.all(np.abs(deq - hf) <= bound)
        checked += 1
    assert checked == P


def test_w4_sorted_pipeline_equals_dense_loop():
    cfg = small_cfg()
    x = oracle.activations_f32(cfg)
    ids, tw = oracle.route_cfg(cfg, synth.logits(cfg))
    w = oracle.expert_weights(cfg, range(cfg.E))
    a_c, a_s = oracle.fp8_quant_blocks(x, 1, 128)
    bm = 32
    al = oracle.align(ids, cfg.E, bm)
    h_q, h_s = oracle.w4_w13_silu(a_c, a_s, w[0], w[1], al, bm, cfg.T, cfg.k, cfg.H, cfg.I)
    out = oracle.w4_w2_combine(h_q, h_s, w[2], w[3], al, bm, tw, cfg.T, cfg.k, cfg.H, cfg.I)
    dense = oracle.w4_moe_tokens(x, ids, tw, *w, I=cfg.I)
    assert np.array_equal(out, dense)


def test_w4_layer_tracks_fp64_layer():
    cfg = small_cfg(T=16, H=256, I=128, E=8, k=2, route="softmax", n_group=1, topk_group=1, scaling=1.0,
                    x_dtype=synth.DTYPE_F32, w_sigma=0.02)
    x = oracle.activations_f32(cfg)
    ids, tw = oracle.route_cfg(cfg, synth.logits(cfg))
    w = oracle.expert_weights(cfg, range(cfg.E))
    out = oracle.w4_moe_tokens(x, ids, tw, *w, I=cfg.I)
    ref = np.zeros((cfg.T, cfg.H))
    for t in range(cfg.T):
        for j in range(cfg.k):
            e = ids[t, j]
            gu = synth.w13_f32(cfg, e).astype(np.float64) @ x[t].astype(np.float64)
            g, u = gu[: cfg.I], gu[cfg.I:]
            ref[t] += float(tw[t, j]) * (synth.w2_f32(cfg, e).astype(np.float64) @ (g / (1 + np.exp(-g)) * u))
    cos = (out.astype(np.float64) * ref).sum() / np.linalg.norm(out) / np.linalg.norm(ref)
    assert cos >= 0.97, cos  # measured 0.981: int4 groups of 128 cost ~2% against fp64
