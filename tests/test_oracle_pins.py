"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

None of these compares the oracle with a retyped copy of itself: the checks are
hand-worked values, closed forms, brute force on tiny inputs, invariants and
special cases that reduce to a plain computation done another way (fp64 numpy).
Sources: SGLang PR #3888 (channel-wise INT8 fused MoE, int32 accumulator),
the jiqizhixin Meituan INT8 DeepSeek R1 article ("Quantization exploration":
block-wise [128,128] weights with per-token-group activations; channel-wise
weights with per-token activations and one dequantization after the INT8
matmul), SGLang PR #8273 (offsets = zero-padded cumsum of per-expert counts).
"""
import itertools
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U = 2.0 ** -24  # fp32 unit roundoff


def small_cfg(name="ds-small", index=20, T=48, H=512, I=256, E=16, k=4, route="sigmoid", n_group=4,
              topk_group=2, scaling=2.5, mode="channel", x_dtype=synth.DTYPE_BF16, w_sigma=0.006):
    return synth.MoEConfig(name=name, index=index, T=T, H=H, I=I, E=E, k=k, route=route, n_group=n_group,
                           topk_group=topk_group, routed_scaling=scaling, renormalize=True, x_dtype=x_dtype,
                           x_sigma=1.0, outlier_threshold=synth.OUTLIER_THRESHOLD, outlier_mult=20.0,
                           w_sigma=w_sigma, scale_mode=mode)


def layer(cfg):
    x = oracle.activations_f32(cfg)
    ids, tw = oracle.route_cfg(cfg, synth.logits(cfg))
    w = oracle.expert_weights(cfg, range(cfg.E))
    return x, ids, tw, w


def pipeline(cfg, x, ids, tw, w, block_m):
    """The sorted-row pipeline: quant -> align -> GEMM1+SiLU+requant -> GEMM2+combine."""
    block = cfg.scale_mode == "block"
    a_q, a_s = oracle.quant_per_token(x, 128 if block else 0)
    al = oracle.align(ids, cfg.E, block_m)
    h_q, h_s = oracle.w13_silu(a_q, a_s, w[0], w[1], al, block_m, cfg.T, cfg.k, cfg.H, cfg.I, block)
    out = oracle.w2_combine(h_q, h_s, w[2], w[3], al, block_m, tw, cfg.T, cfg.k, cfg.H, cfg.I, block)
    return out, dict(a_q=a_q, a_s=a_s, al=al, h_q=h_q, h_s=h_s)


# ---------------------------------------------------------------- generator

def test_splitmix64_reference_outputs():
    # First outputs of SplitMix64 from state 1234567 (the generator's published reference run).
    assert list(synth.splitmix64(3, 1234567)) == [6457827717110365317, 3203168211198807973,
                                                  9817491932198370423]


def test_generator_is_a_function_of_the_index():
    a = synth.normal(1000, 5, synth.STREAM_MISC, 0)
    b = synth.normal(300, 5, synth.STREAM_MISC, 700)
    assert np.array_equal(a[700:], b)
    cfg = synth.CONFIGS["decode"]
    x_all = synth.activations(small_cfg(T=8))
    x_tail = synth.activations(small_cfg(T=8), slice(5, 8))
    assert np.array_equal(x_all[5:], x_tail)
    assert not np.array_equal(synth.normal(100, 1, 1), synth.normal(100, 2, 1))
    assert synth.logits(cfg, slice(3, 4)).shape == (1, 256)


def test_generator_moments():
    z = synth.normal(2_000_000, 9, synth.STREAM_MISC).astype(np.float64)
    assert abs(z.mean()) < 5e-3
    assert abs(z.var() - 1.0) < 5e-3
    assert np.abs(z).max() <= 6.0
    # 1% outliers x20 in the activation generator
    x = synth.bf16_bits_to_f32(synth.activations(small_cfg(T=64, H=4096)))
    frac = np.mean(np.abs(x) > 6.5)
    assert 0.007 < frac < 0.011


# ---------------------------------------------------------------- P1/P2 quantization

def _golden_rows():
    rows = []
    with open(os.path.join(GOLDEN, "quant_rounding.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            xs, s, qs = line.split("|")
            rows.append((np.array(xs.split(), np.float32), np.float32(s), np.array(qs.split(), np.int8)))
    return rows


def test_quant_hand_worked_values():
    for x, s, q in _golden_rows():
        qq, ss = oracle.quant_per_token(x[None, :])
        assert ss[0] == s, (x, ss[0], s)
        assert np.array_equal(qq[0], q), (x, qq[0], q)


def _check_roundtrip(x, q, s, br, bc):
    x64 = x.astype(np.float64)
    s_full = np.repeat(np.repeat(s.astype(np.float64), br, 0), bc, 1)[: x.shape[0], : x.shape[1]]
    assert np.abs(q.astype(np.int32)).max() <= 127
    err = np.abs(x64 - q.astype(np.float64) * s_full)
    # half a step, plus the fp32 rounding of x/s before round-half-even: |x/s| <= 127.5,
    # so that rounding moves the quotient by at most 127.5 * 2^-24 steps
    assert np.all(err <= s_full * (0.5 + 128 * U)), (err / s_full).max()
    # the element of largest magnitude in each block lands on +-127 (unless the scale hit the floor)
    rows, cols = x.shape
    for bi in range(s.shape[0]):
        for bj in range(s.shape[1]):
            blk = x64[bi * br:(bi + 1) * br, bj * bc:(bj + 1) * bc]
            qb = q[bi * br:(bi + 1) * br, bj * bc:(bj + 1) * bc]
            if np.abs(blk).max() / 127 > 1e-8:
                i = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
                assert abs(int(qb[i])) == 127


@pytest.mark.parametrize("group", [0, 128])
def test_quant_roundtrip_activations(group):
    x = synth.bf16_bits_to_f32(synth.activations(small_cfg(T=32, H=1024)))
    x = np.concatenate([x, np.zeros((1, 1024), np.float32), np.full((1, 1024), 3e-9, np.float32)])
    q, s = oracle.quant_per_token(x, group)
    s2 = s.reshape(x.shape[0], -1)
    _check_roundtrip(x, q, s2, 1, 1024 if group == 0 else group)
    assert np.all(q[-2] == 0) and s2[-2, 0] == np.float32(1e-8)
    assert np.all(s2 >= np.float32(1e-8))


@pytest.mark.parametrize("br,bc", [(1, 384), (128, 128)])
def test_quant_roundtrip_weights(br, bc):
    w = synth.normal(256 * 384, 3, synth.STREAM_MISC, sigma=0.006).reshape(256, 384)
    q, s = oracle.quant_blocks(w, br, bc)
    assert s.shape == ((256 + br - 1) // br, (384 + bc - 1) // bc)
    _check_roundtrip(w, q, s, br, bc)


# ---------------------------------------------------------------- P3 int8 GEMM vs brute force

@pytest.mark.parametrize("K", [64, 128, 256])
def test_grouped_gemm_i32_brute_force(K):
    rng = np.random.default_rng(K)
    T, k, E, N = 24, 3, 5, 40
    a = rng.integers(-127, 128, size=(T, K), dtype=np.int64).astype(np.int8)
    a[0] = 127
    a[1] = -127
    w = rng.integers(-127, 128, size=(E, N, K), dtype=np.int64).astype(np.int8)
    w[:, 0] = 127
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    for bm in (1, 4, 16):
        al = oracle.align(ids, E, bm)
        acc = oracle.grouped_gemm_i32(a, True, w, al, bm, T * k, k)
        for r in range(int(al["num_tiles"][0]) * bm):
            p = al["sorted_pair_ids"][r]
            if p >= T * k:
                continue
            e = ids.reshape(-1)[p]
            ref = w[e].astype(np.int64) @ a[p // k].astype(np.int64)
            assert np.array_equal(acc[r].astype(np.int64), ref)
    # second-GEMM form (A rows indexed by sorted row, no gather)
    al = oracle.align(ids, E, 4)
    R = int(al["num_tiles"][0]) * 4
    h = rng.integers(-127, 128, size=(R, K), dtype=np.int64).astype(np.int8)
    acc = oracle.grouped_gemm_i32(h, False, w, al, 4, T * k, k)
    for r in range(R):
        if al["sorted_pair_ids"][r] < T * k:
            e = al["tile_expert"][r // 4]
            assert np.array_equal(acc[r].astype(np.int64), w[e].astype(np.int64) @ h[r].astype(np.int64))


def test_int32_extremes_do_not_overflow():
    K = 7168
    a = np.full((2, K), 127, np.int8)
    a[1] = -127
    w = np.full((1, 1, K), 127, np.int8)
    ids = np.zeros((2, 1), np.int32)
    al = oracle.align(ids, 1, 1)
    acc = oracle.grouped_gemm_i32(a, True, w, al, 1, 2, 1)
    assert acc[0, 0] == 115_612_672 and acc[1, 0] == -115_612_672


# ---------------------------------------------------------------- P4 channel dequant identity

def test_channel_dequant_identity():
    rng = np.random.default_rng(4)
    T, H, I, E = 16, 256, 512, 3
    h_q = rng.integers(-127, 128, size=(T, I), dtype=np.int64).astype(np.int8)
    h_s = (rng.random(T).astype(np.float32) * 0.01 + 1e-4).astype(np.float32)
    w2 = rng.integers(-127, 128, size=(E, H, I), dtype=np.int64).astype(np.int8)
    w2_s = (rng.random((E, H)).astype(np.float32) * 1e-3 + 1e-5).astype(np.float32)
    ids = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    tw = np.ones((T, 1), np.float32)
    al = oracle.align(ids, E, 1)
    # sorted row r holds pair sorted[r]; feed each pair's own intermediate row
    hq_sorted = np.zeros((int(al["num_tiles"][0]), I), np.int8)
    hs_sorted = np.zeros(int(al["num_tiles"][0]), np.float32)
    for r, p in enumerate(al["sorted_pair_ids"][: len(hs_sorted)]):
        hq_sorted[r], hs_sorted[r] = h_q[p], h_s[p]
    out = oracle.w2_combine(hq_sorted, hs_sorted, w2, w2_s, al, 1, tw, T, 1, H, I, False)
    for t in range(T):
        e = ids[t, 0]
        ref = ((h_q[t].astype(np.float64) * float(h_s[t]))[None, :] *
               (w2[e].astype(np.float64) * w2_s[e].astype(np.float64)[:, None])).sum(1)
        assert np.all(np.abs(out[t] - ref) <= 2.0 ** -21 * np.abs(ref))


# ---------------------------------------------------------------- P5 sorted pipeline == dense per-token loop

@pytest.mark.parametrize("which", ["tiny", "ds-small", "ds-small-block"])
def test_sorted_pipeline_equals_dense_loop(which):
    if which == "tiny":
        cfg = synth.CONFIGS["tiny"]
    else:
        cfg = small_cfg(mode="block" if which.endswith("block") else "channel")
    x, ids, tw, w = layer(cfg)
    dense = oracle.moe_tokens(x, ids, tw, *w, I=cfg.I, block=cfg.scale_mode == "block")
    for bm in (1, 16, 64):
        out, _ = pipeline(cfg, x, ids, tw, w, bm)
        assert np.array_equal(out, dense), bm


# ---------------------------------------------------------------- P6 special cases

def _w8a8_mlp_fp64(x, w13_q, w13_s, w2_q, w2_s, I):
    """W2 . requant(silu(gate) * up) with every step after the int8 products in fp64."""
    a_q, a_s = oracle.quant_per_token(x)
    acc = a_q.astype(np.int64) @ w13_q.astype(np.int64).T
    gu = acc * a_s.astype(np.float64)[:, None] * w13_s.astype(np.float64)[None, :]
    g, u = gu[:, :I], gu[:, I:]
    hf = g / (1 + np.exp(-g)) * u
    hs = np.maximum(np.abs(hf).max(1) / 127, 1e-8)
    hq = np.clip(np.rint(hf / hs[:, None]), -127, 127)
    return (hq @ w2_q.astype(np.float64).T) * hs[:, None] * w2_s.astype(np.float64)[None, :]


def test_single_expert_is_a_plain_w8a8_mlp():
    cfg = small_cfg(E=1, k=1, route="softmax", n_group=1, topk_group=1, scaling=1.0, T=32, H=384, I=256)
    x, ids, tw, w = layer(cfg)
    assert np.all(ids == 0) and np.all(tw == 1.0)
    out = oracle.moe_tokens(x, ids, tw, *w, I=cfg.I, block=False)
    ref = _w8a8_mlp_fp64(x, w[0][0], w[1][0], w[2][0], w[3][0], cfg.I)
    assert np.abs(out - ref).max() <= 1e-3 * np.abs(ref).max()
    # a swapped gate/up (a plausible layout mistake) is caught by the same check
    swapped = np.concatenate([w[0][0][cfg.I:], w[0][0][:cfg.I]])
    swapped_s = np.concatenate([w[1][0][cfg.I:], w[1][0][:cfg.I]])
    bad = oracle.moe_tokens(x, ids, tw, [swapped], [swapped_s], w[2], w[3], I=cfg.I, block=False)
    assert np.abs(bad - ref).max() > 1e-2 * np.abs(ref).max()


def test_all_experts_selected_is_permutation_invariant():
    cfg = small_cfg(E=8, k=8, route="softmax", n_group=1, topk_group=1, scaling=1.0, T=16, H=256, I=128)
    x, ids, tw, w = layer(cfg)
    lg = synth.logits(cfg)
    out = oracle.moe_tokens(x, ids, tw, *w, I=cfg.I, block=False)
    perm = np.random.default_rng(0).permutation(8)
    inv = np.argsort(perm)
    ids2, tw2 = oracle.route(lg[:, perm], 8, oracle.SOFTMAX)
    # new expert j is old expert perm[j]
    w_perm = [[w[i][perm[j]] for j in range(8)] for i in range(4)]
    out2 = oracle.moe_tokens(x, ids2, tw2, *w_perm, I=cfg.I, block=False)
    assert np.array_equal(perm[ids2], ids)
    assert np.array_equal(out, out2)
    del inv


def test_all_tokens_to_one_expert():
    cfg = small_cfg(E=8, k=1, route="softmax", n_group=1, topk_group=1, scaling=1.0, T=40, H=256, I=128)
    x = oracle.activations_f32(cfg)
    lg = synth.logits(cfg)
    lg[:, 5] += 100.0
    ids, tw = oracle.route(lg, 1, oracle.SOFTMAX)
    assert np.all(ids == 5)
    w = oracle.expert_weights(cfg, [5])
    al = oracle.align(ids, 8, 16)
    assert al["counts"][5] == 40 and al["counts"].sum() == 40
    assert int(al["num_tiles"][0]) == 3 and np.all(al["tile_expert"][:3] == 5)
    dense = oracle.moe_tokens(x, ids, tw, *w, I=cfg.I, block=False)
    out, _ = pipeline(cfg, x, ids, tw, w, 16)
    assert np.array_equal(out, dense)


# ---------------------------------------------------------------- P7 block-wise reduces to channel-wise

def test_block_reduces_to_channel():
    rng = np.random.default_rng(7)
    T, H, I, E, k = 24, 512, 128, 4, 2
    x = synth.bf16_bits_to_f32(synth.activations(small_cfg(T=T, H=H)))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    tw = rng.random((T, k)).astype(np.float32)
    w13 = rng.integers(-127, 128, size=(E, 2 * I, H), dtype=np.int64).astype(np.int8)
    w2 = rng.integers(-127, 128, size=(E, H, I), dtype=np.int64).astype(np.int8)
    c13 = (rng.random((E, 2 * I // 128)) * 1e-3 + 1e-4).astype(np.float32)
    c2 = (rng.random((E, H // 128)) * 1e-3 + 1e-4).astype(np.float32)
    # channel scales constant inside each 128-row block; block scales equal along K
    w13_ch = np.repeat(c13, 128, axis=1)
    w2_ch = np.repeat(c2, 128, axis=1)
    w13_bl = np.repeat(c13[:, :, None], H // 128, axis=2)
    w2_bl = np.repeat(c2[:, :, None], I // 128, axis=2)
    a_q, a_t = oracle.quant_per_token(x)
    a_bl = np.repeat(a_t[:, None], H // 128, axis=1)
    bm = 8
    al = oracle.align(ids, E, bm)
    hq_c, hs_c = oracle.w13_silu(a_q, a_t, w13, w13_ch, al, bm, T, k, H, I, False)
    hq_b, hs_b = oracle.w13_silu(a_q, a_bl, w13, w13_bl, al, bm, T, k, H, I, True)
    valid = al["sorted_pair_ids"][: len(hs_c)] < T * k
    # I = 128: one requant group per row, so the two modes requantize identically up to fp32 summation
    rel = np.abs(hs_b[valid, 0] - hs_c[valid]) / hs_c[valid]
    assert rel.max() <= 1e-5
    assert np.mean(hq_b[valid] != hq_c[valid]) <= 1e-3
    assert np.abs(hq_b[valid].astype(int) - hq_c[valid].astype(int)).max() <= 1
    # second GEMM on the same intermediate: per-element bound by the K-block terms
    hs_bl = np.repeat(hs_c[:, None], I // 128, axis=1)
    out_c = oracle.w2_combine(hq_c, hs_c, w2, w2_ch, al, bm, tw, T, k, H, I, False)
    out_b = oracle.w2_combine(hq_c, hs_bl, w2, w2_bl, al, bm, tw, T, k, H, I, True)
    bound = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            r = int(np.nonzero(al["sorted_pair_ids"] == t * k + j)[0][0])
            e = ids[t, j]
            parts = (hq_c[r].astype(np.int64).reshape(I // 128, 128)[None, :, :] *
                     w2[e].astype(np.int64).reshape(H, I // 128, 128)).sum(2)  # [H, nkb]
            # integer partials sum exactly to the channel accumulator
            assert np.array_equal(parts.sum(1), w2[e].astype(np.int64) @ hq_c[r].astype(np.int64))
            terms = np.abs(parts * float(hs_c[r]) * w2_ch[e][:, None].astype(np.float64)).sum(1)
            bound[t] += abs(float(tw[t, j])) * terms
    assert np.all(np.abs(out_b - out_c) <= 1e-5 * bound + 1e-30)


# ---------------------------------------------------------------- P8 align invariants

def _check_align(ids, E, bm, al):
    P = ids.size
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E)
    assert np.array_equal(al["counts"], counts)
    # expert offsets are the zero-padded cumulative sum of the counts
    assert np.array_equal(al["offsets"], np.concatenate([[0], np.cumsum(counts)]))
    pcount = (counts + bm - 1) // bm * bm
    assert np.array_equal(al["padded_offsets"], np.concatenate([[0], np.cumsum(pcount)]))
    nt = int(al["num_tiles"][0])
    assert nt * bm == al["padded_offsets"][-1]
    srt = al["sorted_pair_ids"][: nt * bm]
    real = srt[srt < P]
    assert np.array_equal(np.sort(real), np.flatnonzero(valid))
    assert np.sum(srt == P) == np.sum(pcount - counts)
    for e in range(E):
        seg = srt[al["padded_offsets"][e]: al["padded_offsets"][e + 1]]
        body = seg[: counts[e]]
        assert np.all(flat[body] == e)
        assert np.all(np.diff(body) > 0)
        assert np.all(seg[counts[e]:] == P)
        assert np.all(al["tile_expert"][al["padded_offsets"][e] // bm: al["padded_offsets"][e + 1] // bm] == e)


@pytest.mark.parametrize("bm", [1, 16, 64, 128])
def test_align_invariants(bm):
    rng = np.random.default_rng(bm)
    cases = [
        (rng.integers(0, 256, size=(128, 8)), 256),
        (np.minimum(rng.zipf(1.5, size=(300, 8)) - 1, 63), 64),
        (np.full((50, 1), 3), 8),
        (np.zeros((7, 1)), 1),
        (np.tile(np.arange(8), (5, 1)), 8),
        (np.zeros((0, 4)), 16),
    ]
    for ids, E in cases:
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        _check_align(ids, E, bm, oracle.align(ids, E, bm))


@pytest.mark.parametrize("bm", [1, 16, 64])
def test_align_drops_out_of_range_ids(bm):
    """An id outside [0, E) names no expert: its pair takes no row, the others group as before."""
    rng = np.random.default_rng(100 + bm)
    ids = rng.integers(0, 32, size=(90, 4)).astype(np.int32)
    flat = ids.reshape(-1)
    flat[::5] = -1
    flat[2::9] = 32
    flat[3::11] = -2 ** 31
    flat[1::13] = 2 ** 31 - 1
    al = oracle.align(ids, 32, bm)
    _check_align(ids, 32, bm, al)
    assert int(al["counts"].sum()) == int(((flat >= 0) & (flat < 32)).sum())


def test_combine_skips_dropped_pairs():
    """The combine over a routing with dropped pairs equals the combine over the same routing with
    each dropped pair sent to a real expert at weight 0 (acc + 0 * y == acc for finite y): the
    second path runs the oracle's align and GEMM on other rows, with no pair dropped."""
    T, k, E, H, I = 40, 3, 4, 256, 128
    rng = np.random.default_rng(7)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    tw = rng.uniform(0.1, 1.0, size=(T, k)).astype(np.float32)
    drop = np.zeros((T, k), bool)
    drop.reshape(-1)[::4] = True
    bad = ids.copy()
    bad[drop] = np.where(np.arange(drop.sum()) % 2 == 0, -1, E)
    zeroed = tw.copy()
    zeroed[drop] = 0.0
    w2 = [synth.int8_matrix(H, I, 30 + e) for e in range(E)]
    w2_s = [synth.positive_scales(H, 40 + e, 1e-3, 3e-2) for e in range(E)]
    pair_q = synth.int8_matrix(T * k, I, 50)
    pair_s = synth.positive_scales(T * k, 51, 1e-3, 3e-2)

    def run(routing, weights, bm):
        al = oracle.align(routing, E, bm)
        R = int(al["num_tiles"][0]) * bm
        srt = al["sorted_pair_ids"][:R]
        real = srt < T * k
        h_q = np.zeros((max(R, 1), I), np.int8)
        h_s = np.ones(max(R, 1), np.float32)
        h_q[:R][real] = pair_q[srt[real]]
        h_s[:R][real] = pair_s[srt[real]]
        return oracle.w2_combine(h_q, h_s, w2, w2_s, al, bm, weights, T, k, H, I, False)

    for bm in (1, 16):
        got = run(bad, tw, bm)
        assert np.array_equal(got, run(ids, zeroed, bm))
        assert not np.array_equal(got, run(ids, tw, bm))


# ---------------------------------------------------------------- P9 routing

def test_softmax_routing_brute_force():
    lg = synth.logits(synth.CONFIGS["tiny"])
    ids, w = oracle.route(lg, 2, oracle.SOFTMAX)
    for t in range(lg.shape[0]):
        best = max(itertools.combinations(range(8), 2), key=lambda c: (sum(float(lg[t, i]) for i in c),
                                                                       [-i for i in c]))
        assert set(ids[t]) == set(best)
        assert lg[t, ids[t, 0]] >= lg[t, ids[t, 1]]
        sel = lg[t, ids[t]].astype(np.float64)
        ref = np.exp(sel - sel.max()) / np.exp(sel - sel.max()).sum()
        assert np.all(np.abs(w[t] - ref) <= 4 * U * ref)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= 6 * U)


def test_softmax_ties_go_to_lower_index():
    lg = np.array([[1.0, 3.0, 3.0, 0.5, 3.0]], np.float32)
    ids, w = oracle.route(lg, 2, oracle.SOFTMAX)
    assert list(ids[0]) == [1, 2]
    assert w[0, 0] == w[0, 1] == np.float32(0.5)


def _sig64(l):
    return 1.0 / (1.0 + np.exp(-l.astype(np.float64)))


def test_grouped_sigmoid_routing_brute_force():
    E, ng, tg, k = 8, 4, 2, 2
    lg = synth.normal(200 * E, 11, synth.STREAM_MISC).reshape(200, E)
    ids, w = oracle.route(lg, k, oracle.SIGMOID, ng, tg, True, 2.5)
    for t in range(200):
        s = _sig64(lg[t])
        gscore = [sorted(s[g * 2:(g + 1) * 2])[-1] + sorted(s[g * 2:(g + 1) * 2])[-2] for g in range(ng)]
        best_groups = max(itertools.combinations(range(ng), tg), key=lambda c: sum(gscore[g] for g in c))
        allowed = [e for g in best_groups for e in range(g * 2, g * 2 + 2)]
        best = max(itertools.combinations(allowed, k), key=lambda c: sum(s[e] for e in c))
        got = sum(s[e] for e in ids[t])
        assert got >= sum(s[e] for e in best) - 1e-6
        assert len({e // 2 for e in ids[t]}) <= tg
        ref = s[ids[t]] / s[ids[t]].sum() * 2.5
        assert np.all(np.abs(w[t] - ref) <= 1e-6 * ref)


def test_softmax_routing_without_renormalize_brute_force():
    """renormalize = 0: the weight of a selected expert is its softmax probability over all E
    logits (not over the selected ones), times the routed scaling; the selection is the best
    k-subset by logit sum.  A sum over the selected logits only (the renormalized rule) fails."""
    E = 8
    lg = synth.normal(150 * E, 12, synth.STREAM_MISC).reshape(150, E)
    for k in (1, 2, 3, 8):
        ids, w = oracle.route(lg, k, oracle.SOFTMAX, 1, 1, False, 1.5)
        for t in range(lg.shape[0]):
            best = max(itertools.combinations(range(E), k), key=lambda c: sum(float(lg[t, i]) for i in c))
            assert set(ids[t]) == set(best)
            full = np.exp(lg[t].astype(np.float64) - lg[t].max())
            ref = full[ids[t]] / full.sum() * 1.5
            assert np.all(np.abs(w[t] - ref) <= 16 * U * ref), (k, t)
            if k < E:
                assert w[t].astype(np.float64).sum() < 1.5 * (1 - 1e-4)
        if k == E:  # every expert selected: the probabilities sum to one before the scaling
            assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.5) <= 1.5 * 16 * U)


@pytest.mark.parametrize("renorm", [True, False])
def test_sigmoid_routing_with_correction_bias_brute_force(renorm):
    """A correction bias moves the selection, not the weights: groups and experts are chosen by
    c = sigmoid(l) + bias (group score = sum of its two largest c), the weights are the selected
    sigmoid(l) (normalized if renorm) times the scaling.  Brute force over every group subset and
    expert subset on E = 8; a dropped bias, or weights taken from c, fails."""
    E, ng, tg, k = 8, 4, 2, 3
    T = 300
    lg = synth.normal(T * E, 13, synth.STREAM_MISC).reshape(T, E)
    bias = synth.normal(E, 14, synth.STREAM_MISC, 0, 0.4)
    ids, w = oracle.route(lg, k, oracle.SIGMOID, ng, tg, renorm, 2.5, bias)
    ids0, _ = oracle.route(lg, k, oracle.SIGMOID, ng, tg, renorm, 2.5, None)
    moved = 0
    for t in range(T):
        s = _sig64(lg[t])
        c = s + bias.astype(np.float64)
        gscore = [sum(sorted(c[g * 2:(g + 1) * 2])[-2:]) for g in range(ng)]
        groups = max(itertools.combinations(range(ng), tg), key=lambda gs: sum(gscore[g] for g in gs))
        allowed = [e for g in groups for e in range(g * 2, g * 2 + 2)]
        best = max(itertools.combinations(allowed, k), key=lambda sel: sum(c[e] for e in sel))
        margin = sum(c[e] for e in best) - max(sum(c[e] for e in sel)
                                               for sel in itertools.combinations(allowed, k) if set(sel) != set(best))
        if margin > 1e-5:  # no near-tie between fp32 and fp64 scores
            assert set(ids[t]) == set(best), t
        assert np.all(np.diff(c[ids[t]]) <= 1e-6)  # slots in descending c
        ref = s[ids[t]] / s[ids[t]].sum() * 2.5 if renorm else s[ids[t]] * 2.5
        assert np.all(np.abs(w[t] - ref) <= 1e-6 * ref), t
        moved += set(ids[t]) != set(ids0[t])
    assert moved >= T // 10  # the bias changed many selections


def test_deepseek_routing_invariants():
    cfg = synth.CONFIGS["decode"]
    lg = synth.logits(cfg)
    ids, w = oracle.route_cfg(cfg, lg)
    assert ids.shape == (cfg.T, 8)
    groups = ids // 32
    assert all(len(set(g)) <= 4 for g in groups)
    assert all(len(set(r)) == 8 for r in ids)
    # weights sum to the routed scaling: 8 sigmoid terms, a sum, a divide and a multiply
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 2.5) <= 2.5 * 12 * U)
    s = _sig64(lg)
    for t in range(cfg.T):
        assert np.all(np.diff(s[t, ids[t]]) <= 1e-7)  # slots in descending score


# ---------------------------------------------------------------- P10 fp32 epilogue vs fp64

@pytest.mark.parametrize("mode", ["channel", "block"])
def test_second_gemm_epilogue_vs_fp64(mode):
    cfg = small_cfg(mode=mode)
    x, ids, tw, w = layer(cfg)
    out, st = pipeline(cfg, x, ids, tw, w, 16)
    al, h_q, h_s = st["al"], st["h_q"], st["h_s"]
    ref = np.zeros((cfg.T, cfg.H))
    P = cfg.T * cfg.k
    for r in range(int(al["num_tiles"][0]) * 16):
        p = al["sorted_pair_ids"][r]
        if p >= P:
            continue
        e = al["tile_expert"][r // 16]
        wq = w[2][e].astype(np.float64)
        if mode == "channel":
            y = (wq @ h_q[r].astype(np.float64)) * float(h_s[r]) * w[3][e].astype(np.float64)
        else:
            hq = h_q[r].astype(np.float64) * np.repeat(h_s[r].astype(np.float64), 128)
            wsf = np.repeat(np.repeat(w[3][e].astype(np.float64), 128, 0), 128, 1)
            y = (wq * wsf) @ hq
        ref[p // cfg.k] += float(tw.reshape(-1)[p]) * y
    assert np.abs(out - ref).max() <= 1e-5 * np.abs(ref).max()


# ---------------------------------------------------------------- P11 sanity vs unquantized fp64

def test_quantized_layer_tracks_fp64_layer():
    cfg = synth.CONFIGS["tiny"]
    x, ids, tw, w = layer(cfg)
    out = oracle.moe_tokens(x, ids, tw, *w, I=cfg.I, block=False)
    ref = np.zeros((cfg.T, cfg.H))
    for t in range(cfg.T):
        for j in range(cfg.k):
            e = ids[t, j]
            w13 = synth.w13_f32(cfg, e).astype(np.float64)
            w2 = synth.w2_f32(cfg, e).astype(np.float64)
            gu = w13 @ x[t].astype(np.float64)
            g, u = gu[: cfg.I], gu[cfg.I:]
            ref[t] += float(tw[t, j]) * (w2 @ (g / (1 + np.exp(-g)) * u))
    cos = (out.astype(np.float64) * ref).sum() / np.linalg.norm(out) / np.linalg.norm(ref)
    assert cos >= 0.99, cos


# ---------------------------------------------------------------- dense W8A8 linear

def linear_inputs(M, N, K, seed):
    a_q = synth.int8_matrix(M, K, seed)
    w = synth.int8_matrix(N, K, seed + 1)
    a_s = synth.positive_scales(M, seed + 2, 1e-3, 3e-2)
    w_s = synth.positive_scales(N, seed + 3, 1e-3, 3e-2)
    return a_q, a_s, w, w_s


def test_linear_equals_the_moe_second_gemm_with_one_expert():
    """A dense linear is the grouped second GEMM + combine with one expert, top-1 and combine
    weight 1.0 (0 + 1.0 * y == y): the oracle's other code path (align, sorted rows, combine)
    must give the same bits."""
    M, N, K = 37, 256, 384
    a_q, a_s, w, w_s = linear_inputs(M, N, K, 71)
    got = oracle.linear(a_q, a_s, w, w_s)
    ids = np.zeros((M, 1), dtype=np.int32)
    for bm in (16, 64):
        al = oracle.align(ids, 1, bm)
        R = int(al["num_tiles"][0]) * bm
        h_q = np.zeros((R, K), dtype=np.int8)
        h_s = np.ones(R, dtype=np.float32)
        real = al["sorted_pair_ids"][:R] < M
        h_q[real] = a_q[al["sorted_pair_ids"][:R][real]]
        h_s[real] = a_s[al["sorted_pair_ids"][:R][real]]
        ref = oracle.w2_combine(h_q, h_s, w[None], w_s[None], al, bm, np.ones((M, 1), np.float32), M, 1, N, K,
                                False)
        assert np.array_equal(got, ref)


def test_linear_within_two_roundings_of_fp64():
    """|acc| < 2^24, so (float)acc is exact and the two fp32 products round once each."""
    M, N, K = 9, 256, 256
    a_q, a_s, w, w_s = linear_inputs(M, N, K, 73)
    got = oracle.linear(a_q, a_s, w, w_s).astype(np.float64)
    exact = (a_q.astype(np.float64) @ w.astype(np.float64).T) * a_s.astype(np.float64)[:, None] \
        * w_s.astype(np.float64)[None, :]
    assert np.all(np.abs(got - exact) <= np.abs(exact) * (2.0 ** -23 + 2.0 ** -46))


def test_linear_closed_form_and_row_selection():
    """All-ones operands: out[m, n] = K * a_s[m] * w_s[n] in fp32; a row selection computes only
    those rows."""
    M, N, K = 4, 256, 512
    a_q = np.ones((M, K), np.int8)
    w = np.ones((N, K), np.int8)
    a_s = np.array([0.5, 0.25, 2.0, 1.0], np.float32)
    w_s = np.linspace(0.125, 4.0, N).astype(np.float32)
    got = oracle.linear(a_q, a_s, w, w_s)
    assert np.array_equal(got, (np.float32(K) * a_s[:, None]) * w_s[None, :])
    part = oracle.linear(a_q, a_s, w, w_s, rows=[2])
    assert np.array_equal(part[2], got[2]) and not part[[0, 1, 3]].any()


def test_linear_tracks_the_unquantized_matmul():
    """Per-token activation and per-channel weight quantization of Gaussian data, then the linear:
    close to the fp64 x @ W^T (catches a transposed operand or a swapped scale)."""
    rng_x = synth.normal(64 * 1024, 5, 1, 0).reshape(64, 1024).astype(np.float32)
    W = (synth.normal(512 * 1024, 5, 2, 0).reshape(512, 1024) * 0.02).astype(np.float32)
    a_q, a_s = oracle.quant_per_token(rng_x, 0)
    w_q, w_s = oracle.quant_weight(W, "channel")
    got = oracle.linear(a_q, a_s, w_q, w_s.reshape(-1)).astype(np.float64)
    ref = rng_x.astype(np.float64) @ W.astype(np.float64).T
    cos = (got * ref).sum() / np.linalg.norm(got) / np.linalg.norm(ref)
    assert cos >= 0.999, cos
    assert np.abs(got - ref).max() <= 0.05 * np.abs(ref).max()
