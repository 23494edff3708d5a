"""GPU parity of the W4A8 path (packed int4 weights, FP8 activations) against the CPU oracle,
through the C ABI.

The weights are widened to E4M3 codes exactly (|q| <= 7), so the products and the FP8 MFMA's
K-block sums behave as in the FP8 path (the sum model measured in tests/test_gpu_fp8.py: within
TAU * sum|products| of the exact sum, TAU = 7 * 2^-13 + gamma_17).  Bars, derived the same way:
  - weight quantization: packed bytes and scales bit-exact;
  - second GEMM + combine fed the oracle's intermediate: |got - ref| <= (TAU + u + 2 gamma_(nkb+2)
    + 2 gamma_(k+1)) * 1.01 * B elementwise, B the same computation on magnitudes;
  - first GEMM: every dequantized code and h_scale against the exact fp64 SiLU(g) * u, with g and
    u carrying the bound above, and against the oracle's code with both sides' terms;
  - whole layer: max|err| <= 1e-2 * max|ref| over the checked tokens, the FP8 path's bar (its
    derivation: intermediate FP8 codes one E4M3 step off, test_gpu_fp8.py).
"""
import dataclasses
import sys

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import w8a8_int8_quantized_quant_amd as w8  # noqa: E402

LAYER_BAR = 1e-2  # whole-layer error over max|ref|, as for the FP8 path
from w8a8_int8_quantized_quant_amd import workload  # noqa: E402

DEV = "cuda"
U = 2.0 ** -24
MODE = w8.SCALE_W4A8


def gamma(n):
    return n * U / (1 - n * U)


TAU = 7 * 2.0 ** -13 + gamma(17)


def tol_sums(nkb, k=None):
    t = TAU + U + 2 * gamma(nkb + 2)
    if k is not None:
        t += 2 * gamma(k + 1)
    return t * 1.01


def small_cfg(name, index, T, H, I, E, k, route="softmax", n_group=1, topk_group=1, scaling=1.0,
              x_dtype=synth.DTYPE_BF16, w_sigma=0.006):
    return synth.MoEConfig(name=name, index=index, T=T, H=H, I=I, E=E, k=k, route=route, n_group=n_group,
                           topk_group=topk_group, routed_scaling=scaling, renormalize=True, x_dtype=x_dtype,
                           x_sigma=1.0, outlier_threshold=synth.OUTLIER_THRESHOLD, outlier_mult=20.0,
                           w_sigma=w_sigma, scale_mode="w4a8")


CFG = {
    "w4-tiny": small_cfg("w4-tiny", 80, T=16, H=256, I=128, E=8, k=2, x_dtype=synth.DTYPE_F32, w_sigma=0.02),
    "w4-small": small_cfg("w4-small", 81, T=300, H=512, I=256, E=16, k=4, route="sigmoid", n_group=4,
                          topk_group=2, scaling=2.5),
    "w4-dsv3-e8": small_cfg("w4-dsv3-e8", 82, T=1000, H=7168, I=2048, E=8, k=2),
    # fewer than 32 rows per expert on average: the 64-row tiles of the few-rows case
    "w4-dsv3-e64": small_cfg("w4-dsv3-e64", 83, T=533, H=7168, I=2048, E=64, k=2),
    # fewer than 16 rows per expert on average: the 16-row tiles of the streaming engine
    "w4-dsv3-e64s": small_cfg("w4-dsv3-e64s", 84, T=251, H=7168, I=2048, E=64, k=2),
    # the streaming engine's K loops at K / 128 = 4, 8, 16 and 32 (16-row tiles, few rows per expert)
    "w4-s4": small_cfg("w4-s4", 85, T=100, H=512, I=2048, E=16, k=2),
    "w4-s32": small_cfg("w4-s32", 86, T=100, H=4096, I=1024, E=16, k=2, route="sigmoid", n_group=4,
                        topk_group=2, scaling=2.5),
    "w4-decode": dataclasses.replace(synth.CONFIGS["decode"], name="w4-decode", scale_mode="w4a8"),
    "w4-block": dataclasses.replace(synth.CONFIGS["block"], name="w4-block", scale_mode="w4a8"),
}
SMALL = ("w4-tiny", "w4-small", "w4-s4", "w4-s32")


def dt(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


_layer = {}
_oracle_w = {}


def layer_of(name):
    if name not in _layer:
        _layer.clear()
        torch.cuda.empty_cache()
        say(f"[layer] drawing {name} on the device")
        _layer[name] = workload.make_layer(CFG[name], device=DEV)
    return _layer[name]


def oracle_weights(name, experts):
    cfg = CFG[name]
    cache = _oracle_w.setdefault(name, [[None] * cfg.E for _ in range(4)])
    todo = sorted({int(e) for e in experts if cache[0][int(e)] is None})
    if todo:
        w = oracle.expert_weights(cfg, todo)
        for i in range(4):
            for e in todo:
                cache[i][e] = w[i][e]
    return cache


def block_m_of(cfg):
    return w8.w8a8_moe_pick_block_m(cfg.T, cfg.k, cfg.E)


def align_dev(ids, E, bm):
    al = oracle.align(ids, E, bm)
    return al, {key: dt(v) for key, v in al.items()}


def check_rows(al, bm, P, name, nsample=40, seed=2):
    R = int(al["num_tiles"][0]) * bm
    real = np.nonzero(al["sorted_pair_ids"][:R] < P)[0]
    if name in SMALL:
        return real
    counts = al["counts"]
    order = np.argsort(counts, kind="stable")
    nonempty = order[counts[order] > 0]
    rows = []
    for e in (nonempty[-1], nonempty[0]):
        r0, n = int(al["padded_offsets"][e]), int(counts[e])
        rows += [r0, r0 + n - 1, r0 + min(n - 1, 127), r0 + min(n - 1, 128)]
    rng = np.random.default_rng(seed)
    rows += list(rng.choice(real, size=min(nsample, len(real)), replace=False))
    return np.unique(np.array(rows, dtype=np.int64))


# ------------------------------------------------------------------ weight quantization

@pytest.mark.parametrize("case", ["f32", "bf16", "wide"])
def test_w4_quant_bit_exact(case):
    if case == "f32":
        x = synth.normal(300 * 512, 13, 0, sigma=0.02).reshape(300, 512)
    elif case == "bf16":
        x = synth.activations(CFG["w4-small"])
    else:
        x = synth.normal(64 * 7168, 14, 0, sigma=5.0).reshape(64, 7168)
        x[3, :128] = 0.0
    say(f"[w4 quant] {case} {x.shape}")
    xf = oracle.bf16_to_f32(x) if x.dtype == np.uint16 else x
    rq, rs = oracle.w4_quant(xf)
    xd = dt(x.view(np.int16)).view(torch.bfloat16) if x.dtype == np.uint16 else dt(x)
    q = torch.empty(rq.shape, dtype=torch.uint8, device=DEV)
    s = torch.empty(rs.shape, dtype=torch.float32, device=DEV)
    w8.w8a8_w4a8_quant_weights(xd, q, s)
    assert np.array_equal(host(s), rs)
    assert np.array_equal(host(q), rq)


@pytest.mark.parametrize("name", ["w4-small", "w4-block"])
def test_w4_layer_weights_bit_exact(name):
    cfg = CFG[name]
    L = layer_of(name)
    experts = [0, cfg.E - 1]
    w = oracle_weights(name, experts)
    for e in experts:
        assert np.array_equal(host(L.w13[e]), w[0][e]) and np.array_equal(host(L.w13_scale[e]), w[1][e])
        assert np.array_equal(host(L.w2[e]), w[2][e]) and np.array_equal(host(L.w2_scale[e]), w[3][e])


# ------------------------------------------------------------------ the grouped GEMMs

def run_w13(name, ids):
    cfg = CFG[name]
    bm = block_m_of(cfg)
    L = layer_of(name)
    al, d = align_dev(ids, cfg.E, bm)
    a_q, a_s = oracle.fp8_quant_blocks(oracle.activations_f32(cfg), 1, 128)
    R = w8.w8a8_moe_max_rows(cfg.T, cfg.k, cfg.E, bm)
    h_q = torch.empty((R, cfg.I), dtype=torch.uint8, device=DEV)
    h_s = torch.empty((R, cfg.I // 128), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(w8.w8a8_w13_workspace_bytes(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I, bm, MODE), 256),
                     dtype=torch.uint8, device=DEV)
    w8.w8a8_w4a8_grouped_gemm_w13_silu(dt(a_q), dt(a_s), L.w13, L.w13_scale, d["sorted_pair_ids"],
                                       d["padded_offsets"], d["tile_expert"], d["num_tiles"], cfg.T, cfg.k, bm, h_q,
                                       h_s, ws)
    return al, bm, a_q, a_s, host(h_q), host(h_s)


_dec = {}


def decoded_w13(name, e, w):
    key = (name, e)
    if key not in _dec:
        _dec.clear()
        _dec[key] = oracle.w4_unpack(w[0][e]).astype(np.float64) * np.repeat(w[1][e].astype(np.float64), 128, 1)
    return _dec[key]


def check_w13(name, al, bm, a_q, a_s, gq_all, gs_all, rows):
    cfg = CFG[name]
    I = cfg.I
    w = oracle_weights(name, sorted({int(al["tile_expert"][r // bm]) for r in rows}))
    rq, rs = oracle.w4_w13_silu(a_q, a_s, w[0], w[1], al, bm, cfg.T, cfg.k, cfg.H, I, rows)
    tol = tol_sums(cfg.H // 128)
    worst, off, n = 0.0, 0, 0
    for r in sorted(rows, key=lambda r: int(al["tile_expert"][r // bm])):
        p = int(al["sorted_pair_ids"][r])
        t, e = p // cfg.k, int(al["tile_expert"][r // bm])
        wd = decoded_w13(name, e, w)
        a = oracle.fp8_decode(a_q[t]).astype(np.float64) * np.repeat(a_s[t].astype(np.float64), 128)
        gu, bgu = wd @ a, np.abs(wd) @ np.abs(a)
        g, u, dg, du = gu[:I], gu[I:], tol * bgu[:I], tol * bgu[I:]
        sg = g / (1 + np.exp(-g))
        h = sg * u
        dh = 1.1 * np.abs(u) * dg + np.abs(sg) * du + 1.1 * dg * du + 16 * U * np.abs(h)
        hg, dhg = np.abs(h).reshape(-1, 128), dh.reshape(-1, 128)
        lo = np.maximum((hg - dhg).max(1) / 448, 1e-8) * (1 - 2 * U)
        hi = np.maximum((hg + dhg).max(1) / 448, 1e-8) * (1 + 2 * U)
        gs = gs_all[r].astype(np.float64)
        assert np.all((gs >= lo) & (gs <= hi)), (r, gs, lo, hi)
        sc = np.repeat(gs, 128)
        deq = oracle.fp8_decode(gq_all[r]).astype(np.float64) * sc
        half = 2.0 ** -4 * (np.abs(h) + dh) + 2.0 ** -10 * sc
        assert np.all(np.abs(deq - h) <= (half + dh) * (1 + 1e-6)), r
        rsc = np.repeat(rs[r].astype(np.float64), 128)
        rdeq = oracle.fp8_decode(rq[r]).astype(np.float64) * rsc
        rhalf = 2.0 ** -4 * (np.abs(h) + dh) + 2.0 ** -10 * rsc
        assert np.all(np.abs(deq - rdeq) <= (half + rhalf + 2 * dh) * (1 + 1e-6)), r
        worst = max(worst, float(np.max(np.abs(gs / rs[r] - 1))))
        off += int(np.count_nonzero(gq_all[r] != rq[r]))
        n += I
    say(f"[w4 w13] {name}: rows {len(rows)}, h_s max rel vs oracle {worst:.2e}, codes differing from the "
        f"oracle {off}/{n}")


def w13_rows(al, bm, P, name):
    rows = check_rows(al, bm, P, name)
    if name not in SMALL and len(rows) > 40:
        rows = np.sort(np.random.default_rng(7).choice(rows, 40, replace=False))
    return rows


@pytest.mark.parametrize("name", ["w4-tiny", "w4-small", "w4-s4", "w4-s32", "w4-block"])
def test_w4_first_gemm_silu_requant(name):
    cfg = CFG[name]
    ids, _ = oracle.route_cfg(cfg, synth.logits(cfg))
    al, bm, a_q, a_s, gq, gs = run_w13(name, ids)
    check_w13(name, al, bm, a_q, a_s, gq, gs, w13_rows(al, bm, cfg.T * cfg.k, name))


def run_check_w2(name, ids, tw, tokens):
    cfg = CFG[name]
    bm = block_m_of(cfg)
    L = layer_of(name)
    al, d = align_dev(ids, cfg.E, bm)
    R = w8.w8a8_moe_max_rows(cfg.T, cfg.k, cfg.E, bm)
    h_q = synth.int8_matrix(R, cfg.I, cfg.seed + 100).view(np.uint8).copy()
    h_q[(h_q & 0x7F) == 0x7F] -= 1
    h_s = synth.positive_scales(R * (cfg.I // 128), cfg.seed, 1e-3, 3e-2).reshape(R, cfg.I // 128)
    out = torch.full((cfg.T, cfg.H), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(w8.w8a8_w2_workspace_bytes(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I, bm, MODE), 256),
                     dtype=torch.uint8, device=DEV)
    w8.w8a8_w4a8_grouped_gemm_w2_combine(dt(h_q), dt(h_s), L.w2, L.w2_scale, d["sorted_pair_ids"],
                                         d["padded_offsets"], d["tile_expert"], d["num_tiles"], dt(tw), cfg.T, cfg.k,
                                         bm, out, ws)
    got = host(out)
    assert np.isfinite(got).all()
    w = oracle_weights(name, np.unique(ids[tokens]))
    ref = oracle.w4_w2_combine(h_q, h_s, w[2], w[3], al, bm, tw, cfg.T, cfg.k, cfg.H, cfg.I, tokens)
    wa = [None if x is None else oracle.w4_abs(x) for x in w[2]]
    sa = [None if x is None else np.abs(x) for x in w[3]]
    B = oracle.w4_w2_combine(oracle.fp8_abs(h_q), np.abs(h_s), wa, sa, al, bm, np.abs(tw), cfg.T, cfg.k, cfg.H,
                             cfg.I, tokens).astype(np.float64)
    tol = tol_sums(cfg.I // 128, cfg.k)
    err = np.abs(got[tokens].astype(np.float64) - ref)
    say(f"[w4 w2] {name}: tokens {len(tokens)}, bit-equal {np.mean(got[tokens] == ref):.6f}, "
        f"max err/B {np.max(err / np.maximum(B, 1e-30)):.2e} (tol {tol:.2e})")
    assert np.all(err <= tol * B)


@pytest.mark.parametrize("name", ["w4-tiny", "w4-small", "w4-s4", "w4-s32", "w4-block"])
def test_w4_second_gemm_combine(name):
    cfg = CFG[name]
    ids, tw = oracle.route_cfg(cfg, synth.logits(cfg))
    tokens = np.arange(cfg.T) if name in SMALL else np.sort(np.random.default_rng(3).choice(cfg.T, 6, replace=False))
    run_check_w2(name, ids, tw, tokens)


EDGE_COUNTS = {
    "w4-dsv3-e8": [0, 1, 17, 128, 129, 650, 330, 745],
    "w4-dsv3-e64": [0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129] + [5] * 49,
    "w4-dsv3-e64s": [0, 1, 15, 16, 17, 31, 32, 33, 47, 48, 49] + [4] * 52 + [5],
}


@pytest.mark.parametrize("name", ["w4-dsv3-e8", "w4-dsv3-e64", "w4-dsv3-e64s"])
def test_w4_tile_edges(name):
    """Both W4A8 GEMMs at the DeepSeek-V3 expert shapes with expert row counts straddling the
    128- and 64-row tile and 16-row fragment boundaries (E = 8: 128-row tiles; E = 64, under 32
    rows per expert: 64-row tiles; E = 64, under 16 rows per expert: the streaming engine's
    16-row tiles)."""
    cfg = CFG[name]
    counts = EDGE_COUNTS[name]
    flat = np.repeat(np.arange(cfg.E, dtype=np.int32), counts)
    T = len(flat) // 2
    assert T == cfg.T and max(counts) <= T
    ids = np.stack([flat[:T], flat[T:]], axis=1)
    assert np.all(ids[:, 0] != ids[:, 1])
    ids = np.ascontiguousarray(ids[np.random.default_rng(43).permutation(T)])
    tw = synth.positive_scales(T * 2, cfg.seed, 0.05, 1.0).reshape(T, 2)
    al, bm, a_q, a_s, gq, gs = run_w13(name, ids)
    assert list(al["counts"]) == counts
    rows = set()
    for e, n in enumerate(counts[:17]):  # every boundary case, and two of the 5-row experts
        r0 = int(al["padded_offsets"][e])
        js = {0, 1, 15, 16, 17, n - 2, n - 1}
        for b in (16, 32, 64, 128):
            for m in range(1, n // b + 1):
                js |= {m * b - 1, m * b}
        rows |= {r0 + j for j in js if 0 <= j < n}
    rows = np.array(sorted(rows), dtype=np.int64)
    check_w13(name, al, bm, a_q, a_s, gq, gs, rows)
    tokens = np.unique(al["sorted_pair_ids"][rows] // cfg.k)
    run_check_w2(name, ids, tw, tokens)


# ------------------------------------------------------------------ the whole layer

@pytest.mark.parametrize("name", ["w4-tiny", "w4-small", "w4-s4", "w4-s32", "w4-decode", "w4-block"])
def test_w4_forward_matches_oracle(name):
    cfg = CFG[name]
    say(f"[w4 forward] {name}")
    L = layer_of(name)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device=DEV)
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=DEV)
    tw = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=DEV)
    ws = workload.forward_workspace(L)
    workload.forward(L, out, ws, topk_ids=ids, topk_weights=tw)
    got, ids_d, tw_d = host(out), host(ids), host(tw)
    tokens = np.arange(cfg.T) if name in SMALL else np.sort(np.random.default_rng(4).choice(cfg.T, 8, replace=False))
    x = oracle.activations_f32(cfg)[tokens]
    w = oracle_weights(name, np.unique(ids_d[tokens]))
    ref = oracle.w4_moe_tokens(x, ids_d[tokens], tw_d[tokens], *w, I=cfg.I)
    err = np.abs(got[tokens] - ref).max()
    say(f"[w4 forward] {name}: max err {err:.3e}, max |ref| {np.abs(ref).max():.3e}, "
        f"bit-equal {np.mean(got[tokens] == ref):.4f}")
    assert np.isfinite(got).all()
    assert err <= LAYER_BAR * np.abs(ref).max()
