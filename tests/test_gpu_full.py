"""GPU parity at the full DeepSeek-V3 sizes, through the C ABI, in the launch configuration the
benchmark times (block_m from w8a8_moe_pick_block_m, the engine the library picks for the shape).

Workloads: decode (T=128, staged engine), prefill (T=8192, DMA engine), skew (T=4096, Zipf-skewed
load, ring engine), skew-empty (the same with 30 empty experts, ring engine) and block (T=2048,
128x128 block-wise, ring engine).  One module-scoped fixture per workload holds the device layer and
the oracle's own quantized copy of every active expert (drawn by the shared generator, quantized by
the oracle), so each workload's weights are built once.

What is compared (bars as in test_gpu_parity.py):
  - every expert's weights: device quantization == oracle quantization, bit for bit;
  - activation quantization, routing, align: whole outputs;
  - raw int32 accumulators of both GEMMs: every real row bit for bit against the oracle (at prefill
    65536 rows x 4096, then x 7168, int32), and every real row through an exact projection
    (sum_n acc[r, n] v_n == a[row(r)] . (W_e^T v) for two seeded integer vectors v, exact in
    fp32/fp64 at these magnitudes);
  - first GEMM + SiLU + requant on that row set;
  - second GEMM + combine fed the same intermediate, bit for bit, and the whole layer (5e-3 bar), on
    tokens chosen so that every active expert contributes to at least one checked token.
"""
import sys
from dataclasses import dataclass
from typing import List

import numpy as np
import pytest

import gpu_checks
import oracle
import synth

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import w8a8_int8_quantized_quant_amd as w8  # noqa: E402
from w8a8_int8_quantized_quant_amd import workload  # noqa: E402

DEV = "cuda"
ULP = 2.0 ** -23
FULL = ["decode", "prefill", "skew", "skew-empty", "block"]
ENGINE = {"decode": w8.ENGINE_STAGED, "prefill": w8.ENGINE_DMA, "skew": w8.ENGINE_RING,
          "skew-empty": w8.ENGINE_RING, "block": w8.ENGINE_RING}
# real rows per tile (staged: block_m of the padded rows)
TILE_ROWS = {w8.ENGINE_DMA: (320,), w8.ENGINE_RING: (128,)}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dt(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def oracle_weights_all(cfg, experts):
    return gpu_checks.oracle_weights(torch, DEV, cfg, experts)


@dataclass
class Full:
    name: str
    cfg: synth.MoEConfig
    L: workload.DeviceLayer
    ids: np.ndarray
    tw: np.ndarray
    bm: int
    al: dict
    d: dict
    w: tuple
    active: List[int]
    rows: np.ndarray
    tokens: np.ndarray


def check_rows(al, counts, bm, tiles, P, seed, all_rows=False):
    """Sorted rows to compare whole: per non-empty expert its first and last rows, the rows around
    every boundary of its segment's tiles (each size in `tiles`) and the 16-row fragment boundaries
    of its first and last tiles, and three random rows."""
    R = int(al["num_tiles"][0]) * bm
    if all_rows:
        return np.nonzero(al["sorted_pair_ids"][:R] < P)[0].astype(np.int64)
    rng = np.random.default_rng(seed)
    rows = set()
    for e, n in enumerate(counts):
        n = int(n)
        if n == 0:
            continue
        r0 = int(al["padded_offsets"][e])
        js = {0, 1, 15, 16, n - 2, n - 1, (n // 16) * 16 - 1, (n // 16) * 16}
        for tile in tiles:
            for m in range(1, n // tile + 1):
                js |= {m * tile - 1, m * tile, m * tile + 15, m * tile + 16}
        js |= set(rng.integers(0, n, size=3).tolist())
        rows |= {r0 + j for j in js if 0 <= j < n}
    return np.array(sorted(rows), dtype=np.int64)


def cover_tokens(ids, E, seed, extra=8):
    """Tokens such that every expert that some token selects is selected by at least one of them
    (greedy over a seeded token order), plus `extra` random tokens."""
    rng = np.random.default_rng(seed)
    order = rng.permutation(ids.shape[0])
    need = set(np.unique(ids).tolist())
    pick = []
    for t in order:
        new = need & set(ids[t].tolist())
        if new:
            pick.append(int(t))
            need -= new
        if not need:
            break
    assert not need
    pick += rng.choice(ids.shape[0], size=min(extra, ids.shape[0]), replace=False).tolist()
    return np.unique(np.array(pick, dtype=np.int64))


@pytest.fixture(scope="module", params=FULL)
def full(request):
    name = request.param
    cfg = synth.CONFIGS[name]
    say(f"[full] {name}: drawing the device layer")
    L = workload.make_layer(cfg, device=DEV)
    ids, tw = oracle.route_cfg(cfg, synth.logits(cfg))
    bm = w8.w8a8_moe_pick_block_m(cfg.T, cfg.k, cfg.E)
    al = oracle.align(ids, cfg.E, bm)
    d = {key: dt(v) for key, v in al.items()}
    active = [int(e) for e in np.nonzero(al["counts"])[0]]
    say(f"[full] {name}: oracle weights of {len(active)} active experts, block_m={bm}")
    w = oracle_weights_all(cfg, active)
    engine = w8.w8a8_moe_engine(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I, bm, L.scale_mode)
    tiles = TILE_ROWS.get(engine, (bm,))
    rows = check_rows(al, al["counts"], bm, tiles, cfg.T * cfg.k, 1, all_rows=(name == "decode"))
    tokens = cover_tokens(ids, cfg.E, 2)
    say(f"[full] {name}: {len(rows)} check rows, {len(tokens)} check tokens")
    f = Full(name, cfg, L, ids, tw, bm, al, d, w, active, rows, tokens)
    del L, d, w
    yield f
    f.L = f.d = f.w = None  # release the device layer and the host weights before the next workload
    torch.cuda.empty_cache()


def test_engine_is_the_one_the_workload_names(full):
    cfg = full.cfg
    assert w8.w8a8_moe_engine(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I, full.bm, full.L.scale_mode) == ENGINE[full.name]
    if full.name == "skew-empty":
        assert int((full.al["counts"] == 0).sum()) >= 30
        assert len(full.active) == cfg.E - int((full.al["counts"] == 0).sum())


def test_every_expert_weights_bit_exact(full):
    """Expert weights drawn and quantized on the device equal the oracle's own quantization."""
    L, w = full.L, full.w
    for e in full.active:
        assert np.array_equal(host(L.w13[e]), w[0][e]), e
        assert np.array_equal(host(L.w13_scale[e]), w[1][e]), e
        assert np.array_equal(host(L.w2[e]), w[2][e]), e
        assert np.array_equal(host(L.w2_scale[e]), w[3][e]), e


def test_activation_quant_bit_exact(full):
    cfg = full.cfg
    group = 128 if cfg.scale_mode == "block" else 0
    q = torch.empty((cfg.T, cfg.H), dtype=torch.int8, device=DEV)
    s = torch.empty((cfg.T, cfg.H // 128) if group else (cfg.T,), dtype=torch.float32, device=DEV)
    w8.w8a8_quant_per_token(full.L.x, group, q, s)
    rq, rs = oracle.quant_per_token(oracle.activations_f32(cfg), group)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(s), rs)


def test_routing(full):
    cfg = full.cfg
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=DEV)
    tw = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=DEV)
    w8.moe_topk_route(full.L.logits, cfg.k, full.L.score_fn, cfg.n_group, cfg.topk_group, cfg.renormalize,
                      cfg.routed_scaling, None, ids, tw)
    gpu_checks.check_routing(cfg, host(full.L.logits), host(ids), host(tw), full.ids, full.tw)


@pytest.mark.parametrize("bm", [16, 32, 64, 128])
def test_align_bit_exact(full, bm):
    gpu_checks.check_align_equal(gpu_checks.dev_align(w8, torch, DEV, full.ids, full.cfg.E, bm),
                                 oracle.align(full.ids, full.cfg.E, bm))


def _projection_check(got, real, arow, a, w_list, expert_of, V):
    """sum_n got[r, n] V[n, j] == a[arow[r]] . (W_e^T V[:, j]) for every real row r: both sides are
    exact (|W^T v| < 2^24 in fp32, the dot products < 2^53 in fp64)."""
    lhs = got[real].astype(np.float64) @ V.astype(np.float64)
    rhs = np.empty_like(lhs)
    Vf = V.astype(np.float32)
    for e in np.unique(expert_of):
        sel = np.nonzero(expert_of == e)[0]
        U = (Vf.T @ w_list[e].astype(np.float32)).T  # [K, 2], exact integers
        rhs[sel] = a[arow[sel]].astype(np.float64) @ U.astype(np.float64)
    bad = np.nonzero(np.any(lhs != rhs, axis=1))[0]
    assert len(bad) == 0, f"{len(bad)} rows differ, first sorted rows {real[bad[:8]]}"


def _all_rows_equal(got, a, gather, w_list, al, bm, P, k, real, label):
    """Every real row of `got` bit for bit against the oracle's accumulators, computed in chunks of
    rows (a progress line per chunk: the oracle takes about a minute per GEMM at prefill)."""
    chunks = np.array_split(real, max(1, len(real) // 4096))
    for i, rows in enumerate(chunks):
        ref = oracle.grouped_gemm_i32(a, gather, w_list, al, bm, P, k, rows)
        bad = np.nonzero(np.any(got[rows] != ref[rows], axis=1))[0]
        assert len(bad) == 0, f"{label}: {len(bad)} rows differ, first sorted rows {rows[bad[:8]]}"
        say(f"[i32] {label}: {len(rows)} rows equal ({i + 1}/{len(chunks)})")
        del ref


def test_gemm_i32_bit_exact(full):
    """Raw int32 accumulators of both GEMMs through the engine the workload runs: every real row
    bit for bit against the oracle, and by the exact projection."""
    cfg, al, d, bm = full.cfg, full.al, full.d, full.bm
    P = cfg.T * cfg.k
    R = w8.w8a8_moe_max_rows(cfg.T, cfg.k, cfg.E, bm)
    nt = int(al["num_tiles"][0])
    real = np.nonzero(al["sorted_pair_ids"][: nt * bm] < P)[0]
    pid = al["sorted_pair_ids"][real]
    expert_of = al["tile_expert"][real // bm]
    V = synth.int8_matrix(2, max(2 * cfg.I, cfg.H), cfg.seed + 500).T.astype(np.int32) % 17 - 8  # entries in [-8, 8]
    group = 128 if cfg.scale_mode == "block" else 0
    a_q, _ = oracle.quant_per_token(oracle.activations_f32(cfg), group)
    say(f"[i32] {full.name}: first GEMM, {len(real)} real rows")
    ws = torch.empty(max(w8.w8a8_grouped_gemm_i32_workspace_bytes(True, 2 * cfg.I, cfg.H, cfg.T, cfg.k, cfg.E, bm),
                         256), dtype=torch.uint8, device=DEV)
    out = torch.empty((R, 2 * cfg.I), dtype=torch.int32, device=DEV)
    w8.w8a8_grouped_gemm_i32(dt(a_q), True, full.L.w13, d["sorted_pair_ids"], d["padded_offsets"], d["tile_expert"],
                             d["num_tiles"], cfg.T, cfg.k, bm, out, ws)
    got = host(out)
    del out
    _projection_check(got, real, pid // cfg.k, a_q, full.w[0], expert_of, V[: 2 * cfg.I])
    _all_rows_equal(got, a_q, True, full.w[0], al, bm, P, cfg.k, real, f"{full.name} first GEMM")
    del got
    say(f"[i32] {full.name}: second GEMM")
    h = synth.int8_matrix(R, cfg.I, cfg.seed)
    ws2 = torch.empty(max(w8.w8a8_grouped_gemm_i32_workspace_bytes(False, cfg.H, cfg.I, cfg.T, cfg.k, cfg.E, bm),
                          256), dtype=torch.uint8, device=DEV)
    out2 = torch.empty((R, cfg.H), dtype=torch.int32, device=DEV)
    w8.w8a8_grouped_gemm_i32(dt(h), False, full.L.w2, d["sorted_pair_ids"], d["padded_offsets"], d["tile_expert"],
                             d["num_tiles"], cfg.T, cfg.k, bm, out2, ws2)
    got2 = host(out2)
    del out2
    _projection_check(got2, real, real, h, full.w[2], expert_of, V[: cfg.H])
    _all_rows_equal(got2, h, False, full.w[2], al, bm, P, cfg.k, real, f"{full.name} second GEMM")


def test_first_gemm_silu_requant(full):
    cfg, al, d, bm = full.cfg, full.al, full.d, full.bm
    block = cfg.scale_mode == "block"
    a_q, a_s = oracle.quant_per_token(oracle.activations_f32(cfg), 128 if block else 0)
    R = w8.w8a8_moe_max_rows(cfg.T, cfg.k, cfg.E, bm)
    h_q = torch.empty((R, cfg.I), dtype=torch.int8, device=DEV)
    h_s = torch.empty((R, cfg.I // 128) if block else (R,), dtype=torch.float32, device=DEV)
    mode = w8.SCALE_BLOCK128 if block else w8.SCALE_CHANNEL
    ws = torch.empty(max(w8.w8a8_w13_workspace_bytes(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I, bm, mode), 256),
                     dtype=torch.uint8, device=DEV)
    fn = w8.w8a8_block_grouped_gemm_w13_silu if block else w8.w8a8_grouped_gemm_w13_silu
    fn(dt(a_q), dt(a_s), full.L.w13, full.L.w13_scale, d["sorted_pair_ids"], d["padded_offsets"], d["tile_expert"],
       d["num_tiles"], cfg.T, cfg.k, bm, h_q, h_s, ws)
    rows = full.rows
    say(f"[w13] {full.name}: {len(rows)} rows")
    rq, rs = oracle.w13_silu(a_q, a_s, full.w[0], full.w[1], al, bm, cfg.T, cfg.k, cfg.H, cfg.I, block, rows)
    gq, gs = host(h_q)[rows], host(h_s)[rows]
    rq, rs = rq[rows], rs[rows]
    assert np.all(np.abs(gs - rs) <= 4 * ULP * rs), np.abs(gs / rs - 1).max()
    diff = np.abs(gq.astype(np.int32) - rq.astype(np.int32))
    assert diff.max() <= 1
    assert np.mean(diff > 0) <= 1e-3, np.mean(diff > 0)


def test_second_gemm_combine_bit_exact(full):
    """Fed the same intermediate, the second GEMM + combine is the oracle's fp32 operations in the
    oracle's order: equal bits on tokens that together touch every active expert."""
    cfg, al, d, bm = full.cfg, full.al, full.d, full.bm
    block = cfg.scale_mode == "block"
    R = w8.w8a8_moe_max_rows(cfg.T, cfg.k, cfg.E, bm)
    h_q = synth.int8_matrix(R, cfg.I, cfg.seed + 100)
    h_s = synth.positive_scales(R * (cfg.I // 128 if block else 1), cfg.seed, 1e-3, 3e-2)
    h_s = h_s.reshape(R, cfg.I // 128) if block else h_s
    out = torch.full((cfg.T, cfg.H), float("nan"), dtype=torch.float32, device=DEV)
    mode = w8.SCALE_BLOCK128 if block else w8.SCALE_CHANNEL
    ws = torch.empty(max(w8.w8a8_w2_workspace_bytes(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I, bm, mode), 256),
                     dtype=torch.uint8, device=DEV)
    fn = w8.w8a8_block_grouped_gemm_w2_combine if block else w8.w8a8_grouped_gemm_w2_combine
    fn(dt(h_q), dt(h_s), full.L.w2, full.L.w2_scale, d["sorted_pair_ids"], d["padded_offsets"], d["tile_expert"],
       d["num_tiles"], dt(full.tw), cfg.T, cfg.k, bm, out, ws)
    tokens = full.tokens
    say(f"[w2] {full.name}: {len(tokens)} tokens")
    ref = oracle.w2_combine(h_q, h_s, full.w[2], full.w[3], al, bm, full.tw, cfg.T, cfg.k, cfg.H, cfg.I, block,
                            tokens)
    got = host(out)
    assert np.array_equal(got[tokens], ref)
    assert np.isfinite(got).all()


def test_forward_matches_oracle(full):
    cfg, L = full.cfg, full.L
    out = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device=DEV)
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=DEV)
    tw = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=DEV)
    ws = workload.forward_workspace(L)
    workload.forward(L, out, ws, topk_ids=ids, topk_weights=tw)
    got, gids = host(out), host(ids)
    tokens = full.tokens
    keep = np.all(gids[tokens] == full.ids[tokens], axis=1)
    assert keep.mean() >= 0.95
    tokens = tokens[keep]
    say(f"[forward] {full.name}: {len(tokens)} tokens")
    x = oracle.activations_f32(cfg)[tokens]
    ref = oracle.moe_tokens(x, full.ids[tokens], full.tw[tokens], *full.w, I=cfg.I,
                            block=cfg.scale_mode == "block")
    err = np.abs(got[tokens] - ref).max()
    assert err <= 5e-3 * np.abs(ref).max(), (err, np.abs(ref).max())
    assert np.isfinite(got).all()


def test_forward_past_4gib_of_pair_outputs():
    """DeepSeek-V3 shapes at T = 32768, four times the prefill batch, on the engine the library picks
    for it (the DMA engine): the second GEMM's per-pair fp32 outputs span 7.5 GB, so the rows of the
    later experts sit past byte offset 2^32, where the GEMM's epilogue writes them and the combine reads
    them back.  Tokens with a pair past that mark, the last tokens and a seeded spread match the oracle
    (whole-layer bar); the oracle draws only the experts those tokens use."""
    import dataclasses
    cfg = dataclasses.replace(synth.CONFIGS["prefill"], name="prefill-x4", T=4 * synth.CONFIGS["prefill"].T)
    bm = w8.w8a8_moe_pick_block_m(cfg.T, cfg.k, cfg.E)
    say(f"[4gib] T={cfg.T}: drawing the device layer, block_m={bm}")
    L = workload.make_layer(cfg, device=DEV)
    assert w8.w8a8_moe_engine(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I, bm, L.scale_mode) == w8.ENGINE_DMA
    ids, tw = oracle.route_cfg(cfg, synth.logits(cfg))
    al = oracle.align(ids, cfg.E, bm)
    P = cfg.T * cfg.k
    R = int(al["num_tiles"][0]) * bm
    srt = al["sorted_pair_ids"][:R]
    first_far = (1 << 32) // (cfg.H * 4) + 1  # first sorted row whose fp32 output starts past 2^32 bytes
    assert R > first_far + 1000
    far_pairs = srt[first_far:][srt[first_far:] < P]
    rng = np.random.default_rng(5)
    tokens = np.unique(np.concatenate([
        rng.choice(far_pairs // cfg.k, size=6, replace=False),  # a pair past the 4 GiB mark
        np.array([cfg.T - 1, cfg.T - 2]),                        # the last tokens
        rng.choice(cfg.T, size=4, replace=False),                # a spread
    ]).astype(np.int64))
    assert np.any(np.isin(tokens, far_pairs // cfg.k))
    out = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device=DEV)
    gids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=DEV)
    gtw = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=DEV)
    ws = workload.forward_workspace(L)
    say(f"[4gib] workspace {ws.numel() / 2**30:.1f} GiB; forward")
    workload.forward(L, out, ws, topk_ids=gids, topk_weights=gtw)
    got = host(out[torch.from_numpy(tokens).to(DEV)])
    keep = np.all(host(gids)[tokens] == ids[tokens], axis=1)
    assert keep.sum() >= len(tokens) - 1
    tokens, got = tokens[keep], got[keep]
    experts = np.unique(ids[tokens])
    say(f"[4gib] oracle over {len(tokens)} tokens, {len(experts)} experts")
    w = oracle_weights_all(cfg, experts)
    x = np.concatenate([oracle.activations_f32(cfg, rows=slice(int(t), int(t) + 1)) for t in tokens])
    ref = oracle.moe_tokens(x, ids[tokens], tw[tokens], *w, I=cfg.I, block=False)
    err = np.abs(got - ref).max()
    assert err <= 5e-3 * np.abs(ref).max(), (err, np.abs(ref).max())
    assert np.isfinite(got).all()

