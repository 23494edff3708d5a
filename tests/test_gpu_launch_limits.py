"""GPU parity where a launch would exceed what one dispatch can address.  A dispatch counts the
work-items of its x extent in 32 bits, so the library keeps every grid within 2^20 workgroups:
quantization and routing go in pieces of rows or tokens, the staged GEMM in pieces of its
(row tile, N-tile) items, and the requantization and combine kernels take the rest of their rows
with a grid stride.  Each test here is sized so that one of those paths runs more than once, and
checks rows on both sides of every piece boundary against the oracle; the last one runs a layer of
more than 2^32 activation elements, where an unpieced launch would wrap.

Bars as in test_gpu_parity.py: quantization bit for bit, routing by the near-tie rule, the whole
layer within 5e-3 of the largest reference magnitude.
"""
import dataclasses
import sys

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
PIECE = 1 << 20  # workgroups per launch at most


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def dev_normal(n, seed, sigma=1.0):
    buf = torch.empty(n, dtype=torch.float32, device=DEV)
    synth.dev_normal(buf.data_ptr(), n, seed, synth.STREAM_MISC, 0, sigma, torch.cuda.current_stream().cuda_stream)
    return buf


def rows_f32(seed, cols, rows, sigma=1.0):
    """Host copy of the listed rows of the same fp32 fill."""
    return np.stack([synth.normal(cols, seed, synth.STREAM_MISC, int(r) * cols, sigma) for r in rows])


def test_quant_per_token_rows_in_pieces():
    """2^20 + 37 rows of 128 bf16 values, one scale per row: two launches of the per-row kernel
    (2^20 rows, then 37).  Every row matches the oracle bit for bit."""
    rows, cols = PIECE + 37, 128
    say(f"[pieces] per-token quant rows={rows}")
    x = dev_normal(rows * cols, 11).view(rows, cols).to(torch.bfloat16)
    q = torch.empty((rows, cols), dtype=torch.int8, device=DEV)
    s = torch.full((rows,), -1.0, dtype=torch.float32, device=DEV)
    w8.w8a8_quant_per_token(x, 0, q, s)
    rq, rs = oracle.quant_per_token(x.float().cpu().numpy(), 0)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(s), rs)


def test_quant_per_token_groups_in_pieces():
    """32768 + 37 rows of 1024 fp32 values in groups of 8: 128 wavefronts per row, 2^22 per launch,
    so two launches (32768 rows, then 37).  Every group matches the oracle bit for bit."""
    rows, cols, group = 32768 + 37, 1024, 8
    say(f"[pieces] per-token-group quant rows={rows} group={group}")
    x = dev_normal(rows * cols, 12).view(rows, cols)
    q = torch.empty((rows, cols), dtype=torch.int8, device=DEV)
    s = torch.full((rows, cols // group), -1.0, dtype=torch.float32, device=DEV)
    w8.w8a8_quant_per_token(x, group, q, s)
    rq, rs = oracle.quant_per_token(host(x), group)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(s), rs)


@pytest.mark.parametrize("fp8", [False, True])
def test_quant_blocks_in_pieces(fp8):
    """1027 x 4096 fp32 in 2 x 2 blocks: 2048 blocks across a row, 512 block rows per launch, so
    launches of 512 and 2 block rows, the last block row one row high.  Codes and scales match the
    oracle bit for bit (INT8 and FP8 rules)."""
    rows, cols = 1027, 4096
    say(f"[pieces] block quant {rows}x{cols} 2x2 fp8={fp8}")
    x = dev_normal(rows * cols, 13).view(rows, cols)
    q = torch.empty((rows, cols), dtype=torch.uint8 if fp8 else torch.int8, device=DEV)
    s = torch.full(((rows + 1) // 2, cols // 2), -1.0, dtype=torch.float32, device=DEV)
    if fp8:
        w8.w8a8_fp8_quant_blocks(x, 2, 2, q, s)
        rq, rs = oracle.fp8_quant_blocks(host(x), 2, 2)
    else:
        w8.w8a8_quant_blocks(x, 2, 2, q, s)
        rq, rs = oracle.quant_blocks(host(x), 2, 2)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(s), rs)


def test_w4_quant_rows_in_pieces():
    """8192 + 3 rows of 65536 fp32 weights: 512 groups of 128 per row, 2^22 wavefronts per launch,
    so launches of 8192 rows and 3.  The rows at both ends and on both sides of the boundary match
    the oracle bit for bit (packed codes and scales)."""
    rows, cols = 8192 + 3, 65536
    say(f"[pieces] w4 quant rows={rows} cols={cols}")
    x = dev_normal(rows * cols, 14, 0.006).view(rows, cols)
    q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=DEV)
    s = torch.full((rows, cols // 128), -1.0, dtype=torch.float32, device=DEV)
    w8.w8a8_w4a8_quant_weights(x, q, s)
    check = np.array([0, 1, 8190, 8191, 8192, 8193, rows - 1])
    sel = torch.from_numpy(check).to(DEV)
    rq, rs = oracle.w4_quant(rows_f32(14, cols, check, 0.006))
    assert np.array_equal(host(q[sel]), rq)
    assert np.array_equal(host(s[sel]), rs)
    assert (host(s) > 0).all()  # every row's scales written


def test_route_tokens_in_pieces():
    """2^22 + 77 tokens of the DeepSeek-V3 routing rule (256 experts, sigmoid, 8 groups keep 4,
    top-8): 4 tokens per workgroup, 2^22 tokens per launch, so two launches.  Tokens on both sides
    of the boundary, the last ones and a seeded spread follow the oracle (near-tie rule)."""
    cfg = dataclasses.replace(synth.CONFIGS["prefill"], name="route-pieces", T=4 * PIECE + 77)
    say(f"[pieces] route T={cfg.T}")
    lg = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=DEV)
    synth.dev_logits(lg.data_ptr(), cfg, None, torch.cuda.current_stream().cuda_stream)
    ids = torch.full((cfg.T, cfg.k), -1, dtype=torch.int32, device=DEV)
    tw = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=DEV)
    w8.moe_topk_route(lg, cfg.k, w8.SCORE_SIGMOID, cfg.n_group, cfg.topk_group, cfg.renormalize,
                      cfg.routed_scaling, None, ids, tw)
    rng = np.random.default_rng(15)
    tokens = np.unique(np.concatenate([np.array([0, 4 * PIECE - 1, 4 * PIECE, 4 * PIECE + 1, cfg.T - 1]),
                                       rng.choice(cfg.T, size=59, replace=False)]))
    sel = torch.from_numpy(tokens).to(DEV)
    lgh = np.concatenate([synth.logits(cfg, rows=slice(int(t), int(t) + 1)) for t in tokens])
    ids_o, w_o = oracle.route_cfg(cfg, lgh)
    sub = dataclasses.replace(cfg, T=len(tokens))
    gpu_checks.check_routing(sub, lgh, host(ids[sel]), host(tw[sel]), ids_o, w_o)
    assert (host(ids) >= 0).all()  # every token routed


def _forward_check(cfg, tokens, ids, tw, got, tag):
    tokens = np.asarray(tokens)
    say(f"[{tag}] oracle over {len(tokens)} tokens")
    w = gpu_checks.oracle_weights(torch, DEV, cfg, range(cfg.E))
    x = np.concatenate([oracle.activations_f32(cfg, rows=slice(int(t), int(t) + 1)) for t in tokens])
    ref = oracle.moe_tokens(x, ids[tokens], tw[tokens], *w, I=cfg.I, block=False)
    assert np.isfinite(got).all()
    err = np.abs(got - ref).max()
    assert err <= 5e-3 * np.abs(ref).max(), (err, np.abs(ref).max())


def test_forward_staged_in_pieces():
    """2^20 + 100 tokens, hidden = intermediate = 384 (not multiples of 256: the staged engine),
    8 experts, top-4, 16-row tiles.  The first GEMM's 262k row tiles x 6 N-tiles go in two launches,
    the requantization's 4.19M rows take a second grid-stride pass, and the combine's tokens past
    2^20 another.  Tokens on both sides of 2^20, the last ones, tokens with a pair in the first
    GEMM's second launch or in the requantization's second pass, and a seeded spread match the oracle."""
    cfg = synth.MoEConfig(name="staged-pieces", index=37, T=PIECE + 100, H=384, I=384, E=8, k=4, route="softmax",
                          n_group=1, topk_group=1, routed_scaling=1.0, renormalize=True, x_dtype=synth.DTYPE_BF16,
                          x_sigma=1.0, outlier_threshold=synth.OUTLIER_THRESHOLD, outlier_mult=20.0, w_sigma=0.02,
                          scale_mode="channel")
    bm = 16
    assert w8.w8a8_moe_engine(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I, bm, 0) == w8.ENGINE_STAGED
    say(f"[staged-pieces] T={cfg.T}: drawing the device layer")
    L = workload.make_layer(cfg, device=DEV)
    ids, tw = oracle.route_cfg(cfg, synth.logits(cfg))
    al = oracle.align(ids, cfg.E, bm)
    P = cfg.T * cfg.k
    R = int(al["num_tiles"][0]) * bm
    srt = al["sorted_pair_ids"][:R]
    n13 = cfg.I // 64                      # first-GEMM N-tiles of the staged engine
    first_piece2 = -(-PIECE // n13) * bm   # first sorted row whose every N-tile is in the second launch
    requant2 = 4 * PIECE                   # requantization rows past one grid of 2^20 x 4 wavefronts
    assert R > requant2 and R > first_piece2
    p2 = srt[first_piece2:][srt[first_piece2:] < P]
    p3 = srt[requant2:][srt[requant2:] < P]
    assert len(p3) > 0
    rng = np.random.default_rng(16)
    tokens = np.unique(np.concatenate([
        np.array([0, 1, PIECE - 1, PIECE, PIECE + 1, cfg.T - 2, cfg.T - 1]),
        rng.choice(p2 // cfg.k, size=4, replace=False),
        p3[:4] // cfg.k,
        rng.choice(cfg.T, size=4, replace=False),
    ]).astype(np.int64))
    out = torch.full((cfg.T, cfg.H), float("nan"), dtype=torch.float32, device=DEV)
    gids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=DEV)
    gtw = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=DEV)
    ws = workload.forward_workspace(L, block_m=bm)
    say(f"[staged-pieces] workspace {ws.numel() / 2**30:.1f} GiB; forward")
    workload.forward(L, out, ws, block_m=bm, topk_ids=gids, topk_weights=gtw)
    assert not torch.isnan(out).any().item()  # every token written
    sel = torch.from_numpy(tokens).to(DEV)
    got, gid = host(out[sel]), host(gids[sel])
    keep = np.all(gid == ids[tokens], axis=1)
    assert keep.sum() >= len(tokens) - 1
    _forward_check(cfg, tokens[keep], ids, tw, got[keep], "staged-pieces")


def test_forward_past_2_32_elements():
    """T * H > 2^32: 2^24 + 4096 tokens of a 256-wide layer (8 experts, top-2) on the staged engine.
    The activations, their quantized copy, the fp32 intermediate, the per-pair outputs and the layer
    output each hold more than 2^32 elements, and a grid of one workgroup per token (of 256 threads)
    would count more than 2^32 work-items.  The output starts as NaN; every token is written, and
    tokens on both sides of the 2^32-element mark, tokens with a pair past it, the last ones and a
    seeded spread match the oracle.  About 110 GB of device memory."""
    H = I = 256
    T = (1 << 32) // H + 4096
    cfg = synth.MoEConfig(name="past-2-32", index=36, T=T, H=H, I=I, E=8, k=2, route="softmax", n_group=1,
                          topk_group=1, routed_scaling=1.0, renormalize=True, x_dtype=synth.DTYPE_BF16, x_sigma=1.0,
                          outlier_threshold=synth.OUTLIER_THRESHOLD, outlier_mult=20.0, w_sigma=0.006,
                          scale_mode="channel")
    free, _ = torch.cuda.mem_get_info()
    if free < (150 << 30):
        pytest.skip(f"needs ~150 GB of free device memory, {free / 2**30:.0f} GiB free")
    bm = w8.w8a8_moe_pick_block_m(cfg.T, cfg.k, cfg.E)
    assert w8.w8a8_moe_engine(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I, bm, 0) == w8.ENGINE_STAGED
    say(f"[2^32] T={T}: drawing the device layer, block_m={bm}")
    L = workload.make_layer(cfg, device=DEV)
    ids, tw = oracle.route_cfg(cfg, synth.logits(cfg))
    al = oracle.align(ids, cfg.E, bm)
    P = cfg.T * cfg.k
    R = int(al["num_tiles"][0]) * bm
    srt = al["sorted_pair_ids"][:R]
    far = (1 << 32) // I  # the first sorted row past 2^32 elements of the intermediate (and outputs)
    far_pairs = srt[far:][srt[far:] < P]
    rng = np.random.default_rng(7)
    t0 = (1 << 32) // H  # the first token past 2^32 elements of the activations
    tokens = np.unique(np.concatenate([
        np.array([0, t0 - 1, t0, t0 + 1, T - 2, T - 1]),
        rng.choice(far_pairs // cfg.k, size=4, replace=False),
        rng.choice(T, size=4, replace=False),
    ]).astype(np.int64))
    out = torch.full((cfg.T, cfg.H), float("nan"), dtype=torch.float32, device=DEV)
    gids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=DEV)
    gtw = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=DEV)
    ws = workload.forward_workspace(L)
    say(f"[2^32] workspace {ws.numel() / 2**30:.1f} GiB; forward")
    workload.forward(L, out, ws, topk_ids=gids, topk_weights=gtw)
    assert not torch.isnan(out).any().item()  # every token written
    sel = torch.from_numpy(tokens).to(DEV)
    got, gid = host(out[sel]), host(gids[sel])
    keep = np.all(gid == ids[tokens], axis=1)
    assert keep.sum() >= len(tokens) - 1
    _forward_check(cfg, tokens[keep], ids, tw, got[keep], "2^32")
