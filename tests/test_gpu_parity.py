"""GPU parity: every stage of the HIP path against the CPU oracle, through the C ABI.

Bars (stated once, used below):
  - bit-exact: activation quantization (a_q, a_s), weight quantization, align
    outputs, raw int32 accumulators, the second GEMM + combine when fed the same
    intermediate (same fp32 operations in the same order on both sides);
  - routing: expert ids equal except near-ties, where the oracle's score gap
    between swapped experts is within 5e-7 relative (libm and device expf
    differ in the last bits); weights within 8 ulp;
  - first GEMM epilogue (uses expf): h_scale within 4 ulp, at most 0.1% of
    h_q entries off by one, none by more;
  - whole layer: max|err| <= 5e-3 * max|ref| over the checked tokens.
Full-size workloads are checked on sampled rows / tokens, which the oracle
computes one by one from its own quantized copies of the experts they touch.
"""
import os
import sys

import numpy as np
import pytest

import gpu_checks
import oracle
import synth
from gpu_checks import check_align_equal, check_routing

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import w8a8_int8_quantized_quant_amd as w8  # noqa: E402
from w8a8_int8_quantized_quant_amd import workload  # noqa: E402

DEV = "cuda"
ULP = 2.0 ** -23


def small_cfg(name="ds-small", index=20, T=300, H=512, I=256, E=16, k=4, route="sigmoid", n_group=4, topk_group=2,
              scaling=2.5, mode="channel", x_dtype=synth.DTYPE_BF16):
    return synth.MoEConfig(name=name, index=index, T=T, H=H, I=I, E=E, k=k, route=route, n_group=n_group,
                           topk_group=topk_group, routed_scaling=scaling, renormalize=True, x_dtype=x_dtype,
                           x_sigma=1.0, outlier_threshold=synth.OUTLIER_THRESHOLD, outlier_mult=20.0,
                           w_sigma=0.006, scale_mode=mode)


SMALL = {
    "tiny": synth.CONFIGS["tiny"],
    "ds-small": small_cfg(),
    "ds-small-block": small_cfg(name="ds-small-block", index=21, mode="block", T=257),
    # DeepSeek-V3 expert shapes with few experts: the large-batch GEMM engine at the real K sizes.
    "dsv3-e8": small_cfg(name="dsv3-e8", index=40, T=1000, H=7168, I=2048, E=8, k=2, route="softmax", n_group=1,
                         topk_group=1, scaling=1.0),
    "dsv3-e8-block": small_cfg(name="dsv3-e8-block", index=41, T=1000, H=7168, I=2048, E=8, k=2, route="softmax",
                               n_group=1, topk_group=1, scaling=1.0, mode="block"),
    # 125 rows per expert on average: the mid-batch (128-row tile) engine, channel-wise
    "dsv3-e16": small_cfg(name="dsv3-e16", index=42, T=1000, H=7168, I=2048, E=16, k=2, route="softmax", n_group=1,
                          topk_group=1, scaling=1.0),
}


def cfg_of(name):
    return synth.CONFIGS.get(name) or SMALL[name]


def dt(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# ------------------------------------------------------------------ caches (one device layer at a time)

_layer = {}
_oracle_w = {}


def layer_of(name):
    if name not in _layer:
        _layer.clear()
        torch.cuda.empty_cache()
        say(f"[layer] drawing {name} on the device")
        _layer[name] = workload.make_layer(cfg_of(name), device=DEV)
    return _layer[name]


def oracle_weights(name, experts):
    """Oracle-side quantized weights (own draw + own quantization), cached per workload."""
    cfg = cfg_of(name)
    cache = _oracle_w.setdefault(name, [[None] * cfg.E for _ in range(4)])
    todo = sorted({int(e) for e in experts if cache[0][int(e)] is None})
    if todo:
        w = oracle.expert_weights(cfg, todo)
        for i in range(4):
            for e in todo:
                cache[i][e] = w[i][e]
    return cache


def sample(n, count, seed):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(n, size=min(n, count), replace=False))


def route_host(cfg):
    return oracle.route_cfg(cfg, synth.logits(cfg))


def block_m_of(cfg):
    return w8.w8a8_moe_pick_block_m(cfg.T, cfg.k, cfg.E)


def dev_align(ids_np, E, bm):
    return gpu_checks.dev_align(w8, torch, DEV, ids_np, E, bm)


def oracle_align_dev(ids_np, E, bm):
    """The oracle's align outputs, uploaded (stage inputs for the GEMM tests)."""
    al = oracle.align(ids_np, E, bm)
    d = {key: dt(v) for key, v in al.items()}
    return al, d


# ------------------------------------------------------------------ generator

@pytest.mark.parametrize("name", ["tiny", "decode", "skew"])
def test_device_generator_matches_host(name):
    cfg = cfg_of(name)
    hs = torch.cuda.current_stream().cuda_stream
    x = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16 if cfg.x_dtype else torch.float32, device=DEV)
    synth.dev_activations(x.data_ptr(), cfg, hs)
    xh = synth.activations(cfg)
    got = host(x.view(torch.int16) if cfg.x_dtype else x)
    assert np.array_equal(got.view(xh.dtype), xh)
    lg = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=DEV)
    bias = synth.zipf_bias(cfg)
    bt = None if bias is None else dt(bias)
    synth.dev_logits(lg.data_ptr(), cfg, None if bt is None else bt.data_ptr(), hs)
    assert np.array_equal(host(lg), synth.logits(cfg))
    n = 2 * cfg.I * cfg.H
    buf = torch.empty(100_000, dtype=torch.float32, device=DEV)
    for start in (0, (cfg.E - 1) * n + n - 100_000):
        synth.dev_normal(buf.data_ptr(), 100_000, cfg.seed, synth.STREAM_W13, start, cfg.w_sigma, hs)
        assert np.array_equal(host(buf), synth.normal(100_000, cfg.seed, synth.STREAM_W13, start, cfg.w_sigma))


# ------------------------------------------------------------------ step 1: quantization

@pytest.mark.parametrize("name", ["tiny", "ds-small"])
def test_activation_quant_bit_exact(name):
    cfg = cfg_of(name)
    group = 128 if cfg.scale_mode == "block" else 0
    say(f"[quant] {name} T={cfg.T} H={cfg.H} group={group}")
    xh = synth.activations(cfg)
    x = dt(xh.view(np.int16)).view(torch.bfloat16) if cfg.x_dtype else dt(xh)
    q = torch.empty((cfg.T, cfg.H), dtype=torch.int8, device=DEV)
    s = torch.empty((cfg.T, cfg.H // 128) if group else (cfg.T,), dtype=torch.float32, device=DEV)
    w8.w8a8_quant_per_token(x, group, q, s)
    rq, rs = oracle.quant_per_token(oracle.activations_f32(cfg), group)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(s), rs)


@pytest.mark.parametrize("rows,cols,group,dtype", [(1, 24, 0, "f32"), (7, 100, 0, "f32"), (5, 96, 32, "bf16"),
                                                   (33, 7168, 128, "f32"), (3, 40, 40, "bf16"),
                                                   (2, 1024, 0, "bf16")])
def test_activation_quant_ragged_and_degenerate(rows, cols, group, dtype):
    z = synth.normal(rows * cols, 3, synth.STREAM_MISC, 0).reshape(rows, cols)
    z[0, :] = 0.0                      # all-zero row: scale floor, q = 0
    if rows > 2:
        z[1, :] = 3e-9                 # tiny row: scale floor
        z[2, ::3] = 0.5                # exact halves
    if dtype == "bf16":
        zb = torch.from_numpy(z).to(torch.bfloat16)
        x = zb.to(DEV)
        zf = zb.to(torch.float32).numpy()
    else:
        x = dt(z)
        zf = z
    q = torch.empty((rows, cols), dtype=torch.int8, device=DEV)
    s = torch.empty((rows, cols // group) if group else (rows,), dtype=torch.float32, device=DEV)
    w8.w8a8_quant_per_token(x, group, q, s)
    rq, rs = oracle.quant_per_token(zf, group)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(s), rs)
    assert np.all(host(q)[0] == 0)


@pytest.mark.parametrize("rows,cols,group,dtype,misalign", [
    (3, 8192, 0, "bf16", 0),     # per-row kernel from registers, at its 8192-column limit
    (3, 8200, 0, "f32", 0),      # one chunk past it: the two-pass per-row kernel
    (1, 8, 0, "f32", 0),         # one chunk per row
    (5, 128, 128, "f32", 0),     # one 128-wide group per row (one 16-lane DPP row)
    (7, 384, 128, "bf16", 0),    # 3 groups per row, 21 groups: a wavefront with a partial DPP row set
    (2, 65536, 128, "bf16", 0),  # 512 groups per row
    (4, 1024, 0, "bf16", 1),     # input 2 bytes off 16-byte alignment: the groups / blocks kernels
    (4, 1024, 128, "f32", 1),    # input 4 bytes off: the wavefront-per-group kernel
])
def test_activation_quant_kernel_paths(rows, cols, group, dtype, misalign):
    """Each activation-quantization kernel and the choice between them: the per-row kernel that
    holds a row in registers (rows of at most 8192 columns) and the two-pass one past that, the
    128-wide group kernel (16 lanes per group), and the fallbacks taken for inputs that are not
    16-byte aligned.  Bit for bit against the oracle, with an all-zero row and exact halves."""
    z = synth.normal(rows * cols, 9, synth.STREAM_MISC, 0).reshape(rows, cols)
    z[0, :] = 0.0
    if rows > 1:
        z[1, ::5] = 0.5
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    zt = torch.from_numpy(z).to(tdt)
    zf = zt.to(torch.float32).numpy()
    # a flat buffer with the matrix `misalign` elements in, so its address is off 16-byte alignment
    flat = torch.zeros(rows * cols + 16, dtype=tdt, device=DEV)
    flat[misalign:misalign + rows * cols] = zt.reshape(-1).to(DEV)
    x = flat[misalign:misalign + rows * cols].view(rows, cols)
    assert (x.data_ptr() % 16 == 0) == (misalign == 0)
    q = torch.empty((rows, cols), dtype=torch.int8, device=DEV)
    s = torch.full((rows, cols // group) if group else (rows,), -1.0, dtype=torch.float32, device=DEV)
    w8.w8a8_quant_per_token(x, group, q, s)
    rq, rs = oracle.quant_per_token(zf, group)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(s), rs)
    assert np.all(host(q)[0] == 0)


@pytest.mark.parametrize("shape,block", [((300, 384), (128, 128)), ((256, 7168), (1, 7168)), ((129, 257), (128, 128)),
                                         ((64, 130), (1, 130))])
def test_weight_quant_blocks_bit_exact(shape, block):
    z = synth.normal(shape[0] * shape[1], 4, synth.STREAM_MISC, 0, 0.006).reshape(shape)
    q = torch.empty(shape, dtype=torch.int8, device=DEV)
    nb = ((shape[0] + block[0] - 1) // block[0], (shape[1] + block[1] - 1) // block[1])
    s = torch.empty(nb, dtype=torch.float32, device=DEV)
    w8.w8a8_quant_blocks(dt(z), block[0], block[1], q, s)
    rq, rs = oracle.quant_blocks(z, *block)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(s), rs)


# ------------------------------------------------------------------ step 2: routing

@pytest.mark.parametrize("name", ["tiny", "ds-small"])
def test_routing(name):
    cfg = cfg_of(name)
    say(f"[route] {name}")
    lg = synth.logits(cfg)
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=DEV)
    tw = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=DEV)
    fn = w8.SCORE_SOFTMAX if cfg.route == "softmax" else w8.SCORE_SIGMOID
    w8.moe_topk_route(dt(lg), cfg.k, fn, cfg.n_group, cfg.topk_group, cfg.renormalize, cfg.routed_scaling, None,
                      ids, tw)
    ids_o, w_o = route_host(cfg)
    check_routing(cfg, lg, host(ids), host(tw), ids_o, w_o)


@pytest.mark.parametrize("E,k,ng,tg,fn,renorm,bias", [(8, 8, 1, 1, 0, True, False), (64, 6, 1, 1, 0, False, False),
                                                      (1, 1, 1, 1, 0, True, False), (1024, 8, 16, 4, 1, True, True),
                                                      (72, 5, 1, 1, 1, False, False), (256, 8, 8, 4, 1, True, True),
                                                      (384, 8, 8, 4, 1, True, True), (256, 6, 2, 1, 1, False, True),
                                                      (256, 8, 64, 8, 1, True, False), (64, 4, 64, 8, 1, True, True),
                                                      (512, 8, 32, 4, 1, True, True), (160, 6, 5, 3, 1, True, False)])
def test_routing_variants(E, k, ng, tg, fn, renorm, bias):
    """Group sizes 1, 4, 16, 32, 64 take the in-register group scores; 48 and 128 the per-lane scan."""
    T = 77
    lg = synth.normal(T * E, 5, synth.STREAM_MISC, 0).reshape(T, E)
    b = synth.normal(E, 6, synth.STREAM_MISC, 0, 0.1) if bias else None
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    tw = torch.empty((T, k), dtype=torch.float32, device=DEV)
    w8.moe_topk_route(dt(lg), k, fn, ng, tg, renorm, 1.5, None if b is None else dt(b), ids, tw)
    ids_o, w_o = oracle.route(lg, k, fn, ng, tg, renorm, 1.5, b)
    cfg = small_cfg(T=T, E=E, k=k, route="softmax" if fn == 0 else "sigmoid")
    if b is None:
        check_routing(cfg, lg, host(ids), host(tw), ids_o, w_o)
    else:
        assert np.mean(np.all(host(ids) == ids_o, axis=1)) >= 0.98
        same = np.all(host(ids) == ids_o, axis=1)
        assert (np.abs(host(tw)[same] - w_o[same]) / w_o[same]).max() <= 8 * ULP


# ------------------------------------------------------------------ step 3: align

@pytest.mark.parametrize("name", ["tiny", "ds-small"])
@pytest.mark.parametrize("bm", [16, 32, 64, 128])
def test_align_bit_exact(name, bm):
    cfg = cfg_of(name)
    ids, _ = route_host(cfg)
    check_align_equal(dev_align(ids, cfg.E, bm), oracle.align(ids, cfg.E, bm))


def test_align_edge_cases():
    rng = np.random.default_rng(3)
    cases = [
        (np.full((5000, 1), 3, np.int32), 8),                      # every pair on one expert
        (np.tile(np.arange(8, dtype=np.int32), (300, 1)), 8),       # k = E
        (np.zeros((1, 1), np.int32), 1),                            # one pair, one expert
        (np.zeros((70000, 1), np.int32), 1),                        # E = 1, many chunks
        (rng.integers(0, 1024, size=(3000, 8)).astype(np.int32), 1024),
        (np.minimum(rng.zipf(1.3, size=(2049, 8)) - 1, 255).astype(np.int32), 256),
    ]
    for ids, E in cases:
        for bm in (16, 128):
            check_align_equal(dev_align(ids, E, bm), oracle.align(ids, E, bm))
    # no tokens: counts and offsets zero, no tiles
    d = dev_align(np.zeros((0, 8), np.int32), 256, 16)
    assert int(host(d["num_tiles"])[0]) == 0 and not host(d["counts"]).any() and not host(d["offsets"]).any()


def test_align_drops_out_of_range_ids():
    ids = np.array([[0, 5], [9, 2], [-1, 5], [3, 3]], np.int32)
    d = dev_align(ids, 8, 16)
    valid = ids.reshape(-1)[(ids.reshape(-1) >= 0) & (ids.reshape(-1) < 8)]
    assert np.array_equal(host(d["counts"]), np.bincount(valid, minlength=8))
    srt = host(d["sorted_pair_ids"])[: int(host(d["padded_offsets"])[-1])]
    assert sorted(srt[srt < 8].tolist()) == [0, 1, 3, 5, 6, 7]


def test_align_is_deterministic():
    ids, _ = route_host(cfg_of("prefill"))
    a = dev_align(ids, 256, 64)
    b = dev_align(ids, 256, 64)
    for key in a:
        assert torch.equal(a[key], b[key])


# ------------------------------------------------------------------ steps 4-5: grouped GEMMs

def stage_rows(al, bm, P):
    """Every non-pad sorted row (the small workloads' oracle runs them all in well under a second)."""
    R = int(al["num_tiles"][0]) * bm
    return np.nonzero(al["sorted_pair_ids"][:R] < P)[0]


def run_i32(L, cfg, a, gather, d, bm):
    """Raw int32 accumulators of the first (gather) or second GEMM through the C ABI."""
    R = w8.w8a8_moe_max_rows(cfg.T, cfg.k, cfg.E, bm)
    N, K = (2 * cfg.I, cfg.H) if gather else (cfg.H, cfg.I)
    out = torch.empty((R, N), dtype=torch.int32, device=DEV)
    ws = torch.empty(max(w8.w8a8_grouped_gemm_i32_workspace_bytes(gather, N, K, cfg.T, cfg.k, cfg.E, bm), 256),
                     dtype=torch.uint8, device=DEV)
    w8.w8a8_grouped_gemm_i32(dt(a), gather, L.w13 if gather else L.w2, d["sorted_pair_ids"], d["padded_offsets"],
                             d["tile_expert"], d["num_tiles"], cfg.T, cfg.k, bm, out, ws)
    return host(out)


@pytest.mark.parametrize("bm", [16, 32, 64, 128])
@pytest.mark.parametrize("name", ["tiny", "ds-small"])
def test_gemm_i32_bit_exact(name, bm):
    cfg = cfg_of(name)
    say(f"[gemm_i32] {name} block_m={bm}")
    L = layer_of(name)
    ids, _ = route_host(cfg)
    P = cfg.T * cfg.k
    al, d = oracle_align_dev(ids, cfg.E, bm)
    a_q, _ = oracle.quant_per_token(oracle.activations_f32(cfg), 0)
    R = w8.w8a8_moe_max_rows(cfg.T, cfg.k, cfg.E, bm)
    rows = stage_rows(al, bm, P)
    w = oracle_weights(name, range(cfg.E))
    # first GEMM: gathered token rows x w13
    got = run_i32(L, cfg, a_q, True, d, bm)
    assert np.array_equal(got[rows], oracle.grouped_gemm_i32(a_q, True, w[0], al, bm, P, cfg.k, rows)[rows])
    # second GEMM form: sorted rows of an int8 intermediate x w2
    h = synth.int8_matrix(R, cfg.I, cfg.seed)
    got2 = run_i32(L, cfg, h, False, d, bm)
    assert np.array_equal(got2[rows], oracle.grouped_gemm_i32(h, False, w[2], al, bm, P, cfg.k, rows)[rows])


def test_i32_rejects_bad_calls():
    cfg = cfg_of("ds-small")
    L = layer_of("ds-small")
    bm = 16
    ids, _ = route_host(cfg)
    _, d = oracle_align_dev(ids, cfg.E, bm)
    a = torch.zeros((cfg.T, cfg.H), dtype=torch.int8, device=DEV)
    R = w8.w8a8_moe_max_rows(cfg.T, cfg.k, cfg.E, bm)
    out = torch.empty((R, 2 * cfg.I), dtype=torch.int32, device=DEV)
    need = w8.w8a8_grouped_gemm_i32_workspace_bytes(True, 2 * cfg.I, cfg.H, cfg.T, cfg.k, cfg.E, bm)
    short = torch.empty(max(need - 256, 0), dtype=torch.uint8, device=DEV)
    with pytest.raises(w8.W8A8Error) as ex:
        w8.w8a8_grouped_gemm_i32(a, True, L.w13, d["sorted_pair_ids"], d["padded_offsets"], d["tile_expert"],
                                 d["num_tiles"], cfg.T, cfg.k, bm, out, short)
    assert ex.value.status == w8.W8A8_WORKSPACE_TOO_SMALL


@pytest.mark.parametrize("name", ["tiny", "ds-small", "ds-small-block"])
def test_first_gemm_silu_requant(name):
    cfg = cfg_of(name)
    block = cfg.scale_mode == "block"
    bm = block_m_of(cfg)
    say(f"[w13] {name} block_m={bm}")
    L = layer_of(name)
    ids, _ = route_host(cfg)
    P = cfg.T * cfg.k
    al, d = oracle_align_dev(ids, cfg.E, bm)
    a_q, a_s = oracle.quant_per_token(oracle.activations_f32(cfg), 128 if block else 0)
    R = w8.w8a8_moe_max_rows(cfg.T, cfg.k, cfg.E, bm)
    h_q = torch.empty((R, cfg.I), dtype=torch.int8, device=DEV)
    h_s = torch.empty((R, cfg.I // 128) if block else (R,), dtype=torch.float32, device=DEV)
    mode = w8.SCALE_BLOCK128 if block else w8.SCALE_CHANNEL
    ws = torch.empty(max(w8.w8a8_w13_workspace_bytes(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I, bm, mode), 256),
                     dtype=torch.uint8, device=DEV)
    fn = w8.w8a8_block_grouped_gemm_w13_silu if block else w8.w8a8_grouped_gemm_w13_silu
    fn(dt(a_q), dt(a_s), L.w13, L.w13_scale, d["sorted_pair_ids"], d["padded_offsets"], d["tile_expert"],
       d["num_tiles"], cfg.T, cfg.k, bm, h_q, h_s, ws)
    rows = stage_rows(al, bm, P)
    w = oracle_weights(name, range(cfg.E))
    rq, rs = oracle.w13_silu(a_q, a_s, w[0], w[1], al, bm, cfg.T, cfg.k, cfg.H, cfg.I, block, rows)
    gq, gs = host(h_q)[rows], host(h_s)[rows]
    rq, rs = rq[rows], rs[rows]
    assert np.all(np.abs(gs - rs) <= 4 * ULP * rs), np.abs(gs / rs - 1).max()
    diff = np.abs(gq.astype(np.int32) - rq.astype(np.int32))
    assert diff.max() <= 1
    assert np.mean(diff > 0) <= 1e-3, np.mean(diff > 0)


@pytest.mark.parametrize("name", ["tiny", "ds-small", "ds-small-block"])
def test_second_gemm_combine_bit_exact(name):
    """Fed the same intermediate, the second GEMM + combine performs the oracle's fp32
    operations in the oracle's order, so the output matches bit for bit."""
    cfg = cfg_of(name)
    block = cfg.scale_mode == "block"
    bm = block_m_of(cfg)
    say(f"[w2] {name} block_m={bm}")
    L = layer_of(name)
    ids, tw = route_host(cfg)
    P = cfg.T * cfg.k
    al, d = oracle_align_dev(ids, cfg.E, bm)
    R = w8.w8a8_moe_max_rows(cfg.T, cfg.k, cfg.E, bm)
    h_q = synth.int8_matrix(R, cfg.I, cfg.seed + 100)
    h_s = synth.positive_scales(R * (cfg.I // 128 if block else 1), cfg.seed, 1e-3, 3e-2)
    h_s = h_s.reshape(R, cfg.I // 128) if block else h_s
    out = torch.full((cfg.T, cfg.H), float("nan"), dtype=torch.float32, device=DEV)
    mode = w8.SCALE_BLOCK128 if block else w8.SCALE_CHANNEL
    ws = torch.empty(max(w8.w8a8_w2_workspace_bytes(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I, bm, mode), 256),
                     dtype=torch.uint8, device=DEV)
    fn = w8.w8a8_block_grouped_gemm_w2_combine if block else w8.w8a8_grouped_gemm_w2_combine
    fn(dt(h_q), dt(h_s), L.w2, L.w2_scale, d["sorted_pair_ids"], d["padded_offsets"], d["tile_expert"],
       d["num_tiles"], dt(tw), cfg.T, cfg.k, bm, out, ws)
    tokens = np.arange(cfg.T)
    w = oracle_weights(name, range(cfg.E))
    ref = oracle.w2_combine(h_q, h_s, w[2], w[3], al, bm, tw, cfg.T, cfg.k, cfg.H, cfg.I, block, tokens)
    got = host(out)
    assert np.array_equal(got[tokens], ref)
    assert np.isfinite(got).all()


@pytest.mark.parametrize("name", ["tiny", "dsv3-e8", "dsv3-e16", "dsv3-e8-block"])
def test_second_gemm_combine_after_pairs_are_dropped(name):
    """The pair -> row index the combine reads is written by the second GEMM for this call's pairs
    only.  Two calls with one workspace: the full routing, then the same routing with every 7th pair's
    expert id out of range (the align drops those pairs); the second call still matches the oracle,
    which skips them, bit for bit (staged, DMA, ring and block-wise engines)."""
    cfg = cfg_of(name)
    block = cfg.scale_mode == "block"
    bm = block_m_of(cfg)
    say(f"[w2-drop] {name} block_m={bm}")
    L = layer_of(name)
    ids, tw = route_host(cfg)
    R = w8.w8a8_moe_max_rows(cfg.T, cfg.k, cfg.E, bm)
    h_q = synth.int8_matrix(R, cfg.I, cfg.seed + 200)
    h_s = synth.positive_scales(R * (cfg.I // 128 if block else 1), cfg.seed + 1, 1e-3, 3e-2)
    h_s = h_s.reshape(R, cfg.I // 128) if block else h_s
    mode = w8.SCALE_BLOCK128 if block else w8.SCALE_CHANNEL
    ws = torch.empty(max(w8.w8a8_w2_workspace_bytes(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I, bm, mode), 256),
                     dtype=torch.uint8, device=DEV)
    fn = w8.w8a8_block_grouped_gemm_w2_combine if block else w8.w8a8_grouped_gemm_w2_combine
    w = oracle_weights(name, range(cfg.E))
    dropped = ids.copy()
    flat = dropped.reshape(-1)
    flat[::7] = np.where(np.arange(flat[::7].size) % 2 == 0, -1, cfg.E + 3)
    for routing in (ids, dropped):
        al, d = oracle_align_dev(routing, cfg.E, bm)
        out = torch.full((cfg.T, cfg.H), float("nan"), dtype=torch.float32, device=DEV)
        fn(dt(h_q), dt(h_s), L.w2, L.w2_scale, d["sorted_pair_ids"], d["padded_offsets"], d["tile_expert"],
           d["num_tiles"], dt(tw), cfg.T, cfg.k, bm, out, ws)
        ref = oracle.w2_combine(h_q, h_s, w[2], w[3], al, bm, tw, cfg.T, cfg.k, cfg.H, cfg.I, block)
        assert np.array_equal(host(out), ref)


# Rows per expert for the tile-edge cases: empty, one row, a ragged fragment, exactly one 320-row
# tile, one row past it, several tiles, and ragged multi-tile counts (with 16 experts, the ring engine's
# 128-row tiles: 255 / 256 rows, two rows either side of a tile pair).
EDGE_COUNTS = [0, 1, 17, 320, 321, 650, 330, 361]
EDGE_COUNTS_E16 = [0, 1, 17, 255, 256, 650, 330, 361, 130]


def edge_counts(cfg):
    base = EDGE_COUNTS_E16 if cfg.E == 16 else EDGE_COUNTS
    return base + [0] * (cfg.E - len(base))


def edge_routing(cfg):
    """Top-2 ids with the counts above (two distinct experts per token: no expert holds more than
    T rows, so a sorted run never meets itself T places later), tokens shuffled so each expert's
    rows gather scattered token rows."""
    flat = np.repeat(np.arange(cfg.E, dtype=np.int32), edge_counts(cfg))
    T = len(flat) // 2
    assert T == cfg.T and cfg.k == 2 and max(edge_counts(cfg)) <= T
    ids = np.stack([flat[:T], flat[T:]], axis=1)
    assert np.all(ids[:, 0] != ids[:, 1])
    ids = ids[np.random.default_rng(40).permutation(T)]
    tw = synth.positive_scales(T * 2, cfg.seed, 0.05, 1.0).reshape(T, 2)
    return np.ascontiguousarray(ids), np.ascontiguousarray(tw)


def edge_rows(al, counts):
    """Sorted rows at every 16/64/128/256/320-row boundary of each expert's segment, its first and
    last rows and the edges of its last 16-row fragment."""
    rows = set()
    for e, n in enumerate(counts):
        r0 = int(al["padded_offsets"][e])
        js = {0, 1, 15, 16, 17, n - 2, n - 1, (n // 16) * 16 - 1, (n // 16) * 16}
        for b in (64, 128, 256, 320):
            for m in range(1, n // b + 1):
                js |= {m * b - 1, m * b}
        rows |= {r0 + j for j in js if 0 <= j < n}
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("name", ["dsv3-e8", "dsv3-e16", "dsv3-e8-block"])
def test_large_batch_engine_tile_edges(name):
    """Both GEMM stages at the DeepSeek-V3 expert shapes (channel-wise and block-wise) with
    constructed routing whose expert row counts straddle every tile and fragment boundary:
    bit-exact second GEMM + combine and the first GEMM's requantized intermediate, at the rows on
    those boundaries."""
    cfg = cfg_of(name)
    block = cfg.scale_mode == "block"
    mode = w8.SCALE_BLOCK128 if block else w8.SCALE_CHANNEL
    bm = block_m_of(cfg)
    say(f"[edges] {name} block_m={bm}")
    L = layer_of(name)
    ids, tw = edge_routing(cfg)
    P = cfg.T * cfg.k
    al, d = oracle_align_dev(ids, cfg.E, bm)
    counts = edge_counts(cfg)
    assert list(al["counts"]) == counts
    rows = edge_rows(al, counts)
    R = w8.w8a8_moe_max_rows(cfg.T, cfg.k, cfg.E, bm)
    w = oracle_weights(name, [e for e, n in enumerate(counts) if n])
    engine = w8.w8a8_moe_engine(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I, bm, mode)
    assert engine == {"dsv3-e8": w8.ENGINE_DMA, "dsv3-e16": w8.ENGINE_RING, "dsv3-e8-block": w8.ENGINE_RING}[name]
    if not block:  # raw int32 accumulators of both GEMMs through the same engine, bit for bit
        a8, _ = oracle.quant_per_token(oracle.activations_f32(cfg), 0)
        got = run_i32(L, cfg, a8, True, d, bm)
        assert np.array_equal(got[rows], oracle.grouped_gemm_i32(a8, True, w[0], al, bm, P, cfg.k, rows)[rows])
        h8 = synth.int8_matrix(R, cfg.I, cfg.seed + 7)
        got2 = run_i32(L, cfg, h8, False, d, bm)
        assert np.array_equal(got2[rows], oracle.grouped_gemm_i32(h8, False, w[2], al, bm, P, cfg.k, rows)[rows])

    a_q, a_s = oracle.quant_per_token(oracle.activations_f32(cfg), 128 if block else 0)
    h_q = torch.empty((R, cfg.I), dtype=torch.int8, device=DEV)
    h_s = torch.empty((R, cfg.I // 128) if block else (R,), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(w8.w8a8_w13_workspace_bytes(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I, bm, mode), 256),
                     dtype=torch.uint8, device=DEV)
    fn = w8.w8a8_block_grouped_gemm_w13_silu if block else w8.w8a8_grouped_gemm_w13_silu
    fn(dt(a_q), dt(a_s), L.w13, L.w13_scale, d["sorted_pair_ids"], d["padded_offsets"], d["tile_expert"],
       d["num_tiles"], cfg.T, cfg.k, bm, h_q, h_s, ws)
    rq, rs = oracle.w13_silu(a_q, a_s, w[0], w[1], al, bm, cfg.T, cfg.k, cfg.H, cfg.I, block, rows)
    gq, gs = host(h_q)[rows], host(h_s)[rows]
    rq, rs = rq[rows], rs[rows]
    assert np.all(np.abs(gs - rs) <= 4 * ULP * rs), np.abs(gs / rs - 1).max()
    diff = np.abs(gq.astype(np.int32) - rq.astype(np.int32))
    assert diff.max() <= 1
    assert np.mean(diff > 0) <= 1e-3, np.mean(diff > 0)

    hq2 = synth.int8_matrix(R, cfg.I, cfg.seed + 100)
    hs2 = synth.positive_scales(R * (cfg.I // 128 if block else 1), cfg.seed, 1e-3, 3e-2)
    hs2 = hs2.reshape(R, cfg.I // 128) if block else hs2
    out = torch.full((cfg.T, cfg.H), float("nan"), dtype=torch.float32, device=DEV)
    ws2 = torch.empty(max(w8.w8a8_w2_workspace_bytes(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I, bm, mode), 256),
                      dtype=torch.uint8, device=DEV)
    fn = w8.w8a8_block_grouped_gemm_w2_combine if block else w8.w8a8_grouped_gemm_w2_combine
    fn(dt(hq2), dt(hs2), L.w2, L.w2_scale, d["sorted_pair_ids"], d["padded_offsets"], d["tile_expert"],
       d["num_tiles"], dt(tw), cfg.T, cfg.k, bm, out, ws2)
    tokens = np.unique(al["sorted_pair_ids"][rows] // cfg.k)
    ref = oracle.w2_combine(hq2, hs2, w[2], w[3], al, bm, tw, cfg.T, cfg.k, cfg.H, cfg.I, block, tokens)
    got = host(out)
    assert np.array_equal(got[tokens], ref)
    assert np.isfinite(got).all()


# ------------------------------------------------------------------ the whole layer

@pytest.mark.parametrize("name", ["tiny", "ds-small", "ds-small-block"])
def test_forward_matches_oracle(name):
    cfg = cfg_of(name)
    say(f"[forward] {name}")
    L = layer_of(name)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device=DEV)
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=DEV)
    tw = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=DEV)
    ws = workload.forward_workspace(L)
    workload.forward(L, out, ws, topk_ids=ids, topk_weights=tw)
    got, gids = host(out), host(ids)
    tokens = np.arange(cfg.T)
    lg = synth.logits(cfg, slice(0, cfg.T))[tokens]
    ids_o, tw_o = oracle.route_cfg(cfg, lg)
    keep = np.all(gids[tokens] == ids_o, axis=1)
    assert keep.mean() >= 0.95
    tokens, ids_o, tw_o = tokens[keep], ids_o[keep], tw_o[keep]
    w = oracle_weights(name, np.unique(ids_o))
    x = oracle.activations_f32(cfg)[tokens]
    ref = oracle.moe_tokens(x, ids_o, tw_o, *w, I=cfg.I, block=cfg.scale_mode == "block")
    err = np.abs(got[tokens] - ref).max()
    assert err <= 5e-3 * np.abs(ref).max(), (err, np.abs(ref).max())


@pytest.mark.parametrize("bm", [16, 32, 64, 128])
@pytest.mark.parametrize("name", ["ds-small", "ds-small-block"])
def test_forward_every_block_m(name, bm):
    cfg = cfg_of(name)
    L = layer_of(name)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device=DEV)
    ws = workload.forward_workspace(L, bm)
    workload.forward(L, out, ws, block_m=bm)
    ids_o, tw_o = route_host(cfg)
    w = oracle_weights(name, range(cfg.E))
    ref = oracle.moe_tokens(oracle.activations_f32(cfg), ids_o, tw_o, *w, I=cfg.I, block=cfg.scale_mode == "block")
    assert np.abs(host(out) - ref).max() <= 5e-3 * np.abs(ref).max()


def test_forward_is_deterministic():
    L = layer_of("ds-small")
    cfg = L.cfg
    a = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device=DEV)
    b = torch.empty_like(a)
    ws = workload.forward_workspace(L)
    workload.forward(L, a, ws)
    workload.forward(L, b, ws)
    assert torch.equal(a, b)


def _dense_check(cfg, x_np, logits_np, L, out):
    ids_o, tw_o = oracle.route_cfg(cfg, logits_np)
    w = oracle_weights_custom(cfg, np.unique(ids_o))
    ref = oracle.moe_tokens(x_np, ids_o, tw_o, *w, I=cfg.I, block=cfg.scale_mode == "block")
    err = np.abs(host(out) - ref).max()
    assert err <= 5e-3 * max(np.abs(ref).max(), 1e-30), err


_custom_w = {}


def oracle_weights_custom(cfg, experts):
    key = cfg.name
    if key not in _custom_w:
        _custom_w[key] = oracle.expert_weights(cfg, range(cfg.E))
    return _custom_w[key]


@pytest.mark.parametrize("case", ["one_token", "all_to_one_expert", "k_equals_E", "single_expert", "no_tokens"])
def test_forward_edge_cases(case):
    if case == "one_token":
        cfg = small_cfg(name="one", index=30, T=1)
    elif case == "all_to_one_expert":
        cfg = small_cfg(name="skewone", index=31, T=200, k=1, route="softmax", n_group=1, topk_group=1, scaling=1.0)
    elif case == "k_equals_E":
        cfg = small_cfg(name="kE", index=32, T=40, E=8, k=8, route="softmax", n_group=1, topk_group=1, scaling=1.0)
    elif case == "single_expert":
        cfg = small_cfg(name="E1", index=33, T=50, E=1, k=1, route="softmax", n_group=1, topk_group=1, scaling=1.0)
    else:
        cfg = small_cfg(name="empty", index=34, T=0)
    L = workload.make_layer(cfg, device=DEV)
    if case == "all_to_one_expert":
        L.logits[:, 5] += 100.0
    out = torch.full((max(cfg.T, 1), cfg.H), 7.0, dtype=torch.float32, device=DEV)
    ws = workload.forward_workspace(L)
    workload.forward(L, out[: cfg.T], ws)
    if cfg.T == 0:
        assert torch.all(out == 7.0)
        return
    lg = host(L.logits)
    _dense_check(cfg, oracle.activations_f32(cfg), lg, L, out)


def test_outputs_do_not_spill_past_their_buffers():
    """Guard words after every output buffer stay untouched."""
    cfg = cfg_of("ds-small")
    L = layer_of("ds-small")
    G = 4096
    bm = 16
    R = w8.w8a8_moe_max_rows(cfg.T, cfg.k, cfg.E, bm)
    ids, tw = route_host(cfg)

    def guarded(n, dtype):
        t = torch.full((n + G,), 0x5A if dtype == torch.int8 else 12345, dtype=dtype, device=DEV)
        return t, t[:n]

    cnt_g, cnt = guarded(cfg.E, torch.int32)
    off_g, off = guarded(cfg.E + 1, torch.int32)
    pad_g, pad = guarded(cfg.E + 1, torch.int32)
    srt_g, srt = guarded(R, torch.int32)
    te_g, te = guarded(R // bm, torch.int32)
    nt_g, nt = guarded(1, torch.int32)
    ws = torch.empty(w8.moe_align_workspace_bytes(cfg.T, cfg.k, cfg.E), dtype=torch.uint8, device=DEV)
    w8.moe_align_by_expert(dt(ids), cfg.E, bm, cnt, off, pad, srt, te, nt, ws)
    for full, n in ((cnt_g, cfg.E), (off_g, cfg.E + 1), (pad_g, cfg.E + 1), (srt_g, R), (te_g, R // bm), (nt_g, 1)):
        assert torch.all(full[n:] == 12345)
    hq_g, hq = guarded(R * cfg.I, torch.int8)
    hs_g, hs = guarded(R, torch.float32)
    a_q, a_s = oracle.quant_per_token(oracle.activations_f32(cfg))
    ws1 = torch.empty(w8.w8a8_w13_workspace_bytes(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I, bm), dtype=torch.uint8,
                      device=DEV)
    w8.w8a8_grouped_gemm_w13_silu(dt(a_q), dt(a_s), L.w13, L.w13_scale, srt, pad, te, nt, cfg.T, cfg.k, bm,
                                  hq.view(R, cfg.I), hs, ws1)
    out_g, out = guarded(cfg.T * cfg.H, torch.float32)
    ws2 = torch.empty(w8.w8a8_w2_workspace_bytes(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I, bm), dtype=torch.uint8,
                      device=DEV)
    w8.w8a8_grouped_gemm_w2_combine(hq.view(R, cfg.I), hs, L.w2, L.w2_scale, srt, pad, te, nt, dt(tw), cfg.T,
                                    cfg.k, bm, out.view(cfg.T, cfg.H), ws2)
    assert torch.all(hq_g[R * cfg.I:] == 0x5A)
    assert torch.all(hs_g[R:] == 12345)
    assert torch.all(out_g[cfg.T * cfg.H:] == 12345)
