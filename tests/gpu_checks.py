"""Helpers shared by the GPU parity tests (no test functions here): the routing near-tie rule and
device align + comparison against the oracle's align."""
import numpy as np

import oracle

ULP = 2.0 ** -23


def check_routing(cfg, logits, ids_g, w_g, ids_o, w_o):
    """Expert ids equal except near-ties, where the oracle's score gap between swapped experts is
    within 5e-7 relative (libm and device expf differ in the last bits); weights within 8 ulp."""
    fn = oracle.SOFTMAX if cfg.route == "softmax" else oracle.SIGMOID
    score = logits.astype(np.float64) if fn == oracle.SOFTMAX else 1.0 / (1.0 + np.exp(-logits.astype(np.float64)))
    bad = 0
    same = np.all(ids_g == ids_o, axis=1)
    for t in np.nonzero(~same)[0]:
        A, B = set(ids_o[t]), set(ids_g[t])
        if A == B:
            # same set, slots swapped: only a near-tie can do that
            j = np.nonzero(ids_g[t] != ids_o[t])[0]
            gap = np.abs(score[t, ids_o[t, j]] - score[t, ids_g[t, j]]).max()
        else:
            gap = abs(score[t, list(A)].sum() - score[t, list(B)].sum())
        if gap > 5e-7 * np.abs(score[t]).max():
            bad += 1
    assert bad == 0, f"{bad} tokens differ beyond a near-tie"
    assert (~same).sum() <= max(1, cfg.T // 100)
    rel = np.abs(w_g[same] - w_o[same]) / np.abs(w_o[same])
    assert rel.max() <= 8 * ULP, rel.max()


def dev_align(w8, torch, dev, ids_np, E, bm):
    """Align on the device through the C ABI; returns the output tensors by name."""
    T, k = ids_np.shape
    R = max(w8.w8a8_moe_max_rows(T, k, E, bm), 1)
    o = dict(counts=torch.empty(E, dtype=torch.int32, device=dev),
             offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
             padded_offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
             sorted_pair_ids=torch.full((R,), -7, dtype=torch.int32, device=dev),
             tile_expert=torch.full((max(R // bm, 1),), -7, dtype=torch.int32, device=dev),
             num_tiles=torch.empty(1, dtype=torch.int32, device=dev))
    ws = torch.empty(max(w8.moe_align_workspace_bytes(T, k, E), 256), dtype=torch.uint8, device=dev)
    w8.moe_align_by_expert(torch.from_numpy(np.ascontiguousarray(ids_np)).to(dev), E, bm, o["counts"], o["offsets"],
                           o["padded_offsets"], o["sorted_pair_ids"], o["tile_expert"], o["num_tiles"], ws)
    return o


def check_align_equal(d, al):
    """Device align outputs equal the oracle's (sorted ids and tile experts up to the padded end)."""
    def h(t):
        return t.cpu().numpy()

    nt = int(al["num_tiles"][0])
    assert int(h(d["num_tiles"])[0]) == nt
    for key in ("counts", "offsets", "padded_offsets"):
        assert np.array_equal(h(d[key]), al[key]), key
    R = int(al["padded_offsets"][-1])
    assert np.array_equal(h(d["sorted_pair_ids"])[:R], al["sorted_pair_ids"][:R])
    assert np.array_equal(h(d["tile_expert"])[:nt], al["tile_expert"][:nt])


def oracle_weights(torch, dev, cfg, experts):
    """The oracle's quantized copy of the listed experts (None for the others): fp32 weights drawn
    by the shared generator's device fill (bit-identical to its host fill), quantized by the oracle."""
    import synth

    E = cfg.E
    w13q, w13s, w2q, w2s = [None] * E, [None] * E, [None] * E, [None] * E
    n13, n2 = 2 * cfg.I * cfg.H, cfg.H * cfg.I
    buf = torch.empty(n13, dtype=torch.float32, device=dev)
    hs = torch.cuda.current_stream().cuda_stream

    def host(t):
        torch.cuda.synchronize()
        return t.cpu().numpy()

    for e in experts:
        synth.dev_normal(buf.data_ptr(), n13, cfg.seed, synth.STREAM_W13, int(e) * n13, cfg.w_sigma, hs)
        w13q[e], w13s[e] = oracle.quant_weight(host(buf).reshape(2 * cfg.I, cfg.H), cfg.scale_mode)
        synth.dev_normal(buf.data_ptr(), n2, cfg.seed, synth.STREAM_W2, int(e) * n2, cfg.w_sigma, hs)
        w2q[e], w2s[e] = oracle.quant_weight(host(buf[:n2]).reshape(cfg.H, cfg.I), cfg.scale_mode)
    del buf
    return w13q, w13s, w2q, w2s
