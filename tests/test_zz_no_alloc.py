"""The allocation-free align entry point (moe_align_by_expert_noalloc, for callers that cannot
allocate) against moe_align_by_expert with a caller workspace, through the C ABI: bit-identical
outputs on calls in a row, each smaller than the one before -- the first using most of the library's
4 MiB scratch, the second a smaller batch that also goes through the scratch (more than the 4096
pairs the single-workgroup align takes without one) and finds the first call's contents there, then
a decode batch and a small E on the single-workgroup path.  All are also compared with the oracle's
align."""
import numpy as np
import pytest

import gpu_checks
import oracle

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import w8a8_int8_quantized_quant_amd as w8  # noqa: E402

DEV = "cuda"


def noalloc_align(ids_np, E, bm):
    T, k = ids_np.shape
    R = max(w8.w8a8_moe_max_rows(T, k, E, bm), 1)
    o = dict(counts=torch.full((E,), -3, dtype=torch.int32, device=DEV),
             offsets=torch.full((E + 1,), -3, dtype=torch.int32, device=DEV),
             padded_offsets=torch.full((E + 1,), -3, dtype=torch.int32, device=DEV),
             sorted_pair_ids=torch.full((R,), -7, dtype=torch.int32, device=DEV),
             tile_expert=torch.full((max(R // bm, 1),), -7, dtype=torch.int32, device=DEV),
             num_tiles=torch.full((1,), -3, dtype=torch.int32, device=DEV))
    w8.moe_align_by_expert_noalloc(torch.from_numpy(np.ascontiguousarray(ids_np)).to(DEV), E, bm, o["counts"],
                                   o["offsets"], o["padded_offsets"], o["sorted_pair_ids"], o["tile_expert"],
                                   o["num_tiles"])
    return o


def skewed_ids(T, k, E, seed):
    """k distinct experts per token, popularity skewed (Zipf-like weights over a seeded order)."""
    rng = np.random.default_rng(seed)
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p = p[rng.permutation(E)]
    p /= p.sum()
    # Gumbel top-k: k distinct experts per token drawn with these weights
    g = np.log(p)[None, :] - np.log(-np.log(rng.random((T, E))))
    return np.ascontiguousarray(np.argsort(-g, axis=1)[:, :k].astype(np.int32))


def equal(a, b):
    nt = int(b["num_tiles"].cpu()[0])
    assert int(a["num_tiles"].cpu()[0]) == nt
    for key in ("counts", "offsets", "padded_offsets"):
        assert torch.equal(a[key], b[key]), key
    R = int(b["padded_offsets"].cpu()[-1])
    assert torch.equal(a["sorted_pair_ids"][:R], b["sorted_pair_ids"][:R])
    assert torch.equal(a["tile_expert"][:nt], b["tile_expert"][:nt])


@pytest.mark.parametrize("bm", [16, 128])
def test_noalloc_align_matches_workspace_align(bm):
    assert w8.moe_align_noalloc_scratch_bytes() == 4 << 20
    # 100000 tokens x top-8 (800k pairs: 3.9 of the 4 MiB), then 2000 x top-8 (16k pairs, the scratch
    # again), then a decode batch and a small E (one workgroup, no scratch)
    for T, k, E, seed in ((100000, 8, 256, 1), (2000, 8, 256, 4), (128, 8, 256, 2), (300, 2, 8, 3)):
        ids = skewed_ids(T, k, E, seed + bm)
        need = w8.moe_align_workspace_bytes(T, k, E)
        assert need <= w8.moe_align_noalloc_scratch_bytes()
        print(f"[noalloc] T={T} k={k} E={E} block_m={bm} scratch bytes used {need}", flush=True)
        got = noalloc_align(ids, E, bm)
        ref = gpu_checks.dev_align(w8, torch, DEV, ids, E, bm)
        torch.cuda.synchronize()
        equal(got, ref)
        gpu_checks.check_align_equal(got, oracle.align(ids, E, bm))


def test_noalloc_align_rejects_more_pairs_than_its_scratch():
    T, k, E = 131072, 8, 256  # 1M pairs: 4 MiB of ranks alone
    assert w8.moe_align_workspace_bytes(T, k, E) > w8.moe_align_noalloc_scratch_bytes()
    ids = torch.zeros((T, k), dtype=torch.int32, device=DEV)
    o = {n: torch.empty(1, dtype=torch.int32, device=DEV) for n in ("c", "o", "p", "s", "t", "n")}
    with pytest.raises(w8.W8A8Error) as ex:
        w8.moe_align_by_expert_noalloc(ids, E, 16, o["c"], o["o"], o["p"], o["s"], o["t"], o["n"])
    assert ex.value.status == w8.W8A8_UNSUPPORTED_SHAPE
