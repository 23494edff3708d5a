"""GPU parity of the dense W8A8 linear (w8a8_linear) against the CPU oracle, through the C ABI.

int32 products are exact and the epilogue is the oracle's two fp32 products in the oracle's order,
so every checked output must match bit for bit."""
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

DEV = "cuda"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def inputs(M, N, K, seed):
    a_q = synth.int8_matrix(M, K, seed)
    w = synth.int8_matrix(N, K, seed + 1)
    a_s = synth.positive_scales(M, seed + 2, 1e-3, 3e-2)
    w_s = synth.positive_scales(N, seed + 3, 1e-3, 3e-2)
    return a_q, a_s, w, w_s


def run(a_q, a_s, w, w_s, guard=0):
    M, N = a_q.shape[0], w.shape[0]
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    out = torch.full((M * N + guard,), float("nan"), dtype=torch.float32, device=DEV)
    N, K = w.shape
    ws = torch.empty(max(w8.w8a8_linear_workspace_bytes(M, N, K), 256), dtype=torch.uint8, device=DEV)
    w8.w8a8_linear(d(a_q), d(a_s), d(w), d(w_s), out[: M * N].view(M, N), ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("M,N,K", [(1, 256, 256), (5, 256, 4096), (37, 512, 768), (333, 768, 1024), (640, 256, 512),
                                   (1000, 1536, 7168), (100, 512, 2048), (16, 768, 6144), (64, 1024, 3072),
                                   (128, 512, 5120)])
def test_linear_bit_exact(M, N, K):
    """Every plan: at most 128 rows on the ring engine (K = 2048 unsplit, 4096 in two slices, 6144 in
    three) or, with K not a multiple of 2048, on 128 x 128 DMA tiles (3072 and 5120 split two and four
    ways); more rows on 320 x 256 DMA tiles (7168 split four ways at 1000 rows)."""
    say(f"[linear] M={M} N={N} K={K}")
    a_q, a_s, w, w_s = inputs(M, N, K, 100 + M)
    got = run(a_q, a_s, w, w_s, guard=64)
    ref = oracle.linear(a_q, a_s, w, w_s)
    assert np.array_equal(got[: M * N].reshape(M, N), ref)
    assert np.isnan(got[M * N:]).all()  # nothing written past the output


def test_linear_decode_shape_full():
    """A decode-sized output projection: 128 tokens, N = 7168, K = 16384 (a 117 MB weight stream)."""
    M, N, K = 128, 7168, 16384
    say(f"[linear] M={M} N={N} K={K}")
    a_q, a_s, w, w_s = inputs(M, N, K, 7)
    got = run(a_q, a_s, w, w_s).reshape(M, N)
    assert np.array_equal(got, oracle.linear(a_q, a_s, w, w_s))


@pytest.mark.parametrize("K", [2048, 16384])
def test_linear_prefill_shape_sampled(K):
    """8192 tokens x N = 7168 (K = 16384: the attention output projection the benchmark times,
    unsplit): the rows around every 320-row tile edge, the first and last rows, and a random
    sample, computed one by one by the oracle."""
    M, N = 8192, 7168
    say(f"[linear] M={M} N={N} K={K}")
    a_q, a_s, w, w_s = inputs(M, N, K, 11)
    got = run(a_q, a_s, w, w_s).reshape(M, N)
    edges = {0, 1, M - 2, M - 1} | {m for t in range(320, M, 320) for m in (t - 1, t)}
    rng = np.random.default_rng(5)
    rows = sorted(edges | set(rng.choice(M, 32, replace=False).tolist()))
    ref = oracle.linear(a_q, a_s, w, w_s, rows=rows)
    assert np.array_equal(got[rows], ref[rows])
    assert np.isfinite(got).all()


def test_linear_is_deterministic_and_handles_no_rows():
    M, N, K = 700, 512, 1024
    a_q, a_s, w, w_s = inputs(M, N, K, 13)
    assert np.array_equal(run(a_q, a_s, w, w_s), run(a_q, a_s, w, w_s))
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    out = torch.empty((0, N), dtype=torch.float32, device=DEV)
    w8.w8a8_linear(d(a_q[:0]), d(a_s[:0]), d(w), d(w_s), out, None)
    torch.cuda.synchronize()
