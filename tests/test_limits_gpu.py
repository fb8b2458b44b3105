"""GPU parity at the size limits the kernels carry: more gathered GEMV rows than one
launch's grid holds (rows go in launches of 65535), the largest expert count the
counting sort keeps in LDS (8192) for the indexed gather and gather_mm, an expert
count far above the rows for the sorted gather, and tall or wide dense problems.
Outputs are checked against the oracle (whole, or sampled where the oracle would be
slow), and every output must be written."""

import numpy as np
import pytest

import bit_matmul_amd as bm
import oracle
from bit_matmul_amd import inputs as I
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = G.torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    bm.lib()
    yield
    t.cuda.synchronize()


def test_gather_qmv_beyond_one_grid():
    """70000 gathered GEMV rows: two launches of the row grid (65535 + 4465)."""
    t = G.torch()
    g = I.random_indexed(300, 70000, 16, 8, 128, 4, seed=1)
    x, w = G.bf16_tensor(g.x), G.u32_tensor(g.w)
    s, b = G.bf16_tensor(g.scales), G.bf16_tensor(g.biases)
    y = t.full((g.B, g.N), 12345.0, dtype=t.float32, device=G.dev())
    bm.bitmm_gather_qmv(x, w, s, b, G.i32_tensor(g.token_idx), G.i32_tensor(g.expert_idx), y, 4)
    ref = oracle.gather_qmm_indexed(g.x, g.w, g.scales, g.biases, g.token_idx, g.expert_idx, 4)
    G.assert_close(G.to_f64(y), ref, "f32", "70000 rows")


@pytest.mark.parametrize("bits", [4, 8])
def test_indexed_gather_max_experts(bits):
    """E = 8192, the most experts the sort's LDS counters hold; most experts get no row."""
    t = G.torch()
    g = I.random_indexed(500, 6000, 8192, 40, 128, bits, seed=2)
    x, w = G.bf16_tensor(g.x), G.u32_tensor(g.w)
    s, b = G.bf16_tensor(g.scales), G.bf16_tensor(g.biases)
    y = t.full((g.B, g.N), 12345.0, dtype=t.bfloat16, device=G.dev())
    ws = t.empty(bm.bitmm_gather_qmm_indexed_workspace_bytes(g.B, g.N, g.E), dtype=t.uint8, device=G.dev())
    bm.bitmm_gather_qmm_indexed(x, w, s, b, G.i32_tensor(g.token_idx), G.i32_tensor(g.expert_idx), y, ws, bits)
    ref = oracle.gather_qmm_indexed(g.x, g.w, g.scales, g.biases, g.token_idx, g.expert_idx, bits)
    G.assert_close(G.to_f64(y), ref, "bf16", "E=8192")
    assert int(ws[:4].cpu().numpy().view(np.uint32)[0]) == 0


def test_gather_mm_max_experts():
    t = G.torch()
    g = I.random_gather_mm(500, 6000, 8192, 40, 64, "bf16", "nk", seed=3)
    y = t.full((g.B, g.N), 12345.0, dtype=t.float32, device=G.dev())
    ws = t.empty(bm.bitmm_gather_mm_workspace_bytes(g.B, g.N, g.E), dtype=t.uint8, device=G.dev())
    bm.bitmm_gather_mm(G.bf16_tensor(g.x), G.bf16_tensor(g.w), G.i32_tensor(g.token_idx),
                       G.i32_tensor(g.expert_idx), y, ws)
    ref = oracle.gather_mm(g.x, g.w, g.token_idx, g.expert_idx)
    G.assert_close(G.to_f64(y), ref, "f32", "gather_mm E=8192")


def test_sorted_gather_many_more_experts_than_rows():
    """100000 experts, 300 sorted rows: almost every workgroup finds an empty expert."""
    rng = np.random.default_rng(4)
    E = 100000
    idx = np.sort(rng.integers(0, E, 300)).astype(np.int32)
    counts = np.bincount(idx, minlength=E)
    g = I.random_gather(list(counts), N=32, K=64, bits=4, seed=4)
    y, ws = G.run_gather(g, "bf16")
    ref = oracle.gather_qmm(g.x, g.w, g.scales, g.biases, g.expert_idx, 4)
    G.assert_close(G.to_f64(y), ref, "bf16", "E=100000")
    assert int(ws[:4].cpu().numpy().view(np.uint32)[0]) == 0


@pytest.mark.parametrize("fn,M,N,K", [("bitmm_qmv", 1, 1 << 17, 64), ("bitmm_qmm", 4096, 96, 256),
                                      ("bitmm_qmm", 5, 70000, 128), ("bitmm_qmv", 1, 3, 32768)])
def test_dense_extremes(fn, M, N, K):
    """A very wide GEMV (131072 outputs), a tall GEMM (4096 rows), a wide small-M
    product, and a long K with few outputs; sampled outputs against the oracle."""
    d = I.random_dense(M, N, K, 4, seed=M + N + K)
    got = G.to_f64(G.run_dense(fn, d, "f32"))
    r, c = G.sample_points(M, N, 2000, seed=5)
    want = oracle.qmm_points(d.x, d.w, d.scales, d.biases, r, c, 4)
    rule = "f32" if (fn == "bitmm_qmv" or M < 8) else "bf16"
    G.assert_close(got[r, c], want, rule, f"{fn} M{M} N{N} K{K}")
