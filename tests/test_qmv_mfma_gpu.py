"""GPU parity of the matrix-core small-M GEMV (2 to 8 activation rows; more in launches of
8), through the C ABI, on every launch configuration it has, each checked on every output
against the oracle:

* steps of four weight rows per workgroup and steps in flight per wave, chosen by the
  number of steps per compute unit: 1/1 (small N), 2/2, 5/2, 8/2 and, at 8 bits, 8/1;
* chunks per lane 1, 2 and 4 (by K), with K tails that leave lanes of the last wave idle;
* scales and biases staged in LDS by 4-byte copies, by 2-byte copies (an odd number of
  groups per row, or arrays only 2-byte aligned), or loaded per lane (the staged span would
  not fit);
* one row group (up to 4 rows) and two (5 to 8 rows), and more than 8 rows through
  bitmm_qmv;
* bf16 and f32 outputs, and integer-valued inputs whose f32 results must be exact.
"""

import numpy as np
import pytest

import bit_matmul_amd as bm
import oracle
from bit_matmul_amd import inputs as I
from tests import gpu_util as G
from tests.pins import integer_exact_problem

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = G.torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    bm.lib()
    yield
    t.cuda.synchronize()


# (M, N, K, bits, group): N sets the steps per compute unit (256 CUs: N <= 2048 -> 1/1,
# <= 4096 -> 2/2, <= 10240 -> 5/2, beyond -> 8/2, or 8/1 at 8 bits), K the chunks per lane.
SHAPES = [
    (2, 3000, 512, 4, 64),      # 2/2, C 1
    (6, 4001, 384, 8, 64),      # 2/2, two row groups, 8-bit, C 1
    (3, 5000, 4160, 4, 64),     # 5/2, C 2 with a partial last wave
    (8, 4100, 320, 2, 64),      # 5/2, 2-bit, K tail inside one wave
    (5, 6001, 1024, 8, 128),    # 5/2, 8-bit, group 128
    (4, 10300, 256, 4, 32),     # 8/2, group 32
    (7, 10241, 192, 8, 64),     # 8/1 (8-bit), odd group count -> 2-byte staging
    (3, 10300, 12288, 4, 64),   # 8/2, C 4
    (2, 10244, 6144, 8, 64),    # 8/1, 8-bit C 4
    (3, 10300, 8192, 4, 32),    # 8/2, staged span too large -> per-lane scale loads
    (5, 333, 24576, 2, 128),    # 1/1, 2-bit C 4
]


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K,bits,group", SHAPES)
def test_qmv_mfma_paths(M, N, K, bits, group, out):
    d = I.random_dense(M, N, K, bits, seed=M * 7 + N + K + bits, group=group)
    got = G.to_f64(G.run_dense("bitmm_qmv", d, out))
    ref = oracle.qmm(d.x, d.w, d.scales, d.biases, bits, group=group)
    G.assert_close(got, ref, out, f"qmv-mfma M{M} N{N} K{K} b{bits} g{group}")


def test_qmv_mfma_unaligned_scales():
    """Scale and bias arrays only 2-byte aligned: the 2-byte staging copies."""
    t = G.torch()
    d = I.random_dense(3, 5003, 1024, 4, seed=3)
    x, w, s, b = G.dense_to_dev(d)
    s_buf = t.empty(s.numel() + 1, dtype=t.bfloat16, device=G.dev())
    b_buf = t.empty(b.numel() + 1, dtype=t.bfloat16, device=G.dev())
    s_buf[1:].copy_(s.view(-1))
    b_buf[1:].copy_(b.view(-1))
    s1 = s_buf[1:].view(s.shape)
    b1 = b_buf[1:].view(b.shape)
    assert s1.data_ptr() % 4 == 2
    y = t.empty((d.M, d.N), dtype=t.float32, device=G.dev())
    bm.bitmm_qmv(x, w, s1, b1, y, d.bits)
    ref = oracle.qmm(d.x, d.w, d.scales, d.biases, d.bits)
    G.assert_close(G.to_f64(y), ref, "f32", "unaligned scales")


@pytest.mark.parametrize("M", [9, 11, 16, 17])
def test_qmv_more_than_eight_rows(M):
    """bitmm_qmv with more than 8 rows: launches of 8 (and the rest)."""
    d = I.random_dense(M, 700, 512, 4, seed=M)
    got = G.to_f64(G.run_dense("bitmm_qmv", d, "f32"))
    G.assert_close(got, oracle.qmm(d.x, d.w, d.scales, d.biases, 4), "f32", f"qmv M{M}")


@pytest.mark.parametrize("M,N,K,bits", [(3, 10300, 1024, 4), (8, 10241, 512, 8), (5, 4500, 2048, 2),
                                        (2, 3000, 5120, 4)])
def test_qmv_mfma_integer_exact(M, N, K, bits):
    """Every product and partial sum exact in f32: the f32 output equals the exact result
    and the bf16 output its round-to-nearest-even."""
    x, w, s, b, y4 = integer_exact_problem(M, N, K, bits, seed=M + N)
    d = I.Dense("exact", x, w, s, b, bits)
    exact = y4.astype(np.float64) / 4.0
    got32 = G.to_f64(G.run_dense("bitmm_qmv", d, "f32"))
    assert np.array_equal(got32, exact), np.max(np.abs(got32 - exact))
    got16 = G.run_dense("bitmm_qmv", d, "bf16")
    want16 = oracle.f64_to_bf16(exact).reshape(exact.shape)
    assert np.array_equal(got16.view(G.torch().int16).cpu().numpy().view(np.uint16), want16)
