"""GPU parity at quantization groups of 32 and 128 along K (the format's other group
sizes; 64 is covered everywhere else), for every entry point and kernel form.

GEMV paths (qmv, qmm with M < 8, gather_qmv) keep products exact: f32 outputs are held
to the f32 rule. Matrix-core paths (qmm with M >= 8, both grouped GEMMs) are held to
the bf16 rule. Integer-valued inputs must match exactly.
"""

import numpy as np
import pytest

import bit_matmul_amd as bm
import oracle
from bit_matmul_amd import inputs as I
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

GROUPS = [32, 128]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = G.torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    bm.lib()
    yield
    t.cuda.synchronize()


def oracle_dense(d):
    return oracle.qmm(d.x, d.w, d.scales, d.biases, d.bits, group=d.group)


# qmv: decode kernel (K <= 10240 at 4 bits), split-K kernel, general kernel; M < 8 on the
# split-K kernel; M >= 8 on the matrix-core tile (scales staged in LDS while K / group
# <= 80 and even, fetched per group beyond).
GEMV_SHAPES = [(1, 300, 1024), (1, 70, 12288), (1, 40, 20480), (3, 133, 5120), (5, 40, 2048),
               (7, 33, 384)]
MFMA_SHAPES = [(8, 70, 256), (40, 129, 1024), (300, 200, 2048), (96, 64, 2560), (70, 66, 5120),
               (130, 96, 3072), (8, 70, 10368)]


@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", GEMV_SHAPES)
def test_gemv_groups(M, N, K, out, bits, group):
    if K % group:
        pytest.skip("K not a multiple of the group")
    d = I.random_dense(M, N, K, bits, seed=M + N + K + group, group=group)
    got = G.to_f64(G.run_dense("bitmm_qmv", d, out))
    G.assert_close(got, oracle_dense(d), out, f"qmv g{group} M{M} N{N} K{K} b{bits}")


@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M,N,K", MFMA_SHAPES)
def test_mfma_groups(M, N, K, bits, group):
    if K % group:
        pytest.skip("K not a multiple of the group")
    d = I.random_dense(M, N, K, bits, seed=3 * M + N + K + group, group=group)
    got = G.to_f64(G.run_dense("bitmm_qmm", d, "bf16"))
    G.assert_close(got, oracle_dense(d), "bf16", f"qmm g{group} M{M} N{N} K{K} b{bits}")


@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("fn,M", [("bitmm_qmv", 1), ("bitmm_qmm", 3), ("bitmm_qmm", 130)])
def test_integer_exact_groups(fn, M, bits, group):
    """x in {-2..2}, scales powers of two per group, b = -2^(bits-1) s: every weight,
    product and sum is exact in f32 on every path."""
    rng = np.random.default_rng(M + bits + group)
    N, K = 97, 2048
    xi = rng.integers(-2, 3, size=(M, K))
    q = rng.integers(0, 1 << bits, size=(N, K))
    s4 = rng.choice([1, 2, 4, 8], size=(N, K // group))
    half = 1 << (bits - 1)
    d = I.Dense("exact", I.to_bf16_bits(xi.astype(np.float64)), I.pack_codes(q, bits),
                I.to_bf16_bits(s4 / 4.0), I.to_bf16_bits(-half * s4 / 4.0), bits, group)
    w4 = np.repeat(s4, group, axis=1) * (q - half)
    exact = (xi.astype(np.int64) @ w4.T.astype(np.int64)) / 4.0
    assert np.array_equal(oracle_dense(d), exact)
    assert np.array_equal(G.to_f64(G.run_dense(fn, d, "f32")), exact)


@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("N,K", [(96, 1024), (70, 2816), (64, 5120), (50, 1152)])
def test_gather_groups(N, K, bits, group):
    if K % group:
        pytest.skip("K not a multiple of the group")
    g = I.random_gather([37, 0, 5, 70, 33], N=N, K=K, bits=bits, seed=N + K + group, group=group)
    y, ws = G.run_gather(g, "bf16")
    ref = oracle.gather_qmm(g.x, g.w, g.scales, g.biases, g.expert_idx, bits, group=group)
    G.assert_close(G.to_f64(y), ref, "bf16", f"gather g{group} N{N} K{K} b{bits}")
    assert int(ws[:4].cpu().numpy().view(np.uint32)[0]) == 0


def _indexed_dev(g):
    return (G.bf16_tensor(g.x), G.u32_tensor(g.w), G.bf16_tensor(g.scales), G.bf16_tensor(g.biases),
            None if g.token_idx is None else G.i32_tensor(g.token_idx), G.i32_tensor(g.expert_idx))


@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("K", [704 + 64, 2816])
def test_indexed_groups(K, bits, group):
    if K % group:
        pytest.skip("K not a multiple of the group")
    t = G.torch()
    g = I.random_indexed(30, 300, 6, 90, K, bits, seed=K + group, group=group)
    x, w, s, b, tok, exp = _indexed_dev(g)
    y = t.empty((g.B, g.N), dtype=t.bfloat16, device=G.dev())
    ws = t.empty(bm.bitmm_gather_qmm_indexed_workspace_bytes(g.B, g.N, g.E), dtype=t.uint8, device=G.dev())
    bm.bitmm_gather_qmm_indexed(x, w, s, b, tok, exp, y, ws, bits, group_size=group)
    ref = oracle.gather_qmm_indexed(g.x, g.w, g.scales, g.biases, g.token_idx, g.expert_idx, bits,
                                    group=group)
    G.assert_close(G.to_f64(y), ref, "bf16", f"gather_indexed g{group} K{K} b{bits}")


@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("K", [2816, 12288])
def test_gather_qmv_groups(K, bits, group):
    t = G.torch()
    g = I.random_indexed(3, 16, 8, 77, K, bits, seed=K + bits + group, group=group)
    x, w, s, b, tok, exp = _indexed_dev(g)
    y = t.empty((g.B, g.N), dtype=t.float32, device=G.dev())
    bm.bitmm_gather_qmv(x, w, s, b, tok, exp, y, bits, group_size=group)
    ref = oracle.gather_qmm_indexed(g.x, g.w, g.scales, g.biases, g.token_idx, g.expert_idx, bits,
                                    group=group)
    G.assert_close(G.to_f64(y), ref, "f32", f"gather_qmv g{group} K{K} b{bits}")
