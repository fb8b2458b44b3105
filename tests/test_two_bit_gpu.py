"""GPU parity for 2-bit codes (16 per word, LSB first; groups of 64 and 128) on every
entry point: the GEMV paths (qmv, qmm with M < 8, gather_qmv; the split-K kernel up to
3 rows, the general kernel with codes spread to nibbles beyond) are held to the f32
rule, the matrix-core paths (qmm with M >= 8, both grouped GEMMs) to the bf16 rule;
integer-valued inputs must match exactly."""

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


SHAPES = [(1, 300, 1024), (1, 70, 5120), (3, 133, 2048), (2, 61, 16384), (3, 45, 5120), (5, 40, 4096),
          (7, 33, 384), (1, 9, 20480),
          # past the decode (K <= 20480), split-K and matrix-core GEMV (K <= 32768) ranges:
          # the general kernel, one row and launches of four rows
          (1, 37, 24576), (2, 21, 40960), (4, 19, 40960),
          (8, 70, 256), (40, 129, 1024), (300, 200, 2048), (96, 64, 2560), (70, 66, 5120)]


@pytest.mark.parametrize("group", [64, 128])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_two_bit_dense(M, N, K, group):
    if K % group:
        pytest.skip("K not a multiple of the group")
    d = I.random_dense(M, N, K, 2, seed=M + N + K + group, group=group)
    want = oracle.qmm(d.x, d.w, d.scales, d.biases, 2, group=group)
    for out in ("bf16", "f32"):
        got = G.to_f64(G.run_dense("bitmm_qmm", d, out))
        rule = "bf16" if (M >= 8 or out == "bf16") else "f32"
        G.assert_close(got, want, rule, f"2-bit qmm g{group} M{M} N{N} K{K} {out}")
    if M < 8:
        got = G.to_f64(G.run_dense("bitmm_qmv", d, "f32"))
        G.assert_close(got, want, "f32", f"2-bit qmv g{group} M{M} N{N} K{K}")


@pytest.mark.parametrize("fn,M", [("bitmm_qmv", 1), ("bitmm_qmm", 2), ("bitmm_qmm", 3), ("bitmm_qmm", 5),
                                  ("bitmm_qmm", 130)])
def test_two_bit_integer_exact(fn, M):
    rng = np.random.default_rng(M)
    N, K = 97, 2048
    xi = rng.integers(-2, 3, size=(M, K))
    q = rng.integers(0, 4, size=(N, K))
    s4 = rng.choice([1, 2, 4, 8], size=(N, K // 64))
    d = I.Dense("exact", I.to_bf16_bits(xi.astype(np.float64)), I.pack_codes(q, 2),
                I.to_bf16_bits(s4 / 4.0), I.to_bf16_bits(-2 * s4 / 4.0), 2)
    w4 = np.repeat(s4, 64, axis=1) * (q - 2)
    exact = (xi.astype(np.int64) @ w4.T.astype(np.int64)) / 4.0
    assert np.array_equal(oracle.qmm(d.x, d.w, d.scales, d.biases, 2), exact)
    assert np.array_equal(G.to_f64(G.run_dense(fn, d, "f32")), exact)


@pytest.mark.parametrize("group", [64, 128])
@pytest.mark.parametrize("N,K", [(96, 1024), (70, 2816), (50, 768)])
def test_two_bit_gather(N, K, group):
    if K % group:
        pytest.skip("K not a multiple of the group")
    g = I.random_gather([37, 0, 5, 70, 33], N=N, K=K, bits=2, seed=N + K, group=group)
    y, ws = G.run_gather(g, "bf16")
    ref = oracle.gather_qmm(g.x, g.w, g.scales, g.biases, g.expert_idx, 2, group=group)
    G.assert_close(G.to_f64(y), ref, "bf16", f"2-bit gather g{group} N{N} K{K}")
    assert int(ws[:4].cpu().numpy().view(np.uint32)[0]) == 0


@pytest.mark.parametrize("K", [768, 2816])
def test_two_bit_indexed_and_gather_qmv(K):
    t = G.torch()
    for B, out, rule in ((300, t.bfloat16, "bf16"), (12, t.float32, "f32")):
        g = I.random_indexed(30, B, 6, 90, K, 2, seed=K + B)
        x, w = G.bf16_tensor(g.x), G.u32_tensor(g.w)
        s, b = G.bf16_tensor(g.scales), G.bf16_tensor(g.biases)
        tok, e = G.i32_tensor(g.token_idx), G.i32_tensor(g.expert_idx)
        y = t.empty((g.B, g.N), dtype=out, device=G.dev())
        ref = oracle.gather_qmm_indexed(g.x, g.w, g.scales, g.biases, g.token_idx, g.expert_idx, 2)
        if B > 100:
            ws = t.empty(bm.bitmm_gather_qmm_indexed_workspace_bytes(g.B, g.N, g.E), dtype=t.uint8,
                         device=G.dev())
            bm.bitmm_gather_qmm_indexed(x, w, s, b, tok, e, y, ws, 2)
        else:
            bm.bitmm_gather_qmv(x, w, s, b, tok, e, y, 2)
        G.assert_close(G.to_f64(y), ref, rule, f"2-bit indexed/gather_qmv K{K} B{B}")
