"""GPU parity of the gathered GEMV (MoE decode, bitmm_gather_qmv) against the oracle.

Row r of the output reads activation row token_idx[r] (row r without a token index)
and the weights of expert expert_idx[r], in any order. The GEMV paths keep every
product exact and accumulate in f32, so f32 outputs are held to the f32 rule
(|y - y_ref| <= 1e-4 max|y_ref|) and bf16 outputs to the bf16 rule; integer-valued
inputs must match exactly; out-of-range ids must give zero rows.
"""

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


def run(g, out="bf16", token_idx="same", expert_idx=None):
    t = G.torch()
    x, w, s, b = G.bf16_tensor(g.x), G.u32_tensor(g.w), G.bf16_tensor(g.scales), G.bf16_tensor(g.biases)
    tok = g.token_idx if isinstance(token_idx, str) else token_idx
    exp = g.expert_idx if expert_idx is None else expert_idx
    tt = None if tok is None else G.i32_tensor(tok)
    et = G.i32_tensor(exp)
    y = t.empty((exp.shape[0], g.N), dtype=t.bfloat16 if out == "bf16" else t.float32, device=G.dev())
    y.fill_(12345.0)  # every output must be written
    bm.bitmm_gather_qmv(x, w, s, b, tt, et, y, g.bits)
    return G.to_f64(y)


def ref(g, token_idx="same", expert_idx=None):
    tok = g.token_idx if isinstance(token_idx, str) else token_idx
    exp = g.expert_idx if expert_idx is None else expert_idx
    return oracle.gather_qmm_indexed(g.x, g.w, g.scales, g.biases, tok, exp, g.bits)


# Shapes reaching each GEMV kernel form for one activation row: the decode kernel
# (K up to 10240 at 4 bits, 5120 at 8), the split-K kernel (up to 16384 / 8192), the
# general kernel beyond.
SHAPES = [(1, 8, 16, 64, 2816), (3, 24, 8, 200, 704), (2, 5, 3, 33, 192), (4, 16, 6, 70, 12288),
          (2, 7, 3, 45, 6144), (2, 6, 4, 40, 20480), (1, 1, 1, 1, 64)]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("tokens", [True, False])
@pytest.mark.parametrize("T,B,E,N,K", SHAPES)
def test_gather_qmv_random(T, B, E, N, K, tokens, out, bits):
    g = I.random_indexed(T, B, E, N, K, bits, seed=T + B + E + N + K + bits, with_tokens=tokens)
    G.assert_close(run(g, out), ref(g), out, f"gather_qmv T{T} B{B} E{E} N{N} K{K} b{bits}")


@pytest.mark.parametrize("bits,K", [(4, 24576), (8, 12288), (2, 24576)])
def test_gather_qmv_general_kernel(bits, K):
    """Gathered rows with K past the decode and split-K kernels' range: the general
    kernel."""
    g = I.random_indexed(3, 10, 5, 77, K, bits, seed=bits)
    G.assert_close(run(g, "f32"), ref(g), "f32", f"general kernel b{bits} K{K}")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("K", [704, 2816, 12288, 20480])
def test_gather_qmv_invalid_ids(K, bits):
    """Out-of-range token or expert ids give zero rows; the other rows are unaffected."""
    g = I.random_indexed(4, 9, 6, 50, K, bits, seed=K)
    tok = g.token_idx.copy()
    exp = g.expert_idx.copy()
    tok[1], exp[3], exp[5], tok[7] = 4, 6, -1, -3
    got = run(g, "f32", token_idx=tok, expert_idx=exp)
    want = ref(g, token_idx=tok, expert_idx=exp)
    for r in (1, 3, 5, 7):
        assert np.all(got[r] == 0.0), r
    G.assert_close(got, want, "f32", "invalid ids")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("K", [704, 2816, 12288])
def test_gather_qmv_integer_exact(K, bits):
    """Integer-valued x, power-of-two scales, b = -2^(bits-1) s: every product and sum is
    exact in f32, so f32 outputs must equal the oracle exactly."""
    rng = np.random.default_rng(K + bits)
    T, B, E, N = 3, 12, 5, 40
    xi = rng.integers(-2, 3, size=(T, K))
    q = rng.integers(0, 1 << bits, size=(E, N, K))
    s4 = rng.choice([1, 2, 4, 8], size=(E, N, K // 64))
    half = 1 << (bits - 1)
    g = I.GatherIndexed("exact", I.to_bf16_bits(xi.astype(np.float64)), I.pack_codes(q, bits),
                        I.to_bf16_bits(s4 / 4.0), I.to_bf16_bits(-half * s4 / 4.0),
                        rng.integers(0, T, B).astype(np.int32), rng.integers(0, E, B).astype(np.int32),
                        bits)
    exact = np.empty((B, N))
    for r in range(B):
        e, t = g.expert_idx[r], g.token_idx[r]
        w4 = np.repeat(s4[e], 64, axis=1) * (q[e] - half)
        exact[r] = (w4.astype(np.int64) @ xi[t].astype(np.int64)) / 4.0
    assert np.array_equal(ref(g), exact)
    assert np.array_equal(run(g, "f32"), exact)


@pytest.mark.parametrize("bits", [4, 8])
def test_gather_qmv_constant_per_expert_and_token(bits):
    """q = 0, b[e] = e + 1, x[t,:] = (t mod 7) + 1: y[r,n] = K (e_r + 1)((t_r mod 7) + 1);
    a mis-gathered token or expert gives a wrong integer."""
    T, E, N, K = 9, 6, 130, 2816
    tok = np.array([3, 0, 8, 8, 1, 5, 2, 7, 4, 6, 0], dtype=np.int32)
    exp = np.array([5, 0, 2, 2, 4, 1, 3, 0, 5, 1, 4], dtype=np.int32)
    w = np.zeros((E, N, K * bits // 32), dtype=np.uint32)
    s = I.to_bf16_bits(np.full((E, N, K // 64), 0.5))
    b = I.to_bf16_bits(np.broadcast_to((np.arange(E) + 1.0)[:, None, None], (E, N, K // 64)))
    xv = (np.arange(T) % 7 + 1).astype(np.float64)
    x = I.to_bf16_bits(np.broadcast_to(xv[:, None], (T, K)))
    g = I.GatherIndexed("const", x, w, s, b, tok, exp, bits)
    want = K * (exp[:, None] + 1.0) * xv[tok][:, None] * np.ones((1, N))
    assert np.array_equal(run(g, "f32"), want)


@pytest.mark.parametrize("which", ["up", "down"])
@pytest.mark.parametrize("tokens", [1, 4])
def test_moe_decode(which, tokens):
    """The MoE decode step at the expert dims (E=128, top-8, K/N = 2816/704 and 704/2816),
    every output against the oracle."""
    g = I.moe_decode(which, tokens)
    G.assert_close(run(g, "bf16"), ref(g), "bf16", g.name)
    G.assert_close(run(g, "f32"), ref(g), "f32", g.name)


def test_gather_qmv_matches_qmv_rows():
    """A gathered row equals bitmm_qmv of that token's activations with that expert's
    weights, bit for bit (same kernels, same order of operations)."""
    t = G.torch()
    g = I.random_indexed(3, 6, 4, 96, 2816, 4, seed=11)
    got = run(g, "f32")
    for r in range(g.B):
        e, tk = int(g.expert_idx[r]), int(g.token_idx[r])
        d = I.Dense("row", g.x[tk:tk + 1], g.w[e], g.scales[e], g.biases[e], 4)
        y = G.to_f64(G.run_dense("bitmm_qmv", d, "f32"))
        assert np.array_equal(y[0], got[r]), r
    t.cuda.synchronize()


def test_gather_qmv_empty():
    t = G.torch()
    g = I.random_indexed(2, 3, 2, 16, 128, 4, seed=1)
    x, w, s, b = G.bf16_tensor(g.x), G.u32_tensor(g.w), G.bf16_tensor(g.scales), G.bf16_tensor(g.biases)
    e0 = t.empty((0,), dtype=t.int32, device=G.dev())
    y0 = t.empty((0, g.N), dtype=t.bfloat16, device=G.dev())
    bm.bitmm_gather_qmv(x, w, s, b, None, e0, y0, 4)
    t.cuda.synchronize()
