"""GPU parity of the indexed expert-gathered GEMM (bitmm_gather_qmm_indexed).

Row r of the output reads activation row token_idx[r] (row r without a token index)
and the weights of expert expert_idx[r]; rows come in any order. The matrix-core path
rounds w to bf16 before the product, so both output types are held to the bf16 rule,
except for integer-valued inputs, which must match exactly. Out-of-range ids give
zero rows and flag the first one in workspace word 0.
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
    B = exp.shape[0]
    y = t.empty((B, g.N), dtype=t.bfloat16 if out == "bf16" else t.float32, device=G.dev())
    y.fill_(12345.0)  # every output must be written
    ws = t.empty(bm.bitmm_gather_qmm_indexed_workspace_bytes(B, g.N, g.E), dtype=t.uint8, device=G.dev())
    bm.bitmm_gather_qmm_indexed(x, w, s, b, tt, et, y, ws, g.bits)
    flag = int(ws[:4].cpu().numpy().view(np.uint32)[0])
    return G.to_f64(y), flag


def ref(g, token_idx="same", expert_idx=None, rows=None, cols=None):
    tok = g.token_idx if isinstance(token_idx, str) else token_idx
    exp = g.expert_idx if expert_idx is None else expert_idx
    return oracle.gather_qmm_indexed(g.x, g.w, g.scales, g.biases, tok, exp, g.bits,
                                     rows=rows, cols=cols)


# (T, B, E, N, K): a few rows per expert (one 32-row tile), ~36 per expert (64-row tiles),
# ~100 per expert (a row-tile loop), and K covering every scale/bias staging mode
# (G = 3, 11, 29, 44 staged; G = 50 per group).
SHAPES = [(10, 40, 16, 96, 192), (50, 576, 16, 130, 704), (64, 300, 3, 70, 1856),
          (40, 360, 10, 200, 2816), (30, 200, 5, 64, 3200)]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("tokens", [True, False])
@pytest.mark.parametrize("T,B,E,N,K", SHAPES)
def test_indexed_random(T, B, E, N, K, tokens, out, bits):
    g = I.random_indexed(T, B, E, N, K, bits, seed=T + B + E + N + K + bits, with_tokens=tokens)
    got, flag = run(g, out)
    assert flag == 0
    G.assert_close(got, ref(g), "bf16", f"gather_indexed T{T} B{B} E{E} N{N} K{K} b{bits} {out}")


@pytest.mark.parametrize("bits", [4, 8])
def test_indexed_invalid_ids(bits):
    g = I.random_indexed(12, 90, 6, 70, 704, bits, seed=3)
    tok = g.token_idx.copy()
    exp = g.expert_idx.copy()
    tok[17], exp[5], exp[40], tok[88] = 12, 6, -2, -1
    got, flag = run(g, "f32", token_idx=tok, expert_idx=exp)
    assert flag == 5 + 1
    for r in (5, 17, 40, 88):
        assert np.all(got[r] == 0.0), r
    G.assert_close(got, ref(g, token_idx=tok, expert_idx=exp), "bf16", "invalid ids")


@pytest.mark.parametrize("bits", [4, 8])
def test_indexed_integer_exact(bits):
    """Integer x, power-of-two scales, b = -2^(bits-1) s: w is bf16-exact and every sum is
    exact in f32, so the f32 output equals the oracle exactly, rows in any order."""
    rng = np.random.default_rng(40 + bits)
    T, B, E, N, K = 20, 150, 5, 90, 2816
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
    got, _ = run(g, "f32")
    assert np.array_equal(got, exact)


@pytest.mark.parametrize("bits", [4, 8])
def test_indexed_constant_per_expert_and_token(bits):
    """q = 0, b[e] = e + 1, x[t,:] = (t mod 7) + 1: y[r,n] = K (e_r + 1)((t_r mod 7) + 1)."""
    rng = np.random.default_rng(bits)
    T, E, N, K, B = 23, 9, 140, 704, 130
    tok = rng.integers(0, T, B).astype(np.int32)
    exp = rng.integers(0, E, B).astype(np.int32)
    w = np.zeros((E, N, K * bits // 32), dtype=np.uint32)
    s = I.to_bf16_bits(np.full((E, N, K // 64), 0.5))
    b = I.to_bf16_bits(np.broadcast_to((np.arange(E) + 1.0)[:, None, None], (E, N, K // 64)))
    xv = (np.arange(T) % 7 + 1).astype(np.float64)
    x = I.to_bf16_bits(np.broadcast_to(xv[:, None], (T, K)))
    g = I.GatherIndexed("const", x, w, s, b, tok, exp, bits)
    want = K * (exp[:, None] + 1.0) * xv[tok][:, None] * np.ones((1, N))
    got, _ = run(g, "f32")
    assert np.array_equal(got, want)


def test_moe_prefill_token_index():
    """The MoE prefill up projection read through the token index (x = the 573 hidden
    rows, not their 4584 replicas), rows in routing (token-major) order: each row equals
    the sorted, replicated gather's row bit for bit, and sampled rows match the oracle."""
    t = G.torch()
    gs = I.moe_gather("up")
    order = np.argsort(gs.token_of_row * 1000 + gs.expert_idx, kind="stable")  # token-major
    hidden = np.empty((I.MOE_TOKENS, gs.K), dtype=np.uint16)
    hidden[gs.token_of_row] = gs.x
    gi = I.GatherIndexed("up_tok", hidden, gs.w, gs.scales, gs.biases,
                         np.ascontiguousarray(gs.token_of_row[order]),
                         np.ascontiguousarray(gs.expert_idx[order]), gs.bits)
    got, flag = run(gi, "bf16")
    assert flag == 0
    ys, _ = G.run_gather(gs, "bf16")
    assert np.array_equal(got, G.to_f64(ys)[order])
    r, c = G.sample_points(gi.B, gi.N, 300, seed=4)
    want = ref(gi, rows=r, cols=c)
    G.assert_close(got[r, c], want, "bf16", "moe prefill up, token index")
    t.cuda.synchronize()


def test_indexed_deterministic():
    g = I.random_indexed(30, 400, 8, 96, 704, 4, seed=9)
    first, _ = run(g, "f32")
    for _ in range(5):
        again, _ = run(g, "f32")
        assert np.array_equal(first, again)


@pytest.mark.parametrize("tokens", [573, 46])
@pytest.mark.parametrize("which", ["up", "down"])
def test_moe_prefill_indexed_sampled(which, tokens):
    """The benchmark's indexed MoE prefill workloads as timed (routing order; up through
    the token index): the 573-token prompt and the 46-token one below the grouped path's
    gate (about three rows per expert). Sampled outputs against the oracle, and the rows
    equal the sorted gather's rows of the same routing bit for bit."""
    gi = I.moe_prefill_indexed(which, tokens=tokens)
    got, flag = run(gi, "bf16")
    assert flag == 0
    r, c = G.sample_points(gi.B, gi.N, 400, seed=tokens)
    G.assert_close(got[r, c], ref(gi, rows=r, cols=c), "bf16", gi.name)
    gs = I.moe_gather(which, tokens=tokens)
    ys, _ = G.run_gather(gs, "bf16")
    order = np.argsort(gs.token_of_row.astype(np.int64) * (gs.E + 1) + gs.expert_idx, kind="stable")
    assert np.array_equal(got, G.to_f64(ys)[order])
