"""GPU parity of the dense grouped product (bitmm_gather_mm) against the oracle.

Row r of the output reads activation row token_idx[r] (row r without a token index)
and the weights of expert expert_idx[r], rows in any order; W is stored [E, N, K] or
[E, K, N]; x and W are both bf16 or both binary16. Products are exact in f32 and the
accumulation is f32, so f32 outputs are held to the f32 rule (|y - y_ref| <= 1e-4
max|y_ref|) and 16-bit outputs to the bf16 rule; integer-valued inputs must match
exactly, and their 16-bit outputs must be the oracle's round-to-nearest-even of the
exact value. Out-of-range ids give zero rows and flag the first one in workspace
word 0.
"""

import numpy as np
import pytest

import bit_matmul_amd as bm
import oracle
from bit_matmul_amd import inputs as I
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

RULE = {"bf16": "bf16", "f16": "bf16", "f32": "f32"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = G.torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    bm.lib()
    yield
    t.cuda.synchronize()


def out_dtype(out):
    t = G.torch()
    return {"bf16": t.bfloat16, "f16": t.float16, "f32": t.float32}[out]


def run(g, out="bf16", token_idx="same", expert_idx=None):
    t = G.torch()
    x, w = G.half_tensor(g.x, g.dtype), G.half_tensor(g.w, g.dtype)
    tok = g.token_idx if isinstance(token_idx, str) else token_idx
    exp = g.expert_idx if expert_idx is None else expert_idx
    tt = None if tok is None else G.i32_tensor(tok)
    et = G.i32_tensor(exp)
    B = exp.shape[0]
    y = t.empty((B, g.N), dtype=out_dtype(out), device=G.dev())
    y.fill_(12345.0)  # every output must be written
    ws = t.empty(bm.bitmm_gather_mm_workspace_bytes(B, g.N, g.E), dtype=t.uint8, device=G.dev())
    bm.bitmm_gather_mm(x, w, tt, et, y, ws, g.layout)
    flag = int(ws[:4].cpu().numpy().view(np.uint32)[0])
    return y, flag


def ref(g, token_idx="same", expert_idx=None, rows=None, cols=None):
    tok = g.token_idx if isinstance(token_idx, str) else token_idx
    exp = g.expert_idx if expert_idx is None else expert_idx
    return oracle.gather_mm(g.x, g.w, tok, exp, g.dtype, g.layout, rows=rows, cols=cols)


# (T, B, E, N, K): a few rows per expert (one 32-row block), ~36 per expert (two
# blocks), ~100 per expert (the row-tile loop); K with a full last stage (K % 128 == 0)
# and with a ragged last stage (64-k stages below K = 2048 for [N, K] storage and
# always for [K, N]; 128-k stages above); N ragged against the 128-column block, the
# 32-column wave slice and 8 (the 16-byte output stores).
SHAPES = [(10, 40, 16, 96, 128), (50, 576, 16, 130, 704), (64, 300, 3, 70, 1808),
          (40, 360, 10, 200, 2816), (30, 200, 5, 64, 144), (7, 9, 4, 8, 16), (20, 64, 2, 136, 1040),
          (12, 50, 4, 72, 2064)]


@pytest.mark.parametrize("layout", ["nk", "kn"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("T,B,E,N,K", SHAPES)
def test_gather_mm_random(T, B, E, N, K, dtype, layout):
    if layout == "kn" and N % 8:
        pytest.skip("[K, N] storage needs N a multiple of 8")
    g = I.random_gather_mm(T, B, E, N, K, dtype, layout, seed=T + B + E + N + K)
    want = ref(g)
    for out in ("bf16", "f16", "f32"):
        y, flag = run(g, out)
        assert flag == 0
        G.assert_close(G.to_f64(y), want, RULE[out], f"gather_mm {g.name} -> {out}")


@pytest.mark.parametrize("layout", ["nk", "kn"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_gather_mm_without_token_index(dtype, layout):
    g = I.random_gather_mm(0, 150, 6, 72, 704, dtype, layout, seed=3, with_tokens=False)
    y, flag = run(g, "f32")
    assert flag == 0
    G.assert_close(G.to_f64(y), ref(g), "f32", "no token index")


@pytest.mark.parametrize("layout", ["nk", "kn"])
def test_gather_mm_invalid_ids(layout):
    g = I.random_gather_mm(12, 90, 6, 72, 704, "bf16", layout, seed=5)
    tok = g.token_idx.copy()
    exp = g.expert_idx.copy()
    tok[17], exp[5], exp[40], tok[88] = 12, 6, -2, -1
    y, flag = run(g, "f32", token_idx=tok, expert_idx=exp)
    got = G.to_f64(y)
    assert flag == 5 + 1
    for r in (5, 17, 40, 88):
        assert np.all(got[r] == 0.0), r
    G.assert_close(got, ref(g, token_idx=tok, expert_idx=exp), "f32", "invalid ids")


@pytest.mark.parametrize("layout", ["nk", "kn"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_gather_mm_integer_exact(dtype, layout):
    """Integer x and W: every product and partial sum is an integer below 2^24, exact in
    f32, so the f32 output equals the oracle exactly and each 16-bit output is the
    round-to-nearest-even of the exact value."""
    rng = np.random.default_rng(40 + len(dtype) + len(layout))
    T, B, E, N, K = 20, 150, 5, 88, 1040
    xi = rng.integers(-8, 9, size=(T, K)).astype(np.float64)
    wi = rng.integers(-8, 9, size=(E, N, K)).astype(np.float64)
    wl = wi if layout == "nk" else np.ascontiguousarray(np.transpose(wi, (0, 2, 1)))
    enc = I.to_bf16_bits if dtype == "bf16" else I.to_f16_bits
    g = I.GatherMM("exact", enc(xi), enc(wl), rng.integers(0, T, B).astype(np.int32),
                   rng.integers(0, E, B).astype(np.int32), dtype, layout)
    exact = np.stack([wi[g.expert_idx[r]] @ xi[g.token_idx[r]] for r in range(B)])
    assert np.array_equal(ref(g), exact)
    y, _ = run(g, "f32")
    assert np.array_equal(G.to_f64(y), exact)
    y, _ = run(g, "bf16")
    assert np.array_equal(y.view(G.torch().int16).cpu().numpy().view(np.uint16), oracle.f64_to_bf16(exact))
    y, _ = run(g, "f16")
    assert np.array_equal(y.view(G.torch().int16).cpu().numpy().view(np.uint16), oracle.f64_to_f16(exact))


@pytest.mark.parametrize("layout", ["nk", "kn"])
def test_gather_mm_constant_per_expert_and_token(layout):
    """W[e] = e + 1, x[t,:] = (t mod 7) + 1: y[r,n] = K (e_r + 1)((t_r mod 7) + 1); a
    mis-gathered token or expert gives a wrong integer."""
    rng = np.random.default_rng(2)
    T, E, N, K, B = 23, 9, 136, 704, 130
    tok = rng.integers(0, T, B).astype(np.int32)
    exp = rng.integers(0, E, B).astype(np.int32)
    shape = (E, N, K) if layout == "nk" else (E, K, N)
    w = I.to_bf16_bits(np.broadcast_to((np.arange(E) + 1.0)[:, None, None], shape))
    xv = (np.arange(T) % 7 + 1).astype(np.float64)
    x = I.to_bf16_bits(np.broadcast_to(xv[:, None], (T, K)))
    g = I.GatherMM("const", x, w, tok, exp, "bf16", layout)
    want = K * (exp[:, None] + 1.0) * xv[tok][:, None] * np.ones((1, N))
    y, _ = run(g, "f32")
    assert np.array_equal(G.to_f64(y), want)


@pytest.mark.parametrize("which", ["up", "down"])
def test_moe_gather_mm(which):
    """The non-quantized MoE prefill at the expert dims (573 tokens, 8 of 128 experts,
    K/N = 2816/704 and 704/2816, bf16, [E, N, K]), the shapes and launch the benchmark
    times: sampled outputs against the oracle, and the whole output deterministic."""
    g = I.moe_gather_mm(which)
    y, flag = run(g, "bf16")
    assert flag == 0
    got = G.to_f64(y)
    r, c = G.sample_points(g.B, g.N, 400, seed=7)
    G.assert_close(got[r, c], ref(g, rows=r, cols=c), "bf16", g.name)
    y2, _ = run(g, "bf16")
    assert np.array_equal(G.to_f64(y2), got)


def test_moe_gather_mm_transposed_layout_matches():
    """The same MoE up projection with W stored [E, K, N] gives the same bits as [E, N, K]
    (same k order in every MFMA)."""
    g = I.moe_gather_mm("up", layout="kn")
    y, _ = run(g, "f32")
    wt = np.ascontiguousarray(np.transpose(g.w, (0, 2, 1)))
    g2 = I.GatherMM("nk", g.x, wt, g.token_idx, g.expert_idx, "bf16", "nk")
    y2, _ = run(g2, "f32")
    assert np.array_equal(G.to_f64(y), G.to_f64(y2))
    r, c = G.sample_points(g.B, g.N, 200, seed=8)
    G.assert_close(G.to_f64(y)[r, c], ref(g, rows=r, cols=c), "f32", "moe up, [K, N]")


def test_gather_mm_empty():
    t = G.torch()
    g = I.random_gather_mm(2, 3, 2, 16, 128, "bf16", "nk", seed=1)
    x, w = G.half_tensor(g.x, "bf16"), G.half_tensor(g.w, "bf16")
    e0 = t.empty((0,), dtype=t.int32, device=G.dev())
    y0 = t.empty((0, g.N), dtype=t.bfloat16, device=G.dev())
    ws = t.empty(256, dtype=t.uint8, device=G.dev())
    bm.bitmm_gather_mm(x, w, None, e0, y0, ws)
    t.cuda.synchronize()
