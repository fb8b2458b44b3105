"""GPU parity: the HIP kernels, called through the C ABI, against the CPU oracle.

Small problems are compared on every output; the full-size workloads (decode GEMV
at hidden 5120, prefill GEMM M=600 and M=3, their 8-bit twins, the MoE gather in
both orientations) on sampled outputs the oracle computes one by one, plus
properties that hold at any size (finite, deterministic). Integer-valued inputs
must match exactly; the constant-per-expert case exposes any mis-gathered row.
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


def oracle_dense(d):
    return oracle.qmm(d.x, d.w, d.scales, d.biases, d.bits)


# ---------------------------------------------------------------------------
# Small problems: every output
# ---------------------------------------------------------------------------

QMV_SHAPES = [(1, 1, 64), (1, 256, 512), (1, 300, 640), (1, 257, 192), (1, 64, 8192 + 64),
              (1, 70, 12288), (2, 77, 320), (3, 133, 5120), (3, 37, 16384), (4, 66, 8192),
              (5, 40, 576), (6, 45, 8256), (7, 19, 128), (8, 33, 256), (11, 50, 192)]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", QMV_SHAPES)
def test_qmv_small(M, N, K, bits, out):
    d = I.random_dense(M, N, K, bits, seed=M + N + K)
    got = G.to_f64(G.run_dense("bitmm_qmv", d, out))
    G.assert_close(got, oracle_dense(d), out, f"qmv M{M} N{N} K{K} b{bits}")


# Every GEMV kernel form, reached through the shapes that select it (one row: the decode
# kernel up to K = 10240 at 4 bits and 5120 at 8, then the split-K kernel up to 16384 and
# 8192, then the general kernel; 2 to 8 rows: the matrix-core GEMV up to K = 16384 and
# 8192, then the general kernel).
EVERY_KERNEL = [(1, 300, 640, 4), (1, 33, 192, 8), (1, 200, 12288, 4), (1, 200, 6144, 8),
                (1, 100, 20480, 4), (1, 100, 10240, 8), (3, 130, 20480, 4), (6, 50, 10240, 8),
                (3, 130, 5120, 4), (8, 40, 576, 8)]


@pytest.mark.parametrize("M,N,K,bits", EVERY_KERNEL)
def test_qmv_every_kernel(M, N, K, bits):
    """Each GEMV kernel form against the oracle, f32 output, where the exact-product rule
    applies."""
    d = I.random_dense(M, N, K, bits, seed=11 * M + N + K)
    got = G.to_f64(G.run_dense("bitmm_qmv", d, "f32"))
    G.assert_close(got, oracle_dense(d), "f32", f"qmv M{M} N{N} K{K} b{bits}")


# The LDS-ring GEMV at its layout edges: one row; R-row steps with a ragged last
# step (N odd, N = 4k+1); idle chunk slots (K/chunk not a multiple of lanes per
# row); 16, 32 and 64 lanes per row; 1 to 5 chunks per lane (K up to 10240 at 4
# bits, 5120 at 8 bits); N smaller and larger than the number of waves.
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("N,K", [(1, 64), (5, 5120), (4099, 5120), (257, 512), (33, 192),
                                 (2048, 10240), (100, 2816), (3001, 1344)])
def test_qmv_dma_layouts(N, K, bits, out):
    d = I.random_dense(1, N, K, bits, seed=N + 3 * K + bits)
    got = G.to_f64(G.run_dense("bitmm_qmv", d, out))
    G.assert_close(got, oracle_dense(d), out, f"qmv[dma] N{N} K{K} b{bits}")


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("N", [32771, 65539, 131075, 262147])
def test_qmv_dma_steps_per_wave(N, bits):
    """The decode kernel with several steps per wave: at K = 256 a step is four rows (16
    lanes x one chunk each), and past 8192, 16384 and 32768 steps each wave owns 2, 4 and
    8 consecutive steps (straight-line code with up to four steps in flight); N leaves a
    ragged last step and a ragged last wave."""
    d = I.random_dense(1, N, 256, bits, seed=N + bits)
    got = G.to_f64(G.run_dense("bitmm_qmv", d, "f32"))
    G.assert_close(got, oracle_dense(d), "f32", f"qmv[dma] N{N} b{bits}")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", [(1, 130, 320), (2, 64, 128), (3, 200, 640), (5, 33, 192),
                                   (7, 129, 1024)])
def test_qmm_small_m(M, N, K, bits, out):
    d = I.random_dense(M, N, K, bits, seed=7 * M + N + K)
    got = G.to_f64(G.run_dense("bitmm_qmm", d, out))
    G.assert_close(got, oracle_dense(d), out, f"qmm-smallM M{M} N{N} K{K} b{bits}")


MFMA_SHAPES = [(8, 16, 64), (9, 100, 192), (16, 128, 128), (33, 70, 320), (130, 300, 576),
               (129, 257, 1024), (257, 129, 192), (200, 513, 448),
               # K loops of one group, two, three (one unrolled pass), four; M at and
               # just past a multiple of 320 rows, three times 320 and one row more
               (96, 40, 64), (300, 200, 128), (65, 1000, 704), (320, 128, 192),
               (321, 131, 256), (641, 96, 320),
               # scales and biases staged in LDS up to 80 groups (G even), fetched per
               # group beyond
               (100, 70, 5120), (70, 66, 5248)]


# One shape for each row-tile size of the matrix-core GEMM (1, 2, 4, 6, 8 and 10 blocks
# of 32 rows), each with a ragged last row tile and a ragged last column block. The
# dispatch picks the size from M, N and the device's compute units; these shapes make
# each pick on a 256-CU device, where the kernel-choice record is checked too. K = 192
# fetches scales per group (odd group count), K = 128, 256 and 320 stage them in LDS.
TILE_SHAPES = [(20, 130, 320, 1), (45, 16500, 128, 2), (250, 11000, 192, 4), (300, 11000, 256, 6),
               (400, 13000, 192, 8), (577, 11111, 256, 10)]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M,N,K,mb", TILE_SHAPES)
def test_qmm_mfma_each_row_tile(M, N, K, mb, bits):
    d = I.random_dense(M, N, K, bits, seed=M + N + K + bits)
    got = G.to_f64(G.run_dense("bitmm_qmm", d, "bf16"))
    rec = bm.bitmm_last_launches()
    if G.torch().cuda.get_device_properties(G.dev()).multi_processor_count == 256:
        assert len(rec) == 1 and rec[0].startswith(f"qmm_mfma_kernel<MmTile4<{bits}, {mb}, "), rec
    G.assert_close(got, oracle_dense(d), "bf16", f"qmm tile MB{mb} M{M} N{N} K{K} b{bits}")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M,N,K", [(257, 129, 192), (96, 128, 192), (300, 700, 704), (64, 129, 320)])
def test_qmm_tail_bodies_wait_for_their_copies(M, N, K, bits):
    """Regression: the K groups left after the unrolled loop of four (here 3, 3, 11 and 5
    groups) run one body each with the activation copies of the next group landing
    during the body before. With 32-row tiles a body is four MFMAs long, so a wait that
    passes early shows as a few wrong rows; it did when the wait counted weight loads
    that those bodies never issued. Several calls, since a race need not show in one."""
    d = I.random_dense(M, N, K, bits, seed=M * N + K + bits)
    ref = oracle_dense(d)
    for rep in range(4):
        got = G.to_f64(G.run_dense("bitmm_qmm", d, "bf16"))
        G.assert_close(got, ref, "bf16", f"qmm tail M{M} N{N} K{K} b{bits} call {rep}")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M,K", [(200, 1024), (40, 2048)])
def test_qmm_mfma_misaligned_scales(M, K, bits):
    """Scale and bias arrays that are only 2-byte aligned take the per-group path."""
    t = G.torch()
    d = I.random_dense(M, 150, K, bits, seed=M + K)
    x, w, s, b = G.dense_to_dev(d)

    def shift(a):
        buf = t.empty(a.numel() + 1, dtype=a.dtype, device=a.device)
        v = buf[1:].view(a.shape)
        v.copy_(a)
        return v
    s, b = shift(s), shift(b)
    assert s.data_ptr() % 4 == 2
    y = t.empty((d.M, d.N), dtype=t.bfloat16, device=G.dev())
    bm.bitmm_qmm(x, w, s, b, y, bits)
    G.assert_close(G.to_f64(y), oracle_dense(d), "bf16", f"qmm misaligned M{M} K{K} b{bits}")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", MFMA_SHAPES)
def test_qmm_mfma_small(M, N, K, bits, out):
    d = I.random_dense(M, N, K, bits, seed=3 * M + N + K)
    got = G.to_f64(G.run_dense("bitmm_qmm", d, out))
    # The matrix-core path rounds w to bf16 before the product, so it is held to the
    # bf16 rule for both output types.
    G.assert_close(got, oracle_dense(d), "bf16", f"qmm-mfma M{M} N{N} K{K} b{bits} {out}")


GATHER_COUNTS = [
    [5, 0, 3, 17, 1, 0, 64, 70, 2],      # empty experts, one > 64 rows
    [1],                                  # one expert, one row
    [0, 0, 9],                            # leading empty experts
    [40] * 6,
    [3, 129, 0, 1],                       # a segment spanning three row blocks
    # 64-row launch (mean 30 rows): experts of 5 and 32 rows run the 32-row tile, 33 and
    # 37 the launch's, 70 two row tiles
    [37, 0, 5, 70, 33, 32],
    # 128-row launch (mean 64 rows): 10 rows the 32-row tile, 33, 50 and 64 the 64-row
    # tile, 65, 100 and 120 the launch's, 129 two row tiles
    [100, 10, 50, 0, 120, 33, 64, 65, 129],
]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("ci", range(len(GATHER_COUNTS)))
@pytest.mark.parametrize("N,K", [(200, 192), (64, 576), (129, 128)])
def test_gather_small(ci, N, K, bits, out):
    g = I.random_gather(GATHER_COUNTS[ci], N=N, K=K, bits=bits, seed=ci + N + K)
    y, ws = G.run_gather(g, out)
    ref = oracle.gather_qmm(g.x, g.w, g.scales, g.biases, g.expert_idx, bits)
    G.assert_close(G.to_f64(y), ref, "bf16", f"gather {GATHER_COUNTS[ci]} N{N} K{K} b{bits}")
    w = ws.cpu().numpy().view(np.uint32)
    assert w[0] == 0
    exp_off = np.searchsorted(g.expert_idx, np.arange(g.E + 1), side="left")
    assert np.array_equal(w[1:g.E + 2].view(np.int32), exp_off)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("N,K", [(96, 1856), (70, 3200), (64, 2816), (40, 704), (48, 512)])
@pytest.mark.parametrize("misaligned", [False, True])
def test_gather_scale_staging(N, K, bits, misaligned):
    """Every way the grouped GEMM can fetch scales and biases: staged in LDS by 4-byte
    copies (G even, arrays 4-byte aligned), by 2-byte copies (G odd, or the arrays only
    2-byte aligned), and loaded per group (G > 48), on ragged expert segments."""
    t = G.torch()
    g = I.random_gather([37, 0, 5, 70, 33], N=N, K=K, bits=bits, seed=N + K + bits)
    x, w, s, b, e = G.gather_to_dev(g)
    if misaligned:  # views that start 2 bytes into a fresh allocation
        def shift(a):
            buf = t.empty(a.numel() + 1, dtype=a.dtype, device=a.device)
            v = buf[1:].view(a.shape)
            v.copy_(a)
            return v
        s, b = shift(s), shift(b)
        assert s.data_ptr() % 4 == 2 and b.data_ptr() % 4 == 2
    y = t.empty((g.B, g.N), dtype=t.bfloat16, device=G.dev())
    ws = t.empty(bm.bitmm_gather_qmm_workspace_bytes(g.B, g.N, g.E), dtype=t.uint8, device=G.dev())
    bm.bitmm_gather_qmm(x, w, s, b, e, y, ws, g.bits)
    ref = oracle.gather_qmm(g.x, g.w, g.scales, g.biases, g.expert_idx, bits)
    G.assert_close(G.to_f64(y), ref, "bf16", f"gather staging N{N} K{K} b{bits} mis{misaligned}")


# ---------------------------------------------------------------------------
# Exact cases
# ---------------------------------------------------------------------------

def _exact_dense(M, N, K, bits, seed):
    x, w, s, b, y4 = integer_exact_problem(M, N, K, bits, seed)
    d = I.Dense("exact", x, w, s, b, bits)
    return d, y4.astype(np.float64) / 4.0


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("fn,M,N,K", [("bitmm_qmv", 1, 300, 5120), ("bitmm_qmm", 3, 257, 5120),
                                      ("bitmm_qmm", 64, 300, 5120), ("bitmm_qmm", 130, 129, 192)])
def test_integer_exact(fn, M, N, K, bits):
    """Every weight, product and partial sum is exact in f32: outputs must match the
    exact result bit for bit (f32) and its round-to-nearest-even bf16 (bf16)."""
    d, exact = _exact_dense(M, N, K, bits, seed=M * N + bits)
    assert np.array_equal(oracle_dense(d), exact)
    got32 = G.to_f64(G.run_dense(fn, d, "f32"))
    assert np.array_equal(got32, exact), np.max(np.abs(got32 - exact))
    got16 = G.run_dense(fn, d, "bf16")
    t = G.torch()
    bits16 = got16.view(t.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(bits16, oracle.f64_to_bf16(exact))


@pytest.mark.parametrize("bits", [4, 8])
def test_gather_integer_exact(bits):
    counts = [7, 0, 30, 66, 1]
    N, K = 90, 2816
    E = len(counts)
    idx = np.repeat(np.arange(E, dtype=np.int32), counts)
    B = idx.size
    rng = np.random.default_rng(bits)
    xi = rng.integers(-2, 3, size=(B, K))
    q = rng.integers(0, 1 << bits, size=(E, N, K))
    s4 = rng.choice([1, 2, 4, 8], size=(E, N, K // 64))
    half = 1 << (bits - 1)
    g = I.Gather("exact", I.to_bf16_bits(xi.astype(np.float64)), I.pack_codes(q, bits),
                 I.to_bf16_bits(s4 / 4.0), I.to_bf16_bits(-half * s4 / 4.0), idx, bits)
    exact = np.empty((B, N))
    for e in range(E):
        rows = idx == e
        w4 = np.repeat(s4[e], 64, axis=1) * (q[e] - half)
        exact[rows] = (xi[rows].astype(np.int64) @ w4.T.astype(np.int64)) / 4.0
    assert np.array_equal(oracle.gather_qmm(g.x, g.w, g.scales, g.biases, idx, bits), exact)
    y, _ = G.run_gather(g, "f32")
    assert np.array_equal(G.to_f64(y), exact)


@pytest.mark.parametrize("bits", [4, 8])
def test_constant_per_expert(bits):
    """q = 0, b[e] = e + 1, x[r,:] = (r mod 7) + 1: y[r,n] = K (e_r + 1)((r mod 7) + 1)."""
    counts = [3, 0, 50, 1, 0, 70, 9, 2]
    E, N, K = len(counts), 150, 704
    idx = np.repeat(np.arange(E, dtype=np.int32), counts)
    B = idx.size
    w = np.zeros((E, N, K * bits // 32), dtype=np.uint32)
    s = I.to_bf16_bits(np.full((E, N, K // 64), 0.5))
    b = I.to_bf16_bits(np.broadcast_to((np.arange(E) + 1.0)[:, None, None], (E, N, K // 64)))
    xv = (np.arange(B) % 7 + 1).astype(np.float64)
    x = I.to_bf16_bits(np.broadcast_to(xv[:, None], (B, K)))
    g = I.Gather("const", x, w, s, b, idx, bits)
    exp = K * (idx[:, None] + 1.0) * xv[:, None] * np.ones((1, N))
    y, _ = G.run_gather(g, "f32")
    assert np.array_equal(G.to_f64(y), exp)


# ---------------------------------------------------------------------------
# Precondition violations and degenerate inputs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind,row", [("unsorted", 5), ("negative", 0), ("too_large", 11)])
def test_gather_violation_flag(kind, row):
    g = I.random_gather([4, 4, 4], N=70, K=128, bits=4, seed=1)
    idx = g.expert_idx.copy()
    if kind == "unsorted":
        idx[row] = 0           # 1 after a 1 ... -> 0 breaks the order at row 5
    elif kind == "negative":
        idx[row] = -1
    else:
        idx[row] = 3           # E = 3
    y, ws = G.run_gather(g, "bf16", idx=idx)
    flag = int(ws[:4].cpu().numpy().view(np.uint32)[0])
    assert flag == row + 1
    assert np.all(G.to_f64(y) == 0.0)


def test_empty_problems():
    t = G.torch()
    x = t.empty((0, 128), dtype=t.bfloat16, device=G.dev())
    w = t.zeros((16, 16), dtype=t.int32, device=G.dev())
    s = t.zeros((16, 2), dtype=t.bfloat16, device=G.dev())
    y = t.empty((0, 16), dtype=t.bfloat16, device=G.dev())
    bm.bitmm_qmv(x, w, s, s, y, 4)
    bm.bitmm_qmm(x, w, s, s, y, 4)
    g = I.random_gather([0, 0], N=16, K=128, bits=4)
    yg, _ = G.run_gather(g, "bf16")
    assert yg.shape == (0, 16)


# ---------------------------------------------------------------------------
# Full-size workloads: sampled outputs, in the configuration the benchmark times
# ---------------------------------------------------------------------------

FULL_DENSE = [(1, 5120, 4), (1, 13824, 4), (600, 13824, 4), (3, 13824, 4),
              (1, 5120, 8), (1, 13824, 8), (600, 13824, 8), (3, 13824, 8)]


def test_tiny_qmv_full():
    d = I.tiny_qmv()
    for out in ("bf16", "f32"):
        got = G.to_f64(G.run_dense("bitmm_qmv", d, out))
        G.assert_close(got, oracle_dense(d), out, f"tiny qmv {out}")


@pytest.mark.parametrize("M,N,bits", FULL_DENSE)
def test_hidden5120_full_size(M, N, bits):
    """The hidden-5120 workloads at their real sizes: every output of the decode GEMV and
    of the 3-row GEMM against the oracle; the 600-row GEMM (42 G multiply-adds for the
    oracle) on sampled outputs plus its corners and last row and column."""
    d = I.hidden5120(M, N, bits)
    fn = "bitmm_qmv" if M == 1 else "bitmm_qmm"
    exact_path = M < 8
    ref_all = oracle_dense(d) if M < 8 else None
    for out in (("bf16", "f32") if exact_path else ("bf16",)):
        y = G.run_dense(fn, d, out)
        y2 = G.run_dense(fn, d, out)
        t = G.torch()
        assert t.equal(y, y2), "not deterministic"
        got = G.to_f64(y)
        assert np.all(np.isfinite(got))
        if ref_all is not None:
            G.assert_close(got, ref_all, out, f"{d.name} {out}")
        else:
            r, c = G.sample_points(d.M, d.N, 3000, seed=M + N)
            ref = oracle.qmm_points(d.x, d.w, d.scales, d.biases, r, c, bits)
            G.assert_close(got[r, c], ref, out, f"{d.name} {out}")


@pytest.mark.parametrize("which", ["up", "down"])
def test_moe_gather_full_size(which):
    g = I.moe_gather(which)
    y, ws = G.run_gather(g, "bf16")
    y2, _ = G.run_gather(g, "bf16")
    t = G.torch()
    assert t.equal(y, y2)
    wsn = ws.cpu().numpy().view(np.uint32)
    assert wsn[0] == 0
    got = G.to_f64(y)
    # every output (9.1 G multiply-adds for the oracle, a few seconds on the host cores)
    ref = oracle.gather_qmm(g.x, g.w, g.scales, g.biases, g.expert_idx, g.bits)
    G.assert_close(got, ref, "bf16", g.name)


# ---------------------------------------------------------------------------
# Determinism, streams, cross-op consistency
# ---------------------------------------------------------------------------

def test_repeat_bitwise_identical():
    t = G.torch()
    d = I.random_dense(1, 777, 2048, 4, seed=9)
    m = I.random_dense(96, 300, 1024, 8, seed=10)
    g = I.random_gather([20, 0, 50, 7], N=160, K=384, bits=4, seed=11)
    for _ in range(2):
        a = [G.run_dense("bitmm_qmv", d) for _ in range(10)]
        b = [G.run_dense("bitmm_qmm", m) for _ in range(10)]
        c = [G.run_gather(g)[0] for _ in range(10)]
        for seq in (a, b, c):
            for v in seq[1:]:
                assert t.equal(v, seq[0])


def test_side_stream_matches_default():
    t = G.torch()
    d = I.random_dense(130, 300, 640, 4, seed=12)
    ref = G.run_dense("bitmm_qmm", d)
    s1, s2 = t.cuda.Stream(), t.cuda.Stream()
    with t.cuda.stream(s1):
        y1 = G.run_dense("bitmm_qmm", d, stream=s1)
    with t.cuda.stream(s2):
        y2 = G.run_dense("bitmm_qmm", d, stream=s2)
    t.cuda.synchronize()
    assert t.equal(y1, ref) and t.equal(y2, ref)


def test_cross_op_consistency():
    """qmm at M=1 is the GEMV; the first rows of an M=600 GEMM agree with M=3;
    a single-expert gather agrees with qmm. The gather and the dense GEMM may use
    different matrix-core tiles (the same bf16 weights, another f32 summation order),
    so that last pair is held to f32 rounding, not bit equality."""
    t = G.torch()
    d1 = I.random_dense(1, 500, 1024, 4, seed=13)
    assert t.equal(G.run_dense("bitmm_qmv", d1), G.run_dense("bitmm_qmm", d1))
    big = I.hidden5120(64, 2048, 4)
    small = I.Dense("first3", big.x[:3].copy(), big.w, big.scales, big.biases, 4)
    yb = G.to_f64(G.run_dense("bitmm_qmm", big, "f32"))[:3]
    ys = G.to_f64(G.run_dense("bitmm_qmm", small, "f32"))
    G.assert_close(yb, ys, "bf16", "M=64 rows 0-2 vs M=3")
    g = I.random_gather([300], N=200, K=512, bits=8, seed=14)
    dg = I.Dense("e0", g.x, g.w[0], g.scales[0], g.biases[0], 8)
    yg, _ = G.run_gather(g, "f32")
    ym = G.run_dense("bitmm_qmm", dg, "f32")
    G.assert_close(G.to_f64(yg), G.to_f64(ym), "f32", "one-expert gather vs qmm")
