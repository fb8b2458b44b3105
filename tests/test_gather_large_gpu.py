"""GPU parity of the grouped GEMMs' row bookkeeping at large and awkward id arrays.

The prepare kernel (sorted form) and the counting sort (indexed form) each run as one
workgroup of 1024 threads that strides over the ids; here B reaches 16 to 20 thousand
rows (16 to 20 ids per thread, row tiles looping within one expert), the precondition
breaks at the first, a middle and the last row, invalid ids sit at thread-stride
boundaries, and the id arrays are only 4-byte aligned. Every output is checked, with
the status word, the expert offsets and the zeroed rows of invalid ids.
"""

import numpy as np
import pytest

import bit_matmul_amd as bm
import oracle
from bit_matmul_amd import inputs as I
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

BIG = 16384


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = G.torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    bm.lib()
    yield
    t.cuda.synchronize()


# Per-expert row counts: 16 thousand rows and more, empty experts, runs of row tiles.
SORTED_COUNTS = [
    [6000, 0, 5000, 5384],          # 16384
    [6000, 0, 5000, 5385],          # 16385
    [1, 9000, 0, 0, 8500, 3000],    # 20501
    [4096, 4096, 4096, 4095],       # 16383
]


@pytest.mark.parametrize("counts", SORTED_COUNTS)
def test_sorted_large_batches(counts):
    g = I.random_gather(counts, N=64, K=128, bits=4, seed=sum(counts))
    y, ws = G.run_gather(g, "f32")
    ref = oracle.gather_qmm(g.x, g.w, g.scales, g.biases, g.expert_idx, 4)
    G.assert_close(G.to_f64(y), ref, "bf16", f"gather B{g.B}")
    w = ws.cpu().numpy().view(np.uint32)
    assert w[0] == 0
    exp_off = np.searchsorted(g.expert_idx, np.arange(g.E + 1), side="left")
    assert np.array_equal(w[1:g.E + 2].view(np.int32), exp_off)


@pytest.mark.parametrize("B,row", [(16384, 16383), (16384, 255), (16385, 16384), (20000, 17000),
                                   (20000, 3)])
def test_sorted_violation_large(B, row):
    """An unsorted id at `row` (the last row, a thread-stride boundary, deep inside):
    status = row + 1 and every output zero."""
    g = I.random_gather([B // 2, B - B // 2], N=40, K=128, bits=4, seed=B + row)
    idx = g.expert_idx.copy()
    idx[row] = 1 if idx[row] == 0 else 0
    if row == 0 or idx[row - 1] <= idx[row]:   # make sure the row itself breaks the order
        idx[:row] = 1
        idx[row] = 0
    first = int(np.flatnonzero((idx[1:] < idx[:-1]))[0]) + 1
    t = G.torch()
    x, w, s, b, e = G.gather_to_dev(g, idx)
    y = t.full((g.B, g.N), 7.0, dtype=t.float32, device=G.dev())
    ws = t.empty(bm.bitmm_gather_qmm_workspace_bytes(g.B, g.N, g.E), dtype=t.uint8, device=G.dev())
    bm.bitmm_gather_qmm(x, w, s, b, e, y, ws, g.bits)
    flag = int(ws[:4].cpu().numpy().view(np.uint32)[0])
    assert flag == first + 1
    assert np.all(G.to_f64(y) == 0.0)


def _run_indexed(g, tok, exp, out="f32"):
    t = G.torch()
    x, w, s, b = G.bf16_tensor(g.x), G.u32_tensor(g.w), G.bf16_tensor(g.scales), G.bf16_tensor(g.biases)
    tt = None if tok is None else G.i32_tensor(tok)
    et = G.i32_tensor(exp)
    B = exp.shape[0]
    y = t.full((B, g.N), 12345.0, dtype=t.bfloat16 if out == "bf16" else t.float32, device=G.dev())
    ws = t.empty(bm.bitmm_gather_qmm_indexed_workspace_bytes(B, g.N, g.E), dtype=t.uint8, device=G.dev())
    bm.bitmm_gather_qmm_indexed(x, w, s, b, tt, et, y, ws, g.bits)
    return G.to_f64(y), int(ws[:4].cpu().numpy().view(np.uint32)[0])


@pytest.mark.parametrize("B,E", [(BIG, 3), (BIG - 1, 7), (BIG + 1, 3), (19000, 40)])
@pytest.mark.parametrize("tokens", [True, False])
def test_indexed_large_batches(B, E, tokens):
    T = 300
    g = I.random_indexed(T, B, E, 72, 128, 4, seed=B + E, with_tokens=tokens)
    got, flag = _run_indexed(g, g.token_idx, g.expert_idx)
    assert flag == 0
    ref = oracle.gather_qmm_indexed(g.x, g.w, g.scales, g.biases, g.token_idx, g.expert_idx, 4)
    G.assert_close(got, ref, "bf16", f"indexed B{B} E{E}")


@pytest.mark.parametrize("B", [BIG, BIG + 100])
def test_indexed_invalid_ids_large(B):
    """Invalid expert and token ids spread over the batch, the last row among them: those
    rows are zero, the status word names the first."""
    T, E = 50, 5
    g = I.random_indexed(T, B, E, 70, 128, 4, seed=B)
    tok = g.token_idx.copy()
    exp = g.expert_idx.copy()
    deep = 4 * (15 * 256 + 7) + 3
    bad = [17, deep, B - 1, 4000, 4 * 9]
    tok[17], exp[deep], exp[B - 1], tok[4000], exp[4 * 9] = T, E, -1, -3, E + 7
    got, flag = _run_indexed(g, tok, exp)
    assert flag == min(bad) + 1
    for r in bad:
        assert np.all(got[r] == 0.0), r
    ref = oracle.gather_qmm_indexed(g.x, g.w, g.scales, g.biases, tok, exp, 4)
    G.assert_close(got, ref, "bf16", f"indexed invalid B{B}")


def _misaligned(t, a):
    """A view of a's values that starts 4 bytes into a fresh allocation."""
    buf = t.empty(a.numel() + 1, dtype=a.dtype, device=a.device)
    v = buf[1:]
    v.copy_(a)
    assert v.data_ptr() % 16 == 4
    return v


def test_sorted_misaligned_ids():
    """Ids only 4-byte aligned (a view 4 bytes into an allocation)."""
    t = G.torch()
    g = I.random_gather([5, 0, 40, 12, 300], N=64, K=128, bits=4, seed=3)
    x, w, s, b, e = G.gather_to_dev(g)
    e1 = _misaligned(t, e)
    y = t.empty((g.B, g.N), dtype=t.float32, device=G.dev())
    ws = t.empty(bm.bitmm_gather_qmm_workspace_bytes(g.B, g.N, g.E), dtype=t.uint8, device=G.dev())
    bm.bitmm_gather_qmm(x, w, s, b, e1, y, ws, g.bits)
    ref = oracle.gather_qmm(g.x, g.w, g.scales, g.biases, g.expert_idx, 4)
    G.assert_close(G.to_f64(y), ref, "bf16", "misaligned ids")
    wsv = ws.cpu().numpy().view(np.uint32)
    assert wsv[0] == 0
    exp_off = np.searchsorted(g.expert_idx, np.arange(g.E + 1), side="left")
    assert np.array_equal(wsv[1:g.E + 2].view(np.int32), exp_off)


@pytest.mark.parametrize("which", ["tok", "exp"])
def test_indexed_misaligned_ids(which):
    """Token or expert ids only 4-byte aligned."""
    t = G.torch()
    g = I.random_indexed(40, 500, 9, 70, 128, 4, seed=5)
    x, w, s, b = G.bf16_tensor(g.x), G.u32_tensor(g.w), G.bf16_tensor(g.scales), G.bf16_tensor(g.biases)
    tt, et = G.i32_tensor(g.token_idx), G.i32_tensor(g.expert_idx)
    if which == "tok":
        tt = _misaligned(t, tt)
    else:
        et = _misaligned(t, et)
    y = t.full((g.B, g.N), 12345.0, dtype=t.float32, device=G.dev())
    ws = t.empty(bm.bitmm_gather_qmm_indexed_workspace_bytes(g.B, g.N, g.E), dtype=t.uint8, device=G.dev())
    bm.bitmm_gather_qmm_indexed(x, w, s, b, tt, et, y, ws, g.bits)
    assert int(ws[:4].cpu().numpy().view(np.uint32)[0]) == 0
    ref = oracle.gather_qmm_indexed(g.x, g.w, g.scales, g.biases, g.token_idx, g.expert_idx, 4)
    G.assert_close(G.to_f64(y), ref, "bf16", f"indexed misaligned {which}")
