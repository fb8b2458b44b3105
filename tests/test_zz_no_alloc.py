"""The allocation-free gather entry point, bitmm_gather_qmm_noalloc, called through the C
ABI, against bitmm_gather_qmm with a workspace of its own on the same inputs: the two
share their kernels, so the outputs must be bitwise identical. Calls in a row on one
GPU share the library's static workspace; the second call is smaller than the first, so
a stale offset or status word from the first call would show.
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


def _both(g, out, idx=None):
    """(y from bitmm_gather_qmm, its status word, y from the no-alloc entry, its status)."""
    t = G.torch()
    y_ws, ws = G.run_gather(g, out, idx)
    x, w, s, b, e = G.gather_to_dev(g, idx)
    y = t.full((g.B, g.N), 7.0, dtype=t.bfloat16 if out == "bf16" else t.float32, device=G.dev())
    status = t.full((1,), -1, dtype=t.int32, device=G.dev())
    bm.bitmm_gather_qmm_noalloc(x, w, s, b, e, y, g.bits, group_size=getattr(g, "group", 64), status=status)
    t.cuda.synchronize()
    ws0 = int(ws[:4].cpu().numpy().view(np.uint32)[0])
    return y_ws, ws0, y, int(status.cpu().numpy().view(np.uint32)[0])


def _bits_equal(a, b):
    t = G.torch()
    v = t.int16 if a.dtype == t.bfloat16 else t.int32
    return bool(t.equal(a.view(v), b.view(v)))


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_noalloc_matches_workspace_entry_two_calls(out):
    # first call: 40 experts (some empty, one past a 64-row tile), then a smaller one
    counts1 = [3, 0, 70, 1, 0, 0, 12, 36, 5, 0] * 4
    g1 = I.random_gather(counts1, N=200, K=320, bits=4, seed=11)
    g2 = I.random_gather([2, 5, 0, 9], N=96, K=128, bits=8, seed=12)
    for g in (g1, g2):
        y_ws, ws0, y, st = _both(g, out)
        assert ws0 == 0 and st == 0
        assert _bits_equal(y, y_ws), f"no-alloc output differs from the workspace entry ({g.name})"
        ref = oracle.gather_qmm(g.x, g.w, g.scales, g.biases, g.expert_idx, g.bits)
        G.assert_close(G.to_f64(y), ref, "bf16", g.name)


def test_noalloc_moe_shape_then_small():
    g1 = I.moe_gather("down")
    y_ws, ws0, y, st = _both(g1, "bf16")
    assert ws0 == 0 and st == 0 and _bits_equal(y, y_ws)
    g2 = I.random_gather([1, 0, 4], N=64, K=64, bits=4, seed=13)
    y_ws, ws0, y, st = _both(g2, "bf16")
    assert ws0 == 0 and st == 0 and _bits_equal(y, y_ws)


def test_noalloc_precondition_status():
    g = I.random_gather([4, 6, 3, 5], N=64, K=128, bits=4, seed=14)
    bad = g.expert_idx.copy()
    bad[9] = 0  # decreasing at row 9
    y_ws, ws0, y, st = _both(g, "bf16", idx=bad)
    assert ws0 == 10 and st == 10
    assert not G.torch().any(y.float() != 0).item()
    # a valid call right after: the status word is rewritten
    y_ws, ws0, y, st = _both(g, "bf16")
    assert st == 0 and _bits_equal(y, y_ws)
