"""Every entry point captured into a HIP graph (torch.cuda.CUDAGraph) and replayed:
each replay must equal the eager call bit for bit, with eager work and host
synchronisation between the replays, and a replay after the inputs change in place
must equal the eager call on the new inputs (the graph re-reads its buffers; no call
records a memset or keeps state between launches)."""

import numpy as np
import pytest

import bit_matmul_amd as bm
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


def _dense(fn, M, N, K, bits):
    t = G.torch()
    d = I.random_dense(M, N, K, bits, seed=M + N + K + bits)
    args = list(G.dense_to_dev(d))
    y = t.empty((M, N), dtype=t.bfloat16, device=G.dev())
    return (lambda: getattr(bm, fn)(*args, y, bits)), y, args[0]


def _gather(bits):
    t = G.torch()
    g = I.random_gather([40, 0, 70, 9, 33], N=130, K=704, bits=bits, seed=bits)
    x, w, s, b, e = G.gather_to_dev(g)
    y = t.empty((g.B, g.N), dtype=t.bfloat16, device=G.dev())
    ws = t.empty(bm.bitmm_gather_qmm_workspace_bytes(g.B, g.N, g.E), dtype=t.uint8, device=G.dev())
    return (lambda: bm.bitmm_gather_qmm(x, w, s, b, e, y, ws, bits)), y, x


def _indexed(kind):
    t = G.torch()
    g = I.random_indexed(20, 150 if kind == "qmm" else 12, 6, 96, 2816, 4, seed=7)
    x, w = G.bf16_tensor(g.x), G.u32_tensor(g.w)
    s, b = G.bf16_tensor(g.scales), G.bf16_tensor(g.biases)
    tok, e = G.i32_tensor(g.token_idx), G.i32_tensor(g.expert_idx)
    y = t.empty((g.B, g.N), dtype=t.float32, device=G.dev())
    if kind == "qmm":
        ws = t.empty(bm.bitmm_gather_qmm_indexed_workspace_bytes(g.B, g.N, g.E), dtype=t.uint8, device=G.dev())
        return (lambda: bm.bitmm_gather_qmm_indexed(x, w, s, b, tok, e, y, ws, 4)), y, x
    return (lambda: bm.bitmm_gather_qmv(x, w, s, b, tok, e, y, 4)), y, x


def _gather_mm(layout):
    t = G.torch()
    g = I.random_gather_mm(30, 200, 5, 136, 1040, "bf16", layout, seed=5)
    x, w = G.bf16_tensor(g.x), G.bf16_tensor(g.w)
    tok, e = G.i32_tensor(g.token_idx), G.i32_tensor(g.expert_idx)
    y = t.empty((g.B, g.N), dtype=t.bfloat16, device=G.dev())
    ws = t.empty(bm.bitmm_gather_mm_workspace_bytes(g.B, g.N, g.E), dtype=t.uint8, device=G.dev())
    return (lambda: bm.bitmm_gather_mm(x, w, tok, e, y, ws, layout)), y, x


CASES = {
    "qmv": lambda: _dense("bitmm_qmv", 1, 13824 // 8, 5120, 4),
    "qmv_split": lambda: _dense("bitmm_qmm", 3, 1000, 5120, 8),
    "qmm_mfma": lambda: _dense("bitmm_qmm", 200, 300, 2048, 4),
    "gather_qmm": lambda: _gather(4),
    "gather_qmm_indexed": lambda: _indexed("qmm"),
    "gather_qmv": lambda: _indexed("qmv"),
    "gather_mm_nk": lambda: _gather_mm("nk"),
    "gather_mm_kn": lambda: _gather_mm("kn"),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replays_match_eager(name):
    t = G.torch()
    call, y, x = CASES[name]()
    call()
    t.cuda.synchronize()
    eager = y.clone()
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    graph = t.cuda.CUDAGraph()
    with t.cuda.graph(graph, stream=side):
        call()
    t.cuda.synchronize()
    other, y2, _ = CASES["qmm_mfma" if name != "qmm_mfma" else "qmv"]()
    for i in range(4):
        y.fill_(1234.0)
        graph.replay()
        t.cuda.synchronize()
        assert t.equal(y, eager), f"{name}: replay {i} differs from the eager call"
        other()              # eager work of another kernel between replays
        _ = (y2 * 2).sum().item()
    # the graph reads its input buffers anew: change x in place, compare with eager
    x.copy_(x.flip(0) if x.shape[0] > 1 else -x)
    call()
    t.cuda.synchronize()
    eager2 = y.clone()
    assert not t.equal(eager2, eager)
    y.fill_(1234.0)
    graph.replay()
    t.cuda.synchronize()
    assert t.equal(y, eager2), f"{name}: replay after an input change differs"
    del graph
