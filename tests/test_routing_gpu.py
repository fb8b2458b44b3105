"""Which kernel each call enqueues, from the library's kernel-choice record
(bitmm_last_launches): the shape rules of the dispatch, pinned on the shapes the
benchmark and the pages' workloads use. The inputs are zeros (the choice depends on
shapes, code width, group size and alignment only); the parity of every kernel named
here is checked elsewhere on real values.
"""

import pytest

import bit_matmul_amd as bm
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


def dense(fn, M, N, K, bits, group=64):
    t = G.torch()
    x = t.zeros((M, K), dtype=t.bfloat16, device=G.dev())
    w = t.zeros((N, K * bits // 32), dtype=t.int32, device=G.dev())
    s = t.zeros((N, K // group), dtype=t.bfloat16, device=G.dev())
    y = t.empty((M, N), dtype=t.bfloat16, device=G.dev())
    getattr(bm, fn)(x, w, s, s, y, bits, group_size=group)
    return bm.bitmm_last_launches()


def one(rec):
    assert len(rec) == 1, rec
    return rec[0]


@pytest.mark.parametrize("M,N,K,bits,want", [
    # decode GEMV at hidden 5120: one row x 64 lanes x 3 chunks, two steps per wave at
    # N = 13824 (1728 workgroups of 4 waves), one at N = 5120
    (1, 13824, 5120, 4, "qmv_dma_kernel<4, 64, 3, 2> grid=1728x1 block=256"),
    (1, 5120, 5120, 4, "qmv_dma_kernel<4, 64, 3, 1> grid=1280x1 block=256"),
    (1, 13824, 5120, 8, "qmv_dma_kernel<8, 64, 5, 2> "),
    (1, 13824, 5120, 2, "qmv_dma_kernel<2, 32, 3, 1> "),
    (1, 256, 512, 4, "qmv_dma_kernel<4, 16, 1, 1> "),   # the tiny config: 16 chunks per row
    # one row past the decode kernel's K range: split-K up to 16384 at 4 bits, then general
    (1, 4096, 12288, 4, "qmv_split_kernel<4, 1, "),
    (1, 4096, 24576, 4, "qmv_kernel<4, 1, "),
])
def test_qmv_routes(M, N, K, bits, want):
    r = one(dense("bitmm_qmv", M, N, K, bits))
    assert r.startswith(want), r


@pytest.mark.parametrize("M,bits,want", [
    (2, 4, "qmv_mfma_kernel<4, 2, 8, 2, 1, 1> "),   # small M: the matrix-core GEMV
    (3, 4, "qmv_mfma_kernel<4, 2, 8, 2, 1, 1> "),
    (3, 8, "qmv_mfma_kernel<8, 4, 8, 1, 1, 1> "),
    (5, 4, "qmv_mfma_kernel<4, 2, 8, 2, 1, 2> "),   # two row groups
    (8, 4, "qmv_mfma_kernel<4, 2, 8, 2, 1, 2> "),   # M = 8 stays on the GEMV where it fits
    (9, 4, "qmm_mfma_kernel<MmTile4<4, 1, 4, 4, 2, 1, 80, false, true>> "),
    (64, 4, "qmm_mfma_kernel<MmTile4<4, 1, 4, 4, 2, 1, 80, false, true>> grid=216x1"),  # 2 x 108 tiles
    (128, 4, "qmm_mfma_kernel<MmTile4<4, 2, 4, 4, 2, 1, 80, false, true>> grid=216x1"),
    (300, 4, "qmm_mfma_kernel<MmTile4<4, 6, 4, 4, 2, 1, 80, false, true>> grid=216x1"),
    (600, 4, "qmm_mfma_kernel<MmTile4<4, 10, 4, 4, 2, 1, 80, false, true>> grid=216x1 block=256 lds=163840"),
    (600, 8, "qmm_mfma_kernel<MmTile4<8, 10, 4, 4, 2, 1, 80, false, true>> grid=216x1"),
    (600, 2, "qmm_mfma_kernel<MmTile4<2, 10, 4, 4, 2, 1, 80, false, false>> grid=216x1"),
])
def test_qmm_routes_hidden5120(M, bits, want):
    r = one(dense("bitmm_qmm", M, 13824, 5120, bits))
    assert r.startswith(want), r


@pytest.mark.parametrize("M,N,K,want", [
    # Narrow N: smaller row tiles, so that the grid fills the CUs in one round
    (600, 5120, 13824, "qmm_mfma_kernel<MmTile4<4, 4, 4, 4, 2, 0, 0, false, true>> grid=200x1"),
    (600, 5120, 5120, "qmm_mfma_kernel<MmTile4<4, 4, 4, 4, 2, 1, 80, false, true>> grid=200x1"),
    (600, 2048, 5120, "qmm_mfma_kernel<MmTile4<4, 2, 4, 4, 2, 1, 80, false, true>> grid=160x1"),
    (600, 700, 512, "qmm_mfma_kernel<MmTile4<4, 1, 4, 4, 2, 1, 80, false, true>> grid=114x1"),
    # Large M: rounds of 256 tiles; 2048 rows at N = 5120 in 11 tiles of 192 rows
    (2048, 5120, 5120, "qmm_mfma_kernel<MmTile4<4, 6, 4, 4, 2, 1, 80, false, true>> grid=440x1"),
])
def test_qmm_row_tile_choice(M, N, K, want):
    assert one(dense("bitmm_qmm", M, N, K, 4)).startswith(want)


def test_qmm_group32_loads_scales_per_group():
    """G = 160 groups per row do not fit the staging area: per-lane scale loads."""
    assert one(dense("bitmm_qmm", 600, 13824, 5120, 4, group=32)).startswith(
        "qmm_mfma_kernel<MmTile4<4, 10, 4, 4, 2, 0, 0, false, true>> ")


def test_qmm_more_than_eight_small_rows_run_in_launches_of_eight():
    """bitmm_qmv with M = 17: launches of 8, 8 and 1 rows."""
    rec = dense("bitmm_qmv", 17, 700, 512, 4)
    assert len(rec) == 3, rec
    assert all(r.startswith("qmv_mfma_kernel<4, ") for r in rec[:2])


def _moe_sorted(E, rows_per_expert, N, K, bits=4):
    t = G.torch()
    B = E * rows_per_expert
    x = t.zeros((B, K), dtype=t.bfloat16, device=G.dev())
    w = t.zeros((E, N, K * bits // 32), dtype=t.int32, device=G.dev())
    s = t.zeros((E, N, K // 64), dtype=t.bfloat16, device=G.dev())
    idx = t.arange(E, dtype=t.int32, device=G.dev()).repeat_interleave(rows_per_expert)
    return x, w, s, idx, B


@pytest.mark.parametrize("which,N,K,tile", [
    ("up", 704, 2816, "MmTile4<4, 2, 4, 4, 2, 1, 48, false, true>"),
    ("down", 2816, 704, "MmTile4<4, 2, 4, 4, 2, 2, 12, false, true>"),   # G = 11 (odd): 2-byte staging
])
def test_gather_routes_moe(which, N, K, tile):
    """MoE prefill, ~36 rows per expert: the prepare pass, then 64-row tiles, one
    workgroup per (expert, 128-column block)."""
    t = G.torch()
    E = 128
    x, w, s, idx, B = _moe_sorted(E, 36, N, K)
    y = t.empty((B, N), dtype=t.bfloat16, device=G.dev())
    ws = t.empty(bm.bitmm_gather_qmm_workspace_bytes(B, N, E), dtype=t.uint8, device=G.dev())
    bm.bitmm_gather_qmm(x, w, s, s, idx, y, ws, 4)
    rec = bm.bitmm_last_launches()
    assert len(rec) == 2, rec
    assert rec[0].startswith("gather_prepare_kernel grid=1x1 block=1024")
    tiles_n = (N + 127) // 128
    assert rec[1].startswith(f"gather_qmm_kernel<4, {tile}> grid={E * tiles_n}x1 block=256")


def test_gather_indexed_and_small_batch_routes():
    """Rows in routing order: the counting sort, then the gathered-row tile; at ~3 rows
    per expert (the 46-token prompt) 32-row tiles."""
    t = G.torch()
    E, N, K, T = 128, 704, 2816, 46
    B = T * 8
    x = t.zeros((T, K), dtype=t.bfloat16, device=G.dev())
    w = t.zeros((E, N, K // 8), dtype=t.int32, device=G.dev())
    s = t.zeros((E, N, K // 64), dtype=t.bfloat16, device=G.dev())
    tok = t.arange(T, dtype=t.int32, device=G.dev()).repeat_interleave(8)
    exp = (t.arange(B, dtype=t.int32, device=G.dev()) * 37) % E
    y = t.empty((B, N), dtype=t.bfloat16, device=G.dev())
    ws = t.empty(bm.bitmm_gather_qmm_indexed_workspace_bytes(B, N, E), dtype=t.uint8, device=G.dev())
    bm.bitmm_gather_qmm_indexed(x, w, s, s, tok, exp, y, ws, 4)
    rec = bm.bitmm_last_launches()
    assert len(rec) == 2, rec
    assert rec[0].startswith("gather_sort_kernel grid=1x1 block=1024")
    assert rec[1].startswith("gather_qmm_indexed_kernel<4, MmTile4<4, 1, 4, 4, 2, 1, 48, true, true>> ")


def test_gather_noalloc_same_kernels():
    t = G.torch()
    E, N, K = 16, 704, 2816
    x, w, s, idx, B = _moe_sorted(E, 36, N, K)
    y = t.empty((B, N), dtype=t.bfloat16, device=G.dev())
    bm.bitmm_gather_qmm_noalloc(x, w, s, s, idx, y, 4)
    rec = bm.bitmm_last_launches()
    assert [r.split(" ")[0] for r in rec] == [
        "gather_prepare_kernel", "gather_qmm_kernel<4,"], rec


def test_gather_qmv_routes():
    """MoE decode: the decode GEMV with one grid row per gathered row."""
    t = G.torch()
    E, N, K, T = 128, 704, 2816, 1
    x = t.zeros((T, K), dtype=t.bfloat16, device=G.dev())
    w = t.zeros((E, N, K // 8), dtype=t.int32, device=G.dev())
    s = t.zeros((E, N, K // 64), dtype=t.bfloat16, device=G.dev())
    tok = t.zeros(8, dtype=t.int32, device=G.dev())
    exp = t.arange(8, dtype=t.int32, device=G.dev()) * 9
    y = t.empty((8, N), dtype=t.bfloat16, device=G.dev())
    bm.bitmm_gather_qmv(x, w, s, s, tok, exp, y, 4)
    r = one(bm.bitmm_last_launches())
    assert r.startswith("qmv_dma_kernel<4, 32, 3, 1> ") and "x8 block=256" in r, r


def test_gather_mm_routes():
    t = G.torch()
    E, N, K, B = 16, 704, 2816, 16 * 36
    x = t.zeros((B, K), dtype=t.bfloat16, device=G.dev())
    w = t.zeros((E, N, K), dtype=t.bfloat16, device=G.dev())
    exp = t.arange(E, dtype=t.int32, device=G.dev()).repeat_interleave(36)
    y = t.empty((B, N), dtype=t.bfloat16, device=G.dev())
    ws = t.empty(bm.bitmm_gather_mm_workspace_bytes(B, N, E), dtype=t.uint8, device=G.dev())
    bm.bitmm_gather_mm(x, w, None, exp, y, ws)
    rec = bm.bitmm_last_launches()
    assert [r.split(" ")[0] for r in rec] == ["gather_sort_kernel", "gather_mm_kernel<MmTileD<0,"], rec


def test_record_resets_per_call():
    dense("bitmm_qmv", 1, 256, 512, 4)
    assert len(bm.bitmm_last_launches()) == 1
    t = G.torch()
    x = t.zeros((0, 512), dtype=t.bfloat16, device=G.dev())
    w = t.zeros((256, 64), dtype=t.int32, device=G.dev())
    s = t.zeros((256, 8), dtype=t.bfloat16, device=G.dev())
    y = t.empty((0, 256), dtype=t.bfloat16, device=G.dev())
    bm.bitmm_qmv(x, w, s, s, y, 4)           # an empty problem enqueues nothing
    assert bm.bitmm_last_launches() == []
