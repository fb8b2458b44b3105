"""Host-side tests of the C ABI: no GPU needed.

The library must load, export every function ``include/bitmm.h`` declares, and
reject bad arguments with the documented status before touching the device.
Pointer arguments here are fake addresses: validation never dereferences them.
"""

import ctypes
import os
import re

import pytest

import bit_matmul_amd as bm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitmm.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bitmm_\w+)\s*\(", text)))


def header_enum(name):
    text = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(rf"\b({name}_\w+)\s*=\s*(\d+)", text)}


@pytest.fixture(scope="module")
def L():
    return bm.lib()


def gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def test_exports_every_declared_function(L):
    names = header_functions()
    assert set(names) == {"bitmm_abi_version", "bitmm_status_string", "bitmm_last_launches",
                          "bitmm_qmv", "bitmm_qmm",
                          "bitmm_gather_qmm_workspace_bytes", "bitmm_gather_qmm",
                          "bitmm_gather_qmm_noalloc", "bitmm_gather_qmv", "bitmm_gather_qmm_indexed_workspace_bytes",
                          "bitmm_gather_qmm_indexed", "bitmm_gather_mm_workspace_bytes",
                          "bitmm_gather_mm"}
    for n in names:
        assert hasattr(L, n), f"libbitmm.so does not export {n}"


def test_launch_record_is_empty_after_a_rejected_call(L):
    """Every call starts a fresh kernel-choice record; a call rejected by validation (here
    a code width the library does not take) enqueues nothing and leaves it empty. The
    query copies nothing into a NULL or zero-length buffer and returns the full length."""
    assert L.bitmm_qmv(*dense_args(bits=3)) == bm.BITMM_ERR_UNSUPPORTED
    assert bm.bitmm_last_launches() == []
    buf = ctypes.create_string_buffer(b"xyz", 4)
    assert L.bitmm_last_launches(buf, 0) == 0
    assert buf.value == b"xyz"
    assert L.bitmm_last_launches(None, 16) == 0
    assert L.bitmm_last_launches(buf, 4) == 0 and buf.value == b""


def test_abi_version_matches_header(L):
    text = open(HEADER).read()
    v = int(re.search(r"#define BITMM_ABI_VERSION (\d+)", text).group(1))
    assert bm.bitmm_abi_version() == v


def test_status_codes_match_header_and_have_strings(L):
    codes = header_enum("BITMM")
    for k, v in codes.items():
        if k.startswith(("BITMM_OUT_", "BITMM_DTYPE_", "BITMM_LAYOUT_")):
            assert getattr(bm, k) == v, k
            continue
        assert getattr(bm, k) == v, k
        s = bm.bitmm_status_string(v)
        assert s and s != "unknown status"
    assert bm.bitmm_status_string(99) == "unknown status"
    assert bm.BITMM_OUT_BF16 == codes["BITMM_OUT_BF16"] and bm.BITMM_OUT_F32 == codes["BITMM_OUT_F32"]


A = 0x10000  # fake, 256-byte aligned addresses


def dense_args(**kw):
    a = dict(x=A, w=A + 0x1000, s=A + 0x2000, b=A + 0x3000, y=A + 0x4000, M=1, N=256, K=512,
             bits=4, group=64, out=0, stream=0)
    a.update(kw)
    return [ctypes.c_void_p(a["x"]), ctypes.c_void_p(a["w"]), ctypes.c_void_p(a["s"]),
            ctypes.c_void_p(a["b"]), ctypes.c_void_p(a["y"]), a["M"], a["N"], a["K"], a["bits"],
            a["group"], a["out"], ctypes.c_void_p(a["stream"])]


DENSE_CASES = [
    (dict(bits=3), bm.BITMM_ERR_UNSUPPORTED),
    (dict(bits=2, group=32), bm.BITMM_ERR_UNSUPPORTED),  # 2 bits: groups of 64 and 128
    (dict(bits=1), bm.BITMM_ERR_UNSUPPORTED),
    (dict(bits=16), bm.BITMM_ERR_UNSUPPORTED),
    (dict(group=16), bm.BITMM_ERR_UNSUPPORTED),
    (dict(group=256), bm.BITMM_ERR_UNSUPPORTED),
    (dict(group=48), bm.BITMM_ERR_UNSUPPORTED),
    (dict(out=2), bm.BITMM_ERR_UNSUPPORTED),
    (dict(K=100), bm.BITMM_ERR_SHAPE),
    (dict(K=96, group=32), bm.BITMM_ERR_SHAPE),    # K must also be a multiple of 64
    (dict(K=576, group=128), bm.BITMM_ERR_SHAPE),  # and of the group size
    (dict(K=0), bm.BITMM_ERR_SHAPE),
    (dict(K=-64), bm.BITMM_ERR_SHAPE),
    (dict(M=-1), bm.BITMM_ERR_SHAPE),
    (dict(N=-5), bm.BITMM_ERR_SHAPE),
    (dict(M=1 << 31), bm.BITMM_ERR_SHAPE),
    (dict(K=3355456), bm.BITMM_ERR_UNSUPPORTED),   # 320 * K * 2 >= 2^31 (32-bit tile offsets)
    (dict(K=3355392), None),                       # the largest multiple of 64 below the limit
    (dict(M=0), bm.BITMM_OK),                      # empty problem: nothing enqueued
    (dict(N=0), bm.BITMM_OK),
    (dict(M=0, x=0, y=0), bm.BITMM_OK),            # pointers unused when empty
    (dict(x=0), bm.BITMM_ERR_NULL),
    (dict(w=0), bm.BITMM_ERR_NULL),
    (dict(s=0), bm.BITMM_ERR_NULL),
    (dict(b=0), bm.BITMM_ERR_NULL),
    (dict(y=0), bm.BITMM_ERR_NULL),
    (dict(x=A + 8), bm.BITMM_ERR_ALIGN),
    (dict(w=A + 4), bm.BITMM_ERR_ALIGN),
    (dict(s=A + 1), bm.BITMM_ERR_ALIGN),
    (dict(b=A + 3), bm.BITMM_ERR_ALIGN),
    (dict(y=A + 1), bm.BITMM_ERR_ALIGN),
    (dict(y=A + 2, out=1), bm.BITMM_ERR_ALIGN),
    (dict(s=A + 2, b=A + 6, y=A + 2), None),       # 2-byte alignment is enough -> device
]


@pytest.mark.parametrize("fn", ["bitmm_qmv", "bitmm_qmm"])
@pytest.mark.parametrize("kw,expected", DENSE_CASES)
def test_dense_validation(L, fn, kw, expected):
    if expected is None:
        if gpu_present():
            pytest.skip("fake pointers would reach a real device")
        expected = bm.BITMM_ERR_DEVICE
    assert getattr(L, fn)(*dense_args(**kw)) == expected


def test_dense_valid_without_device(L):
    """With every argument valid and no GPU the call reports BITMM_ERR_DEVICE."""
    if gpu_present():
        pytest.skip("fake pointers would reach a real device")
    for fn in (L.bitmm_qmv, L.bitmm_qmm):
        for bits in (2, 4, 8):
            for M in (1, 3, 8, 600):
                for group in (32, 64, 128):
                    if bits == 2 and group == 32:
                        continue
                    assert fn(*dense_args(bits=bits, M=M, out=1, group=group)) == bm.BITMM_ERR_DEVICE


def gather_args(**kw):
    a = dict(x=A, w=A + 0x1000, s=A + 0x2000, b=A + 0x3000, idx=A + 0x4000, y=A + 0x5000,
             B=4584, N=704, K=2816, E=128, bits=4, group=64, out=0, ws=A + 0x6000,
             ws_bytes=1 << 20, stream=0)
    a.update(kw)
    return [ctypes.c_void_p(a["x"]), ctypes.c_void_p(a["w"]), ctypes.c_void_p(a["s"]),
            ctypes.c_void_p(a["b"]), ctypes.c_void_p(a["idx"]), ctypes.c_void_p(a["y"]), a["B"],
            a["N"], a["K"], a["E"], a["bits"], a["group"], a["out"], ctypes.c_void_p(a["ws"]),
            a["ws_bytes"], ctypes.c_void_p(a["stream"])]


GATHER_CASES = [
    (dict(bits=5), bm.BITMM_ERR_UNSUPPORTED),
    (dict(bits=2, group=32), bm.BITMM_ERR_UNSUPPORTED),
    (dict(bits=2, group=128), None),
    (dict(group=16), bm.BITMM_ERR_UNSUPPORTED),
    (dict(out=-1), bm.BITMM_ERR_UNSUPPORTED),
    (dict(E=0), bm.BITMM_ERR_SHAPE),
    (dict(K=700), bm.BITMM_ERR_SHAPE),
    (dict(B=-1), bm.BITMM_ERR_SHAPE),
    (dict(B=0), bm.BITMM_OK),
    (dict(N=0), bm.BITMM_OK),
    (dict(idx=0), bm.BITMM_ERR_NULL),
    (dict(x=0), bm.BITMM_ERR_NULL),
    (dict(ws=0), bm.BITMM_ERR_WORKSPACE),
    (dict(ws_bytes=16), bm.BITMM_ERR_WORKSPACE),
    (dict(idx=A + 2), bm.BITMM_ERR_ALIGN),
    (dict(ws=A + 8), bm.BITMM_ERR_ALIGN),
    (dict(x=A + 2), bm.BITMM_ERR_ALIGN),
    (dict(), None),
]


@pytest.mark.parametrize("kw,expected", GATHER_CASES)
def test_gather_validation(L, kw, expected):
    if expected is None:
        if gpu_present():
            pytest.skip("fake pointers would reach a real device")
        expected = bm.BITMM_ERR_DEVICE
    assert L.bitmm_gather_qmm(*gather_args(**kw)) == expected


def noalloc_args(**kw):
    a = dict(x=A, w=A + 0x1000, s=A + 0x2000, b=A + 0x3000, idx=A + 0x4000, y=A + 0x5000,
             B=4584, N=704, K=2816, E=128, bits=4, group=64, out=0, status=A + 0x6000, stream=0)
    a.update(kw)
    return [ctypes.c_void_p(a["x"]), ctypes.c_void_p(a["w"]), ctypes.c_void_p(a["s"]),
            ctypes.c_void_p(a["b"]), ctypes.c_void_p(a["idx"]), ctypes.c_void_p(a["y"]), a["B"],
            a["N"], a["K"], a["E"], a["bits"], a["group"], a["out"], ctypes.c_void_p(a["status"]),
            ctypes.c_void_p(a["stream"])]


NOALLOC_CASES = [
    (dict(bits=5), bm.BITMM_ERR_UNSUPPORTED),
    (dict(group=16), bm.BITMM_ERR_UNSUPPORTED),
    (dict(out=2), bm.BITMM_ERR_UNSUPPORTED),
    (dict(E=16383), bm.BITMM_ERR_UNSUPPORTED),  # beyond the static workspace
    (dict(E=16383, B=0), bm.BITMM_ERR_UNSUPPORTED),
    (dict(E=0), bm.BITMM_ERR_SHAPE),
    (dict(K=700), bm.BITMM_ERR_SHAPE),
    (dict(B=-1), bm.BITMM_ERR_SHAPE),
    (dict(B=0), bm.BITMM_OK),
    (dict(N=0), bm.BITMM_OK),
    (dict(idx=0), bm.BITMM_ERR_NULL),
    (dict(y=0), bm.BITMM_ERR_NULL),
    (dict(idx=A + 2), bm.BITMM_ERR_ALIGN),
    (dict(status=A + 2), bm.BITMM_ERR_ALIGN),
    (dict(x=A + 2), bm.BITMM_ERR_ALIGN),
    (dict(), None),
    (dict(status=0), None),    # the status word is optional
    (dict(E=16382), None),     # the largest expert count the static workspace holds
]


@pytest.mark.parametrize("kw,expected", NOALLOC_CASES)
def test_gather_noalloc_validation(L, kw, expected):
    if expected is None:
        if gpu_present():
            pytest.skip("fake pointers would reach a real device")
        expected = bm.BITMM_ERR_DEVICE
    assert L.bitmm_gather_qmm_noalloc(*noalloc_args(**kw)) == expected


def gqmv_args(**kw):
    a = dict(x=A, w=A + 0x1000, s=A + 0x2000, b=A + 0x3000, tok=A + 0x4000, idx=A + 0x5000,
             y=A + 0x6000, B=8, N=704, K=2816, E=128, T=1, bits=4, group=64, out=0, stream=0)
    a.update(kw)
    return [ctypes.c_void_p(a["x"]), ctypes.c_void_p(a["w"]), ctypes.c_void_p(a["s"]),
            ctypes.c_void_p(a["b"]), ctypes.c_void_p(a["tok"]), ctypes.c_void_p(a["idx"]),
            ctypes.c_void_p(a["y"]), a["B"], a["N"], a["K"], a["E"], a["T"], a["bits"],
            a["group"], a["out"], ctypes.c_void_p(a["stream"])]


GQMV_CASES = [
    (dict(bits=2, group=32), bm.BITMM_ERR_UNSUPPORTED),  # 2 bits: groups of 64 and 128
    (dict(bits=1), bm.BITMM_ERR_UNSUPPORTED),
    (dict(bits=16), bm.BITMM_ERR_UNSUPPORTED),
    (dict(group=256), bm.BITMM_ERR_UNSUPPORTED),
    (dict(out=7), bm.BITMM_ERR_UNSUPPORTED),
    (dict(K=704, group=128), bm.BITMM_ERR_SHAPE),
    (dict(E=0), bm.BITMM_ERR_SHAPE),
    (dict(K=0), bm.BITMM_ERR_SHAPE),
    (dict(K=96), bm.BITMM_ERR_SHAPE),
    (dict(T=-1), bm.BITMM_ERR_SHAPE),
    (dict(B=-2), bm.BITMM_ERR_SHAPE),
    (dict(B=1 << 31), bm.BITMM_ERR_SHAPE),
    (dict(B=0), bm.BITMM_OK),
    (dict(N=0, idx=0), bm.BITMM_OK),
    (dict(idx=0), bm.BITMM_ERR_NULL),
    (dict(w=0), bm.BITMM_ERR_NULL),
    (dict(x=0), bm.BITMM_ERR_NULL),
    (dict(y=0), bm.BITMM_ERR_NULL),
    (dict(tok=A + 2), bm.BITMM_ERR_ALIGN),
    (dict(idx=A + 6), bm.BITMM_ERR_ALIGN),
    (dict(x=A + 8), bm.BITMM_ERR_ALIGN),
    (dict(y=A + 1), bm.BITMM_ERR_ALIGN),
    (dict(y=A + 2, out=1), bm.BITMM_ERR_ALIGN),
    (dict(), None),            # token index given
    (dict(tok=0), None),       # no token index: row r reads x row r
    (dict(x=0, T=0), None),    # no activation rows: every row is a zero row
]


@pytest.mark.parametrize("kw,expected", GQMV_CASES)
def test_gather_qmv_validation(L, kw, expected):
    if expected is None:
        if gpu_present():
            pytest.skip("fake pointers would reach a real device")
        expected = bm.BITMM_ERR_DEVICE
    assert L.bitmm_gather_qmv(*gqmv_args(**kw)) == expected


def gidx_args(**kw):
    a = dict(x=A, w=A + 0x1000, s=A + 0x2000, b=A + 0x3000, tok=A + 0x4000, idx=A + 0x5000,
             y=A + 0x6000, B=4584, N=704, K=2816, E=128, T=573, bits=4, group=64, out=0,
             ws=A + 0x7000, ws_bytes=1 << 20, stream=0)
    a.update(kw)
    return [ctypes.c_void_p(a["x"]), ctypes.c_void_p(a["w"]), ctypes.c_void_p(a["s"]),
            ctypes.c_void_p(a["b"]), ctypes.c_void_p(a["tok"]), ctypes.c_void_p(a["idx"]),
            ctypes.c_void_p(a["y"]), a["B"], a["N"], a["K"], a["E"], a["T"], a["bits"],
            a["group"], a["out"], ctypes.c_void_p(a["ws"]), a["ws_bytes"],
            ctypes.c_void_p(a["stream"])]


GIDX_CASES = [
    (dict(bits=3), bm.BITMM_ERR_UNSUPPORTED),
    (dict(bits=2, group=32), bm.BITMM_ERR_UNSUPPORTED),
    (dict(bits=2), None),
    (dict(group=16), bm.BITMM_ERR_UNSUPPORTED),
    (dict(out=2), bm.BITMM_ERR_UNSUPPORTED),
    (dict(E=8193), bm.BITMM_ERR_UNSUPPORTED),
    (dict(T=1 << 20, K=1024), bm.BITMM_ERR_UNSUPPORTED),
    (dict(E=0), bm.BITMM_ERR_SHAPE),
    (dict(K=100), bm.BITMM_ERR_SHAPE),
    (dict(T=-1), bm.BITMM_ERR_SHAPE),
    (dict(B=-1), bm.BITMM_ERR_SHAPE),
    (dict(B=0), bm.BITMM_OK),
    (dict(N=0), bm.BITMM_OK),
    (dict(idx=0), bm.BITMM_ERR_NULL),
    (dict(y=0), bm.BITMM_ERR_NULL),
    (dict(ws=0), bm.BITMM_ERR_WORKSPACE),
    (dict(ws_bytes=4 * (4584 + 130) - 1), bm.BITMM_ERR_WORKSPACE),
    (dict(ws=A + 4), bm.BITMM_ERR_ALIGN),
    (dict(tok=A + 1), bm.BITMM_ERR_ALIGN),
    (dict(w=A + 4), bm.BITMM_ERR_ALIGN),
    (dict(), None),
    (dict(tok=0, T=4584), None),
]


@pytest.mark.parametrize("kw,expected", GIDX_CASES)
def test_gather_qmm_indexed_validation(L, kw, expected):
    if expected is None:
        if gpu_present():
            pytest.skip("fake pointers would reach a real device")
        expected = bm.BITMM_ERR_DEVICE
    assert L.bitmm_gather_qmm_indexed(*gidx_args(**kw)) == expected


def gmm_args(**kw):
    a = dict(x=A, w=A + 0x1000, tok=A + 0x4000, idx=A + 0x5000, y=A + 0x6000, B=4584, N=704,
             K=2816, E=128, T=573, dtype=0, layout=0, out=0, ws=A + 0x7000, ws_bytes=1 << 20,
             stream=0)
    a.update(kw)
    return [ctypes.c_void_p(a["x"]), ctypes.c_void_p(a["w"]), ctypes.c_void_p(a["tok"]),
            ctypes.c_void_p(a["idx"]), ctypes.c_void_p(a["y"]), a["B"], a["N"], a["K"], a["E"],
            a["T"], a["dtype"], a["layout"], a["out"], ctypes.c_void_p(a["ws"]), a["ws_bytes"],
            ctypes.c_void_p(a["stream"])]


GMM_CASES = [
    (dict(dtype=2), bm.BITMM_ERR_UNSUPPORTED),
    (dict(dtype=-1), bm.BITMM_ERR_UNSUPPORTED),
    (dict(layout=2), bm.BITMM_ERR_UNSUPPORTED),
    (dict(out=3), bm.BITMM_ERR_UNSUPPORTED),
    (dict(K=100), bm.BITMM_ERR_UNSUPPORTED),              # K a multiple of 16
    (dict(layout=1, N=700), bm.BITMM_ERR_UNSUPPORTED),    # [K, N] rows of 16-byte chunks
    (dict(layout=0, N=700), None),                         # [N, K]: any N
    (dict(E=8193), bm.BITMM_ERR_UNSUPPORTED),
    (dict(T=1 << 20, K=1024), bm.BITMM_ERR_UNSUPPORTED),  # activation offsets are 32-bit
    (dict(N=1 << 17, K=1 << 14), bm.BITMM_ERR_UNSUPPORTED),  # one expert's W over 2 GiB
    (dict(E=0), bm.BITMM_ERR_SHAPE),
    (dict(K=0), bm.BITMM_ERR_SHAPE),
    (dict(T=-1), bm.BITMM_ERR_SHAPE),
    (dict(B=-1), bm.BITMM_ERR_SHAPE),
    (dict(N=-1), bm.BITMM_ERR_SHAPE),
    (dict(B=0), bm.BITMM_OK),
    (dict(N=0, layout=1), bm.BITMM_OK),
    (dict(idx=0), bm.BITMM_ERR_NULL),
    (dict(w=0), bm.BITMM_ERR_NULL),
    (dict(y=0), bm.BITMM_ERR_NULL),
    (dict(x=0), bm.BITMM_ERR_NULL),
    (dict(x=0, T=0, tok=0, B=4), None),                  # no activation rows: x unused
    (dict(ws=0), bm.BITMM_ERR_WORKSPACE),
    (dict(ws_bytes=4 * (4584 + 130) - 1), bm.BITMM_ERR_WORKSPACE),
    (dict(ws=A + 4), bm.BITMM_ERR_ALIGN),
    (dict(tok=A + 1), bm.BITMM_ERR_ALIGN),
    (dict(w=A + 8), bm.BITMM_ERR_ALIGN),
    (dict(x=A + 8), bm.BITMM_ERR_ALIGN),
    (dict(y=A + 2, out=1), bm.BITMM_ERR_ALIGN),
    (dict(y=A + 2, out=2), None),
    (dict(dtype=1, layout=1, out=2), None),
    (dict(), None),
    (dict(tok=0, T=4584), None),
]


@pytest.mark.parametrize("kw,expected", GMM_CASES)
def test_gather_mm_validation(L, kw, expected):
    if expected is None:
        if gpu_present():
            pytest.skip("fake pointers would reach a real device")
        expected = bm.BITMM_ERR_DEVICE
    assert L.bitmm_gather_mm(*gmm_args(**kw)) == expected


def test_gather_mm_workspace_size(L):
    ws = bm.bitmm_gather_mm_workspace_bytes
    assert ws(4584, 704, 128) >= 4 * (4584 + 128 + 2)
    assert ws(4584, 704, 128) % 256 == 0
    assert ws(-1, 1, 1) == 0 and ws(1, 1, 0) == 0
    need = ws(4584, 704, 128)
    if not gpu_present():
        assert L.bitmm_gather_mm(*gmm_args(ws_bytes=need)) == bm.BITMM_ERR_DEVICE
    assert L.bitmm_gather_mm(*gmm_args(ws_bytes=need - 1)) == bm.BITMM_ERR_WORKSPACE


def test_indexed_workspace_size(L):
    ws = bm.bitmm_gather_qmm_indexed_workspace_bytes
    assert ws(4584, 704, 128) >= 4 * (4584 + 128 + 2)
    assert ws(4584, 704, 128) % 256 == 0
    assert ws(0, 1, 1) > 0
    assert ws(-1, 1, 1) == 0 and ws(1, 1, 0) == 0


def test_workspace_size(L):
    ws = bm.bitmm_gather_qmm_workspace_bytes
    assert ws(4584, 704, 128) >= 4 * (128 + 2)
    assert ws(4584, 704, 128) % 256 == 0
    assert ws(1, 1, 1) >= 12
    assert ws(0, 0, 1) > 0
    assert ws(-1, 1, 1) == 0
    assert ws(1, 1, 0) == 0
    # exactly the documented minimum is accepted by validation
    need = ws(4584, 704, 128)
    if not gpu_present():
        assert L.bitmm_gather_qmm(*gather_args(ws_bytes=need)) == bm.BITMM_ERR_DEVICE
    assert L.bitmm_gather_qmm(*gather_args(ws_bytes=need - 1)) == bm.BITMM_ERR_WORKSPACE


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library the binding raises instead of falling back."""
    monkeypatch.setattr(bm, "_lib", None)
    monkeypatch.setattr(bm, "LIB_PATH", str(tmp_path / "libbitmm.so"))
    with pytest.raises(RuntimeError, match="missing"):
        bm.lib()
