"""Python access to the CPU oracle (``oracle.c``): test infrastructure only.

It covers the affine group-wise quantized products (qmm, gather_qmm and the indexed
gather) and the dense grouped product gather_mm.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` use this package. The library under ``bit_matmul_amd`` never
imports it, and it never imports the library.

Arrays are numpy: bf16 tensors as uint16 bit patterns, packed codes as uint32,
expert ids as int32. Results are float64.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

# Plain C, no fast-math, no FMA contraction: every operation is the one written.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(force: bool = True, src: str = SRC_PATH, out: str = LIB_PATH) -> str:
    """Compile the oracle with gcc (also run by ``__graft_entry__.build``)."""
    if force or not os.path.exists(out):
        tmp = out + f".tmp{os.getpid()}"
        subprocess.run(["gcc", *CFLAGS, "-I", _HERE, src, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, out)
    return out


class Oracle:
    """ctypes view of one compiled oracle library (the default one, or a test build)."""

    def __init__(self, path: str = LIB_PATH):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_f64_to_bf16_rne.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_bf16_rne.restype = ctypes.c_uint16
        lib.oracle_f64_to_bf16_array.argtypes = [P, P, I64]
        lib.oracle_f64_to_bf16_array.restype = None
        lib.oracle_code.argtypes = [P, I64, I]
        lib.oracle_code.restype = ctypes.c_uint32
        lib.oracle_weight.argtypes = [P, P, P, I64, I, I]
        lib.oracle_weight.restype = ctypes.c_double
        lib.oracle_default_threads.argtypes = []
        lib.oracle_default_threads.restype = I
        lib.oracle_qmm.argtypes = [P, P, P, P, I64, I64, I64, I, I, P, I]
        lib.oracle_qmm.restype = I
        lib.oracle_qmm_points.argtypes = [P, P, P, P, I64, I64, I64, I, I, P, P, I64, P, I]
        lib.oracle_qmm_points.restype = I
        lib.oracle_gather_qmm.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I, I, P, I]
        lib.oracle_gather_qmm.restype = I
        lib.oracle_gather_qmm_points.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I, I,
                                                 P, P, I64, P, I]
        lib.oracle_gather_qmm_points.restype = I
        lib.oracle_gather_qmm_indexed.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I64, I, I,
                                                  P, I]
        lib.oracle_gather_qmm_indexed.restype = I
        lib.oracle_gather_qmm_indexed_points.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64,
                                                         I64, I, I, P, P, I64, P, I]
        lib.oracle_gather_qmm_indexed_points.restype = I
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_f64_to_f16_rne.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_f16_rne.restype = ctypes.c_uint16
        lib.oracle_f64_to_f16_array.argtypes = [P, P, I64]
        lib.oracle_f64_to_f16_array.restype = None
        lib.oracle_f16_to_f64_array.argtypes = [P, P, I64]
        lib.oracle_f16_to_f64_array.restype = None
        lib.oracle_gather_mm.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, I, I, P, I]
        lib.oracle_gather_mm.restype = I
        lib.oracle_gather_mm_points.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, I, I, P, P,
                                                I64, P, I]
        lib.oracle_gather_mm_points.restype = I
        self.lib = lib
        self.path = path

    def default_threads(self) -> int:
        return int(self.lib.oracle_default_threads())

    def bf16_to_f64(self, h: int) -> float:
        return float(self.lib.oracle_bf16_to_f64(int(h)))

    def f64_to_bf16(self, v) -> np.ndarray:
        """Round doubles to bf16 bit patterns (nearest, ties to even)."""
        v, pv = _c(v, np.float64)
        out = np.empty(v.shape, dtype=np.uint16)
        self.lib.oracle_f64_to_bf16_array(pv, out.ctypes.data_as(ctypes.c_void_p), v.size)
        return out

    def f16_to_f64(self, h) -> np.ndarray:
        """Widen binary16 bit patterns to float64 (exact)."""
        h, ph = _c(h, np.uint16)
        out = np.empty(h.shape, dtype=np.float64)
        self.lib.oracle_f16_to_f64_array(ph, out.ctypes.data_as(ctypes.c_void_p), h.size)
        return out

    def f64_to_f16(self, v) -> np.ndarray:
        """Round doubles to binary16 bit patterns (nearest, ties to even)."""
        v, pv = _c(v, np.float64)
        out = np.empty(v.shape, dtype=np.uint16)
        self.lib.oracle_f64_to_f16_array(pv, out.ctypes.data_as(ctypes.c_void_p), v.size)
        return out

    def gather_mm(self, x, w, token_idx, expert_idx, dtype: str = "bf16", layout: str = "nk",
                  threads: int = 0, rows=None, cols=None) -> np.ndarray:
        """Dense grouped product, y[B,N] (float64) or y at the points (rows[i], cols[i]):
        row r reads x row token_idx[r] (row r when token_idx is None) and the weights of
        expert expert_idx[r]; w is [E, N, K] (layout "nk") or [E, K, N] ("kn"); x and w
        are bf16 or binary16 ("f16") bit patterns."""
        x, px = _c(x, np.uint16)
        w, pw = _c(w, np.uint16)
        e, pe = _c(expert_idx, np.int32)
        dt = {"bf16": 0, "f16": 1}[dtype]
        lay = {"nk": 0, "kn": 1}[layout]
        T, K = x.shape
        E = w.shape[0]
        N = w.shape[1] if lay == 0 else w.shape[2]
        B = e.shape[0]
        if w.shape != ((E, N, K) if lay == 0 else (E, K, N)) or e.ndim != 1:
            raise ValueError("oracle.gather_mm: inconsistent shapes")
        if token_idx is None:
            pt = None
            if T != B:
                raise ValueError("oracle.gather_mm: x rows must equal B without token_idx")
        else:
            t, pt = _c(token_idx, np.int32)
            if t.shape != (B,):
                raise ValueError("oracle.gather_mm: token_idx shape")
        if rows is None:
            y = np.empty((B, N), dtype=np.float64)
            _check(self.lib.oracle_gather_mm(px, pw, pt, pe, B, N, K, E, T, dt, lay,
                                             y.ctypes.data_as(ctypes.c_void_p), int(threads)))
            return y
        r, pr = _c(rows, np.int64)
        c, pc = _c(cols, np.int64)
        if r.shape != c.shape:
            raise ValueError("oracle.gather_mm: rows and cols differ in shape")
        y = np.empty(r.shape, dtype=np.float64)
        _check(self.lib.oracle_gather_mm_points(px, pw, pt, pe, B, N, K, E, T, dt, lay, pr, pc,
                                                r.size, y.ctypes.data_as(ctypes.c_void_p),
                                                int(threads)))
        return y

    def code(self, row_words, k: int, bits: int) -> int:
        w, pw = _c(row_words, np.uint32)
        return int(self.lib.oracle_code(pw, int(k), int(bits)))

    def weight(self, row_words, row_scales, row_biases, k: int, bits: int,
               group: int = 64) -> float:
        w, pw = _c(row_words, np.uint32)
        s, ps = _c(row_scales, np.uint16)
        b, pb = _c(row_biases, np.uint16)
        return float(self.lib.oracle_weight(pw, ps, pb, int(k), int(bits), int(group)))

    def qmm(self, x, w, scales, biases, bits: int, group: int = 64,
            threads: int = 0) -> np.ndarray:
        """y[M,N] (float64) = x[M,K] . dequant(w)^T."""
        x, px = _c(x, np.uint16)
        w, pw = _c(w, np.uint32)
        s, ps = _c(scales, np.uint16)
        b, pb = _c(biases, np.uint16)
        M, K = x.shape
        N = w.shape[0]
        if w.shape != (N, K * bits // 32) or s.shape != (N, K // group) or b.shape != s.shape:
            raise ValueError("oracle.qmm: inconsistent shapes")
        y = np.empty((M, N), dtype=np.float64)
        _check(self.lib.oracle_qmm(px, pw, ps, pb, M, N, K, bits, group,
                                   y.ctypes.data_as(ctypes.c_void_p), int(threads)))
        return y

    def qmm_points(self, x, w, scales, biases, rows, cols, bits: int, group: int = 64,
                   threads: int = 0) -> np.ndarray:
        """The outputs (rows[i], cols[i]) of qmm, computed one by one."""
        x, px = _c(x, np.uint16)
        w, pw = _c(w, np.uint32)
        s, ps = _c(scales, np.uint16)
        b, pb = _c(biases, np.uint16)
        r, pr = _c(rows, np.int64)
        c, pc = _c(cols, np.int64)
        M, K = x.shape
        N = w.shape[0]
        if w.shape != (N, K * bits // 32) or s.shape != (N, K // group) or r.shape != c.shape:
            raise ValueError("oracle.qmm_points: inconsistent shapes")
        y = np.empty(r.shape, dtype=np.float64)
        _check(self.lib.oracle_qmm_points(px, pw, ps, pb, M, N, K, bits, group, pr, pc, r.size,
                                          y.ctypes.data_as(ctypes.c_void_p), int(threads)))
        return y

    def gather_qmm(self, x, w, scales, biases, expert_idx, bits: int, group: int = 64,
                   threads: int = 0) -> np.ndarray:
        """y[B,N] (float64): row r uses expert expert_idx[r]."""
        x, px = _c(x, np.uint16)
        w, pw = _c(w, np.uint32)
        s, ps = _c(scales, np.uint16)
        b, pb = _c(biases, np.uint16)
        e, pe = _c(expert_idx, np.int32)
        B, K = x.shape
        E, N = w.shape[0], w.shape[1]
        if (w.shape != (E, N, K * bits // 32) or s.shape != (E, N, K // group)
                or b.shape != s.shape or e.shape != (B,)):
            raise ValueError("oracle.gather_qmm: inconsistent shapes")
        y = np.empty((B, N), dtype=np.float64)
        _check(self.lib.oracle_gather_qmm(px, pw, ps, pb, pe, B, N, K, E, bits, group,
                                          y.ctypes.data_as(ctypes.c_void_p), int(threads)))
        return y

    def gather_qmm_points(self, x, w, scales, biases, expert_idx, rows, cols, bits: int,
                          group: int = 64, threads: int = 0) -> np.ndarray:
        x, px = _c(x, np.uint16)
        w, pw = _c(w, np.uint32)
        s, ps = _c(scales, np.uint16)
        b, pb = _c(biases, np.uint16)
        e, pe = _c(expert_idx, np.int32)
        r, pr = _c(rows, np.int64)
        c, pc = _c(cols, np.int64)
        B, K = x.shape
        E, N = w.shape[0], w.shape[1]
        if (w.shape != (E, N, K * bits // 32) or s.shape != (E, N, K // group)
                or e.shape != (B,) or r.shape != c.shape):
            raise ValueError("oracle.gather_qmm_points: inconsistent shapes")
        y = np.empty(r.shape, dtype=np.float64)
        _check(self.lib.oracle_gather_qmm_points(px, pw, ps, pb, pe, B, N, K, E, bits, group,
                                                 pr, pc, r.size,
                                                 y.ctypes.data_as(ctypes.c_void_p),
                                                 int(threads)))
        return y

    def gather_qmm_indexed(self, x, w, scales, biases, token_idx, expert_idx, bits: int,
                           group: int = 64, threads: int = 0, rows=None, cols=None) -> np.ndarray:
        """y[B,N] (float64), or y at the points (rows[i], cols[i]): row r reads x row
        token_idx[r] (row r when token_idx is None) and expert expert_idx[r]."""
        x, px = _c(x, np.uint16)
        w, pw = _c(w, np.uint32)
        s, ps = _c(scales, np.uint16)
        b, pb = _c(biases, np.uint16)
        e, pe = _c(expert_idx, np.int32)
        T, K = x.shape
        E, N = w.shape[0], w.shape[1]
        B = e.shape[0]
        if token_idx is None:
            pt = None
            if T != B:
                raise ValueError("oracle.gather_qmm_indexed: x rows must equal B without token_idx")
        else:
            t, pt = _c(token_idx, np.int32)
            if t.shape != (B,):
                raise ValueError("oracle.gather_qmm_indexed: token_idx shape")
        if (w.shape != (E, N, K * bits // 32) or s.shape != (E, N, K // group)
                or b.shape != s.shape or e.ndim != 1):
            raise ValueError("oracle.gather_qmm_indexed: inconsistent shapes")
        if rows is None:
            y = np.empty((B, N), dtype=np.float64)
            _check(self.lib.oracle_gather_qmm_indexed(px, pw, ps, pb, pt, pe, B, N, K, E, T, bits,
                                                      group, y.ctypes.data_as(ctypes.c_void_p),
                                                      int(threads)))
            return y
        r, pr = _c(rows, np.int64)
        c, pc = _c(cols, np.int64)
        if r.shape != c.shape:
            raise ValueError("oracle.gather_qmm_indexed: rows and cols differ in shape")
        y = np.empty(r.shape, dtype=np.float64)
        _check(self.lib.oracle_gather_qmm_indexed_points(px, pw, ps, pb, pt, pe, B, N, K, E, T,
                                                         bits, group, pr, pc, r.size,
                                                         y.ctypes.data_as(ctypes.c_void_p),
                                                         int(threads)))
        return y


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _check(rc):
    if rc < 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return rc


_default = None


def get() -> Oracle:
    """The oracle built from ``oracle.c`` (compiled on first use if missing or stale)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
            build(force=True)
        _default = Oracle(LIB_PATH)
    return _default


def default_threads() -> int:
    return get().default_threads()


def bf16_to_f64(h):
    return get().bf16_to_f64(h)


def f64_to_bf16(v):
    return get().f64_to_bf16(v)


def code(row_words, k, bits):
    return get().code(row_words, k, bits)


def f16_to_f64(h):
    return get().f16_to_f64(h)


def f64_to_f16(v):
    return get().f64_to_f16(v)


def gather_mm(x, w, token_idx, expert_idx, dtype="bf16", layout="nk", threads=0, rows=None,
              cols=None):
    return get().gather_mm(x, w, token_idx, expert_idx, dtype, layout, threads, rows, cols)


def weight(row_words, row_scales, row_biases, k, bits, group=64):
    return get().weight(row_words, row_scales, row_biases, k, bits, group)


def qmm(x, w, scales, biases, bits, group=64, threads=0):
    return get().qmm(x, w, scales, biases, bits, group, threads)


def qmm_points(x, w, scales, biases, rows, cols, bits, group=64, threads=0):
    return get().qmm_points(x, w, scales, biases, rows, cols, bits, group, threads)


def gather_qmm(x, w, scales, biases, expert_idx, bits, group=64, threads=0):
    return get().gather_qmm(x, w, scales, biases, expert_idx, bits, group, threads)


def gather_qmm_indexed(x, w, scales, biases, token_idx, expert_idx, bits, group=64, threads=0,
                       rows=None, cols=None):
    return get().gather_qmm_indexed(x, w, scales, biases, token_idx, expert_idx, bits, group,
                                    threads, rows, cols)


def gather_qmm_points(x, w, scales, biases, expert_idx, rows, cols, bits, group=64, threads=0):
    return get().gather_qmm_points(x, w, scales, biases, expert_idx, rows, cols, bits, group,
                                   threads)
