"""Shared helpers for the GPU tests: move seeded inputs to the device, call the
library through its binding, and compare with the oracle under the tolerances
the workload states:

    bf16 output:  |y - y_ref| <= 1e-2 * max|y_ref| + 1e-3
    f32 output:   |y - y_ref| <= 1e-4 * max|y_ref|    (paths that keep w exact)

max|y_ref| is taken over the whole output of the call, or over the sampled
outputs when only a sample is computed (never larger, so never looser).
"""

from __future__ import annotations

import numpy as np

import bit_matmul_amd as bm
from bit_matmul_amd import inputs as I


def torch():
    import torch as t
    return t


def dev():
    return torch().device("cuda:0")


def bf16_tensor(a_u16):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).view(t.bfloat16).to(dev())


def f16_tensor(a_u16):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).view(t.float16).to(dev())


def half_tensor(a_u16, dtype):
    """bf16 ("bf16") or binary16 ("f16") bit patterns as a device tensor of that type."""
    return bf16_tensor(a_u16) if dtype == "bf16" else f16_tensor(a_u16)


def u32_tensor(a_u32):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a_u32).view(np.int32)).to(dev())


def i32_tensor(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def dense_to_dev(d):
    return (bf16_tensor(d.x), u32_tensor(d.w), bf16_tensor(d.scales), bf16_tensor(d.biases))


def gather_to_dev(g, idx=None):
    return (bf16_tensor(g.x), u32_tensor(g.w), bf16_tensor(g.scales), bf16_tensor(g.biases),
            i32_tensor(g.expert_idx if idx is None else idx))


def to_f64(y):
    t = torch()
    if y.dtype == t.bfloat16:
        return I.bf16_bits_to_f64(y.view(t.int16).cpu().numpy().view(np.uint16))
    return y.double().cpu().numpy()


def run_dense(fn_name, d, out="bf16", stream=None):
    t = torch()
    x, w, s, b = dense_to_dev(d)
    y = t.empty((d.M, d.N), dtype=t.bfloat16 if out == "bf16" else t.float32, device=dev())
    getattr(bm, fn_name)(x, w, s, b, y, d.bits, group_size=getattr(d, "group", 64), stream=stream)
    return y


def run_gather(g, out="bf16", idx=None):
    t = torch()
    x, w, s, b, e = gather_to_dev(g, idx)
    y = t.empty((g.B, g.N), dtype=t.bfloat16 if out == "bf16" else t.float32, device=dev())
    ws = t.empty(bm.bitmm_gather_qmm_workspace_bytes(g.B, g.N, g.E), dtype=t.uint8, device=dev())
    bm.bitmm_gather_qmm(x, w, s, b, e, y, ws, g.bits, group_size=getattr(g, "group", 64))
    return y, ws


def tolerance(ref, out):
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    return 1e-2 * scale + 1e-3 if out == "bf16" else 1e-4 * scale


def assert_close(got, ref, out, what=""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    tol = tolerance(ref, out)
    worst = int(np.argmax(err)) if err.size else 0
    assert err.size == 0 or err.flat[worst] <= tol, (
        f"{what}: max error {err.flat[worst]:.3e} > tol {tol:.3e} at flat index {worst} "
        f"(got {got.flat[worst]!r}, ref {ref.flat[worst]!r})")
    return float(err.max()) if err.size else 0.0


def sample_points(rows, cols, count, seed=0):
    """Random outputs plus the four corners and the last row/column."""
    rng = np.random.default_rng(seed)
    r = rng.integers(0, rows, count)
    c = rng.integers(0, cols, count)
    extra_r = np.array([0, 0, rows - 1, rows - 1] + [rows - 1] * 8 + list(range(min(rows, 8))))
    extra_c = np.array([0, cols - 1, 0, cols - 1] + list(rng.integers(0, cols, 8)) + [cols - 1] * min(rows, 8))
    return np.concatenate([r, extra_r]).astype(np.int64), np.concatenate([c, extra_c]).astype(np.int64)
