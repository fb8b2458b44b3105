"""bitmm: affine group-wise quantized matmul for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libbitmm.so`` (C ABI in ``include/bitmm.h``). The
functions carry the C names and only marshal arguments: they check that the torch
tensors match the shapes, dtypes and device the C call expects, pass raw device
pointers and the current HIP stream, and turn a non-OK status into ``BitmmError``.
Every step of the computation runs in the library's HIP kernels; there is no
fallback path. PyTorch is used only for device memory and streams.

Tensor conventions (all contiguous, on the GPU):
    x        torch.bfloat16 [M, K]
    w        torch.int32 (bit pattern of uint32 words) [N, K*bits/32] or [E, N, K*bits/32]
    scales   torch.bfloat16 [N, K/64] or [E, N, K/64]
    biases   same as scales
    y        torch.bfloat16 or torch.float32 [M, N]
    expert_idx  torch.int32 [B]
    workspace   torch.uint8 [>= bitmm_gather_qmm_workspace_bytes(B, N, E)]
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbitmm.so")

BITMM_OK = 0
BITMM_ERR_NULL = 1
BITMM_ERR_SHAPE = 2
BITMM_ERR_UNSUPPORTED = 3
BITMM_ERR_ALIGN = 4
BITMM_ERR_WORKSPACE = 5
BITMM_ERR_DEVICE = 6
BITMM_ERR_LAUNCH = 7

BITMM_OUT_BF16 = 0
BITMM_OUT_F32 = 1
BITMM_OUT_F16 = 2

BITMM_DTYPE_BF16 = 0
BITMM_DTYPE_F16 = 1

BITMM_LAYOUT_NK = 0
BITMM_LAYOUT_KN = 1

GROUP = 64

__all__ = [
    "BitmmError", "lib", "bitmm_abi_version", "bitmm_status_string", "bitmm_last_launches",
    "bitmm_qmv", "bitmm_qmm",
    "bitmm_gather_qmm_workspace_bytes", "bitmm_gather_qmm", "bitmm_gather_qmm_noalloc", "bitmm_gather_qmv",
    "bitmm_gather_qmm_indexed_workspace_bytes", "bitmm_gather_qmm_indexed", "qmv", "qmm",
    "gather_qmm", "gather_qmv", "gather_qmm_indexed", "bitmm_gather_mm_workspace_bytes",
    "bitmm_gather_mm", "gather_mm",
]


class BitmmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {bitmm_status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libbitmm.so. Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m bit_matmul_amd.build` "
                "(bitmm has no CPU or framework fallback)")
        try:  # share torch's HIP runtime (same soname) when torch is present
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        L.bitmm_abi_version.argtypes = []
        L.bitmm_abi_version.restype = I
        L.bitmm_status_string.argtypes = [I]
        L.bitmm_status_string.restype = ctypes.c_char_p
        L.bitmm_last_launches.argtypes = [ctypes.c_char_p, SZ]
        L.bitmm_last_launches.restype = SZ
        dense = [P, P, P, P, P, I64, I64, I64, I, I, I, P]
        L.bitmm_qmv.argtypes = dense
        L.bitmm_qmv.restype = I
        L.bitmm_qmm.argtypes = dense
        L.bitmm_qmm.restype = I
        L.bitmm_gather_qmm_workspace_bytes.argtypes = [I64, I64, I64]
        L.bitmm_gather_qmm_workspace_bytes.restype = SZ
        L.bitmm_gather_qmm.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I, I, I, P, SZ, P]
        L.bitmm_gather_qmm.restype = I
        L.bitmm_gather_qmm_noalloc.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I, I, I, P, P]
        L.bitmm_gather_qmm_noalloc.restype = I
        L.bitmm_gather_qmv.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I, I, I, P]
        L.bitmm_gather_qmv.restype = I
        L.bitmm_gather_qmm_indexed_workspace_bytes.argtypes = [I64, I64, I64]
        L.bitmm_gather_qmm_indexed_workspace_bytes.restype = SZ
        L.bitmm_gather_qmm_indexed.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I, I,
                                               I, P, SZ, P]
        L.bitmm_gather_qmm_indexed.restype = I
        L.bitmm_gather_mm_workspace_bytes.argtypes = [I64, I64, I64]
        L.bitmm_gather_mm_workspace_bytes.restype = SZ
        L.bitmm_gather_mm.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, I, I, I, P, SZ, P]
        L.bitmm_gather_mm.restype = I
        _lib = L
    return _lib


def bitmm_abi_version() -> int:
    return int(lib().bitmm_abi_version())


def bitmm_status_string(status: int) -> str:
    return lib().bitmm_status_string(int(status)).decode()


def bitmm_last_launches() -> list:
    """The kernels this thread's most recent bitmm_* call enqueued, one string each."""
    n = int(lib().bitmm_last_launches(None, 0))
    buf = ctypes.create_string_buffer(n + 1)
    lib().bitmm_last_launches(buf, n + 1)
    return [line for line in buf.value.decode().split("\n") if line]


def bitmm_gather_qmm_workspace_bytes(B: int, N: int, E: int) -> int:
    return int(lib().bitmm_gather_qmm_workspace_bytes(int(B), int(N), int(E)))


def bitmm_gather_qmm_indexed_workspace_bytes(B: int, N: int, E: int) -> int:
    return int(lib().bitmm_gather_qmm_indexed_workspace_bytes(int(B), int(N), int(E)))


# ---------------------------------------------------------------------------
# Marshalling helpers
# ---------------------------------------------------------------------------

def bitmm_gather_mm_workspace_bytes(B: int, N: int, E: int) -> int:
    return int(lib().bitmm_gather_mm_workspace_bytes(int(B), int(N), int(E)))


def _torch():
    import torch
    return torch


def _stream_ptr(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def _expect(t, name, dtype, shape, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _out_code(y):
    torch = _torch()
    if y.dtype == torch.bfloat16:
        return BITMM_OUT_BF16
    if y.dtype == torch.float32:
        return BITMM_OUT_F32
    raise TypeError(f"y must be bfloat16 or float32, got {y.dtype}")


def _out_code_any(y):
    """bitmm_out code of y for bitmm_gather_mm (bf16, f32 or float16)."""
    torch = _torch()
    if y.dtype == torch.float16:
        return BITMM_OUT_F16
    return _out_code(y)


def _dense(fn, where, x, w, scales, biases, y, bits, group_size, stream):
    torch = _torch()
    M, K = x.shape
    N = w.shape[0]
    dev = x.device
    _expect(x, "x", torch.bfloat16, (M, K), dev)
    if K % group_size:
        raise ValueError(f"K={K} is not a multiple of group_size={group_size}")
    _expect(w, "w", torch.int32, (N, K * bits // 32), dev)
    _expect(scales, "scales", torch.bfloat16, (N, K // group_size), dev)
    _expect(biases, "biases", torch.bfloat16, (N, K // group_size), dev)
    _expect(y, "y", y.dtype, (M, N), dev)
    st = fn(_ptr(x), _ptr(w), _ptr(scales), _ptr(biases), _ptr(y), M, N, K, int(bits),
            int(group_size), _out_code(y), _stream_ptr(stream, dev))
    if st != BITMM_OK:
        raise BitmmError(st, where)
    return y


# ---------------------------------------------------------------------------
# The C entry points
# ---------------------------------------------------------------------------

def bitmm_qmv(x, w, scales, biases, y, bits: int, group_size: int = GROUP, stream=None):
    """y[M, N] = x[M, K] * dequant(w)^T with the GEMV kernel (decode)."""
    return _dense(lib().bitmm_qmv, "bitmm_qmv", x, w, scales, biases, y, bits, group_size, stream)


def bitmm_qmm(x, w, scales, biases, y, bits: int, group_size: int = GROUP, stream=None):
    """y[M, N] = x[M, K] * dequant(w)^T; M < 8 -> GEMV kernel, else matrix-core GEMM."""
    return _dense(lib().bitmm_qmm, "bitmm_qmm", x, w, scales, biases, y, bits, group_size, stream)


def bitmm_gather_qmm(x, w, scales, biases, expert_idx, y, workspace, bits: int,
                     group_size: int = GROUP, stream=None):
    """y[r, :] = x[r, :] * dequant(w[expert_idx[r]])^T, rows sorted by expert."""
    torch = _torch()
    B, K = x.shape
    E, N = w.shape[0], w.shape[1]
    dev = x.device
    _expect(x, "x", torch.bfloat16, (B, K), dev)
    if K % group_size:
        raise ValueError(f"K={K} is not a multiple of group_size={group_size}")
    _expect(w, "w", torch.int32, (E, N, K * bits // 32), dev)
    _expect(scales, "scales", torch.bfloat16, (E, N, K // group_size), dev)
    _expect(biases, "biases", torch.bfloat16, (E, N, K // group_size), dev)
    _expect(expert_idx, "expert_idx", torch.int32, (B,), dev)
    _expect(y, "y", y.dtype, (B, N), dev)
    if workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the same device")
    st = lib().bitmm_gather_qmm(_ptr(x), _ptr(w), _ptr(scales), _ptr(biases), _ptr(expert_idx),
                                _ptr(y), B, N, K, E, int(bits), int(group_size), _out_code(y),
                                _ptr(workspace), workspace.numel(), _stream_ptr(stream, dev))
    if st != BITMM_OK:
        raise BitmmError(st, "bitmm_gather_qmm")
    return y


def bitmm_gather_qmm_noalloc(x, w, scales, biases, expert_idx, y, bits: int, group_size: int = GROUP,
                             status=None, stream=None):
    """bitmm_gather_qmm without a workspace: the library's static per-GPU workspace is
    used and nothing is allocated. `status` (optional int32 tensor of one element on the
    device) receives the precondition status word (0, or 1 + the first offending row)."""
    torch = _torch()
    B, K = x.shape
    E, N = w.shape[0], w.shape[1]
    dev = x.device
    _expect(x, "x", torch.bfloat16, (B, K), dev)
    if K % group_size:
        raise ValueError(f"K={K} is not a multiple of group_size={group_size}")
    _expect(w, "w", torch.int32, (E, N, K * bits // 32), dev)
    _expect(scales, "scales", torch.bfloat16, (E, N, K // group_size), dev)
    _expect(biases, "biases", torch.bfloat16, (E, N, K // group_size), dev)
    _expect(expert_idx, "expert_idx", torch.int32, (B,), dev)
    _expect(y, "y", y.dtype, (B, N), dev)
    if status is not None:
        _expect(status, "status", torch.int32, (1,), dev)
    st = lib().bitmm_gather_qmm_noalloc(_ptr(x), _ptr(w), _ptr(scales), _ptr(biases), _ptr(expert_idx),
                                        _ptr(y), B, N, K, E, int(bits), int(group_size), _out_code(y),
                                        None if status is None else _ptr(status), _stream_ptr(stream, dev))
    if st != BITMM_OK:
        raise BitmmError(st, "bitmm_gather_qmm_noalloc")
    return y


def bitmm_gather_qmm_indexed(x, w, scales, biases, token_idx, expert_idx, y, workspace, bits: int,
                             group_size: int = GROUP, stream=None):
    """y[r, :] = x[token_idx[r], :] * dequant(w[expert_idx[r]])^T (MoE prefill, rows in any
    order, token_idx may be None); out-of-range ids give zero rows (workspace word 0 flags
    the first)."""
    torch = _torch()
    T, K = x.shape
    E, N = w.shape[0], w.shape[1]
    B = expert_idx.shape[0]
    dev = x.device
    _expect(x, "x", torch.bfloat16, (T, K), dev)
    if K % group_size:
        raise ValueError(f"K={K} is not a multiple of group_size={group_size}")
    _expect(w, "w", torch.int32, (E, N, K * bits // 32), dev)
    _expect(scales, "scales", torch.bfloat16, (E, N, K // group_size), dev)
    _expect(biases, "biases", torch.bfloat16, (E, N, K // group_size), dev)
    _expect(expert_idx, "expert_idx", torch.int32, (B,), dev)
    if token_idx is not None:
        _expect(token_idx, "token_idx", torch.int32, (B,), dev)
    _expect(y, "y", y.dtype, (B, N), dev)
    if workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the same device")
    st = lib().bitmm_gather_qmm_indexed(_ptr(x), _ptr(w), _ptr(scales), _ptr(biases),
                                        _ptr(token_idx), _ptr(expert_idx), _ptr(y), B, N, K, E, T,
                                        int(bits), int(group_size), _out_code(y), _ptr(workspace),
                                        workspace.numel(), _stream_ptr(stream, dev))
    if st != BITMM_OK:
        raise BitmmError(st, "bitmm_gather_qmm_indexed")
    return y


def bitmm_gather_qmv(x, w, scales, biases, token_idx, expert_idx, y, bits: int,
                     group_size: int = GROUP, stream=None):
    """y[r, :] = x[token_idx[r], :] * dequant(w[expert_idx[r]])^T (MoE decode); token_idx
    may be None (row r reads x[r]); any order; out-of-range ids give zero rows."""
    torch = _torch()
    T, K = x.shape
    E, N = w.shape[0], w.shape[1]
    B = expert_idx.shape[0]
    dev = x.device
    _expect(x, "x", torch.bfloat16, (T, K), dev)
    if K % group_size:
        raise ValueError(f"K={K} is not a multiple of group_size={group_size}")
    _expect(w, "w", torch.int32, (E, N, K * bits // 32), dev)
    _expect(scales, "scales", torch.bfloat16, (E, N, K // group_size), dev)
    _expect(biases, "biases", torch.bfloat16, (E, N, K // group_size), dev)
    _expect(expert_idx, "expert_idx", torch.int32, (B,), dev)
    if token_idx is not None:
        _expect(token_idx, "token_idx", torch.int32, (B,), dev)
    _expect(y, "y", y.dtype, (B, N), dev)
    st = lib().bitmm_gather_qmv(_ptr(x), _ptr(w), _ptr(scales), _ptr(biases), _ptr(token_idx),
                                _ptr(expert_idx), _ptr(y), B, N, K, E, T, int(bits),
                                int(group_size), _out_code(y), _stream_ptr(stream, dev))
    if st != BITMM_OK:
        raise BitmmError(st, "bitmm_gather_qmv")
    return y


# ---------------------------------------------------------------------------
# Allocating conveniences (torch allocates the output; the kernels do the work)
# ---------------------------------------------------------------------------

def qmv(x, w, scales, biases, bits: int, out_dtype=None, stream=None):
    torch = _torch()
    y = torch.empty((x.shape[0], w.shape[0]), dtype=out_dtype or torch.bfloat16, device=x.device)
    return bitmm_qmv(x, w, scales, biases, y, bits, stream=stream)


def qmm(x, w, scales, biases, bits: int, out_dtype=None, stream=None):
    torch = _torch()
    y = torch.empty((x.shape[0], w.shape[0]), dtype=out_dtype or torch.bfloat16, device=x.device)
    return bitmm_qmm(x, w, scales, biases, y, bits, stream=stream)


def gather_qmm(x, w, scales, biases, expert_idx, bits: int, out_dtype=None, workspace=None,
               stream=None):
    """Returns (y, workspace); workspace word 0 is the precondition status."""
    torch = _torch()
    B, N, E = x.shape[0], w.shape[1], w.shape[0]
    y = torch.empty((B, N), dtype=out_dtype or torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(bitmm_gather_qmm_workspace_bytes(B, N, E), 256),
                                dtype=torch.uint8, device=x.device)
    bitmm_gather_qmm(x, w, scales, biases, expert_idx, y, workspace, bits, stream=stream)
    return y, workspace


def gather_qmv(x, w, scales, biases, token_idx, expert_idx, bits: int, out_dtype=None,
               stream=None):
    torch = _torch()
    y = torch.empty((expert_idx.shape[0], w.shape[1]), dtype=out_dtype or torch.bfloat16,
                    device=x.device)
    return bitmm_gather_qmv(x, w, scales, biases, token_idx, expert_idx, y, bits, stream=stream)


def gather_qmm_indexed(x, w, scales, biases, token_idx, expert_idx, bits: int, out_dtype=None,
                       workspace=None, stream=None):
    """Returns (y, workspace); workspace word 0 flags the first row with an out-of-range id."""
    torch = _torch()
    B, N, E = expert_idx.shape[0], w.shape[1], w.shape[0]
    y = torch.empty((B, N), dtype=out_dtype or torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(bitmm_gather_qmm_indexed_workspace_bytes(B, N, E), 256),
                                dtype=torch.uint8, device=x.device)
    bitmm_gather_qmm_indexed(x, w, scales, biases, token_idx, expert_idx, y, workspace, bits,
                             stream=stream)
    return y, workspace


def bitmm_gather_mm(x, w, token_idx, expert_idx, y, workspace, layout: str = "nk", stream=None):
    """Dense grouped product: y[r, :] = x[token_idx[r], :] * W[expert_idx[r]]^T (rows in any
    order, token_idx may be None). x and w are both bfloat16 or both float16; w is
    [E, N, K] (layout "nk") or [E, K, N] ("kn"); y is bfloat16, float16 or float32.
    Out-of-range ids give zero rows (workspace word 0 flags the first)."""
    torch = _torch()
    T, K = x.shape
    lay = {"nk": BITMM_LAYOUT_NK, "kn": BITMM_LAYOUT_KN}[layout]
    E = w.shape[0]
    N = w.shape[1] if lay == BITMM_LAYOUT_NK else w.shape[2]
    B = expert_idx.shape[0]
    dev = x.device
    if x.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"x must be bfloat16 or float16, got {x.dtype}")
    dt = BITMM_DTYPE_BF16 if x.dtype == torch.bfloat16 else BITMM_DTYPE_F16
    _expect(x, "x", x.dtype, (T, K), dev)
    _expect(w, "w", x.dtype, (E, N, K) if lay == BITMM_LAYOUT_NK else (E, K, N), dev)
    _expect(expert_idx, "expert_idx", torch.int32, (B,), dev)
    if token_idx is not None:
        _expect(token_idx, "token_idx", torch.int32, (B,), dev)
    _expect(y, "y", y.dtype, (B, N), dev)
    if workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the same device")
    st = lib().bitmm_gather_mm(_ptr(x), _ptr(w), _ptr(token_idx), _ptr(expert_idx), _ptr(y), B, N,
                               K, E, T, dt, lay, _out_code_any(y), _ptr(workspace),
                               workspace.numel(), _stream_ptr(stream, dev))
    if st != BITMM_OK:
        raise BitmmError(st, "bitmm_gather_mm")
    return y


def gather_mm(x, w, token_idx, expert_idx, layout: str = "nk", out_dtype=None, workspace=None,
              stream=None):
    """Returns (y, workspace); y has x's dtype unless out_dtype is given."""
    torch = _torch()
    B, E = expert_idx.shape[0], w.shape[0]
    N = w.shape[1] if layout == "nk" else w.shape[2]
    y = torch.empty((B, N), dtype=out_dtype or x.dtype, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(bitmm_gather_mm_workspace_bytes(B, N, E), 256),
                                dtype=torch.uint8, device=x.device)
    bitmm_gather_mm(x, w, token_idx, expert_idx, y, workspace, layout, stream=stream)
    return y, workspace
