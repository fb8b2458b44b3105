"""Seeded synthetic inputs for the affine group-quantized matmul.

This module only draws random tensors and lays them out in the storage
format the library consumes. It performs none of the matmul's arithmetic:
no unpacking, no dequantization, no accumulation. Both the HIP path and the
CPU oracle are fed from here, so neither side can influence what the other
one is checked on.

Storage format (the contract in ``include/bitmm.h``):

* bf16 tensors are ``uint16`` arrays holding the bf16 bit pattern.
* Packed codes are ``uint32`` words along K, LSB first: code ``j`` of a word
  occupies bits ``[bits*j, bits*(j+1))`` and word ``i`` of a row holds
  ``k = i*(32//bits) + j``.
* Scales and biases are bf16 ``[..., N, K // 64]``, one pair per group of 64
  consecutive K.

Workloads follow the shapes the pages measure (the mlxcel Volta pages: dense
hidden size 5120 with a 13824-wide projection; a MoE layer of 128 experts,
top-8 routing, expert dims 2816 / 704, 573 prompt tokens). Every draw uses
``numpy.random.default_rng(SeedSequence([seed, tag, ...]))`` with a separate
stream per tensor:

    tag 1 = activations, 2 = codes, 3 = scales, 4 = routing, 5 = second
    activations (MoE down-projection input), 6 = dense weights (gather_mm)

Value distributions: scale ~ U[0.001, 0.02] rounded to bf16; bias =
-2**(bits-1) * scale (exact in bf16); codes uniform over [0, 2**bits); dense
activations N(0, 1) (U[-1, 1] for the tiny case), rounded to bf16.
"""

from __future__ import annotations

import numpy as np

GROUP = 64

TAG_X = 1
TAG_Q = 2
TAG_SCALE = 3
TAG_ROUTE = 4
TAG_X2 = 5
TAG_W = 6


def rng_for(seed: int, tag: int, *extra: int) -> np.random.Generator:
    """Independent generator for one tensor: SeedSequence([seed, tag, *extra])."""
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(tag), *map(int, extra)]))


# ---------------------------------------------------------------------------
# bf16 storage helpers (input side only)
# ---------------------------------------------------------------------------

def to_bf16_bits(a) -> np.ndarray:
    """Round float64 values to bf16 (round to nearest, ties to even) -> uint16 bits.

    Done directly from float64 (no float32 double rounding): each finite value
    is written as r * 2**(e-8) with r an integer in [128, 256], rounded with
    ``np.rint`` (ties to even). Inputs must be finite and inside the normal bf16
    range, which every distribution drawn here is; zeros are allowed.
    """
    a = np.asarray(a, dtype=np.float64)
    if not np.all(np.isfinite(a)):
        raise ValueError("to_bf16_bits: non-finite input")
    mag = np.abs(a)
    nz = mag > 0
    if np.any(mag[nz] < 2.0 ** -126) or np.any(mag >= 2.0 ** 128):
        raise ValueError("to_bf16_bits: value outside the normal bf16 range")
    m, e = np.frexp(mag)                     # mag = m * 2**e, m in [0.5, 1)
    r = np.rint(np.ldexp(m, 8))              # integer in [128, 256]
    carry = r == 256
    r = np.where(carry, 128, r)
    e = e + carry
    expo = (e - 1 + 127).astype(np.int64)
    if np.any(expo[nz] >= 255):
        raise ValueError("to_bf16_bits: rounds to infinity")
    bits = (expo << 7) | (r.astype(np.int64) - 128)
    bits = np.where(nz, bits, 0)
    bits = bits | np.where(np.signbit(a), 0x8000, 0)
    return bits.astype(np.uint16)


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even) -> uint16 bits, for large
    draws made in float32 (bf16 is the upper half of a binary32). Finite inputs only."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + r) >> np.uint32(16)).astype(np.uint16)


def to_f16_bits(a) -> np.ndarray:
    """Round values to IEEE binary16 with numpy (nearest, ties to even) -> uint16 bits."""
    return np.asarray(a).astype(np.float16).view(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def pack_codes(q, bits: int) -> np.ndarray:
    """Pack unsigned codes [..., K] into uint32 words [..., K*bits//32], LSB first."""
    q = np.asarray(q)
    if bits not in (2, 4, 8):
        raise ValueError("bits must be 2, 4 or 8")
    per = 32 // bits
    if q.shape[-1] % per:
        raise ValueError("K must be a multiple of 32/bits")
    if q.size and (q.min() < 0 or q.max() >= (1 << bits)):
        raise ValueError("code out of range")
    qw = q.astype(np.uint32).reshape(*q.shape[:-1], q.shape[-1] // per, per)
    shifts = (np.arange(per, dtype=np.uint32) * bits).astype(np.uint32)
    return np.bitwise_or.reduce(qw << shifts, axis=-1).astype(np.uint32)


def random_words(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform random uint32 words: every packed code is uniform over [0, 2**bits)."""
    return rng.integers(0, 0xFFFFFFFF, size=shape, dtype=np.uint32, endpoint=True)


def random_scales(rng: np.random.Generator, shape) -> np.ndarray:
    """Scales ~ U[0.001, 0.02], rounded to bf16 (uint16 bits)."""
    return to_bf16_bits(rng.uniform(0.001, 0.02, size=shape))


def bias_for_scales(scale_bits: np.ndarray, bits: int) -> np.ndarray:
    """bias = -2**(bits-1) * scale; a power-of-two multiple, so exact in bf16."""
    return to_bf16_bits(-(2.0 ** (bits - 1)) * bf16_bits_to_f64(scale_bits))


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

class Dense:
    """One qmv / qmm problem: y[M,N] = x[M,K] . dequant(w)^T."""

    def __init__(self, name, x, w, scales, biases, bits, group: int = GROUP):
        self.name = name
        self.x, self.w, self.scales, self.biases = x, w, scales, biases
        self.bits, self.group = bits, group
        self.M, self.K = x.shape
        self.N = w.shape[0]
        assert w.shape == (self.N, self.K * bits // 32)
        assert scales.shape == biases.shape == (self.N, self.K // group)

    def algorithmic_bytes(self, out_bytes: int = 2) -> int:
        """Codes + scales + biases + x + y, each moved once."""
        return (self.w.nbytes + self.scales.nbytes + self.biases.nbytes
                + self.x.nbytes + self.M * self.N * out_bytes)

    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


class Gather:
    """One expert-sorted problem: y[r,:] = x[r,:] . dequant(w[expert_idx[r]])^T."""

    def __init__(self, name, x, w, scales, biases, expert_idx, bits, token_of_row=None,
                 group: int = GROUP):
        self.name = name
        self.x, self.w, self.scales, self.biases = x, w, scales, biases
        self.expert_idx = expert_idx
        self.token_of_row = token_of_row
        self.bits, self.group = bits, group
        self.B, self.K = x.shape
        self.E, self.N = w.shape[0], w.shape[1]
        assert w.shape == (self.E, self.N, self.K * bits // 32)
        assert scales.shape == biases.shape == (self.E, self.N, self.K // group)
        assert expert_idx.shape == (self.B,) and expert_idx.dtype == np.int32

    def algorithmic_bytes(self, out_bytes: int = 2) -> int:
        return (self.w.nbytes + self.scales.nbytes + self.biases.nbytes + self.x.nbytes
                + self.B * self.N * out_bytes + self.expert_idx.nbytes)

    def flops(self) -> int:
        return 2 * self.B * self.N * self.K


class GatherIndexed:
    """Indexed gather: y[r,:] = x[token_idx[r],:] . dequant(w[expert_idx[r]])^T, rows in
    any order (token_idx None: row r reads x row r)."""

    def __init__(self, name, x, w, scales, biases, token_idx, expert_idx, bits, group: int = GROUP):
        self.name = name
        self.x, self.w, self.scales, self.biases = x, w, scales, biases
        self.token_idx, self.expert_idx = token_idx, expert_idx
        self.bits, self.group = bits, group
        self.T, self.K = x.shape
        self.E, self.N = w.shape[0], w.shape[1]
        self.B = expert_idx.shape[0]
        assert w.shape == (self.E, self.N, self.K * bits // 32)
        assert scales.shape == biases.shape == (self.E, self.N, self.K // group)
        assert expert_idx.dtype == np.int32
        assert token_idx is None or (token_idx.shape == (self.B,) and token_idx.dtype == np.int32)

    def algorithmic_bytes(self, out_bytes: int = 2) -> int:
        """Weights of every distinct expert the rows use (streamed once), the activation
        rows they read, the ids and the outputs."""
        used = np.unique(self.expert_idx[(self.expert_idx >= 0) & (self.expert_idx < self.E)])
        per_expert = (self.w[0].nbytes + self.scales[0].nbytes + self.biases[0].nbytes)
        rows = self.T if self.token_idx is None else np.unique(self.token_idx).size
        ids = self.expert_idx.nbytes + (0 if self.token_idx is None else self.token_idx.nbytes)
        return (used.size * per_expert + rows * self.K * 2 + ids + self.B * self.N * out_bytes)

    def flops(self) -> int:
        return 2 * self.B * self.N * self.K


class GatherMM:
    """Dense grouped product: y[r,:] = x[token_idx[r],:] . W[expert_idx[r]]^T, rows in any
    order (token_idx None: row r reads x row r). x and w are bf16 (dtype "bf16") or
    binary16 ("f16") bit patterns; w is [E, N, K] (layout "nk") or [E, K, N] ("kn")."""

    def __init__(self, name, x, w, token_idx, expert_idx, dtype: str = "bf16", layout: str = "nk"):
        self.name = name
        self.x, self.w = x, w
        self.token_idx, self.expert_idx = token_idx, expert_idx
        self.dtype, self.layout = dtype, layout
        self.T, self.K = x.shape
        self.E = w.shape[0]
        self.N = w.shape[1] if layout == "nk" else w.shape[2]
        self.B = expert_idx.shape[0]
        assert x.dtype == np.uint16 and w.dtype == np.uint16 and dtype in ("bf16", "f16")
        assert w.shape == ((self.E, self.N, self.K) if layout == "nk" else (self.E, self.K, self.N))
        assert expert_idx.dtype == np.int32
        assert token_idx is None or (token_idx.shape == (self.B,) and token_idx.dtype == np.int32)

    def algorithmic_bytes(self, out_bytes: int = 2) -> int:
        """Weights of every distinct expert the rows use (streamed once), the activation
        rows they read, the ids and the outputs."""
        used = np.unique(self.expert_idx[(self.expert_idx >= 0) & (self.expert_idx < self.E)])
        rows = self.T if self.token_idx is None else np.unique(self.token_idx).size
        ids = self.expert_idx.nbytes + (0 if self.token_idx is None else self.token_idx.nbytes)
        return used.size * self.w[0].nbytes + rows * self.K * 2 + ids + self.B * self.N * out_bytes

    def flops(self) -> int:
        return 2 * self.B * self.N * self.K


def _encode(a, dtype: str) -> np.ndarray:
    return to_bf16_bits(a) if dtype == "bf16" else to_f16_bits(a)


def random_gather_mm(T: int, B: int, E: int, N: int, K: int, dtype: str = "bf16",
                     layout: str = "nk", seed: int = 0, with_tokens: bool = True) -> GatherMM:
    """Arbitrary dense grouped product: random token and expert per row (repeats, any
    order); x ~ N(0, 1), W ~ N(0, 0.02^2) like a trained projection."""
    rng = rng_for(seed, TAG_ROUTE, 11, T, B, E, N, K)
    exp = rng.integers(0, E, B).astype(np.int32)
    tok = rng.integers(0, T, B).astype(np.int32) if with_tokens else None
    rows = T if with_tokens else B
    x = _encode(rng_for(seed, TAG_X, 11, rows, K).standard_normal(size=(rows, K)), dtype)
    wshape = (E, N, K) if layout == "nk" else (E, K, N)
    w = _encode(0.02 * rng_for(seed, TAG_W, E, N, K).standard_normal(size=wshape), dtype)
    return GatherMM(f"gather_mm_T{rows}_B{B}_E{E}_K{K}_N{N}_{dtype}_{layout}", x, w, tok, exp,
                    dtype, layout)


def moe_gather_mm(which: str, dtype: str = "bf16", layout: str = "nk", seed: int = 0,
                  tokens: int = None, E: int = None, top_k: int = None, hidden: int = None,
                  inter: int = None) -> GatherMM:
    """The MoE prefill of a non-quantized checkpoint: the routing of ``moe_gather`` (573
    tokens, 8 of 128 experts each) in routing (token-major) order, dense weights.

    ``which="up"``:   K=hidden, N=inter; x = the hidden states [tokens, hidden], read
                      through the token index.
    ``which="down"``: K=inter, N=hidden; x = one N(0,1) row per output row [B, inter].
    Weights ~ N(0, 0.02^2), drawn in float32 and rounded to the operand type.
    """
    tokens = MOE_TOKENS if tokens is None else tokens
    E = MOE_E if E is None else E
    top_k = MOE_TOPK if top_k is None else top_k
    hidden = MOE_HIDDEN if hidden is None else hidden
    inter = MOE_INTER if inter is None else inter
    idx, tok = moe_routing(seed, tokens, E, top_k)
    order = np.argsort(tok.astype(np.int64) * (E + 1) + idx, kind="stable")
    exp = np.ascontiguousarray(idx[order])
    B = exp.shape[0]
    enc32 = f32_to_bf16_bits if dtype == "bf16" else to_f16_bits
    if which == "up":
        K, N = hidden, inter
        x = enc32(rng_for(seed, TAG_X, 6, tokens, hidden).standard_normal(size=(tokens, hidden),
                                                                          dtype=np.float32))
        tk = np.ascontiguousarray(tok[order])
    elif which == "down":
        K, N = inter, hidden
        x = enc32(rng_for(seed, TAG_X2, 6, B, inter).standard_normal(size=(B, inter), dtype=np.float32))
        tk = None
    else:
        raise ValueError("which must be 'up' or 'down'")
    wshape = (E, N, K) if layout == "nk" else (E, K, N)
    w32 = rng_for(seed, TAG_W, E, N, K).standard_normal(size=wshape, dtype=np.float32)
    w32 *= np.float32(0.02)
    w = enc32(w32)
    del w32
    return GatherMM(f"gather_mm_{which}_B{B}_E{E}_K{K}_N{N}_{dtype}_{layout}", x, w, tk, exp,
                    dtype, layout)


def _dense_weights(seed: int, N: int, K: int, bits: int, sub: int = 0, group: int = GROUP):
    w = random_words(rng_for(seed, TAG_Q, bits, N, K, sub), (N, K * bits // 32))
    s = random_scales(rng_for(seed, TAG_SCALE, N, K, sub), (N, K // group))
    return w, s, bias_for_scales(s, bits)


def tiny_qmv(seed: int = 0) -> Dense:
    """M=1, K=512, N=256, 4-bit; activations U[-1, 1]."""
    M, K, N, bits = 1, 512, 256, 4
    x = to_bf16_bits(rng_for(seed, TAG_X, 0).uniform(-1.0, 1.0, size=(M, K)))
    w, s, b = _dense_weights(seed, N, K, bits, sub=0)
    return Dense("qmv_K512_N256_b4", x, w, s, b, bits)


_DENSE_M, _DENSE_K, _DENSE_N = 600, 5120, 13824


def _dense_x(seed: int) -> np.ndarray:
    return to_bf16_bits(rng_for(seed, TAG_X, 1).standard_normal(size=(_DENSE_M, _DENSE_K)))


def hidden5120(M: int, N: int, bits: int, seed: int = 0) -> Dense:
    """Dense problems at hidden size 5120.

    All share one draw of activations [600, 5120] (M rows take the first M),
    one draw of scales [13824, 80] and one draw of codes per bit width
    [13824, 5120] (N columns take the first N rows of W). So the decode GEMV at
    N=5120 sees the first 5120 output rows of the prefill weight, M=3 sees the
    first three prefill tokens, and the 8-bit problems use identical
    activations and scales.
    """
    if not (1 <= M <= _DENSE_M and 1 <= N <= _DENSE_N and bits in (4, 8)):
        raise ValueError("hidden5120: M <= 600, N <= 13824, bits in {4, 8}")
    x = _dense_x(seed)[:M]
    w = random_words(rng_for(seed, TAG_Q, bits, _DENSE_N, _DENSE_K, 0),
                     (_DENSE_N, _DENSE_K * bits // 32))[:N]
    s = random_scales(rng_for(seed, TAG_SCALE, _DENSE_N, _DENSE_K, 0),
                      (_DENSE_N, _DENSE_K // GROUP))[:N]
    b = bias_for_scales(s, bits)
    kind = "qmv" if M == 1 else "qmm"
    return Dense(f"{kind}_M{M}_K{_DENSE_K}_N{N}_b{bits}", x, np.ascontiguousarray(w),
                 np.ascontiguousarray(s), np.ascontiguousarray(b), bits)


MOE_TOKENS, MOE_E, MOE_TOPK = 573, 128, 8
MOE_HIDDEN, MOE_INTER = 2816, 704


def moe_routing(seed: int = 0, tokens: int = MOE_TOKENS, E: int = MOE_E, top_k: int = MOE_TOPK):
    """Each token picks top_k distinct experts uniformly; pairs flattened
    token-major, then stable-sorted by expert. Returns (expert_idx, token_of_row)."""
    rng = rng_for(seed, TAG_ROUTE, tokens, E, top_k)
    choice = np.stack([rng.choice(E, top_k, replace=False) for _ in range(tokens)])
    experts = choice.reshape(-1).astype(np.int32)
    tokens_of = np.repeat(np.arange(tokens, dtype=np.int32), top_k)
    order = np.argsort(experts, kind="stable")
    return np.ascontiguousarray(experts[order]), np.ascontiguousarray(tokens_of[order])


def moe_gather(which: str, seed: int = 0, tokens: int = MOE_TOKENS, E: int = MOE_E,
               top_k: int = MOE_TOPK, hidden: int = MOE_HIDDEN, inter: int = MOE_INTER,
               bits: int = 4) -> Gather:
    """MoE prefill, expert-sorted rows.

    ``which="up"``:   K=hidden, N=inter; x row r is hidden-state row token_of_row[r].
    ``which="down"``: K=inter, N=hidden; x is a fresh N(0,1) draw [B, inter].
    """
    idx, tok = moe_routing(seed, tokens, E, top_k)
    B = idx.shape[0]
    if which == "up":
        K, N = hidden, inter
        h = to_bf16_bits(rng_for(seed, TAG_X, 4, tokens, hidden).standard_normal(size=(tokens, hidden)))
        x = np.ascontiguousarray(h[tok])
    elif which == "down":
        K, N = inter, hidden
        x = to_bf16_bits(rng_for(seed, TAG_X2, B, inter).standard_normal(size=(B, inter)))
    else:
        raise ValueError("which must be 'up' or 'down'")
    w = random_words(rng_for(seed, TAG_Q, bits, E, N, K), (E, N, K * bits // 32))
    s = random_scales(rng_for(seed, TAG_SCALE, E, N, K), (E, N, K // GROUP))
    b = bias_for_scales(s, bits)
    return Gather(f"gather_{which}_B{B}_E{E}_K{K}_N{N}_b{bits}", x, w, s, b, idx, bits, tok)


def moe_prefill_indexed(which: str, seed: int = 0, tokens: int = MOE_TOKENS, E: int = MOE_E,
                        top_k: int = MOE_TOPK, hidden: int = MOE_HIDDEN, inter: int = MOE_INTER,
                        bits: int = 4) -> GatherIndexed:
    """MoE prefill as the routing produces it: rows token-major (expert ids unsorted).

    ``which="up"``:   x = the hidden states [tokens, hidden], each row reads its token's
                      row through the token index (no replicas).
    ``which="down"``: x = one activation row per output row [B, inter], no token index.
    Same routing, activations and weights as ``moe_gather``, so each output row equals
    the corresponding row of the sorted problem.
    """
    g = moe_gather(which, seed, tokens, E, top_k, hidden, inter, bits)
    order = np.argsort(g.token_of_row.astype(np.int64) * (E + 1) + g.expert_idx, kind="stable")
    exp = np.ascontiguousarray(g.expert_idx[order])
    if which == "up":
        x = np.empty((tokens, g.K), dtype=np.uint16)
        x[g.token_of_row] = g.x
        tok = np.ascontiguousarray(g.token_of_row[order])
    else:
        x = np.ascontiguousarray(g.x[order])
        tok = None
    return GatherIndexed(f"gather_indexed_{which}_B{g.B}_E{E}_K{g.K}_N{g.N}_b{bits}", x, g.w,
                         g.scales, g.biases, tok, exp, bits)


def moe_decode(which: str, tokens: int = 1, seed: int = 0, E: int = MOE_E, top_k: int = MOE_TOPK,
               hidden: int = MOE_HIDDEN, inter: int = MOE_INTER, bits: int = 4) -> GatherIndexed:
    """MoE decode step: each of `tokens` tokens picks top_k distinct experts uniformly;
    output rows are token-major (expert ids unsorted), B = tokens * top_k.

    ``which="up"``:   K=hidden, N=inter; row r reads hidden-state row token_idx[r].
    ``which="down"``: K=inter, N=hidden; each row reads its own activation row (a fresh
                      N(0,1) draw [B, inter]), no token index.
    The expert weights are the same draws as ``moe_gather``'s (one MoE layer's experts).
    """
    rng = rng_for(seed, TAG_ROUTE, tokens, E, top_k, 1)
    experts = np.concatenate([rng.choice(E, top_k, replace=False) for _ in range(tokens)])
    experts = np.ascontiguousarray(experts.astype(np.int32))
    B = experts.shape[0]
    if which == "up":
        K, N = hidden, inter
        x = to_bf16_bits(rng_for(seed, TAG_X, 6, tokens, hidden).standard_normal(size=(tokens, hidden)))
        tok = np.repeat(np.arange(tokens, dtype=np.int32), top_k)
    elif which == "down":
        K, N = inter, hidden
        x = to_bf16_bits(rng_for(seed, TAG_X2, 6, B, inter).standard_normal(size=(B, inter)))
        tok = None
    else:
        raise ValueError("which must be 'up' or 'down'")
    w = random_words(rng_for(seed, TAG_Q, bits, E, N, K), (E, N, K * bits // 32))
    s = random_scales(rng_for(seed, TAG_SCALE, E, N, K), (E, N, K // GROUP))
    b = bias_for_scales(s, bits)
    return GatherIndexed(f"moe_decode_{which}_T{tokens}_B{B}_E{E}_K{K}_N{N}_b{bits}", x, w, s, b,
                         tok, experts, bits)


def random_indexed(T: int, B: int, E: int, N: int, K: int, bits: int, seed: int = 0,
                   with_tokens: bool = True, group: int = GROUP) -> GatherIndexed:
    """Arbitrary indexed gather: random token and expert per row (repeats, any order)."""
    rng = rng_for(seed, TAG_ROUTE, 9, T, B, E, N, K)
    exp = rng.integers(0, E, B).astype(np.int32)
    tok = rng.integers(0, T, B).astype(np.int32) if with_tokens else None
    rows = T if with_tokens else B
    x = to_bf16_bits(rng_for(seed, TAG_X, 9, rows, K).standard_normal(size=(rows, K)))
    w = random_words(rng_for(seed, TAG_Q, bits, E, N, K, 9), (E, N, K * bits // 32))
    s = random_scales(rng_for(seed, TAG_SCALE, E, N, K, 9), (E, N, K // group))
    b = bias_for_scales(s, bits)
    return GatherIndexed(f"indexed_T{rows}_B{B}_E{E}_K{K}_N{N}_b{bits}", x, w, s, b, tok, exp, bits,
                         group)


def random_dense(M: int, N: int, K: int, bits: int, seed: int = 0, x_dist: str = "normal",
                 group: int = GROUP) -> Dense:
    """Arbitrary-shape dense problem with the standard value distributions."""
    rx = rng_for(seed, TAG_X, 7, M, N, K)
    xf = rx.standard_normal(size=(M, K)) if x_dist == "normal" else rx.uniform(-1, 1, size=(M, K))
    w, s, b = _dense_weights(seed, N, K, bits, sub=7, group=group)
    gname = "" if group == GROUP else f"_g{group}"
    return Dense(f"dense_M{M}_K{K}_N{N}_b{bits}{gname}", to_bf16_bits(xf), w, s, b, bits, group)


def random_gather(counts, N: int, K: int, bits: int, seed: int = 0, group: int = GROUP) -> Gather:
    """Expert-sorted problem with explicit per-expert row counts (zeros allowed)."""
    counts = np.asarray(counts, dtype=np.int64)
    E = counts.shape[0]
    idx = np.repeat(np.arange(E, dtype=np.int32), counts)
    B = idx.shape[0]
    x = to_bf16_bits(rng_for(seed, TAG_X, 8, B, N, K).standard_normal(size=(B, K)))
    w = random_words(rng_for(seed, TAG_Q, bits, E, N, K, 8), (E, N, K * bits // 32))
    s = random_scales(rng_for(seed, TAG_SCALE, E, N, K, 8), (E, N, K // group))
    b = bias_for_scales(s, bits)
    return Gather(f"gather_B{B}_E{E}_K{K}_N{N}_b{bits}", x, w, s, b, idx, bits, group=group)
