"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``check_*`` function takes an oracle object (``oracle.Oracle``) and raises
AssertionError if it disagrees with what the definition of the computation
(w = s*q + b per group along K, y = x . W^T, summed exactly; for the dense
grouped product gather_mm, y = x . W^T with W stored [N, K] or [K, N]), the bf16
and binary16 formats, or the documented code layout fix. They run against the real oracle
in ``test_oracle_pins.py`` and against oracles with planted mistakes in
``test_oracle_mutants.py`` (each planted mistake must trip at least one pin).

None of these recomputes the oracle's formula the oracle's way: the
brute-force path unpacks with a byte view instead of word shifts and uses
numpy's float64 matmul; the exact cases compare against integer arithmetic or
a closed form; the layout and rounding cases against hand-written fixtures.
"""

from __future__ import annotations

import os
import sys

import numpy as np

from bit_matmul_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# Independent numpy reference for tiny shapes (brute force, "library routine")
# ---------------------------------------------------------------------------

def numpy_codes(w: np.ndarray, bits: int) -> np.ndarray:
    """Codes [..., K] from packed words via a little-endian byte view."""
    assert sys.byteorder == "little"
    by = np.ascontiguousarray(w).view(np.uint8)  # byte j of word i = bits [8j, 8j+8)
    if bits == 8:
        return by.astype(np.int64)
    if bits == 2:           # k = 4*byte + i in bits [2i, 2i+2) of the byte
        parts = [(by >> (2 * i)) & 0x03 for i in range(4)]
        return np.stack(parts, axis=-1).reshape(*by.shape[:-1], by.shape[-1] * 4).astype(np.int64)
    lo = by & 0x0F          # k = 2*byte
    hi = by >> 4            # k = 2*byte + 1
    return np.stack([lo, hi], axis=-1).reshape(*by.shape[:-1], by.shape[-1] * 2).astype(np.int64)


def numpy_dequant(w, s, b, bits, group=64):
    q = numpy_codes(w, bits).astype(np.float64)
    sf = np.repeat(I.bf16_bits_to_f64(s), group, axis=-1)
    bf = np.repeat(I.bf16_bits_to_f64(b), group, axis=-1)
    return sf * q + bf


def numpy_qmm(x, w, s, b, bits, group=64):
    return np.matmul(I.bf16_bits_to_f64(x), numpy_dequant(w, s, b, bits, group).T)


# ---------------------------------------------------------------------------
# Fixture readers
# ---------------------------------------------------------------------------

def read_bf16_golden():
    rows = []
    with open(os.path.join(GOLDEN, "bf16_rne.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tok = line.split()
            v = {"inf": np.inf, "-inf": -np.inf, "nan": np.nan}.get(tok[0])
            if v is None:
                v = float.fromhex(tok[0])
            rows.append((v, int(tok[1], 16)))
    return rows


def read_f16_golden():
    """(value, bits, exact) rows of tests/golden/f16_rne.txt."""
    rows = []
    with open(os.path.join(GOLDEN, "f16_rne.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tok = line.split()
            v = {"inf": np.inf, "-inf": -np.inf, "nan": np.nan, "0": 0.0, "-0": -0.0}.get(tok[0])
            if v is None:
                v = float.fromhex(tok[0])
            rows.append((v, int(tok[1], 16), tok[2] == "exact"))
    return rows


def read_unpack_golden():
    rows = []
    with open(os.path.join(GOLDEN, "unpack_codes.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tok = line.split()
            rows.append((int(tok[0]), int(tok[1], 16), [int(t) for t in tok[2:]]))
    return rows


# ---------------------------------------------------------------------------
# Pins
# ---------------------------------------------------------------------------

def check_bf16_golden(O):
    for v, bits in read_bf16_golden():
        got = int(O.f64_to_bf16(np.array([v]))[0])
        assert got == bits, f"bf16({v!r}) = {got:#06x}, expected {bits:#06x}"


def check_bf16_vs_torch(O):
    """float32 -> bfloat16 in torch rounds to nearest even: same bits for every
    float32 input (a float32 converts to double exactly)."""
    import torch
    rng = np.random.default_rng(11)
    u = rng.integers(0, 1 << 32, size=4000, dtype=np.uint64).astype(np.uint32)
    # add exact ties and near-ties: low 16 bits 0x8000, 0x7fff, 0x8001
    hi = u & np.uint32(0xFFFF0000)
    u = np.concatenate([u, hi | 0x8000, hi | 0x7FFF, hi | 0x8001]).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f64_to_bf16(f.astype(np.float64))
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches vs torch, first {f[bad[0]]!r}"


def check_unpack_golden(O):
    for bits, word, codes in read_unpack_golden():
        for k, c in enumerate(codes):
            got = O.code(np.array([word], dtype=np.uint32), k, bits)
            assert got == c, f"bits={bits} word={word:#010x} k={k}: {got} != {c}"
    # multi-word rows: element k lives in word k // (32/bits)
    for bits in (2, 4, 8):
        per = 32 // bits
        q = (np.arange(5 * per) * 7 + 3) % (1 << bits)
        row = I.pack_codes(q, bits)
        for k in range(q.size):
            assert O.code(row, k, bits) == q[k]


def check_weight_definition(O):
    """w = s*q + b with the group of k; exact for bf16 s, b (checked in Fractions)."""
    from fractions import Fraction
    rng = np.random.default_rng(5)
    for bits in (2, 4, 8):
        K = 256
        q = rng.integers(0, 1 << bits, size=K)
        row = I.pack_codes(q, bits)
        s = I.to_bf16_bits(rng.uniform(-3, 3, size=K // 64))
        b = I.to_bf16_bits(rng.uniform(-3, 3, size=K // 64))
        for k in range(K):
            g = k // 64
            exp = Fraction(float(I.bf16_bits_to_f64(s[g]))) * int(q[k]) + Fraction(
                float(I.bf16_bits_to_f64(b[g])))
            assert Fraction(O.weight(row, s, b, k, bits)) == exp, (bits, k)


def check_brute_force(O):
    """Tiny shapes: oracle == numpy byte-view unpack + float64 matmul."""
    for bits in (2, 4, 8):
        for M in (1, 2, 3, 5):
            for N in (1, 3, 8, 17):
                for K in (64, 128, 192):
                    d = I.random_dense(M, N, K, bits, seed=M * 1000 + N * 10 + K)
                    ref = numpy_qmm(d.x, d.w, d.scales, d.biases, bits)
                    got = O.qmm(d.x, d.w, d.scales, d.biases, bits)
                    err = np.max(np.abs(got - ref))
                    assert err <= 1e-12 * max(1.0, np.max(np.abs(ref))), (bits, M, N, K, err)


def check_brute_force_groups(O):
    """Groups of 32 and 128 along K: oracle == numpy (byte-view unpack, scales and
    biases repeated over their group, float64 matmul), dense and indexed gather."""
    for group in (32, 128):
        for bits in (2, 4, 8):
            for M, N, K in ((1, 5, 128), (3, 8, 256), (2, 17, 384)):
                d = I.random_dense(M, N, K, bits, seed=M * 100 + N + K + group, group=group)
                ref = numpy_qmm(d.x, d.w, d.scales, d.biases, bits, group)
                got = O.qmm(d.x, d.w, d.scales, d.biases, bits, group=group)
                assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max()), (group, bits, M, N, K)
            g = I.random_indexed(3, 9, 4, 7, 256, bits, seed=group + bits, group=group)
            got = O.gather_qmm_indexed(g.x, g.w, g.scales, g.biases, g.token_idx, g.expert_idx,
                                       bits, group=group)
            xf = I.bf16_bits_to_f64(g.x)
            ref = np.stack([numpy_dequant(g.w[e], g.scales[e], g.biases[e], bits, group) @ xf[t]
                            for t, e in zip(g.token_idx, g.expert_idx)])
            assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max()), (group, bits)


def integer_exact_problem(M, N, K, bits, seed):
    """x in {-2..2}, s in {1/4,1/2,1,2} per group, b = -2**(bits-1)*s: every
    weight, product and partial sum is an exact multiple of 1/4 below 2**24/4."""
    rng = np.random.default_rng(seed)
    xi = rng.integers(-2, 3, size=(M, K))
    q = rng.integers(0, 1 << bits, size=(N, K))
    s4 = rng.choice([1, 2, 4, 8], size=(N, K // 64))           # 4*s
    half = 1 << (bits - 1)
    x = I.to_bf16_bits(xi.astype(np.float64))
    s = I.to_bf16_bits(s4 / 4.0)
    b = I.to_bf16_bits(-half * s4 / 4.0)
    w = I.pack_codes(q, bits)
    w4 = np.repeat(s4, 64, axis=1) * (q - half)                 # 4*w, integers
    y4 = xi.astype(np.int64) @ w4.T.astype(np.int64)            # 4*y, exact
    return x, w, s, b, y4


def check_integer_exact(O):
    for bits in (2, 4, 8):
        for (M, N, K) in ((3, 17, 192), (1, 40, 640), (9, 5, 5120)):
            x, w, s, b, y4 = integer_exact_problem(M, N, K, bits, seed=K + bits)
            got = O.qmm(x, w, s, b, bits)
            assert np.array_equal(got * 4.0, y4.astype(np.float64)), (bits, M, N, K)


def check_one_hot(O):
    """x = I_K gives y[k][n] = w[n][k]; with s = 1, b = -2**(bits-1) the weight
    is q - 2**(bits-1). Codes q[n][k] = (k + n) mod 2**bits put every value at
    every position inside a word."""
    for bits, K, N in ((4, 128, 16), (8, 256, 64)):
        per = 32 // bits
        kk, nn = np.meshgrid(np.arange(K), np.arange(N))
        q = (kk + nn) % (1 << bits)
        seen = {(int(k % per), int(v)) for k, v in zip(kk.ravel(), q.ravel())}
        assert len(seen) == per * (1 << bits)
        w = I.pack_codes(q, bits)
        s = I.to_bf16_bits(np.ones((N, K // 64)))
        b = I.to_bf16_bits(np.full((N, K // 64), -float(1 << (bits - 1))))
        x = I.to_bf16_bits(np.eye(K))
        got = O.qmm(x, w, s, b, bits)
        assert np.array_equal(got, (q.T - (1 << (bits - 1))).astype(np.float64)), bits


def check_closed_form(O):
    """x = 1, q = c everywhere: y[n] = 64 * sum_g (c*s[n,g] + b[n,g])."""
    from fractions import Fraction
    rng = np.random.default_rng(3)
    for bits in (2, 4, 8):
        K, N = 320, 6
        for c in (0, 1, (1 << bits) - 1):
            w = I.pack_codes(np.full((N, K), c), bits)
            s = I.to_bf16_bits(rng.uniform(0.001, 0.02, size=(N, K // 64)))
            b = I.to_bf16_bits(rng.uniform(-0.1, 0.1, size=(N, K // 64)))
            x = I.to_bf16_bits(np.ones((1, K)))
            got = O.qmm(x, w, s, b, bits)[0]
            sf, bf = I.bf16_bits_to_f64(s), I.bf16_bits_to_f64(b)
            for n in range(N):
                exact = 64 * sum(Fraction(float(sf[n, g])) * c + Fraction(float(bf[n, g]))
                                 for g in range(K // 64))
                assert abs(Fraction(got[n]) - exact) <= Fraction(1, 10 ** 12) * (1 + abs(exact)), (
                    bits, c, n)


def check_bias_linearity(O):
    """y(b) - y(0) = sum_g b[n,g] * X_g with X_g the group sums of x."""
    for bits in (2, 4, 8):
        d = I.random_dense(4, 9, 256, bits, seed=21)
        zero = np.zeros_like(d.biases)
        y1 = O.qmm(d.x, d.w, d.scales, d.biases, bits)
        y0 = O.qmm(d.x, d.w, d.scales, zero, bits)
        xf = I.bf16_bits_to_f64(d.x)
        Xg = xf.reshape(d.M, d.K // 64, 64).sum(axis=2)             # [M, G]
        ref = Xg @ I.bf16_bits_to_f64(d.biases).T                   # [M, N]
        assert np.max(np.abs((y1 - y0) - ref)) <= 1e-12 * (1 + np.max(np.abs(ref))), bits


def check_constant_per_expert(O):
    """q = 0, b[e] = e + 1, x[r,:] = (r mod 7) + 1: y[r,n] = K (e_r+1) ((r mod 7)+1)
    exactly; a mis-gathered expert or a misplaced row gives a wrong integer."""
    counts = [3, 0, 5, 1, 0, 4, 9]
    E, N, K = len(counts), 11, 192
    idx = np.repeat(np.arange(E, dtype=np.int32), counts)
    B = idx.size
    for bits in (2, 4, 8):
        w = np.zeros((E, N, K * bits // 32), dtype=np.uint32)
        s = I.to_bf16_bits(np.full((E, N, K // 64), 0.5))
        b = I.to_bf16_bits(np.broadcast_to((np.arange(E) + 1.0)[:, None, None], (E, N, K // 64)))
        xv = (np.arange(B) % 7 + 1).astype(np.float64)
        x = I.to_bf16_bits(np.broadcast_to(xv[:, None], (B, K)))
        got = O.gather_qmm(x, w, s, b, idx, bits)
        exp = K * (idx[:, None] + 1.0) * xv[:, None] * np.ones((1, N))
        assert np.array_equal(got, exp), bits


def check_invalid_expert_rows(O):
    """Rows whose id is outside [0, E) come out as zero rows."""
    g = I.random_gather([2, 3], N=5, K=128, bits=4, seed=2)
    idx = g.expert_idx.copy()
    idx[1] = -1
    idx[4] = 2
    got = O.gather_qmm(g.x, g.w, g.scales, g.biases, idx, 4)
    assert np.all(got[1] == 0) and np.all(got[4] == 0)
    assert np.all(got[[0, 2, 3]] != 0)


def check_gather_consistency(O):
    """Per-expert slices of gather_qmm equal qmm on that expert's rows and
    weights; E = 1 equals qmm; permuting rows within a segment permutes outputs."""
    for bits in (2, 4, 8):
        g = I.random_gather([4, 0, 7, 2, 5], N=13, K=192, bits=bits, seed=bits)
        y = O.gather_qmm(g.x, g.w, g.scales, g.biases, g.expert_idx, bits)
        for e in range(g.E):
            rows = np.nonzero(g.expert_idx == e)[0]
            if rows.size == 0:
                continue
            ye = O.qmm(g.x[rows], g.w[e], g.scales[e], g.biases[e], bits)
            assert np.array_equal(y[rows], ye), (bits, e)
        one = O.gather_qmm(g.x, g.w[:1], g.scales[:1], g.biases[:1],
                           np.zeros(g.B, dtype=np.int32), bits)
        assert np.array_equal(one, O.qmm(g.x, g.w[0], g.scales[0], g.biases[0], bits))
        perm = np.arange(g.B)
        seg = np.nonzero(g.expert_idx == 2)[0]
        perm[seg] = seg[::-1]
        yp = O.gather_qmm(g.x[perm], g.w, g.scales, g.biases, g.expert_idx, bits)
        assert np.array_equal(yp, y[perm])


def check_repack_8bit(O):
    """Codes below 16 stored as 8-bit give the same result as stored as 4-bit, and codes
    below 4 the same again stored as 2-bit."""
    rng = np.random.default_rng(9)
    N, K, M = 7, 192, 3
    s = I.random_scales(rng, (N, K // 64))
    b = I.to_bf16_bits(rng.uniform(-0.2, 0.2, size=(N, K // 64)))
    x = I.to_bf16_bits(rng.standard_normal((M, K)))
    q = rng.integers(0, 16, size=(N, K))
    y4 = O.qmm(x, I.pack_codes(q, 4), s, b, 4)
    y8 = O.qmm(x, I.pack_codes(q, 8), s, b, 8)
    assert np.array_equal(y4, y8)
    q = rng.integers(0, 4, size=(N, K))
    y2 = O.qmm(x, I.pack_codes(q, 2), s, b, 2)
    assert np.array_equal(y2, O.qmm(x, I.pack_codes(q, 4), s, b, 4))
    assert np.array_equal(y2, O.qmm(x, I.pack_codes(q, 8), s, b, 8))


def check_points_and_threads(O):
    """Point evaluation equals the full result; thread count changes nothing."""
    d = I.random_dense(6, 37, 320, 4, seed=4)
    full = O.qmm(d.x, d.w, d.scales, d.biases, 4, threads=1)
    assert np.array_equal(full, O.qmm(d.x, d.w, d.scales, d.biases, 4, threads=3))
    rng = np.random.default_rng(1)
    r = rng.integers(0, d.M, 50)
    c = rng.integers(0, d.N, 50)
    assert np.array_equal(O.qmm_points(d.x, d.w, d.scales, d.biases, r, c, 4), full[r, c])
    g = I.random_gather([3, 1, 4], N=9, K=128, bits=8, seed=6)
    gy = O.gather_qmm(g.x, g.w, g.scales, g.biases, g.expert_idx, 8, threads=2)
    r = rng.integers(0, g.B, 30)
    c = rng.integers(0, g.N, 30)
    assert np.array_equal(
        O.gather_qmm_points(g.x, g.w, g.scales, g.biases, g.expert_idx, r, c, 8), gy[r, c])


def _indexed_problem(T, B, E, N, K, bits, seed):
    """Random tokens and experts per output row, unsorted, with repeats."""
    rng = np.random.default_rng(seed)
    x = I.to_bf16_bits(rng.standard_normal((T, K)))
    w = I.random_words(rng, (E, N, K * bits // 32))
    s = I.random_scales(rng, (E, N, K // 64))
    b = I.to_bf16_bits(rng.uniform(-0.2, 0.2, size=(E, N, K // 64)))
    tok = rng.integers(0, T, B).astype(np.int32)
    exp = rng.integers(0, E, B).astype(np.int32)
    return x, w, s, b, tok, exp


def check_indexed_brute_force(O):
    """The indexed gather (row r reads x[token_idx[r]] and expert expert_idx[r], any
    order) against numpy: rows gathered by fancy indexing, each expert dequantized
    densely with the byte-view unpacker, float64 matmul."""
    for bits in (2, 4, 8):
        for T, B, E, N, K in ((1, 8, 16, 9, 128), (3, 7, 5, 17, 192), (6, 20, 4, 3, 64)):
            x, w, s, b, tok, exp = _indexed_problem(T, B, E, N, K, bits, seed=T * 100 + B + bits)
            got = O.gather_qmm_indexed(x, w, s, b, tok, exp, bits)
            xf = I.bf16_bits_to_f64(x)
            ref = np.empty((B, N))
            for r in range(B):
                W = numpy_dequant(w[exp[r]], s[exp[r]], b[exp[r]], bits)
                ref[r] = W @ xf[tok[r]]
            assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max()), (bits, T, B)
            # without a token index, row r reads activation row r
            xr = x[tok]
            assert np.array_equal(O.gather_qmm_indexed(xr, w, s, b, None, exp, bits), got)


def check_indexed_constant(O):
    """q = 0, b[e] = e + 1, x[t,:] = (t mod 7) + 1, tokens and experts unsorted:
    y[r,n] = K (e_r + 1)((tok_r mod 7) + 1) exactly; a mis-gathered token or expert
    gives a wrong integer. Out-of-range ids give zero rows."""
    T, E, N, K = 9, 6, 5, 128
    tok = np.array([3, 0, 8, 8, 1, 5, 2, 7, 4, 6, 0, 9, -1, 2], dtype=np.int32)
    exp = np.array([5, 0, 2, 2, 4, 1, 3, 0, 5, 1, 4, 1, 2, 6], dtype=np.int32)
    for bits in (2, 4, 8):
        w = np.zeros((E, N, K * bits // 32), dtype=np.uint32)
        s = I.to_bf16_bits(np.full((E, N, K // 64), 0.5))
        b = I.to_bf16_bits(np.broadcast_to((np.arange(E) + 1.0)[:, None, None], (E, N, K // 64)))
        xv = (np.arange(T) % 7 + 1).astype(np.float64)
        x = I.to_bf16_bits(np.broadcast_to(xv[:, None], (T, K)))
        got = O.gather_qmm_indexed(x, w, s, b, tok, exp, bits)
        ok = (tok >= 0) & (tok < T) & (exp >= 0) & (exp < E)
        want = np.where(ok[:, None], K * (exp[:, None] + 1.0) * xv[np.clip(tok, 0, T - 1)][:, None], 0.0)
        assert np.array_equal(got, want * np.ones((1, N))), bits
        assert np.array_equal(got[~ok], np.zeros((int((~ok).sum()), N)))


def check_indexed_points(O):
    """Point evaluation of the indexed gather equals its full result."""
    x, w, s, b, tok, exp = _indexed_problem(4, 12, 3, 10, 128, 4, seed=5)
    full = O.gather_qmm_indexed(x, w, s, b, tok, exp, 4, threads=2)
    rng = np.random.default_rng(3)
    r = rng.integers(0, 12, 40)
    c = rng.integers(0, 10, 40)
    assert np.array_equal(O.gather_qmm_indexed(x, w, s, b, tok, exp, 4, rows=r, cols=c), full[r, c])


# ---------------------------------------------------------------------------
# binary16 and the dense grouped product (gather_mm)
# ---------------------------------------------------------------------------

def check_f16_golden(O):
    """Rounding to binary16 and widening back, against hand-derived bit patterns."""
    for v, bits, exact in read_f16_golden():
        got = int(O.f64_to_f16(np.array([v]))[0])
        assert got == bits, f"f16({v!r}) = {got:#06x}, expected {bits:#06x}"
        if exact:
            back = float(O.f16_to_f64(np.array([bits], dtype=np.uint16))[0])
            assert back == v and np.signbit(back) == np.signbit(v), f"f16 {bits:#06x} -> {back!r}"


def check_f16_vs_numpy(O):
    """Widening: every one of the 65536 patterns against numpy's float16. Rounding:
    numpy converts float64 to float16 to nearest even in one step; random doubles,
    exact ties and near-ties at every exponent agree bit for bit."""
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float64)
    got = O.f16_to_f64(h)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    rng = np.random.default_rng(21)
    v = rng.standard_normal(3000) * np.exp2(rng.integers(-30, 18, 3000))
    fin = ref[np.isfinite(ref)]
    mids = (np.sort(np.unique(fin))[1:] + np.sort(np.unique(fin))[:-1]) / 2  # exact ties
    v = np.concatenate([v, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf)])
    with np.errstate(over="ignore"):
        want = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(O.f64_to_f16(v), want)


def _dense_problem(T, B, E, N, K, dtype, layout, seed):
    """Random x and W (bf16 or binary16 bit patterns), tokens and experts unsorted."""
    rng = np.random.default_rng(seed)
    xv = rng.standard_normal((T, K))
    wshape = (E, N, K) if layout == "nk" else (E, K, N)
    wv = rng.standard_normal(wshape) * 0.1
    if dtype == "bf16":
        x, w = I.to_bf16_bits(xv), I.to_bf16_bits(wv)
    else:
        x, w = xv.astype(np.float16).view(np.uint16), wv.astype(np.float16).view(np.uint16)
    tok = rng.integers(0, T, B).astype(np.int32)
    exp = rng.integers(0, E, B).astype(np.int32)
    return x, w, tok, exp


def _numpy_operand(h, dtype):
    return I.bf16_bits_to_f64(h) if dtype == "bf16" else h.view(np.float16).astype(np.float64)


def check_gather_mm_brute_force(O):
    """gather_mm against numpy: rows gathered by fancy indexing, operands widened by
    numpy (bf16 by a 16-bit shift, binary16 by numpy's own float16), each expert's
    [N, K] matrix (the [K, N] layout transposed by numpy) in a float64 matmul."""
    for dtype in ("bf16", "f16"):
        for layout in ("nk", "kn"):
            for T, B, E, N, K in ((1, 8, 16, 9, 16), (3, 7, 5, 17, 40), (6, 20, 4, 3, 7)):
                x, w, tok, exp = _dense_problem(T, B, E, N, K, dtype, layout,
                                                seed=T * 100 + B + len(dtype) + len(layout))
                got = O.gather_mm(x, w, tok, exp, dtype, layout)
                xf = _numpy_operand(x, dtype)
                wf = _numpy_operand(w, dtype)
                if layout == "kn":
                    wf = np.ascontiguousarray(np.transpose(wf, (0, 2, 1)))
                ref = np.stack([wf[exp[r]] @ xf[tok[r]] for r in range(B)])
                assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max()), \
                    (dtype, layout, T, B)
                # without a token index, row r reads activation row r
                assert np.array_equal(O.gather_mm(x[tok], w, None, exp, dtype, layout), got)


def check_gather_mm_integer_exact(O):
    """Integer-valued x and W (exact in both formats): every sum is an integer that
    int64 arithmetic gives exactly; the two layouts agree with each other."""
    rng = np.random.default_rng(8)
    T, B, E, N, K = 5, 12, 3, 11, 48
    xi = rng.integers(-8, 9, size=(T, K))
    wi = rng.integers(-8, 9, size=(E, N, K))
    tok = rng.integers(0, T, B).astype(np.int32)
    exp = rng.integers(0, E, B).astype(np.int32)
    want = np.stack([wi[exp[r]] @ xi[tok[r]] for r in range(B)]).astype(np.float64)
    for dtype in ("bf16", "f16"):
        if dtype == "bf16":
            x, w = I.to_bf16_bits(xi.astype(np.float64)), I.to_bf16_bits(wi.astype(np.float64))
        else:
            x, w = xi.astype(np.float16).view(np.uint16), wi.astype(np.float16).view(np.uint16)
        assert np.array_equal(O.gather_mm(x, w, tok, exp, dtype, "nk"), want), dtype
        wt = np.ascontiguousarray(np.transpose(w, (0, 2, 1)))
        assert np.array_equal(O.gather_mm(x, wt, tok, exp, dtype, "kn"), want), dtype


def check_gather_mm_constant(O):
    """W[e] = e + 1 everywhere, x[t,:] = (t mod 7) + 1: y[r,n] = K (e_r + 1)((t_r mod 7) + 1)
    exactly (a mis-gathered token or expert gives a wrong integer); out-of-range ids
    give zero rows."""
    T, E, N, K = 9, 6, 5, 32
    tok = np.array([3, 0, 8, 8, 1, 5, 2, 7, 4, 6, 0, 9, -1, 2], dtype=np.int32)
    exp = np.array([5, 0, 2, 2, 4, 1, 3, 0, 5, 1, 4, 1, 2, 6], dtype=np.int32)
    xv = (np.arange(T) % 7 + 1).astype(np.float64)
    ok = (tok >= 0) & (tok < T) & (exp >= 0) & (exp < E)
    want = np.where(ok[:, None], K * (exp[:, None] + 1.0) * xv[np.clip(tok, 0, T - 1)][:, None], 0.0)
    want = want * np.ones((1, N))
    wv = np.broadcast_to((np.arange(E) + 1.0)[:, None, None], (E, N, K))
    for dtype in ("bf16", "f16"):
        enc = I.to_bf16_bits if dtype == "bf16" else (lambda a: np.asarray(a).astype(np.float16).view(np.uint16))
        x = enc(np.broadcast_to(xv[:, None], (T, K)))
        w = enc(wv)
        assert np.array_equal(O.gather_mm(x, w, tok, exp, dtype, "nk"), want), dtype
        wt = np.ascontiguousarray(np.transpose(w, (0, 2, 1)))
        assert np.array_equal(O.gather_mm(x, wt, tok, exp, dtype, "kn"), want), dtype


def check_gather_mm_points(O):
    """Point evaluation equals the full result, for either layout and thread count."""
    for layout in ("nk", "kn"):
        x, w, tok, exp = _dense_problem(4, 12, 3, 10, 24, "bf16", layout, seed=6)
        full = O.gather_mm(x, w, tok, exp, "bf16", layout, threads=3)
        rng = np.random.default_rng(4)
        r = rng.integers(0, 12, 40)
        c = rng.integers(0, 10, 40)
        assert np.array_equal(O.gather_mm(x, w, tok, exp, "bf16", layout, rows=r, cols=c), full[r, c])
        assert np.array_equal(O.gather_mm(x, w, tok, exp, "bf16", layout, threads=1), full)


ALL_CHECKS = [
    check_bf16_golden,
    check_bf16_vs_torch,
    check_unpack_golden,
    check_weight_definition,
    check_brute_force,
    check_brute_force_groups,
    check_integer_exact,
    check_one_hot,
    check_closed_form,
    check_bias_linearity,
    check_constant_per_expert,
    check_invalid_expert_rows,
    check_gather_consistency,
    check_repack_8bit,
    check_points_and_threads,
    check_indexed_brute_force,
    check_indexed_constant,
    check_indexed_points,
    check_f16_golden,
    check_f16_vs_numpy,
    check_gather_mm_brute_force,
    check_gather_mm_integer_exact,
    check_gather_mm_constant,
    check_gather_mm_points,
]
