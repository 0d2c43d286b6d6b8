"""Exact rational brute force for tiny inputs (test infrastructure only).

Pure-Python ``fractions.Fraction`` arithmetic: no rounding anywhere.  Used by
the tests to pin the C oracle's block exponent, FP4 rounding, dequantisation
and logits on small cases.  It is written from the definitions, separately
from ``fp4idx_oracle.c`` (decode by table lookup on reshaped pool views, dot
products as exact rational sums).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

# e2m1 magnitudes by 3-bit code (OCP MX v1.0, FP4 E2M1)
GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
        Fraction(6)]


def exact(x) -> Fraction:
    """Exact rational value of a finite float."""
    return Fraction(float(x))


def block_exponent(amax) -> int:
    """Smallest integer e with 6 * 2^e >= amax, clamped to [-127, 127]."""
    a = exact(amax)
    if a == 0:
        return -127
    e = -127
    while e < 127 and Fraction(6) * Fraction(2) ** e < a:
        e += 1
    return e


def e2m1_code(z, e: int) -> int:
    """Nearest grid magnitude to |z| / 2^e, ties to the even code; sign bit 3."""
    v = abs(exact(z)) / Fraction(2) ** e
    best, bd = 0, abs(v - GRID[0])
    for c in range(1, 8):
        d = abs(v - GRID[c])
        if d < bd or (d == bd and c % 2 == 0):
            best, bd = c, d
    neg = np.signbit(np.float32(z))
    return best | (8 if neg else 0)


def decode_vector(codes64: np.ndarray, scales4: np.ndarray):
    """128 exact values from 64 packed bytes (low nibble = even element) and
    4 UE8M0 scale bytes."""
    out = []
    for i in range(128):
        b = int(codes64[i // 2])
        c = (b >> 4) if (i & 1) else (b & 15)
        m = GRID[c & 7]
        if c & 8:
            m = -m
        out.append(m * Fraction(2) ** (int(scales4[i // 32]) - 127))
    return out


def pool_token(payload: np.ndarray, scale: np.ndarray, slot: int):
    """Read one token's 64 + 4 bytes through the page shapes
    payload [P, 1, 4, 64, 16] and scale [P, 1, 4, 64]."""
    P = payload.size // 4096
    pv = payload.reshape(P, 1, 4, 64, 16)
    sv = scale.reshape(P, 1, 4, 64)
    page, t = divmod(int(slot), 64)
    codes = pv[page, 0, :, t, :].reshape(64)
    sc = sv[page, 0, :, t]
    return codes, sc


def logit(qcodes, qscales, w, kcodes, kscales) -> Fraction:
    """sum_h w_h * ReLU(qhat_h . khat), exactly.  qcodes [H,64], qscales [H,4]."""
    kv = decode_vector(kcodes, kscales)
    total = Fraction(0)
    for h in range(qcodes.shape[0]):
        qv = decode_vector(qcodes[h], qscales[h])
        d = sum((a * b for a, b in zip(qv, kv)), Fraction(0))
        if d > 0:
            total += exact(w[h]) * d
    return total


def logit_terms(qvecs, w, kv):
    """(L, T, A) exactly for dequantised vectors: L = sum_h w_h ReLU(q_h . k),
    T = sum_h |w_h| ReLU(q_h . k) and A = sum_h |w_h| sum_i |q_hi k_i| (the
    scales a floating-point evaluation's error is measured against).
    qvecs: H lists of exact values, w: H floats, kv: the token's exact values."""
    L = T = A = Fraction(0)
    for h, qv in enumerate(qvecs):
        d = sum((a * b for a, b in zip(qv, kv)), Fraction(0))
        a = sum((abs(x * y) for x, y in zip(qv, kv)), Fraction(0))
        wh = exact(w[h])
        if d > 0:
            L += wh * d
            T += abs(wh) * d
        A += abs(wh) * a
    return L, T, A


# ---- FP8 E4M3 (OCP OFP8 v1.0): bias 7, 3 mantissa bits, no infinities, S.1111.111 NaN

def e4m3_magnitude(code: int) -> Fraction:
    """Exact magnitude of an e4m3 code (sign bit ignored); codes 0x7F/0xFF are NaN."""
    ex, m = (code >> 3) & 15, code & 7
    if ex == 0:
        return Fraction(m, 8) * Fraction(2) ** -6
    return (1 + Fraction(m, 8)) * Fraction(2) ** (ex - 7)


def fp8_exponent(amax) -> int:
    """Smallest integer e with 448 * 2^e >= amax, clamped to [-127, 127]."""
    a = exact(amax)
    if a == 0:
        return -127
    e = -127
    while e < 127 and Fraction(448) * Fraction(2) ** e < a:
        e += 1
    return e


def e4m3_code(z, e: int) -> int:
    """Nearest e4m3 magnitude to |z| / 2^e, ties to the even code; sign bit 7."""
    v = abs(exact(z)) / Fraction(2) ** e
    best, bd = 0, v
    for c in range(1, 127):
        d = abs(v - e4m3_magnitude(c))
        if d < bd or (d == bd and c % 2 == 0):
            best, bd = c, d
    neg = np.signbit(np.float32(z))
    return best | (0x80 if neg else 0)


def fp8_pool_token(pool: np.ndarray, slot: int):
    """One token of the fused FP8 pool through its page shape: 64 x 128 code
    bytes, then 64 fp32 scales."""
    P = pool.size // 8448
    pages = pool.reshape(P, 8448)
    page, t = divmod(int(slot), 64)
    codes = pages[page, :8192].reshape(64, 128)[t]
    scale = pages[page, 8192:].view(np.float32)[t]
    return codes, scale


def fp8_decode(codes, scale):
    """128 exact values of an FP8 token (codes + fp32 power-of-two scale)."""
    s = exact(scale)
    return [(-1 if c & 0x80 else 1) * e4m3_magnitude(int(c)) * s for c in codes]
