"""Pins for the CPU oracle: each test checks it against something other than
itself (closed forms, a textbook matrix, exact rational arithmetic, brute
force, invariants, the layout the pages print).  CPU only."""
import json
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

from oracle import brute
from sparse_attention_fp4_fp4idx_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
H128 = scipy.linalg.hadamard(128).astype(np.int64)   # Sylvester order


def f32bits(x):
    return int(np.float32(x).view(np.uint32))


# ---------------------------------------------------------------- Hadamard

def test_hadamard_constant_is_nearest_float_to_inverse_sqrt128(orc):
    C = orc.hadamard_scale()
    getcontext().prec = 60
    exact = Decimal(1) / Decimal(128).sqrt()
    c = Decimal(Fraction(float(C)).numerator) / Decimal(Fraction(float(C)).denominator)
    ulp = Decimal(float(np.spacing(C)))
    assert abs(c - exact) <= ulp / 2
    assert f32bits(C) == 0x3DB504F3


def test_fwht_equals_sylvester_matrix_on_small_integers(orc):
    """|x| <= 4 integers: every butterfly sum is exact in fp32, so the fast
    transform must equal fp32(C * (H x)) with H from scipy, bit for bit."""
    rng = np.random.default_rng(1)
    C = orc.hadamard_scale()
    for _ in range(50):
        x = rng.integers(-4, 5, 128)
        got = orc.fwht128(x.astype(np.float32))
        want = np.float32(C) * (H128 @ x).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_fwht_basis_vectors_give_hadamard_columns(orc):
    C = orc.hadamard_scale()
    for i in (0, 1, 5, 64, 127):
        e = np.zeros(128, np.float32)
        e[i] = 1.0
        got = orc.fwht128(e)
        assert np.array_equal(got, (np.float32(C) * H128[:, i].astype(np.float32)))


def test_fwht_orthonormal_involution_and_parseval(orc):
    rng = np.random.default_rng(2)
    for _ in range(20):
        x = rng.standard_normal(128).astype(np.float32)
        y = orc.fwht128(x)
        xx = orc.fwht128(y)
        assert np.allclose(xx, x, rtol=0, atol=1e-5 * np.abs(x).max())
        assert abs(np.linalg.norm(y.astype(np.float64)) / np.linalg.norm(x.astype(np.float64)) - 1) < 1e-6
        # against the exact orthonormal transform in fp64
        ref = (H128 @ x.astype(np.float64)) / np.sqrt(128.0)
        assert np.max(np.abs(y - ref)) <= 1e-5 * np.abs(ref).max()


def test_fwht_sign_flip_of_stage_breaks_matrix_pin(orc):
    """Sanity of the pin itself: a transform with one stage's sign swapped is
    a different matrix, which the integer pin above would reject."""
    x = np.zeros(128); x[3] = 1
    wrong = H128.copy(); wrong[:, 3] *= -1
    assert not np.array_equal(H128 @ x, wrong @ x)


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_constant_vector_closed_form(orc):
    g = np.ones(128, np.float32)
    for a in (0.5, 3.0, -2.0, 1.0, 7.25):
        for eps in (0.0, 1e-6):
            y = orc.rmsnorm128(np.full(128, a, np.float32), g, eps)
            exact = a / np.sqrt(a * a + np.float64(np.float32(eps)))
            assert np.all(np.abs(y - exact) <= 4 * np.spacing(np.float32(abs(exact))))


def test_rmsnorm_power_of_two_scale_invariance(orc):
    rng = np.random.default_rng(3)
    g = W.f32_from_bf16(W.norm_weight(rng))
    x = W.f32_from_bf16(W.bf16_normal(rng, 128))
    y0 = orc.rmsnorm128(x, g, 0.0)
    for k in (-3, 1, 5):
        yk = orc.rmsnorm128(x * np.float32(2.0 ** k), g, 0.0)
        assert np.array_equal(y0.view(np.uint32), yk.view(np.uint32))


def test_rmsnorm_unit_mean_square_and_exact_bound(orc):
    rng = np.random.default_rng(4)
    for _ in range(20):
        x = W.f32_from_bf16(W.bf16_normal(rng, 128))
        y = orc.rmsnorm128(x, np.ones(128, np.float32), 1e-6)
        assert abs(np.mean(y.astype(np.float64) ** 2) - 1.0) < 1e-5
        # exact sum of squares (rational), then the real-valued normalisation
        S = sum(Fraction(float(v)) ** 2 for v in x)
        ms = float(S / 128)
        exact = x.astype(np.float64) / np.sqrt(ms + float(np.float32(1e-6)))
        assert np.max(np.abs(y - exact) / np.abs(exact).max()) < 2e-6


def test_rmsnorm_weight_is_applied_last(orc):
    rng = np.random.default_rng(5)
    x = W.f32_from_bf16(W.bf16_normal(rng, 128))
    y1 = orc.rmsnorm128(x, np.ones(128, np.float32), 1e-6)
    g = np.float32(2.0) ** rng.integers(-2, 3, 128).astype(np.float32)   # powers of two: exact product
    yg = orc.rmsnorm128(x, g, 1e-6)
    assert np.array_equal(yg, y1 * g)


# ---------------------------------------------------------------- RoPE

def test_rope_position_zero_is_identity(orc):
    tab = W.f32_from_bf16(W.rope_table(4))
    assert np.all(tab[0, :32] == 1) and np.all(tab[0, 32:] == 0)
    rng = np.random.default_rng(6)
    y = rng.standard_normal(128).astype(np.float32)
    assert np.array_equal(orc.rope64(y, tab[0]), y)


def test_rope_unit_vectors_pick_table_entries(orc):
    tab = W.f32_from_bf16(W.rope_table(100))
    cs = tab[97]
    for j in (0, 7, 31):
        e = np.zeros(128, np.float32); e[j] = 1
        out = orc.rope64(e, cs)
        assert out[j] == cs[j] and out[j + 32] == cs[32 + j]
        e = np.zeros(128, np.float32); e[j + 32] = 1
        out = orc.rope64(e, cs)
        assert out[j] == -cs[32 + j] and out[j + 32] == cs[j]
    e = np.zeros(128, np.float32); e[64:] = np.arange(64)
    assert np.array_equal(orc.rope64(e, cs), e)


def test_rope_is_a_complex_rotation(orc):
    tab = W.f32_from_bf16(W.rope_table(5000))
    rng = np.random.default_rng(7)
    for p in (1, 123, 4999):
        y = rng.standard_normal(128).astype(np.float32)
        out = orc.rope64(y, tab[p])
        z = (y[:32].astype(np.float64) + 1j * y[32:64]) * (tab[p, :32].astype(np.float64) + 1j * tab[p, 32:])
        assert np.max(np.abs(out[:32] - z.real)) < 1e-6 * 8
        assert np.max(np.abs(out[32:64] - z.imag)) < 1e-6 * 8
        assert np.array_equal(out[64:], y[64:])


# ---------------------------------------------------------------- FP4 / UE8M0

def test_golden_e2m1_grid_matches_oracle_codes(orc):
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_grid.txt")) if l.strip() and not l.startswith("#")]
    for code_s, val_s in rows:
        code, val = int(code_s), float(val_s)
        for e in (-5, 0, 3):
            z = np.float32(val * 2.0 ** e)
            if val == 0.0:
                z = np.float32(-0.0) if code == 8 else np.float32(0.0)
            assert orc.e2m1_code(z, e) == code
        # and the exact decoder agrees
        b = np.array([code | (code << 4)] * 64, np.uint8)
        dec = orc.dequant128(b, np.array([127] * 4, np.uint8))
        assert dec[0] == val and dec[1] == val


def test_block_exponent_against_exact_definition(orc):
    edge = []
    for k in (-130, -127, -126, -20, -1, 0, 1, 50, 125):
        base = 6.0 * 2.0 ** k
        for f in (1.0, 1.0 - 2 ** -24, 1.0 + 2 ** -23, 0.5, 0.75, 0.5000001):
            v = np.float32(base * f)
            if np.isfinite(v):
                edge.append(v)
    edge += [np.float32(0.0), np.float32(1e-45), np.float32(1.17e-38), np.float32(3.4e38), np.float32(1.0)]
    rng = np.random.default_rng(8)
    edge += list((rng.standard_normal(300) * 10.0 ** rng.integers(-30, 30, 300)).astype(np.float32))
    for v in edge:
        a = abs(np.float32(v))
        assert orc.block_exponent(a) == brute.block_exponent(a), a


def test_block_max_lands_in_upper_half_of_grid(orc):
    rng = np.random.default_rng(9)
    for _ in range(2000):
        a = np.float32(abs(rng.standard_normal()) * 10.0 ** rng.integers(-20, 20))
        if a == 0:
            continue
        e = orc.block_exponent(a)
        r = Fraction(float(a)) / Fraction(2) ** e
        assert Fraction(3) < r <= Fraction(6)


def test_midpoints_round_to_even_code(orc):
    # midpoint -> expected magnitude code (even)
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for m, c in cases.items():
        for e in (-3, 0, 2):
            assert orc.e2m1_code(np.float32(m * 2.0 ** e), e) == c
            assert orc.e2m1_code(np.float32(-m * 2.0 ** e), e) == c | 8
    # a hair above / below each midpoint goes to the nearer value
    for m, c in cases.items():
        up = np.nextafter(np.float32(m), np.float32(10))
        dn = np.nextafter(np.float32(m), np.float32(-10))
        assert orc.e2m1_code(up, 0) == (c if c % 2 == 1 else max(c, 0)) or orc.e2m1_code(up, 0) == c + 1
        assert orc.e2m1_code(up, 0) in (c, c + 1) and orc.e2m1_code(dn, 0) in (c, c - 1)
    assert orc.e2m1_code(np.float32(-0.0), 0) == 8
    assert orc.e2m1_code(np.float32(-0.1), 0) == 8


def test_e2m1_rounding_exhaustive_band(orc):
    """Every fp32 in [1/8, 8) at exponent 0 (and its negative), plus every
    4099th pattern below 1/8 (zero, subnormals, tiny normals), against an
    independent threshold formulation of nearest-even onto the grid."""
    lo, hi = 0x3E000000, 0x41000000
    step = 1 << 24
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    chunks = [np.arange(0, lo, 4099, dtype=np.uint32)]
    chunks += [np.arange(a, min(a + step, hi), dtype=np.uint32) for a in range(lo, hi, step)]
    for bits in chunks:
        start = int(bits[0])
        v = bits.view(np.float32)
        got = orc.e2m1_codes(v, 0)
        # count of midpoints strictly below v, +1 where v equals a midpoint whose upper neighbour is even
        k = np.searchsorted(mids, v, side="left").astype(np.int64)
        eq = np.isin(v, mids)
        up_even = np.isin(v, mids[[1, 3, 5]])   # 0.75 -> 1.0 (2), 1.75 -> 2 (4), 3.5 -> 4 (6)
        want = k + (eq & up_even)
        want = np.minimum(want, 7)
        assert np.array_equal(got.astype(np.int64), want), start
        gotn = orc.e2m1_codes(-v[1:], 0)
        assert np.array_equal(gotn.astype(np.int64), want[1:] | 8)


def test_e2m1_rounding_matches_fraction_brute_force_sample(orc):
    rng = np.random.default_rng(10)
    for _ in range(400):
        e = int(rng.integers(-127, 126))
        z = np.float32(rng.uniform(-6.5, 6.5) * 2.0 ** e)
        assert orc.e2m1_code(z, e) == brute.e2m1_code(z, e)


# ---------------------------------------------------------------- layout / footprint

def test_golden_split_layout_and_68_byte_footprint(orc):
    lay = json.load(open(os.path.join(GOLDEN, "split_layout.json")))
    assert lay["payload_bytes_per_token"] + lay["scale_bytes_per_token"] == lay["bytes_per_token"] == 68
    pages = 3
    page_payload = int(np.prod(lay["payload_shape_per_page"]))
    page_scale = int(np.prod(lay["scale_shape_per_page"]))
    assert page_payload == 64 * lay["tokens_per_page"] and page_scale == 4 * lay["tokens_per_page"]
    rng = np.random.default_rng(12)
    tab = W.rope_table(64)
    for slot in (0, 63, 64, 130, 191):
        pay = np.full(pages * page_payload, 0xA5, np.uint8)
        sc = np.full(pages * page_scale, 0x5A, np.uint8)
        k = W.bf16_normal(rng, (1, 128))
        orc.write_k(k, np.array([5], np.int32), np.array([slot], np.int32), W.norm_weight(rng), 1e-6, tab, pay, sc)
        # touched bytes = exactly those at [page, 0, :, t, :] and [page, 0, :, t]
        pv = pay.reshape(pages, *lay["payload_shape_per_page"])
        sv = sc.reshape(pages, *lay["scale_shape_per_page"])
        page, t = divmod(slot, 64)
        mask_p = np.zeros(pv.shape, bool); mask_p[page, 0, :, t, :] = True
        mask_s = np.zeros(sv.shape, bool); mask_s[page, 0, :, t] = True
        assert np.all(pv[~mask_p] == 0xA5) and np.all(sv[~mask_s] == 0x5A)
        changed = int(np.sum(pv[mask_p] != 0xA5) + np.sum(sv[mask_s] != 0x5A))
        assert changed <= 68 and np.sum(mask_p) + np.sum(mask_s) == 68
        assert np.all(sv[mask_s] != 0x5A)


def test_negative_slot_skips_and_duplicates_are_rejected(orc):
    tab = W.rope_table(16)
    rng = np.random.default_rng(13)
    pay = np.full(4096, 7, np.uint8); sc = np.full(256, 7, np.uint8)
    k = W.bf16_normal(rng, (2, 128))
    orc.write_k(k, np.array([1, 2], np.int32), np.array([-1, -5], np.int32), W.norm_weight(rng), 1e-6, tab, pay, sc)
    assert np.all(pay == 7) and np.all(sc == 7)
    with pytest.raises(orc.OracleError):
        orc.write_k(k, np.array([1, 2], np.int32), np.array([3, 3], np.int32), W.norm_weight(rng), 1e-6, tab, pay, sc)
    with pytest.raises(orc.OracleError):
        orc.write_k(k, np.array([1, 2], np.int32), np.array([3, 64], np.int32), W.norm_weight(rng), 1e-6, tab, pay, sc)


def test_encoding_decodes_to_the_fp64_pipeline_within_quantisation_error(orc):
    """End-to-end K: decode the pool through the page shapes (brute decoder)
    and compare with RMSNorm -> complex-rotation RoPE -> scipy Hadamard in
    fp64.  Error per element must stay within half an FP4 step at its block
    scale (plus fp32 slack).  Catches nibble order, block order, scale byte,
    sign and operand mix-ups."""
    rng = np.random.default_rng(14)
    tab = W.rope_table(4096)
    n = 64
    k = W.bf16_normal(rng, (n, 128))
    g = W.norm_weight(rng)
    pos = rng.integers(0, 4096, n).astype(np.int32)
    slot = rng.permutation(128)[:n].astype(np.int32)
    pay = np.zeros(2 * 4096, np.uint8); sc = np.zeros(2 * 256, np.uint8)
    orc.write_k(k, pos, slot, g, 1e-6, tab, pay, sc)
    tabf = W.f32_from_bf16(tab).astype(np.float64)
    for i in range(n):
        x = W.f32_from_bf16(k[i]).astype(np.float64)
        y = x / np.sqrt(np.mean(x * x) + 1e-6) * W.f32_from_bf16(g)
        z = (y[:32] + 1j * y[32:64]) * (tabf[pos[i], :32] + 1j * tabf[pos[i], 32:])
        y[:32], y[32:64] = z.real, z.imag
        ref = (H128 @ y) / np.sqrt(128.0)
        codes, scs = brute.pool_token(pay, sc, slot[i])
        dec = np.array([float(v) for v in brute.decode_vector(codes, scs)])
        for j in range(4):
            blk = slice(32 * j, 32 * j + 32)
            e = int(scs[j]) - 127
            assert e == brute.block_exponent(np.float32(np.abs(ref[blk]).max())) or \
                abs(np.abs(ref[blk]).max() / 2.0 ** e - 6) < 1e-4 or abs(np.abs(ref[blk]).max() / 2.0 ** e - 3) < 1e-4
            half_step = np.where(np.abs(ref[blk]) / 2.0 ** e < 2, 0.25, np.where(np.abs(ref[blk]) / 2.0 ** e < 4, 0.5, 1.0))
            assert np.all(np.abs(dec[blk] - ref[blk]) <= half_step * 2.0 ** e + 1e-4), (i, j)


def test_q_pack_matches_k_encoding_without_norm(orc):
    rng = np.random.default_rng(15)
    tab = W.rope_table(512)
    q = W.bf16_normal(rng, (3, 4, 128))
    pos = np.array([0, 17, 511], np.int32)
    w = rng.uniform(0, 1, (3, 4)).astype(np.float32)
    qf, qs, wo = orc.pack_q(q, pos, tab, w, 0.5)
    assert np.array_equal(wo, w * np.float32(0.5))
    for t in range(3):
        for h in range(4):
            c, s = orc.encode_q_head(q[t, h], tab[pos[t]])
            assert np.array_equal(qf[t, h], c) and np.array_equal(qs[t, h], s)
            # Q encoding = K encoding of an input whose RMSNorm is the identity:
            # x with mean square 1 exactly and g = 1, eps = 0 -> r = 1
    x = np.ones(128, np.float32)
    y = orc.rmsnorm128(x, np.ones(128, np.float32), 0.0)
    assert np.array_equal(y, x)
    kq = W.bf16_from_f32(np.ones(128, np.float32))
    ck, sk = orc.encode_k_token(kq, W.bf16_from_f32(np.ones(128, np.float32)), 0.0, tab[9])
    cq, sq = orc.encode_q_head(kq, tab[9])
    assert np.array_equal(ck, cq) and np.array_equal(sk, sq)


# ---------------------------------------------------------------- logits

def _tiny_logit_problem(rng, H=3, ctx=(5, 70), rows=(1, 2)):
    B = len(rows)
    indptr = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    T = int(indptr[-1])
    row_ctx = np.concatenate([[c] * r for c, r in zip(ctx, rows)]).astype(np.int32)
    pages = [(c + 63) // 64 for c in ctx]
    num_pages = sum(pages) + 1
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.full((B, max(pages)), -1, np.int32)
    cur = 0
    for b in range(B):
        bt[b, :pages[b]] = perm[cur:cur + pages[b]]; cur += pages[b]
    payload, scale = W.random_pool(rng, num_pages, 120, 132)
    qf = rng.integers(0, 256, (T, H, 64)).astype(np.uint8)
    qs = rng.integers(122, 130, (T, H, 4)).astype(np.uint8)
    w = rng.uniform(-1, 1, (T, H)).astype(np.float32)
    return qf, qs, w, indptr, row_ctx, bt, payload, scale


def test_logits_against_exact_rational_brute_force(orc):
    rng = np.random.default_rng(16)
    qf, qs, w, indptr, row_ctx, bt, pay, sc = _tiny_logit_problem(rng)
    out, f64, tol, _ = orc.logits(qf, qs, w, indptr, row_ctx, bt, pay, sc, logits_stride=80, want_f64=True)
    for b in range(len(indptr) - 1):
        for t in range(indptr[b], indptr[b + 1]):
            for s in range(row_ctx[t]):
                kc, ks = brute.pool_token(pay, sc, bt[b, s // 64] * 64 + s % 64)
                ex = brute.logit(qf[t], qs[t], w[t], kc, ks)
                assert f64[t, s] == float(ex) or abs(f64[t, s] - float(ex)) <= 1e-12 * abs(float(ex))
                assert out[t, s] == np.float32(float(ex))
            assert np.all(np.isnan(out[t, row_ctx[t]:]))


def test_logits_special_cases(orc):
    rng = np.random.default_rng(17)
    # one head, w = 1: ReLU(q.k); k = 0 -> 0; q = k -> |q|^2
    pay = np.zeros(4096, np.uint8); sc = np.full(256, 127, np.uint8)
    q = rng.integers(0, 256, (1, 1, 64)).astype(np.uint8)
    qs = np.full((1, 1, 4), 127, np.uint8)
    pay.reshape(1, 1, 4, 64, 16)[0, 0, :, 1, :] = q[0, 0].reshape(4, 16)     # token 1 = q
    neg = q[0, 0] ^ 0x88                                                     # token 2 = -q
    pay.reshape(1, 1, 4, 64, 16)[0, 0, :, 2, :] = neg.reshape(4, 16)
    out = orc.logits(q, qs, np.ones((1, 1), np.float32), np.array([0, 1], np.int32), np.array([3], np.int32),
                     np.array([[0]], np.int32), pay, sc, logits_stride=3)
    qv = np.array([float(v) for v in brute.decode_vector(q[0, 0], qs[0, 0])])
    assert out[0, 0] == 0.0                     # token 0 is all-zero codes
    assert out[0, 1] == np.float32(np.dot(qv, qv))
    assert out[0, 2] == 0.0                     # ReLU of a negative dot product


def test_logits_integer_lut_formulation_agrees(orc):
    """Cross-check the dequantise-and-multiply definition with the integer
    form: per block, sum of (2q)(2k) code products times 2^(eq+ek-2)."""
    rng = np.random.default_rng(18)
    qf, qs, w, indptr, row_ctx, bt, pay, sc = _tiny_logit_problem(rng, H=4, ctx=(33,), rows=(2,))
    out, f64, _, _ = orc.logits(qf, qs, w, indptr, row_ctx, bt, pay, sc, logits_stride=33, want_f64=True)
    twice = np.array([0, 1, 2, 3, 4, 6, 8, 12], np.int64)

    def ints(codes):
        lo, hi = codes & 15, codes >> 4
        c = np.stack([lo, hi], -1).reshape(*codes.shape[:-1], 128).astype(np.int64)
        return np.where(c & 8, -twice[c & 7], twice[c & 7])

    for t in range(2):
        for s in range(33):
            kc, ks = brute.pool_token(pay, sc, bt[0, s // 64] * 64 + s % 64)
            kv = ints(kc[None])[0]
            L = Fraction(0)
            for h in range(4):
                qv = ints(qf[t, h][None])[0]
                d = Fraction(0)
                for j in range(4):
                    iprod = int(np.dot(qv[32 * j:32 * j + 32], kv[32 * j:32 * j + 32]))
                    d += iprod * Fraction(2) ** (int(qs[t, h, j]) + int(ks[j]) - 254 - 2)
                if d > 0:
                    L += Fraction(float(w[t, h])) * d
            assert f64[t, s] == float(L)


def _sample_pairs(rng, row_ctx, n):
    """Random (row, token) pairs over rows with context, plus every such row's
    first and last token and the tokens on both sides of each page boundary."""
    live = np.nonzero(row_ctx > 0)[0]
    rows = rng.choice(live, n)
    toks = (rng.random(n) * row_ctx[rows]).astype(np.int64)
    er, et = [], []
    for t in live:
        c = int(row_ctx[t])
        for s in {0, c - 1, *[p for b in range(64, c, 64) for p in (b - 1, b)]}:
            er.append(t); et.append(s)
    return np.concatenate([rows, er]).astype(np.int64), np.concatenate([toks, et]).astype(np.int64)


def test_sampled_logits_checker_equals_full_logits_and_brute_force(orc):
    """orc_logits_sampled (the checker of the full-size GPU logits tests, which
    finds each sample's request from the row and its page from the block
    table) against orc_logits, which walks every row of every request, at
    random (row, token) pairs of a multi-request paged problem with permuted
    page ids and unequal row counts; and, on a subset, against the exact
    rational L, T and A of the brute force read through the page shapes."""
    rng = np.random.default_rng(23)
    qf, qs, w, indptr, row_ctx, bt, pay, sc = _tiny_logit_problem(rng, H=4, ctx=(70, 200, 5, 130),
                                                                   rows=(2, 1, 3, 2))
    stride = 200
    _, f64, tol, absr = orc.logits(qf, qs, w, indptr, row_ctx, bt, pay, sc, logits_stride=stride, want_f64=True)
    rows, toks = _sample_pairs(rng, row_ctx, 300)
    s64, sT, sA = orc.logits_sampled(qf, qs, w, indptr, bt, pay, sc, rows, toks)
    assert np.array_equal(s64, f64[rows, toks])
    assert np.array_equal(sT, tol[rows, toks]) and np.array_equal(sA, absr[rows, toks])
    req = np.searchsorted(indptr, rows, side="right") - 1
    for i in range(0, rows.size, 9):
        t, s, b = int(rows[i]), int(toks[i]), int(req[i])
        kc, ks = brute.pool_token(pay, sc, int(bt[b, s // 64]) * 64 + s % 64)
        kv = brute.decode_vector(kc, ks)
        qv = [brute.decode_vector(qf[t, h], qs[t, h]) for h in range(qf.shape[1])]
        L, T, A = brute.logit_terms(qv, w[t], kv)
        for got, want in ((s64[i], L), (sT[i], T), (sA[i], A)):
            assert abs(got - float(want)) <= 1e-12 * abs(float(want)), (t, s)


# ---------------------------------------------------------------- top-k

def _ref_topk(vals, ctx, k):
    v = vals[:ctx].astype(np.float64)
    order = np.lexsort((np.arange(ctx), -v))[:min(k, ctx)]
    out = np.full(k, -1, np.int32)
    out[:order.size] = np.sort(order)
    return out


def test_topk_full_sort_ties_and_edges(orc):
    rng = np.random.default_rng(19)
    T, S, k = 7, 300, 50
    vals = rng.integers(-5, 6, (T, S)).astype(np.float32)       # heavy ties
    vals[1] = rng.standard_normal(S).astype(np.float32)         # no ties
    vals[2, :] = -0.0; vals[2, ::3] = 0.0                       # signed zeros are equal
    ctx = np.array([300, 299, 120, 50, 10, 0, 1], np.int32)
    got = orc.topk(vals, ctx, k)
    for t in range(T):
        assert np.array_equal(got[t], _ref_topk(vals[t], ctx[t], k)), t
    assert np.all(got[5] == -1)
    assert np.array_equal(got[4][:10], np.arange(10)) and np.all(got[4][10:] == -1)
    assert np.array_equal(got[3], np.arange(50))
    assert np.array_equal(got[2], np.arange(50))                 # all equal -> lowest positions


# ---------------------------------------------------------------- split-pool reader

def test_reader_matches_exact_decoding_through_the_page_shapes(orc):
    """The reader against exact rational decoding of the same bytes read
    through the printed page shapes [P,1,4,64,16] / [P,1,4,64] ([P2]
    Motivation); scale bytes 0..254 cover the subnormal and near-overflow
    ends, and slots outside the pool read as zeros."""
    rng = np.random.default_rng(61)
    P = 3
    pay = rng.integers(0, 256, P * 4096).astype(np.uint8)
    sc = rng.integers(0, 255, P * 256).astype(np.uint8)
    sc[:4] = [0, 1, 253, 254]
    slots = np.array([0, 1, 63, 64, 130, 191, -1, P * 64, 5], np.int32)
    got = orc.read_k(pay, sc, slots)
    for i, s in enumerate(slots):
        if s < 0 or s >= P * 64:
            assert np.all(got[i] == 0.0)
            continue
        codes, scales = brute.pool_token(pay, sc, int(s))
        want = [float(v) for v in brute.decode_vector(codes, scales)]
        assert np.array_equal(got[i], np.array(want)), s
    # a planted token: element 2b in the low nibble, sign bit 8, scale 2^(byte-127)
    pay2 = np.zeros(4096, np.uint8); sc2 = np.full(256, 127, np.uint8)
    pay2[1 * 1024 + 5 * 16 + 0] = 0x9F          # token 5, block 1, byte 0: element 32 = 0xF (-6), element 33 = 0x9 (-0.5)
    sc2[1 * 64 + 5] = 129                       # block 1 of token 5 scaled by 4
    v = orc.read_k(pay2, sc2, np.array([5], np.int32))[0]
    assert v[32] == -24.0 and v[33] == -2.0 and np.count_nonzero(v) == 2


# ---------------------------------------------------------------- FP8 indexer variant

def test_golden_e4m3_values_match_oracle(orc):
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e4m3_ocp_values.txt")) if l.strip() and not l.startswith("#")]
    assert len(rows) >= 10
    for code_s, val_s in rows:
        code, val = int(code_s), float(val_s)
        assert orc.e4m3_value(code) == val and np.signbit(orc.e4m3_value(code)) == np.signbit(val)
        assert float(brute.e4m3_magnitude(code)) == abs(val)
        for e in (-9, 0, 4):      # each grid value scaled by 2^e encodes to its own code
            z = np.float32(val * 2.0 ** e)
            assert orc.e4m3_code(z, e) == code, (code, e)
    mags = [orc.e4m3_value(c) for c in range(127)]
    assert all(a < b for a, b in zip(mags, mags[1:])) and mags[-1] == 448.0


def test_fp8_exponent_against_exact_definition(orc):
    edge = []
    for k in (-140, -127, -126, -20, -1, 0, 1, 50, 119):
        base = 448.0 * 2.0 ** k
        for f in (1.0, 1.0 - 2 ** -24, 1.0 + 2 ** -23, 0.5, 0.5000001, 0.875):
            v = np.float32(base * f)
            if np.isfinite(v):
                edge.append(v)
    edge += [np.float32(0.0), np.float32(1e-45), np.float32(1.17e-38), np.float32(3.4e38), np.float32(1.0)]
    rng = np.random.default_rng(81)
    edge += list((np.abs(rng.standard_normal(300)) * 10.0 ** rng.integers(-30, 30, 300)).astype(np.float32))
    for v in edge:
        a = abs(np.float32(v))
        e = orc.fp8_exponent(a)
        assert e == brute.fp8_exponent(a), a
        if a > 448 * 2.0 ** -127:
            r = Fraction(float(a)) / Fraction(2) ** e
            assert Fraction(224) < r <= Fraction(448)


def test_fp8_codes_match_exact_nearest_even(orc):
    """Codes against rational nearest-with-ties-to-even on random values over
    many binades (subnormal range included), exact midpoints and signed zero."""
    rng = np.random.default_rng(82)
    vals = list((rng.standard_normal(400) * 2.0 ** rng.integers(-12, 10, 400)).astype(np.float32))
    # midpoints between neighbouring grid values (ties must go to the even code)
    for c in list(range(0, 20)) + list(range(60, 70)) + [120, 124, 125]:
        mid = (brute.e4m3_magnitude(c) + brute.e4m3_magnitude(c + 1)) / 2
        vals.append(np.float32(float(mid)))
        vals.append(np.float32(-float(mid)))
    vals += [np.float32(-0.0), np.float32(0.0), np.float32(448.0), np.float32(447.99997)]
    for z in vals:
        for e in (0, -3, 5):
            zz = np.float32(float(z) * 2.0 ** e)
            if abs(float(zz)) / 2.0 ** e > 448 or not np.isfinite(zz):
                continue
            assert orc.e4m3_code(zz, e) == brute.e4m3_code(zz, e), (zz, e)


def test_fp8_pool_footprint_is_132_bytes(orc):
    """Writing one token changes exactly its 128 code bytes and 4 scale bytes
    at the fused page layout, and the scale is a power of two."""
    rng = np.random.default_rng(83)
    tab = W.rope_table(64)
    pool = np.full(2 * 8448, 0xA5, np.uint8)
    k = W.bf16_normal(rng, (1, 128))
    orc.write_k_fp8(k, np.array([7], np.int32), np.array([64 + 9], np.int32), W.norm_weight(rng), 1e-6, tab, pool)
    changed = np.nonzero(pool != 0xA5)[0]
    allowed = set(range(8448 + 9 * 128, 8448 + 10 * 128)) | set(range(8448 + 8192 + 36, 8448 + 8192 + 40))
    assert set(changed.tolist()) <= allowed and len(changed) >= 128
    codes, sc = brute.fp8_pool_token(pool, 64 + 9)
    m, ex = np.frexp(np.float64(sc))
    assert m == 0.5


def test_fp8_encoding_decodes_within_half_a_step_of_the_fp64_pipeline(orc):
    rng = np.random.default_rng(84)
    tab = W.rope_table(4096)
    n = 48
    k = W.bf16_normal(rng, (n, 128)); g = W.norm_weight(rng)
    pos = rng.integers(0, 4096, n).astype(np.int32)
    slot = rng.permutation(128)[:n].astype(np.int32)
    pool = np.zeros(2 * 8448, np.uint8)
    orc.write_k_fp8(k, pos, slot, g, 1e-6, tab, pool)
    tabf = W.f32_from_bf16(tab).astype(np.float64)
    for i in range(n):
        x = W.f32_from_bf16(k[i]).astype(np.float64)
        y = x / np.sqrt(np.mean(x * x) + 1e-6) * W.f32_from_bf16(g)
        z = (y[:32] + 1j * y[32:64]) * (tabf[pos[i], :32] + 1j * tabf[pos[i], 32:])
        y[:32], y[32:64] = z.real, z.imag
        ref = (H128 @ y) / np.sqrt(128.0)
        codes, sc = brute.fp8_pool_token(pool, slot[i])
        dec = np.array([float(v) for v in brute.fp8_decode(codes, sc)])
        s = float(sc)
        a = np.abs(ref) / s
        # half a step at each value's binade (step 2^(k-3), k >= -6), plus fp32 pipeline slack
        kk = np.maximum(np.floor(np.log2(np.maximum(a, 2.0 ** -10))), -6)
        assert np.all(np.abs(dec - ref) <= 0.5 * 2.0 ** (kk - 3) * s * (1 + 1e-6) + 1e-6 * np.abs(ref).max()), i
        assert 224 < np.abs(ref).max() / s <= 448 * (1 + 1e-5)


def test_fp8_q_pack_matches_k_encoding_without_norm(orc):
    rng = np.random.default_rng(85)
    tab = W.rope_table(512)
    q = W.bf16_normal(rng, (2, 3, 128))
    pos = np.array([5, 300], np.int32)
    w = rng.uniform(0, 1, (2, 3)).astype(np.float32)
    qf, qs, wo = orc.pack_q_fp8(q, pos, tab, w, 2.0)
    assert np.array_equal(wo, w * np.float32(2.0))
    for t in range(2):
        for h in range(3):
            c, s = orc.encode_q_head_fp8(q[t, h], tab[pos[t]])
            assert np.array_equal(qf[t, h], c) and qs[t, h] == s
    kq = W.bf16_from_f32(np.ones(128, np.float32))
    ck, sk = orc.encode_k_token_fp8(kq, W.bf16_from_f32(np.ones(128, np.float32)), 0.0, tab[9])
    cq, sq = orc.encode_q_head_fp8(kq, tab[9])
    assert np.array_equal(ck, cq) and sk == sq


def test_fp8_logits_against_exact_rational_brute_force(orc):
    rng = np.random.default_rng(86)
    H, ctx, rows = 3, (5, 70), (1, 2)
    indptr = np.array([0, 1, 3], np.int32)
    row_ctx = np.array([5, 70, 70], np.int32)
    num_pages = 4
    bt = np.array([[2, -1], [0, 3]], np.int32)
    pool = np.zeros(num_pages * 8448, np.uint8)
    pv = pool.reshape(num_pages, 8448)
    codes = rng.integers(0, 256, (num_pages, 8192)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x11                           # no NaN codes
    pv[:, :8192] = codes
    pv[:, 8192:].view(np.float32)[:] = (2.0 ** rng.integers(-12, 4, (num_pages, 64))).astype(np.float32)
    qf = rng.integers(0, 256, (3, H, 128)).astype(np.uint8); qf[(qf & 0x7F) == 0x7F] = 0x22
    qs = (2.0 ** rng.integers(-6, 3, (3, H))).astype(np.float32)
    w = rng.uniform(-1, 1, (3, H)).astype(np.float32)
    out, f64, tol, _ = orc.logits_fp8(qf, qs, w, indptr, row_ctx, bt, pool, logits_stride=80, want_f64=True)
    for b in range(2):
        for t in range(indptr[b], indptr[b + 1]):
            qd = [brute.fp8_decode(qf[t, h], qs[t, h]) for h in range(H)]
            for s in range(row_ctx[t]):
                kc, ks = brute.fp8_pool_token(pool, bt[b, s // 64] * 64 + s % 64)
                kd = brute.fp8_decode(kc, ks)
                ex = sum(Fraction(float(w[t, h])) * max(sum(a * c for a, c in zip(qd[h], kd)), Fraction(0))
                         for h in range(H))
                assert abs(f64[t, s] - float(ex)) <= 1e-12 * abs(float(ex)) + 1e-300
                assert out[t, s] == np.float32(float(ex))


def test_fp8_sampled_logits_checker_equals_full_logits_and_brute_force(orc):
    """orc_logits_fp8_sampled (the checker of the full-size FP8 logits tests)
    against orc_logits_fp8 at random (row, token) pairs of a multi-request
    paged problem with permuted page ids, and on a subset against the exact
    rational L, T and A through the fused page shape."""
    rng = np.random.default_rng(87)
    H = 3
    rows_per = (2, 1, 3)
    ctxs = (130, 64, 200)
    indptr = np.concatenate([[0], np.cumsum(rows_per)]).astype(np.int32)
    row_ctx = np.concatenate([[c] * r for c, r in zip(ctxs, rows_per)]).astype(np.int32)
    row_ctx[4] = 150   # rows of one request with different contexts
    pages = [(c + 63) // 64 for c in ctxs]
    num_pages = sum(pages) + 2
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.full((3, max(pages)), -1, np.int32)
    cur = 0
    for b in range(3):
        bt[b, :pages[b]] = perm[cur:cur + pages[b]]; cur += pages[b]
    pool = np.zeros(num_pages * 8448, np.uint8)
    pv = pool.reshape(num_pages, 8448)
    codes = rng.integers(0, 256, (num_pages, 8192)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x11
    pv[:, :8192] = codes
    pv[:, 8192:].view(np.float32)[:] = (2.0 ** rng.integers(-12, 4, (num_pages, 64))).astype(np.float32)
    T = int(indptr[-1])
    qf = rng.integers(0, 256, (T, H, 128)).astype(np.uint8); qf[(qf & 0x7F) == 0x7F] = 0x22
    qs = (2.0 ** rng.integers(-6, 3, (T, H))).astype(np.float32)
    w = rng.uniform(-1, 1, (T, H)).astype(np.float32)
    _, f64, tol, absr, b16 = orc.logits_fp8(qf, qs, w, indptr, row_ctx, bt, pool, logits_stride=200,
                                             want_f64=True, want_b16=True)
    rows, toks = _sample_pairs(rng, row_ctx, 200)
    s64, sT, sA, sB = orc.logits_fp8_sampled(qf, qs, w, indptr, bt, pool, rows, toks, want_b16=True)
    assert np.array_equal(s64, f64[rows, toks])
    assert np.array_equal(sT, tol[rows, toks]) and np.array_equal(sA, absr[rows, toks])
    assert np.array_equal(sB, b16[rows, toks])
    req = np.searchsorted(indptr, rows, side="right") - 1
    for i in range(0, rows.size, 11):
        t, s, b = int(rows[i]), int(toks[i]), int(req[i])
        kc, ks = brute.fp8_pool_token(pool, int(bt[b, s // 64]) * 64 + s % 64)
        kv = brute.fp8_decode(kc, ks)
        qv = [brute.fp8_decode(qf[t, h], qs[t, h]) for h in range(H)]
        L, Tt, A = brute.logit_terms(qv, w[t], kv)
        # B16: per head the 16 largest |q_i k_i|, exactly
        B = sum(abs(Fraction(float(w[t, h]))) * sum(sorted((abs(a * c) for a, c in zip(qv[h], kv)),
                                                           reverse=True)[:16]) for h in range(H))
        for got, want in ((s64[i], L), (sT[i], Tt), (sA[i], A), (sB[i], B)):
            assert abs(got - float(want)) <= 1e-12 * abs(float(want)), (t, s)
