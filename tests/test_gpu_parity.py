"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: encoder bytes (payload, scale, packed Q) and top-k indices bit-exact;
logits within |gpu - exact| <= 1e-5 * T + 4 * 2^-24 * A, where, for each
(row, token), T = sum_h |w_h| max(d_h, 0) (the quantity the 1e-5 relative
tolerance refers to) and A = sum_h |w_h| sum_i |q_hi k_i| (what the FP4
MFMA's rounding of a head's four block sums can lose when the dot product
cancels; derivation in tests/bars.py).  Each check reports its worst err / T.
Inputs come from the seeded generators; expected values from the oracle only.
"""
import numpy as np
import pytest
import torch

from bars import check_fp4, fp4_bound, in_context
from sparse_attention_fp4_fp4idx_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from sparse_attention_fp4_fp4idx_amd import fp4idx
    fp4idx.load()
    return fp4idx


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bf16(a):
    return dev(a.view(np.int16)).view(torch.bfloat16)


def say(*a):
    print(*a, flush=True)


def check_rows(gpu, f64, T, A, ctx, where):
    """Every row's [0, ctx) against the bar, in one check."""
    m = in_context(ctx, gpu.shape[1])
    check_fp4(gpu[m], f64[:, :gpu.shape[1]][m], T[:, :gpu.shape[1]][m], A[:, :gpu.shape[1]][m], where)


# ---------------------------------------------------------------- K writer

def _write_both(F, orc, k, pos, slot, norm_w, eps, tab, num_pages, k_row_stride=None):
    pay_o = np.full(num_pages * 4096, 0xA5, np.uint8)
    sc_o = np.full(num_pages * 256, 0x5A, np.uint8)
    orc.write_k(k, pos, slot, norm_w, eps, tab, pay_o, sc_o)
    pay_g = dev(np.full(num_pages * 4096, 0xA5, np.uint8))
    sc_g = dev(np.full(num_pages * 256, 0x5A, np.uint8))
    kk = k
    if k_row_stride is not None and k_row_stride != 128:
        kk = np.zeros((k.shape[0], k_row_stride), np.uint16)
        kk[:, :128] = k
        kt = bf16(kk)[:, :128]
    else:
        kt = bf16(kk)
    F.write_k(kt, dev(pos), dev(slot), bf16(norm_w), eps, bf16(tab), pay_g, sc_g)
    torch.cuda.synchronize()
    return pay_o, sc_o, pay_g.cpu().numpy(), sc_g.cpu().numpy()


def test_write_k_small_ragged_bit_exact(F, orc):
    wl = W.small()
    say("write_k small: tokens", wl.k_new.shape[0], "pages", wl.num_pages)
    tab = W.rope_table(wl.max_pos)
    po, so, pg, sg = _write_both(F, orc, wl.k_new, wl.pos_new, wl.slot_new, wl.norm_w, wl.eps, tab, wl.num_pages)
    assert np.array_equal(po, pg) and np.array_equal(so, sg)


@pytest.mark.parametrize("n", [300, 20000])   # a partial block and a multi-wave batch; neither a multiple of the block
def test_write_k_edges_strided_skip_extremes(F, orc, n):
    rng = np.random.default_rng(21)
    tab = W.rope_table(4096)
    k = W.bf16_normal(rng, (n, 128))
    k[0] = 0                                  # all-zero row: amax 0 -> scale byte 0
    k[1] = W.bf16_from_f32(np.full(128, 3.0, np.float32))
    k[2, :] = W.bf16_from_f32(rng.standard_normal(128).astype(np.float32) * 1e-30)   # tiny
    k[3, :] = W.bf16_from_f32(rng.standard_normal(128).astype(np.float32) * 1e30)    # huge
    pos = rng.integers(0, 4096, n).astype(np.int32)
    pos[:2] = [0, 4095]
    pages = (n + 63) // 64 + 2
    slot = rng.permutation(pages * 64)[:n].astype(np.int32)
    slot[5] = -1
    slot[17] = -7
    for eps in (1e-6, 0.0):
        sl = slot.copy()
        if eps == 0.0:
            sl[[0, 2]] = -1   # zero / underflowing rows: 1/sqrt(0) is outside the finite-value contract
        po, so, pg, sg = _write_both(F, orc, k, pos, sl, W.norm_weight(rng), eps, tab, pages, k_row_stride=136)
        assert np.array_equal(po, pg) and np.array_equal(so, sg), eps


def test_write_k_skips_tokens_outside_pool_or_table(F, orc):
    """A slot past the pool or a position outside the table skips the token
    (the kernel's own range checks): the pools equal the oracle's with those
    tokens marked as padding."""
    rng = np.random.default_rng(24)
    n, pages, max_pos = 200, 5, 512
    tab = W.rope_table(max_pos)
    k = W.bf16_normal(rng, (n, 128))
    slot = rng.permutation(pages * 64)[:n].astype(np.int32)
    pos = rng.integers(0, max_pos, n).astype(np.int32)
    gslot, gpos = slot.copy(), pos.copy()
    gslot[[3, 50]] = [pages * 64, 2 ** 31 - 1]
    gpos[[7, 90]] = [max_pos, -2]
    oslot = slot.copy()
    oslot[[3, 50, 7, 90]] = -1
    nw = W.norm_weight(rng)
    pay_o = np.full(pages * 4096, 0xA5, np.uint8); sc_o = np.full(pages * 256, 0x5A, np.uint8)
    orc.write_k(k, pos, oslot, nw, 1e-6, tab, pay_o, sc_o)
    pay_g = dev(np.full(pages * 4096, 0xA5, np.uint8)); sc_g = dev(np.full(pages * 256, 0x5A, np.uint8))
    F.write_k(bf16(k), dev(gpos), dev(gslot), bf16(nw), 1e-6, bf16(tab), pay_g, sc_g)
    torch.cuda.synchronize()
    assert np.array_equal(pay_g.cpu().numpy(), pay_o) and np.array_equal(sc_g.cpu().numpy(), sc_o)


def test_write_k_bulk_65536_bit_exact(F, orc):
    wl = W.make(4, with_q=False)
    say("write_k bulk:", wl.k_new.shape[0], "tokens into", wl.num_pages, "pages")
    tab = W.rope_table(wl.max_pos)
    po, so, pg, sg = _write_both(F, orc, wl.k_new, wl.pos_new, wl.slot_new, wl.norm_w, wl.eps, tab, wl.num_pages)
    assert np.array_equal(po, pg) and np.array_equal(so, sg)


# ---------------------------------------------------------------- Q pack

def _pack_both(F, orc, q, pos, tab, w, w_scale):
    qo, so, wo = orc.pack_q(q, pos, tab, w, w_scale)
    qg, sg, wg = F.pack_q(bf16(q), dev(pos), bf16(tab), dev(w), w_scale)
    torch.cuda.synchronize()
    return (qo, so, wo), (qg.cpu().numpy(), sg.cpu().numpy(), wg.cpu().numpy())


@pytest.mark.parametrize("heads", [64, 16, 32, 48, 112, 128])
def test_pack_q_small_bit_exact(F, orc, heads):
    rng = np.random.default_rng(22 + heads)
    T = 37
    tab = W.rope_table(1 << 14)
    q = W.bf16_normal(rng, (T, heads, 128))
    q[0, 0] = 0
    pos = rng.integers(0, 1 << 14, T).astype(np.int32)
    w = rng.uniform(-1, 1, (T, heads)).astype(np.float32)
    o, g = _pack_both(F, orc, q, pos, tab, w, 0.37)
    for a, b in zip(o, g):
        assert np.array_equal(a, b)


def test_pack_q_edges_zero_and_tiny_rows(F, orc):
    rng = np.random.default_rng(23)
    T, heads = 300, 64            # 19,200 vectors: zero rows, near-underflow heads, signed weights
    tab = W.rope_table(1 << 12)
    q = W.bf16_normal(rng, (T, heads, 128))
    q[0] = 0
    q[1, :5] = W.bf16_from_f32(rng.standard_normal((5, 128)).astype(np.float32) * 1e-36)
    pos = rng.integers(0, 1 << 12, T).astype(np.int32)
    w = rng.uniform(-1, 1, (T, heads)).astype(np.float32)
    o, g = _pack_both(F, orc, q, pos, tab, w, 1.0)
    for a, b in zip(o, g):
        assert np.array_equal(a, b)


def test_pack_q_position_outside_table_encodes_zero(F, orc):
    """Rows whose position is outside the table come out as the encoding of
    the +0 vector (the oracle's quantiser on zeros); the other rows as usual."""
    rng = np.random.default_rng(25)
    T, heads, max_pos = 9, 16, 256
    tab = W.rope_table(max_pos)
    q = W.bf16_normal(rng, (T, heads, 128))
    pos = rng.integers(0, max_pos, T).astype(np.int32)
    gpos = pos.copy()
    gpos[[2, 5]] = [max_pos, -1]
    w = rng.uniform(0, 1, (T, heads)).astype(np.float32)
    qf, qs, wo = orc.pack_q(q, pos, tab, w, 1.0)
    zc, zs = orc.quant128(np.zeros(128, np.float32))
    qf[[2, 5]] = zc
    qs[[2, 5]] = zs
    g = F.pack_q(bf16(q), dev(gpos), bf16(tab), dev(w), 1.0)
    torch.cuda.synchronize()
    for a, b in zip((qf, qs, wo), g):
        assert np.array_equal(a.view(np.uint8), b.cpu().numpy().view(np.uint8))


@pytest.mark.parametrize("n_tok,n_rows", [(64, 64), (1000, 7), (0, 5), (300, 0)])
def test_write_k_pack_q_one_launch_bit_exact(F, orc, n_tok, n_rows):
    """The combined launch produces the oracle's bytes for both halves (either
    side may be empty) and leaves every other pool byte untouched."""
    rng = np.random.default_rng([n_tok, n_rows, 5])
    tab = W.rope_table(1 << 12)
    num_pages = max(1, (n_tok + 63) // 64 + 3)
    k = W.bf16_normal(rng, (n_tok, 128))
    pos_k = rng.integers(0, 1 << 12, n_tok).astype(np.int32)
    slot = rng.permutation(num_pages * 64)[:n_tok].astype(np.int32)
    if n_tok > 2:
        slot[1] = -1                                                # padding token
    nw = W.norm_weight(rng)
    q = W.bf16_normal(rng, (n_rows, 64, 128))
    pos_q = rng.integers(0, 1 << 12, n_rows).astype(np.int32)
    w = rng.uniform(-1, 1, (n_rows, 64)).astype(np.float32)
    pay_o = np.full(num_pages * 4096, 0xA5, np.uint8); sc_o = np.full(num_pages * 256, 0x5A, np.uint8)
    orc.write_k(k, pos_k, slot, nw, 1e-6, tab, pay_o, sc_o)
    qf_o, qs_o, w_o = orc.pack_q(q, pos_q, tab, w, 0.5)
    pay_g = dev(np.full(num_pages * 4096, 0xA5, np.uint8)); sc_g = dev(np.full(num_pages * 256, 0x5A, np.uint8))
    qf_g, qs_g, w_g = F.write_k_pack_q(bf16(k), dev(pos_k), dev(slot), bf16(nw), 1e-6, bf16(tab), pay_g, sc_g,
                                       bf16(q), dev(pos_q), dev(w), 0.5)
    torch.cuda.synchronize()
    assert np.array_equal(pay_g.cpu().numpy(), pay_o) and np.array_equal(sc_g.cpu().numpy(), sc_o)
    assert np.array_equal(qf_g.cpu().numpy(), qf_o) and np.array_equal(qs_g.cpu().numpy(), qs_o)
    assert np.array_equal(w_g.cpu().numpy().view(np.uint32), w_o.view(np.uint32))


@pytest.mark.parametrize("cfg", [2, 3])
def test_pack_q_full_size_bit_exact(F, orc, cfg):
    wl = W.make(cfg)
    say("pack_q", wl.name, "rows", wl.n_rows)
    tab = W.rope_table(wl.max_pos)
    o, g = _pack_both(F, orc, wl.q, wl.pos_q, tab, wl.w, wl.w_scale)
    for a, b in zip(o, g):
        assert np.array_equal(a, b)


# ---------------------------------------------------------------- logits

def bits(x):
    return np.nan_to_num(x, nan=7.0).view(np.uint32)


def _gpu_logits(F, qf, qs, w, wl, payload, scale, stride=None, sentinel=np.nan):
    """The logits through the scheduled call (fp4idx_mqa_logits: plan + run)
    and through the host-bounded call, which must agree bit for bit
    (untouched entries included); returns them."""
    T = qf.shape[0]
    stride = stride or max(1, wl.max_ctx)
    args = (dev(qf), dev(qs), dev(w), dev(wl.req_row_indptr), dev(wl.row_ctx), dev(wl.block_table), dev(payload),
            dev(scale))
    out = torch.full((T, stride), float(sentinel), dtype=torch.float32, device=DEV)
    F.mqa_logits(*args, logits=out)
    ref = torch.full((T, stride), float(sentinel), dtype=torch.float32, device=DEV)
    F.mqa_logits_bounded(*args, wl.max_rows_per_req, wl.max_ctx, logits=ref)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(bits(got), bits(ref.cpu().numpy())), "scheduled and host-bounded logits differ"
    return got


def _encoded_small(orc, wl):
    tab = W.rope_table(wl.max_pos)
    pay = np.zeros(wl.num_pages * 4096, np.uint8)
    sc = np.zeros(wl.num_pages * 256, np.uint8)
    orc.write_k(wl.k_new, wl.pos_new, wl.slot_new, wl.norm_w, wl.eps, tab, pay, sc)
    qf, qs, w = orc.pack_q(wl.q, wl.pos_q, tab, wl.w, wl.w_scale)
    return qf, qs, w, pay, sc


@pytest.mark.parametrize("heads", [64, 16, 128, 48, 80, 96, 112])
def test_logits_small_mixed_all_scores(F, orc, heads):
    wl = W.small(heads=heads)
    qf, qs, w, pay, sc = _encoded_small(orc, wl)
    stride = wl.max_ctx + 5
    gpu = _gpu_logits(F, qf, qs, w, wl, pay, sc, stride=stride)
    ref, f64, T, A = orc.logits(qf, qs, w, wl.req_row_indptr, wl.row_ctx, wl.block_table, pay, sc,
                                logits_stride=stride, want_f64=True)
    check_rows(gpu, f64, T, A, wl.row_ctx, f"small mixed, {heads} heads")
    assert np.all(np.isnan(gpu[~in_context(wl.row_ctx, stride)])), "wrote past a row's context"


def test_logits_rows_per_request_variants(F, orc):
    """Every row-group shape the launcher picks (1, 2, 3/6, 4+, 16 rows per
    request) with ragged contexts and a padded zero-context row."""
    for rows, ctxs in (((1, 1, 1), (64, 1, 200)), ((2, 2), (100, 65)), ((6, 3), (300, 129)),
                       ((5, 4, 7), (77, 300, 16)), ((16, 1), (250, 90)), ((9, 2), (0, 40))):
        wl = W.small(seed=sum(rows) + sum(ctxs), rows=rows, ctxs=ctxs)
        qf, qs, w, pay, sc = _encoded_small(orc, wl)
        gpu = _gpu_logits(F, qf, qs, w, wl, pay, sc)
        ref, f64, T, A = orc.logits(qf, qs, w, wl.req_row_indptr, wl.row_ctx, wl.block_table, pay, sc,
                                    logits_stride=gpu.shape[1], want_f64=True)
        check_rows(gpu, f64, T, A, wl.row_ctx, f"rows per request {rows}")
        assert np.all(np.isnan(gpu[~in_context(wl.row_ctx, gpu.shape[1])]))


@pytest.mark.parametrize("rows,heads", [((3, 3), 64), ((4, 4, 3), 64), ((5, 5), 64), ((8, 7), 64), ((10, 9), 64),
                                        ((12, 12), 64), ((13, 13), 64), ((16, 14), 32), ((4, 4), 128),
                                        ((7, 7), 128), ((6, 5), 16), ((16, 1, 1), 64), ((14, 2, 5), 128),
                                        ((6, 6), 48), ((8, 8), 48), ((5, 5), 80), ((9, 8), 96), ((4, 4), 112),
                                        ((14, 2, 5), 112)])
def test_logits_shared_page_kernel_every_shape(F, orc, rows, heads):
    """Batches with three or more rows per request on average go to the
    shared-page kernel; each rows-per-work-group shape it picks (near-uniform
    row counts by the largest request, far-from-uniform ones with short page
    chunks), every head count, ragged contexts (a row block whose rows need
    different pages, a zero-context row)."""
    ctxs = tuple(64 * 3 + 17 * (i + 1) for i in range(len(rows)))
    wl = W.small(seed=sum(rows) * heads, rows=rows, ctxs=ctxs, heads=heads)
    wl.row_ctx[wl.req_row_indptr[0] + 1] = 0
    wl.row_ctx[wl.req_row_indptr[0]] = 1
    qf, qs, w, pay, sc = _encoded_small(orc, wl)
    gpu = _gpu_logits(F, qf, qs, w, wl, pay, sc)
    ref, f64, T, A = orc.logits(qf, qs, w, wl.req_row_indptr, wl.row_ctx, wl.block_table, pay, sc,
                                logits_stride=gpu.shape[1], want_f64=True)
    check_rows(gpu, f64, T, A, wl.row_ctx, f"shared-page rows {rows} heads {heads}")
    assert np.all(np.isnan(gpu[~in_context(wl.row_ctx, gpu.shape[1])]))


def test_logits_same_bits_from_every_kernel(F, orc):
    """A 16-row request (shared-page kernel, long enough for several page
    chunks) gives the same bits as its rows scored one per request (per-wave
    kernel, one row per wave), as the same request next to a one-row request
    (a non-uniform batch: shared-page kernel, shorter chunks) and as the same
    request next to fifteen one-row requests (under three rows per request
    on average: per-wave kernel, four rows per wave); each batch through the
    scheduled call and the host-bounded call (whose schedules and kernel
    shapes differ again)."""
    rng = np.random.default_rng(17)
    ctx = 40_000  # 625 pages: many page chunks
    pages = (ctx + 63) // 64
    pay, sc = W.random_pool(rng, pages + 3)
    qf, qs, w = _random_q(rng, 16)
    table = rng.permutation(pages + 3)[:pages].astype(np.int32)[None, :]
    row_ctx = (ctx - np.arange(16)[::-1] * 7).astype(np.int32)
    def both(q, qsc, wt, ind, cx, bt, mr):
        """(scheduled, host-bounded) logits of one batch."""
        T = q.shape[0]
        o1 = torch.full((T, ctx), float("nan"), dtype=torch.float32, device=DEV)
        o2 = torch.full((T, ctx), float("nan"), dtype=torch.float32, device=DEV)
        a_ = (dev(q), dev(qsc), dev(wt), dev(ind), dev(cx), dev(bt), dev(pay), dev(sc))
        F.mqa_logits(*a_, logits=o1)
        F.mqa_logits_bounded(*a_, mr, ctx, logits=o2)
        torch.cuda.synchronize()
        return o1.cpu().numpy(), o2.cpu().numpy()
    runs = [both(qf, qs, w, np.array([0, 16], np.int32), row_ctx, table, 16),
            both(qf, qs, w, np.arange(17, dtype=np.int32), row_ctx, np.repeat(table, 16, axis=0), 1)]
    m1, m2 = both(np.concatenate([qf, qf[:1]]), np.concatenate([qs, qs[:1]]), np.concatenate([w, w[:1]]),
                  np.array([0, 16, 17], np.int32), np.concatenate([row_ctx, row_ctx[:1]]),
                  np.repeat(table, 2, axis=0), 16)
    runs.append((m1[:16], m2[:16]))
    pick = np.concatenate([np.arange(16), np.arange(15)])
    s1, s2 = both(qf[pick], qs[pick], w[pick], np.concatenate([[0], np.arange(16, 32)]).astype(np.int32),
                  row_ctx[pick], np.repeat(table, 16, axis=0), 16)
    runs.append((s1[:16], s2[:16]))
    a = runs[0][0]
    for x, y in runs:
        assert np.array_equal(bits(a), bits(x)) and np.array_equal(bits(a), bits(y))
    assert np.array_equal(bits(a[:15]), bits(s1[16:])) and np.array_equal(bits(a[:15]), bits(s2[16:]))
    rows, toks = np.arange(16).repeat(40), (rng.random(640) * row_ctx.repeat(40)).astype(np.int64)
    f64, T, A = orc.logits_sampled(qf, qs, w, np.array([0, 16], np.int32), table, pay, sc, rows, toks)
    check_fp4(a[rows, toks], f64, T, A, "16-row request, 40,000 tokens (sampled)")


def test_logits_multi_row_broken_inputs_stay_in_bounds(F, orc):
    """Broken contract on a multi-row request: a context length past the
    logits row is cut to the row (the next row stays untouched), and a page
    id outside the pool reads page 0 (its tokens are garbage, no other token
    changes, nothing outside the buffers is touched)."""
    wl = W.small(seed=43, rows=(5, 1), ctxs=(300, 60))
    qf, qs, w, pay, sc = _encoded_small(orc, wl)
    stride = 320
    bad_ctx = wl.row_ctx.copy()
    bad_ctx[2] = 1 << 20
    table = wl.block_table.copy()
    table[0, 2] = wl.num_pages + 5  # tokens 128..191 of request 0
    out = torch.full((wl.n_rows + 1, stride), float("nan"), dtype=torch.float32, device=DEV)
    F.mqa_logits_bounded(dev(qf), dev(qs), dev(w), dev(wl.req_row_indptr), dev(bad_ctx), dev(table), dev(pay),
                         dev(sc), wl.max_rows_per_req, wl.max_ctx, logits=out[:wl.n_rows])
    out2 = torch.full((wl.n_rows + 1, stride), float("nan"), dtype=torch.float32, device=DEV)
    F.mqa_logits(dev(qf), dev(qs), dev(w), dev(wl.req_row_indptr), dev(bad_ctx), dev(table), dev(pay), dev(sc),
                 logits=out2[:wl.n_rows])
    torch.cuda.synchronize()
    g = out.cpu().numpy()
    assert np.array_equal(bits(g), bits(out2.cpu().numpy())), "scheduled and host-bounded logits differ"
    _, f64, T, A = orc.logits(qf, qs, w, wl.req_row_indptr, wl.row_ctx, wl.block_table, pay, sc,
                              logits_stride=stride, want_f64=True)
    keep = in_context(wl.row_ctx, stride)
    keep[:5, 128:192] = False                       # the tokens of the broken page id
    check_fp4(g[:wl.n_rows][keep], f64[keep], T[keep], A[keep], "broken multi-row inputs, intact scores")
    for t in range(wl.n_rows):
        c = min(int(bad_ctx[t]), stride)
        assert not np.any(np.isnan(g[t, :c])) and np.all(np.isnan(g[t, c:]))
    assert np.all(np.isnan(g[wl.n_rows]))


def test_logits_broken_indptr_stays_in_bounds(F, orc):
    """A request row range outside [0, n_rows] (a broken indptr) is clamped by
    the kernels to the rows that exist: nothing past the last row of the
    logits (or of the fused call's indices) is written, and a request whose
    range becomes empty writes nothing."""
    wl = W.small(seed=44, rows=(5, 1), ctxs=(300, 60))
    qf, qs, w, pay, sc = _encoded_small(orc, wl)
    T, stride = wl.n_rows, 320
    for ind in (np.array([0, 1 << 20, -5], np.int32), np.array([-3, 2, 1 << 30], np.int32),
                np.array([4, 1, 6], np.int32)):
        for mr in (1, 5):   # per-wave kernel and multi-row kernels
            out = torch.full((T + 2, stride), float("nan"), dtype=torch.float32, device=DEV)
            F.mqa_logits_bounded(dev(qf), dev(qs), dev(w), dev(ind), dev(wl.row_ctx), dev(wl.block_table), dev(pay),
                                 dev(sc), mr, wl.max_ctx, logits=out[:T])
            out2 = torch.full((T + 2, stride), float("nan"), dtype=torch.float32, device=DEV)
            F.mqa_logits(dev(qf), dev(qs), dev(w), dev(ind), dev(wl.row_ctx), dev(wl.block_table), dev(pay),
                         dev(sc), logits=out2[:T])
            idx = torch.full((T + 2, 16), -77, dtype=torch.int32, device=DEV)
            F.mqa_logits_topk(dev(qf), dev(qs), dev(w), dev(ind), dev(wl.row_ctx), dev(wl.block_table), dev(pay),
                              dev(sc), 16, mr, wl.max_ctx, out_idx=idx[:T])
            torch.cuda.synchronize()
            g = out.cpu().numpy()
            g2 = out2.cpu().numpy()
            assert np.all(np.isnan(g[T:])) and np.all(np.isnan(g2[T:])), (ind, mr)
            assert np.all(np.isnan(g2[:T, wl.max_ctx:])), (ind, mr)
            assert np.all(idx.cpu().numpy()[T:] == -77), (ind, mr)
            assert np.all(np.isnan(g[:T, wl.max_ctx:])), (ind, mr)


def _random_q(rng, T, H=64):
    qf = rng.integers(0, 256, (T, H, 64)).astype(np.uint8)
    qs = rng.integers(124, 129, (T, H, 4)).astype(np.uint8)
    w = rng.uniform(0, 1, (T, H)).astype(np.float32)
    return qf, qs, w


def _samples(rng, wl, n):
    rows = rng.integers(0, wl.n_rows, n)
    ctx = wl.row_ctx[rows].astype(np.int64)
    keep = ctx > 0
    rows, ctx = rows[keep], ctx[keep]
    toks = (rng.random(rows.size) * ctx).astype(np.int64)
    # every row's first and last token, and tile / page boundaries
    live = np.nonzero(wl.row_ctx > 0)[0]
    extra_r = np.concatenate([live, live])
    extra_t = np.concatenate([np.zeros(live.size, np.int64), wl.row_ctx[live].astype(np.int64) - 1])
    return np.concatenate([rows, extra_r]), np.concatenate([toks, extra_t])


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_logits_full_size_sampled(F, orc, cfg):
    """Each workload at its real shape (random FP4 pool and Q codes from the
    generator) in the launch configuration the bench times; sampled scores
    against the oracle, and nothing written past any row's context."""
    wl = W.make(cfg, with_q=False)
    rng = np.random.default_rng([cfg, 99])
    pay, sc = W.random_pool(rng, wl.num_pages)
    qf, qs, w = _random_q(rng, wl.n_rows)
    say("logits", wl.name, "scores", wl.scores)
    stride = wl.max_ctx + 3
    gpu = _gpu_logits(F, qf, qs, w, wl, pay, sc, stride=stride)
    rows, toks = _samples(rng, wl, 6000)
    f64, T, A = orc.logits_sampled(qf, qs, w, wl.req_row_indptr, wl.block_table, pay, sc, rows, toks)
    check_fp4(gpu[rows, toks], f64, T, A, f"{wl.name} (sampled)")
    cols = np.arange(stride)[None, :]
    assert np.all(np.isnan(gpu[cols >= wl.row_ctx[:, None]]))
    assert not np.any(np.isnan(gpu[cols < wl.row_ctx[:, None]]))


def test_logits_invariant_to_pages_and_batch(F, orc):
    """Bitwise: permuting physical pages or scoring a request alone gives the
    same logits ([P3] Historical results: identical across page layouts)."""
    wl = W.small(seed=31, rows=(3, 6, 1), ctxs=(500, 257, 64))
    rng = np.random.default_rng(5)
    pay, sc = W.random_pool(rng, wl.num_pages)
    qf, qs, w = _random_q(rng, wl.n_rows)
    base = _gpu_logits(F, qf, qs, w, wl, pay, sc)
    perm = rng.permutation(wl.num_pages)
    inv = np.argsort(perm)
    pay2 = pay.reshape(wl.num_pages, 4096)[perm].reshape(-1)
    sc2 = sc.reshape(wl.num_pages, 256)[perm].reshape(-1)
    wl2 = W.small(seed=31, rows=(3, 6, 1), ctxs=(500, 257, 64))
    wl2.block_table = np.where(wl.block_table >= 0, inv[np.maximum(wl.block_table, 0)], -1).astype(np.int32)
    moved = _gpu_logits(F, qf, qs, w, wl2, pay2, sc2)
    assert np.array_equal(np.nan_to_num(base, nan=7.0).view(np.uint32), np.nan_to_num(moved, nan=7.0).view(np.uint32))
    # request 1 alone
    b = 1
    r0, r1 = wl.req_row_indptr[b], wl.req_row_indptr[b + 1]
    wl3 = W.small(seed=31, rows=(3, 6, 1), ctxs=(500, 257, 64))
    wl3.req_row_indptr = np.array([0, r1 - r0], np.int32)
    wl3.row_ctx = wl.row_ctx[r0:r1].copy()
    wl3.block_table = wl.block_table[b:b + 1].copy()
    alone = _gpu_logits(F, qf[r0:r1], qs[r0:r1], w[r0:r1], wl3, pay, sc, stride=base.shape[1])
    assert np.array_equal(np.nan_to_num(base[r0:r1], nan=7.0).view(np.uint32), np.nan_to_num(alone, nan=7.0).view(np.uint32))


def test_pools_and_logits_past_2_gib(F, orc):
    """64-bit offsets: a payload pool of 8,388,672 pages (34 GB), whose scale
    pool is itself past 2 GiB, and a logits buffer of 4 GiB.  K tokens are
    written to pages on both sides of the 2 GiB payload boundary and past
    the 2 GiB scale boundary, scored through a block table that points at
    them into logits rows that start past 2 GiB, and selected by top-k from
    those rows; bytes, logits and indices against the oracle run on a
    compact pool with the same tokens."""
    P = (1 << 23) + 64                       # scale pool 2 GiB + 16 KiB
    high = np.array([(1 << 19) - 1, 1 << 19, (1 << 19) + 1, (1 << 23) - 1, 1 << 23, (1 << 23) + 5, P - 1],
                    np.int64)                # payload offset 2 GiB = page 2^19; scale offset 2 GiB = page 2^23
    n_pages = high.size
    rng = np.random.default_rng(91)
    tab = W.rope_table(4096)
    n = n_pages * 64
    k = W.bf16_normal(rng, (n, 128))
    pos = rng.integers(0, 4096, n).astype(np.int32)
    nw = W.norm_weight(rng)
    compact_slot = np.arange(n, dtype=np.int32)
    slot = (high[compact_slot // 64] * 64 + compact_slot % 64).astype(np.int32)
    pay_o = np.zeros(n_pages * 4096, np.uint8); sc_o = np.zeros(n_pages * 256, np.uint8)
    orc.write_k(k, pos, compact_slot, nw, 1e-6, tab, pay_o, sc_o)
    say("allocating", P * 4352 / 1e9, "GB of pools")
    pay = torch.empty(P * 4096, dtype=torch.uint8, device=DEV)
    sc = torch.empty(P * 256, dtype=torch.uint8, device=DEV)
    F.write_k(bf16(k), dev(pos), dev(slot), bf16(nw), 1e-6, bf16(tab), pay, sc)
    torch.cuda.synchronize()
    for i, pg in enumerate(high.tolist()):
        assert np.array_equal(pay[pg * 4096:(pg + 1) * 4096].cpu().numpy(), pay_o[i * 4096:(i + 1) * 4096]), pg
        assert np.array_equal(sc[pg * 256:(pg + 1) * 256].cpu().numpy(), sc_o[i * 256:(i + 1) * 256]), pg
    # two requests of two rows; request 0 reads pages 0..3 of the list, request 1 pages 3..6
    T, stride = 4, 1 << 28                   # rows 2 and 3 start at 2 GiB and 3 GiB
    indptr = np.array([0, 2, 4], np.int32)
    ctx = np.array([256, 200, 256, 190], np.int32)
    compact_bt = np.array([[0, 1, 2, 3], [3, 4, 5, 6]], np.int32)
    bt = high[compact_bt].astype(np.int32)
    qf, qs, w = _random_q(rng, T)
    lg = torch.full((T, stride), float("nan"), dtype=torch.float32, device=DEV)
    F.mqa_logits(dev(qf), dev(qs), dev(w), dev(indptr), dev(ctx), dev(bt), pay, sc, logits=lg)
    top = F.topk(lg, dev(ctx), 64, 256)
    torch.cuda.synchronize()
    g = lg[:, :300].cpu().numpy()
    lg[:, :300] = float("nan")
    F.mqa_logits_bounded(dev(qf), dev(qs), dev(w), dev(indptr), dev(ctx), dev(bt), pay, sc, 2, 256, logits=lg)
    torch.cuda.synchronize()
    assert np.array_equal(bits(g), bits(lg[:, :300].cpu().numpy())), "scheduled and host-bounded logits differ"
    del pay, sc
    _, f64, Tt, A = orc.logits(qf, qs, w, indptr, ctx, compact_bt, pay_o, sc_o, logits_stride=300, want_f64=True)
    check_rows(g, f64, Tt, A, ctx, "pools and logits past 2 GiB")
    assert np.all(np.isnan(g[~in_context(ctx, 300)]))
    assert np.array_equal(top.cpu().numpy(), orc.topk(g, ctx, 64))
    del lg
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- top-k

def _gpu_topk(F, logits, ctx, k):
    """fp4idx_topk_bounded at the rows' longest context; fp4idx_topk (sized
    by the logits row) must give the same indices."""
    lg, cx = dev(logits), dev(ctx)
    out = F.topk(lg, cx, k, int(ctx.max(initial=0)))
    plain = F.topk(lg, cx, k)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert np.array_equal(out, plain.cpu().numpy()), "fp4idx_topk and fp4idx_topk_bounded differ"
    return out


def test_topk_edges_and_ties_bit_exact(F, orc):
    rng = np.random.default_rng(41)
    T, S = 12, 5000
    vals = rng.standard_normal((T, S)).astype(np.float32)
    vals[1] = rng.integers(-3, 4, S).astype(np.float32)            # massive ties
    vals[2] = 1.5                                                   # all equal
    vals[3, ::2] = -0.0; vals[3, 1::2] = 0.0                        # signed zeros only
    vals[4] = np.round(vals[4] * 4) / 4                             # quantised
    vals[5] = np.abs(vals[5]) * 1e-40                               # subnormals
    vals[6] = -np.abs(vals[6]) * 1e30                               # large negatives
    vals[7, 100] = 3e38; vals[7, 200] = -3e38                       # extreme range
    ctx = np.array([5000, 5000, 5000, 3000, 4999, 2500, 5000, 5000, 0, 100, 2048, 2049], np.int32)
    for k in (2048, 256, 1, 7):
        got = _gpu_topk(F, vals, ctx, k)
        want = orc.topk(vals, ctx, k)
        assert np.array_equal(got, want), k


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_topk_full_size_bit_exact(F, orc, cfg):
    wl = W.make(cfg, with_q=False)
    rng = np.random.default_rng([cfg, 17])
    T, S = wl.n_rows, wl.max_ctx
    say("topk", wl.name, "rows", T, "ctx", S)
    vals = (rng.standard_normal((T, S)) * 20 + 40).astype(np.float32)
    vals[:, ::97] = np.round(vals[:, ::97])                         # planted ties
    got = _gpu_topk(F, vals, wl.row_ctx, wl.topk)
    want = orc.topk(vals, wl.row_ctx, wl.topk)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("rows,max_ctx", [(300, 8000), (300, 12000), (300, 16000), (300, 18000), (300, 24000),
                                          (300, 30000), (40, 20000), (40, 30000)])
def test_topk_every_register_variant_bit_exact(F, orc, rows, max_ctx):
    """Row counts on both sides of the 1024-thread / 512-thread switch and row
    lengths in every register band (512 threads x 16, 24, 36, 48 and 64 slots;
    1024 x 24 and 32); ragged rows (including ctx 0, ctx < k, ctx = k,
    ctx = k + 1), planted ties and a crowded row."""
    rng = np.random.default_rng([rows, max_ctx])
    vals = (rng.standard_normal((rows, max_ctx)) * 10).astype(np.float32)
    vals[:, ::61] = np.round(vals[:, ::61])                          # ties
    vals[3] = rng.integers(-2, 3, max_ctx).astype(np.float32)        # crowded bins
    ctx = rng.integers(max_ctx // 2, max_ctx + 1, rows).astype(np.int32)
    ctx[:4] = [0, 1000, 2048, 2049]
    ctx[-1] = max_ctx
    got = _gpu_topk(F, vals, ctx, 2048)
    assert np.array_equal(got, orc.topk(vals, ctx, 2048))


@pytest.mark.parametrize("rows", [300, 40])
def test_topk_threshold_bin_paths_bit_exact(F, orc, rows):
    """Values on a 1/8 grid, so every first-cut bin holds one grid value and
    its ties: k = 64 leaves a few dozen candidates in the threshold bin (ranked
    by one wave), k = 256 about a hundred (ranked through LDS), k = 2048 some
    hundreds (exact key rounds).  300 rows of up to 18,000 positions take
    512-thread rows of 36 slots, which re-read the candidates' values; 40 rows
    take 1024-thread rows, which keep them in registers."""
    rng = np.random.default_rng([rows, 7])
    S = 18000
    vals = (np.round(rng.standard_normal((rows, S)) * 8) / 8).astype(np.float32)
    ctx = rng.integers(S - 3000, S + 1, rows).astype(np.int32)
    ctx[-1] = S
    for k in (64, 256, 2048):
        got = _gpu_topk(F, vals, ctx, k)
        assert np.array_equal(got, orc.topk(vals, ctx, k)), k


def test_topk_long_rows_use_global_path(F, orc):
    rng = np.random.default_rng(43)
    T, S = 3, 40000
    vals = rng.standard_normal((T, S)).astype(np.float32)
    vals[1] = np.round(vals[1] * 8)
    ctx = np.array([40000, 39000, 35000], np.int32)
    got = _gpu_topk(F, vals, ctx, 2048)
    assert np.array_equal(got, orc.topk(vals, ctx, 2048))


# ---------------------------------------------------------------- whole chain

def test_chain_small_write_pack_logits_topk(F, orc):
    """write_k -> pack_q -> logits -> top-k on the GPU against the oracle's
    chain.  Top-k sets must match exactly on every row whose gap at the k-th
    value exceeds twice the logits tolerance; other rows must still be a
    valid top-k of the oracle's values within that tolerance."""
    wl = W.small(seed=51, rows=(2, 6, 16, 1), ctxs=(3000, 700, 2100, 300), topk=256)
    tab = W.rope_table(wl.max_pos)
    # oracle chain
    pay_o = np.zeros(wl.num_pages * 4096, np.uint8); sc_o = np.zeros(wl.num_pages * 256, np.uint8)
    orc.write_k(wl.k_new, wl.pos_new, wl.slot_new, wl.norm_w, wl.eps, tab, pay_o, sc_o)
    qf_o, qs_o, w_o = orc.pack_q(wl.q, wl.pos_q, tab, wl.w, wl.w_scale)
    ref, f64, T, A = orc.logits(qf_o, qs_o, w_o, wl.req_row_indptr, wl.row_ctx, wl.block_table, pay_o, sc_o,
                                want_f64=True)
    top_o = orc.topk(ref, wl.row_ctx, wl.topk)
    # GPU chain
    pay_g = torch.zeros(wl.num_pages * 4096, dtype=torch.uint8, device=DEV)
    sc_g = torch.zeros(wl.num_pages * 256, dtype=torch.uint8, device=DEV)
    F.write_k(bf16(wl.k_new), dev(wl.pos_new), dev(wl.slot_new), bf16(wl.norm_w), wl.eps, bf16(tab), pay_g, sc_g)
    qf_g, qs_g, w_g = F.pack_q(bf16(wl.q), dev(wl.pos_q), bf16(tab), dev(wl.w), wl.w_scale)
    lg = F.mqa_logits(qf_g, qs_g, w_g, dev(wl.req_row_indptr), dev(wl.row_ctx), dev(wl.block_table), pay_g, sc_g,
                      max_ctx=wl.max_ctx)
    top_g = F.topk(lg, dev(wl.row_ctx), wl.topk, wl.max_ctx)
    torch.cuda.synchronize()
    assert np.array_equal(pay_g.cpu().numpy(), pay_o) and np.array_equal(sc_g.cpu().numpy(), sc_o)
    assert np.array_equal(qf_g.cpu().numpy(), qf_o) and np.array_equal(qs_g.cpu().numpy(), qs_o)
    lgn = lg.cpu().numpy()
    tg = top_g.cpu().numpy()
    check_rows(lgn, f64, T, A, wl.row_ctx, "chain (encoded K and Q)")
    for t in range(wl.n_rows):
        c = int(wl.row_ctx[t])
        K = min(wl.topk, c)
        sel_g = tg[t, :K]
        assert np.all(tg[t, K:] == -1) and np.all(np.diff(sel_g) > 0)
        tol = fp4_bound(T[t, :c], A[t, :c])
        if K < c:
            srt = np.sort(f64[t, :c])[::-1]
            gap = srt[K - 1] - srt[K]
            if gap > 2 * tol.max():
                assert np.array_equal(sel_g, top_o[t, :K]), f"row {t}"
            else:
                kth = srt[K - 1]
                assert np.all(f64[t, sel_g] >= kth - 2 * tol.max())
        else:
            assert np.array_equal(sel_g, np.arange(c))


# ---------------------------------------------------------------- kernel timing hook

def test_time_next_call_stamps_kernel_and_keeps_results(F, orc):
    """Armed timing events go to the next call's kernel only; the call's result
    is unchanged and the arming is used up by that call."""
    rng = np.random.default_rng(47)
    vals = rng.standard_normal((9, 3000)).astype(np.float32)
    ctx = np.array([3000, 2999, 1, 0, 2048, 2049, 100, 3000, 1500], np.int32)
    want = orc.topk(vals, ctx, 2048)
    lg, cx = dev(vals), dev(ctx)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    F.time_next_call(ev[0], ev[1])
    a = F.topk(lg, cx, 2048, 3000)
    b = F.topk(lg, cx, 2048, 3000)           # not timed: the arming was used up
    F.time_next_call(ev[2], ev[3])
    c = F.topk(lg, cx, 2048, 3000)
    torch.cuda.synchronize()
    for got in (a, b, c):
        assert np.array_equal(got.cpu().numpy(), want)
    t1, t2 = ev[0].elapsed_time(ev[1]), ev[2].elapsed_time(ev[3])
    say("topk kernel ms", t1, t2)
    assert 0.0 < t1 < 100.0 and 0.0 < t2 < 100.0


# ---------------------------------------------------------------- HIP graph capture

def test_chain_graph_replays_match_eager(F):
    """The four calls captured in one HIP graph (in sequence, and with the K
    write on a parallel branch as the benchmark captures it): every replay,
    with eager work and synchronisation between replays, reproduces the eager
    results exactly (pool bytes, packed Q, logits bits, top-k)."""
    wl = W.small(seed=53, rows=(3, 1, 8), ctxs=(2500, 900, 4100), topk=512)
    tab = bf16(W.rope_table(wl.max_pos))
    ins = dict(k=bf16(wl.k_new), pos=dev(wl.pos_new), slot=dev(wl.slot_new), nw=bf16(wl.norm_w), q=bf16(wl.q),
               pq=dev(wl.pos_q), w=dev(wl.w), ind=dev(wl.req_row_indptr), ctx=dev(wl.row_ctx), bt=dev(wl.block_table))
    T, H = wl.n_rows, wl.heads

    def outs():
        return dict(pay=torch.zeros(wl.num_pages * 4096, dtype=torch.uint8, device=DEV),
                    sc=torch.zeros(wl.num_pages * 256, dtype=torch.uint8, device=DEV),
                    qf=torch.empty((T, H, 64), dtype=torch.uint8, device=DEV),
                    qs=torch.empty((T, H, 4), dtype=torch.uint8, device=DEV),
                    wo=torch.empty((T, H), dtype=torch.float32, device=DEV),
                    lg=torch.full((T, wl.max_ctx), -7.0, dtype=torch.float32, device=DEV),
                    top=torch.empty((T, wl.topk), dtype=torch.int32, device=DEV),
                    ws=F.new_workspace(T, wl.n_reqs, wl.max_ctx))

    def chain(o, strm, side=None):
        kw = strm
        if side is not None:   # K write on a parallel branch, joined before the logits
            fork = torch.cuda.Event()
            fork.record(strm)
            side.wait_event(fork)
            kw = side
        F.write_k(ins["k"], ins["pos"], ins["slot"], ins["nw"], wl.eps, tab, o["pay"], o["sc"], stream=kw)
        F.pack_q(ins["q"], ins["pq"], tab, ins["w"], wl.w_scale, o["qf"], o["qs"], o["wo"], stream=strm)
        if side is not None:
            join = torch.cuda.Event()
            join.record(side)
            strm.wait_event(join)
        F.mqa_logits(o["qf"], o["qs"], o["wo"], ins["ind"], ins["ctx"], ins["bt"], o["pay"], o["sc"],
                     logits=o["lg"], workspace=o["ws"], stream=strm)
        F.topk(o["lg"], ins["ctx"], wl.topk, wl.max_ctx, out_idx=o["top"], stream=strm)

    ref = outs()
    chain(ref, torch.cuda.current_stream())
    torch.cuda.synchronize()
    want = {n: v.cpu() for n, v in ref.items()}

    for forked in (False, True):
        o = outs()
        g = torch.cuda.CUDAGraph()
        cap, side = torch.cuda.Stream(), torch.cuda.Stream()
        with torch.cuda.graph(g, stream=cap):
            chain(o, torch.cuda.current_stream(), side if forked else None)
        for rep in range(4):
            for n in ("pay", "sc", "qf", "qs", "wo", "top", "ws"):   # eager work between replays
                o[n].zero_()
            o["lg"].fill_(-7.0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for n, v in want.items():
                if n == "ws":
                    continue
                got = o[n].cpu()
                if n in ("wo", "lg"):
                    assert torch.equal(got.view(torch.int32), v.view(torch.int32)), (forked, rep, n)
                else:
                    assert torch.equal(got, v), (forked, rep, n)


def test_chain_graph_replays_follow_changed_inputs(F, orc):
    """One captured chain (K write, Q pack, logits, top-k) replayed with its
    device inputs rewritten in place between replays, as a serving loop
    reuses a captured decode step: new K rows, positions and slots, new
    query rows, positions and weights, new row-to-request split, context
    lengths and block tables (within the captured row and context bounds).
    The logits call's device schedule is part of the captured graph, so
    each replay plans the new batch.  Every replay equals an eager run of
    the same calls on the same values, bit for bit, and the oracle: pool and
    Q bytes exact, logits within the bar, top-k equal to the oracle's
    selection of the GPU logits."""
    wl = W.small(seed=63, rows=(3, 1, 8), ctxs=(2500, 900, 4100), topk=512)
    tab_np = W.rope_table(wl.max_pos)
    tab = bf16(tab_np)
    T, H, P, B = wl.n_rows, wl.heads, wl.num_pages, wl.n_reqs
    n = wl.k_new.shape[0]
    max_rows, max_ctx = wl.max_rows_per_req, wl.max_ctx
    ins = dict(k=bf16(wl.k_new), pos=dev(wl.pos_new), slot=dev(wl.slot_new), nw=bf16(wl.norm_w), q=bf16(wl.q),
               pq=dev(wl.pos_q), w=dev(wl.w), ind=dev(wl.req_row_indptr), ctx=dev(wl.row_ctx),
               bt=dev(wl.block_table))

    def outs():
        return dict(pay=torch.zeros(P * 4096, dtype=torch.uint8, device=DEV),
                    sc=torch.zeros(P * 256, dtype=torch.uint8, device=DEV),
                    qf=torch.empty((T, H, 64), dtype=torch.uint8, device=DEV),
                    qs=torch.empty((T, H, 4), dtype=torch.uint8, device=DEV),
                    wo=torch.empty((T, H), dtype=torch.float32, device=DEV),
                    lg=torch.full((T, max_ctx), -7.0, dtype=torch.float32, device=DEV),
                    top=torch.empty((T, wl.topk), dtype=torch.int32, device=DEV),
                    ws=F.new_workspace(T, B, max_ctx))

    def chain(o, strm):
        F.write_k(ins["k"], ins["pos"], ins["slot"], ins["nw"], wl.eps, tab, o["pay"], o["sc"], stream=strm)
        F.pack_q(ins["q"], ins["pq"], tab, ins["w"], wl.w_scale, o["qf"], o["qs"], o["wo"], stream=strm)
        F.mqa_logits(o["qf"], o["qs"], o["wo"], ins["ind"], ins["ctx"], ins["bt"], o["pay"], o["sc"],
                     logits=o["lg"], workspace=o["ws"], stream=strm)
        F.topk(o["lg"], ins["ctx"], wl.topk, max_ctx, out_idx=o["top"], stream=strm)

    o = outs()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        chain(o, torch.cuda.current_stream())
    torch.cuda.synchronize()
    rng = np.random.default_rng(64)
    pay_o = np.zeros(P * 4096, np.uint8); sc_o = np.zeros(P * 256, np.uint8)
    cur = dict(k=wl.k_new, pos=wl.pos_new, slot=wl.slot_new, q=wl.q, pq=wl.pos_q, w=wl.w, ind=wl.req_row_indptr,
               ctx=wl.row_ctx, bt=wl.block_table)
    splits = [None, (6, 2, 4), (1, 8, 3)]
    for rep in range(3):
        if rep > 0:   # new values, written into the captured buffers in place
            rows = splits[rep]
            cur = dict(k=W.bf16_normal(rng, (n, 128)), pos=rng.integers(0, wl.max_pos, n).astype(np.int32),
                       slot=rng.permutation(P * 64)[:n].astype(np.int32), q=W.bf16_normal(rng, (T, H, 128)),
                       pq=rng.integers(0, wl.max_pos, T).astype(np.int32),
                       w=rng.uniform(0, 1, (T, H)).astype(np.float32),
                       ind=np.concatenate([[0], np.cumsum(rows)]).astype(np.int32),
                       ctx=rng.integers(0, max_ctx + 1, T).astype(np.int32),
                       bt=np.stack([rng.permutation(P)[:wl.block_table.shape[1]] for _ in range(B)]).astype(np.int32))
            cur["ctx"][[0, T - 1]] = [max_ctx, 0]
            cur["slot"][3] = -1                                      # a padding token
            for name, dst in (("k", "k"), ("q", "q")):
                ins[dst].copy_(bf16(cur[name]))
            for name in ("pos", "slot", "pq", "w", "ind", "ctx", "bt"):
                ins[name].copy_(dev(cur[name]))
            torch.cuda.synchronize()
        # eager run of the same calls on the same values, from the same pool state
        e = outs()
        e["pay"].copy_(o["pay"]); e["sc"].copy_(o["sc"])
        chain(e, torch.cuda.current_stream())
        o["lg"].fill_(-7.0)                                          # entries past the new contexts
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name in ("pay", "sc", "qf", "qs", "top"):
            assert torch.equal(o[name], e[name]), (rep, name)
        lb = torch.full((T, max_ctx), -7.0, dtype=torch.float32, device=DEV)   # the host-bounded call agrees
        F.mqa_logits_bounded(o["qf"], o["qs"], o["wo"], ins["ind"], ins["ctx"], ins["bt"], o["pay"], o["sc"],
                             max_rows, max_ctx, logits=lb)
        torch.cuda.synchronize()
        assert torch.equal(o["lg"].view(torch.int32), lb.view(torch.int32)), rep
        for name in ("wo", "lg"):
            assert torch.equal(o[name].view(torch.int32), e[name].view(torch.int32)), (rep, name)
        # the oracle on the same values (its pool follows the same writes)
        orc.write_k(cur["k"], cur["pos"], cur["slot"], wl.norm_w, wl.eps, tab_np, pay_o, sc_o)
        qf_o, qs_o, w_o = orc.pack_q(cur["q"], cur["pq"], tab_np, cur["w"], wl.w_scale)
        assert np.array_equal(o["pay"].cpu().numpy(), pay_o) and np.array_equal(o["sc"].cpu().numpy(), sc_o), rep
        assert np.array_equal(o["qf"].cpu().numpy(), qf_o) and np.array_equal(o["qs"].cpu().numpy(), qs_o), rep
        lgn = o["lg"].cpu().numpy()
        _, f64, Tt, A = orc.logits(qf_o, qs_o, w_o, cur["ind"], cur["ctx"], cur["bt"], pay_o, sc_o,
                                   logits_stride=max_ctx, want_f64=True)
        check_rows(lgn, f64, Tt, A, cur["ctx"], f"graph replay {rep} on changed inputs")
        assert np.array_equal(o["top"].cpu().numpy(), orc.topk(lgn, cur["ctx"], wl.topk)), rep


# ---------------------------------------------------------------- split-pool reader

def test_read_k_bit_exact_on_random_pool_bytes(F, orc):
    """Every code and every scale byte the writer can store (0..254), slots
    in order, shuffled, repeated, padding (-1) and past the pool: fp32 bits
    equal the oracle's exact values rounded to fp32 (exact, or +-inf)."""
    rng = np.random.default_rng(71)
    P = 40
    pay = rng.integers(0, 256, P * 4096).astype(np.uint8)
    sc = rng.integers(0, 255, P * 256).astype(np.uint8)
    sc[:8] = [0, 1, 2, 126, 127, 128, 253, 254]
    slots = np.concatenate([np.arange(P * 64), rng.integers(0, P * 64, 1000), [-1, P * 64, -7, 5, 5]]).astype(np.int32)
    with np.errstate(over="ignore"):
        want = orc.read_k(pay, sc, slots).astype(np.float32)      # exact values; overflow becomes +-inf
    got = F.read_k(dev(pay), dev(sc), dev(slots))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_read_k_round_trips_the_writer(F, orc):
    """write_k then read_k on the GPU: the values the oracle decodes from its
    own pool, for a strided output."""
    rng = np.random.default_rng(72)
    n, num_pages = 777, 20
    tab = W.rope_table(1 << 12)
    k = W.bf16_normal(rng, (n, 128)); pos = rng.integers(0, 1 << 12, n).astype(np.int32)
    slot = rng.permutation(num_pages * 64)[:n].astype(np.int32); nw = W.norm_weight(rng)
    pay_o = np.zeros(num_pages * 4096, np.uint8); sc_o = np.zeros(num_pages * 256, np.uint8)
    orc.write_k(k, pos, slot, nw, 1e-6, tab, pay_o, sc_o)
    want = orc.read_k(pay_o, sc_o, slot).astype(np.float32)
    pay_g = torch.zeros(num_pages * 4096, dtype=torch.uint8, device=DEV)
    sc_g = torch.zeros(num_pages * 256, dtype=torch.uint8, device=DEV)
    F.write_k(bf16(k), dev(pos), dev(slot), bf16(nw), 1e-6, bf16(tab), pay_g, sc_g)
    out = torch.full((n, 136), 9.0, dtype=torch.float32, device=DEV)
    F.read_k(pay_g, sc_g, dev(slot), out=out[:, :128])
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.array_equal(o[:, :128].view(np.uint32), want.view(np.uint32))
    assert np.all(o[:, 128:] == 9.0)
