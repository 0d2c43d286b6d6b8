"""GPU parity of the FP8 indexer variant (132-byte fused tokens) through the
C ABI against the CPU oracle.

Bars: the writer's and the Q pack's bytes (codes, fp32 scales, weights) and
the top-k indices are bit-exact; logits satisfy
    |gpu - exact| <= 1e-5 * T + 7 * 2^-13 * B16 + 4 * 2^-24 * A
with T = sum_h |w_h| max(d_h, 0), B16 = sum_h |w_h| (the 16 largest
|q_hi k_i| of head h) and A = sum_h |w_h| sum_i |q_hi k_i| per (row, token).
The B16 term comes from the block-scaled FP8 MFMA's arithmetic on gfx950: it
sums each dot product in 16 groups of 8 products and drops the bits of every
product below 2^-13 of its group's largest (measured on the device: a
product 2^14 below the group's largest vanishes, 1.5 * 2^3 next to 2^16
counts as 8; group sums are then added exactly up to fp32 rounding), so a
group loses less than 7 * 2^-13 of its largest product, and the 16 group
maxima sum to at most the 16 largest products (derivation in tests/bars.py).
Inputs come from the seeded generators; expected values from the oracle only.
"""
import numpy as np
import pytest
import torch

from bars import check_fp8, fp8_bound, in_context
from sparse_attention_fp4_fp4idx_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"
PAGE8 = W.FP8_PAGE_BYTES


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


def check_rows(gpu, f64, T, A, B, ctx, where):
    """Every row's [0, ctx) against the FP8 bar, in one check."""
    m = in_context(ctx, gpu.shape[1])
    w = gpu.shape[1]
    check_fp8(gpu[m], f64[:, :w][m], T[:, :w][m], A[:, :w][m], B[:, :w][m], where)


# ---------------------------------------------------------------- K writer

def _write_both(F, orc, k, pos, slot, norm_w, eps, tab, num_pages, k_row_stride=None, gpu_slot=None, gpu_pos=None):
    pool_o = np.full(num_pages * PAGE8, 0xA5, np.uint8)
    orc.write_k_fp8(k, pos, slot, norm_w, eps, tab, pool_o)
    pool_g = dev(np.full(num_pages * PAGE8, 0xA5, np.uint8))
    if k_row_stride is not None and k_row_stride != 128:
        kk = np.zeros((k.shape[0], k_row_stride), np.uint16)
        kk[:, :128] = k
        kt = bf16(kk)[:, :128]
    else:
        kt = bf16(k)
    F.write_k_fp8(kt, dev(pos if gpu_pos is None else gpu_pos), dev(slot if gpu_slot is None else gpu_slot),
                  bf16(norm_w), eps, bf16(tab), pool_g)
    torch.cuda.synchronize()
    return pool_o, pool_g.cpu().numpy()


@pytest.mark.parametrize("n", [300, 20000])
def test_write_k_fp8_edges_strided_skip_extremes(F, orc, n):
    rng = np.random.default_rng(121)
    tab = W.rope_table(4096)
    k = W.bf16_normal(rng, (n, 128))
    k[0] = 0                                  # zero row: scale 2^-127, all codes 0
    k[1] = W.bf16_from_f32(np.full(128, 3.0, np.float32))
    k[2] = W.bf16_from_f32(rng.standard_normal(128).astype(np.float32) * 1e-30)
    k[3] = W.bf16_from_f32(rng.standard_normal(128).astype(np.float32) * 1e30)
    pos = rng.integers(0, 4096, n).astype(np.int32)
    pos[:2] = [0, 4095]
    pages = (n + 63) // 64 + 2
    slot = rng.permutation(pages * 64)[:n].astype(np.int32)
    slot[5] = -1
    slot[17] = -7
    say("write_k_fp8 edges: tokens", n)
    for eps in (1e-6, 0.0):
        sl = slot.copy()
        if eps == 0.0:
            sl[[0, 2]] = -1
        o, g = _write_both(F, orc, k, pos, sl, W.norm_weight(rng), eps, tab, pages, k_row_stride=136)
        assert np.array_equal(o, g), eps


def test_write_k_fp8_workload_bit_exact(F, orc):
    wl = W.make(4, with_q=False)
    n = 16384                                  # a slice of the bulk write keeps the oracle quick
    say("write_k_fp8:", n, "tokens into", wl.num_pages, "pages")
    tab = W.rope_table(wl.max_pos)
    o, g = _write_both(F, orc, wl.k_new[:n], wl.pos_new[:n], wl.slot_new[:n], wl.norm_w, wl.eps, tab, wl.num_pages)
    assert np.array_equal(o, g)


def test_write_k_fp8_skips_tokens_outside_pool_or_table(F, orc):
    """A slot past the pool or a position outside the table skips the token
    (the kernel's own range checks): the pool equals the oracle's with those
    tokens marked as padding."""
    rng = np.random.default_rng(122)
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
    o, g = _write_both(F, orc, k, pos, oslot, W.norm_weight(rng), 1e-6, tab, pages, gpu_slot=gslot, gpu_pos=gpos)
    assert np.array_equal(o, g)


# ---------------------------------------------------------------- Q pack

def _pack_both(F, orc, q, pos, tab, w, w_scale, gpu_pos=None):
    o = orc.pack_q_fp8(q, pos, tab, w, w_scale)
    g = F.pack_q_fp8(bf16(q), dev(pos if gpu_pos is None else gpu_pos), bf16(tab), dev(w), w_scale)
    torch.cuda.synchronize()
    return o, tuple(x.cpu().numpy() for x in g)


def _same(a, b):
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("heads", [64, 16, 32, 80, 128])
def test_pack_q_fp8_bit_exact(F, orc, heads):
    rng = np.random.default_rng(130 + heads)
    T = 37
    tab = W.rope_table(1 << 14)
    q = W.bf16_normal(rng, (T, heads, 128))
    q[0, 0] = 0
    pos = rng.integers(0, 1 << 14, T).astype(np.int32)
    w = rng.uniform(-1, 1, (T, heads)).astype(np.float32)
    o, g = _pack_both(F, orc, q, pos, tab, w, 0.37)
    for a, b in zip(o, g):
        assert _same(a, b)


def test_pack_q_fp8_magnitude_extremes(F, orc):
    """Heads from 1e-36 (scale clamped at 2^-127, subnormal inputs) through
    1e-20 and 1e-15 (both sides of the pre-scaling switch) to 1e30."""
    rng = np.random.default_rng(131)
    T, heads = 40, 64
    tab = W.rope_table(1 << 12)
    q = W.bf16_normal(rng, (T, heads, 128))
    q[0] = 0
    for h, mag in enumerate((1e-36, 1e-30, 1e-25, 1e-20, 1e-18, 1e-15, 1e-10, 1e10, 1e30)):
        q[1:, h] = W.bf16_from_f32(rng.standard_normal((T - 1, 128)).astype(np.float32) * np.float32(mag))
    pos = rng.integers(0, 1 << 12, T).astype(np.int32)
    w = rng.uniform(-1, 1, (T, heads)).astype(np.float32)
    o, g = _pack_both(F, orc, q, pos, tab, w, 1.0)
    for a, b in zip(o, g):
        assert _same(a, b)


def test_pack_q_fp8_position_outside_table_encodes_zero(F, orc):
    """Rows whose position is outside the table come out as the encoding of
    the +0 vector (the oracle's quantiser on zeros); the other rows as usual."""
    rng = np.random.default_rng(132)
    T, heads, max_pos = 9, 16, 256
    tab = W.rope_table(max_pos)
    q = W.bf16_normal(rng, (T, heads, 128))
    pos = rng.integers(0, max_pos, T).astype(np.int32)
    gpos = pos.copy()
    gpos[[2, 5]] = [max_pos, -1]
    w = rng.uniform(0, 1, (T, heads)).astype(np.float32)
    qf, qs, wo = orc.pack_q_fp8(q, pos, tab, w, 1.0)
    zc, zs = orc.quant_fp8_128(np.zeros(128, np.float32))
    qf[[2, 5]] = zc
    qs[[2, 5]] = zs
    g = F.pack_q_fp8(bf16(q), dev(gpos), bf16(tab), dev(w), 1.0)
    torch.cuda.synchronize()
    for a, b in zip((qf, qs, wo), g):
        assert _same(a, b.cpu().numpy())


@pytest.mark.parametrize("n_tok,n_rows", [(64, 64), (1000, 7), (0, 5), (300, 0)])
def test_write_k_pack_q_fp8_one_launch_bit_exact(F, orc, n_tok, n_rows):
    rng = np.random.default_rng([n_tok, n_rows, 8])
    tab = W.rope_table(1 << 12)
    num_pages = max(1, (n_tok + 63) // 64 + 3)
    k = W.bf16_normal(rng, (n_tok, 128))
    pos_k = rng.integers(0, 1 << 12, n_tok).astype(np.int32)
    slot = rng.permutation(num_pages * 64)[:n_tok].astype(np.int32)
    if n_tok > 2:
        slot[1] = -1
    nw = W.norm_weight(rng)
    q = W.bf16_normal(rng, (n_rows, 64, 128))
    pos_q = rng.integers(0, 1 << 12, n_rows).astype(np.int32)
    w = rng.uniform(-1, 1, (n_rows, 64)).astype(np.float32)
    pool_o = np.full(num_pages * PAGE8, 0xA5, np.uint8)
    orc.write_k_fp8(k, pos_k, slot, nw, 1e-6, tab, pool_o)
    qo = orc.pack_q_fp8(q, pos_q, tab, w, 0.5)
    pool_g = dev(np.full(num_pages * PAGE8, 0xA5, np.uint8))
    qg = F.write_k_pack_q_fp8(bf16(k), dev(pos_k), dev(slot), bf16(nw), 1e-6, bf16(tab), pool_g, bf16(q),
                              dev(pos_q), dev(w), 0.5)
    torch.cuda.synchronize()
    assert np.array_equal(pool_g.cpu().numpy(), pool_o)
    for a, b in zip(qo, qg):
        assert _same(a, b.cpu().numpy())


# ---------------------------------------------------------------- logits

def _gpu_logits(F, qf, qs, w, wl, pool, stride=None, sentinel=np.nan):
    T = qf.shape[0]
    stride = stride or max(1, wl.max_ctx)
    out = torch.full((T, stride), float(sentinel), dtype=torch.float32, device=DEV)
    F.mqa_logits_fp8(dev(qf), dev(qs), dev(w), dev(wl.req_row_indptr), dev(wl.row_ctx), dev(wl.block_table),
                     dev(pool), wl.max_rows_per_req, wl.max_ctx, logits=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _encoded_small(orc, wl):
    tab = W.rope_table(wl.max_pos)
    pool = np.zeros(wl.num_pages * PAGE8, np.uint8)
    orc.write_k_fp8(wl.k_new, wl.pos_new, wl.slot_new, wl.norm_w, wl.eps, tab, pool)
    qf, qs, w = orc.pack_q_fp8(wl.q, wl.pos_q, tab, wl.w, wl.w_scale)
    return qf, qs, w, pool


@pytest.mark.parametrize("heads", [64, 16, 128, 48, 112])
def test_logits_fp8_small_mixed_all_scores(F, orc, heads):
    wl = W.small(heads=heads)
    qf, qs, w, pool = _encoded_small(orc, wl)
    stride = wl.max_ctx + 5
    gpu = _gpu_logits(F, qf, qs, w, wl, pool, stride=stride)
    _, f64, T, A, B = orc.logits_fp8(qf, qs, w, wl.req_row_indptr, wl.row_ctx, wl.block_table, pool,
                                     logits_stride=stride, want_f64=True, want_b16=True)
    check_rows(gpu, f64, T, A, B, wl.row_ctx, f"fp8 small mixed, {heads} heads")
    assert np.all(np.isnan(gpu[~in_context(wl.row_ctx, stride)])), "wrote past a row's context"


def test_logits_fp8_rows_per_request_variants(F, orc):
    for rows, ctxs in (((1, 1, 1), (64, 1, 200)), ((2, 2), (100, 65)), ((6, 3), (300, 129)),
                       ((5, 4, 7), (77, 300, 16)), ((16, 1), (250, 90)), ((9, 2), (0, 40))):
        wl = W.small(seed=sum(rows) + sum(ctxs) + 1, rows=rows, ctxs=ctxs)
        qf, qs, w, pool = _encoded_small(orc, wl)
        gpu = _gpu_logits(F, qf, qs, w, wl, pool)
        _, f64, T, A, B = orc.logits_fp8(qf, qs, w, wl.req_row_indptr, wl.row_ctx, wl.block_table, pool,
                                         logits_stride=gpu.shape[1], want_f64=True, want_b16=True)
        check_rows(gpu, f64, T, A, B, wl.row_ctx, f"fp8 rows per request {rows}")
        assert np.all(np.isnan(gpu[~in_context(wl.row_ctx, gpu.shape[1])]))


@pytest.mark.parametrize("heads,rows", [(16, (1, 1, 1)), (48, (2, 1, 2)), (80, (1, 1)), (128, (2, 2, 1)),
                                       (112, (1, 2))])
def test_logits_fp8_one_wave_staging_every_head_count(F, orc, heads, rows):
    """One or two rows per request: one-wave work-groups that stage their
    own FP8 pages through LDS, at every M-tile count; ragged contexts (a
    partial last page, a zero-context row, a context under one page)."""
    ctxs = tuple((70, 0, 700, 130, 1)[: len(rows)])
    wl = W.small(seed=heads + sum(rows), rows=rows, ctxs=ctxs, heads=heads)
    qf, qs, w, pool = _encoded_small(orc, wl)
    gpu = _gpu_logits(F, qf, qs, w, wl, pool)
    _, f64, T, A, B = orc.logits_fp8(qf, qs, w, wl.req_row_indptr, wl.row_ctx, wl.block_table, pool,
                                     logits_stride=gpu.shape[1], want_f64=True, want_b16=True)
    check_rows(gpu, f64, T, A, B, wl.row_ctx, f"fp8 one-wave staging, {heads} heads, rows {rows}")
    assert np.all(np.isnan(gpu[~in_context(wl.row_ctx, gpu.shape[1])]))


def test_logits_fp8_128_heads_many_rows(F, orc):
    """128 heads with more than two rows per request (the row cap for the
    wide FP8 operands)."""
    wl = W.small(seed=77, rows=(5, 3, 1), ctxs=(200, 70, 129), heads=128)
    qf, qs, w, pool = _encoded_small(orc, wl)
    gpu = _gpu_logits(F, qf, qs, w, wl, pool)
    _, f64, T, A, B = orc.logits_fp8(qf, qs, w, wl.req_row_indptr, wl.row_ctx, wl.block_table, pool,
                                     logits_stride=gpu.shape[1], want_f64=True, want_b16=True)
    check_rows(gpu, f64, T, A, B, wl.row_ctx, "fp8 128 heads, 5 rows per request")
    assert np.all(np.isnan(gpu[~in_context(wl.row_ctx, gpu.shape[1])]))


def _samples(rng, wl, n):
    rows = rng.integers(0, wl.n_rows, n)
    ctx = wl.row_ctx[rows].astype(np.int64)
    keep = ctx > 0
    rows, ctx = rows[keep], ctx[keep]
    toks = (rng.random(rows.size) * ctx).astype(np.int64)
    live = np.nonzero(wl.row_ctx > 0)[0]
    extra_r = np.concatenate([live, live])
    extra_t = np.concatenate([np.zeros(live.size, np.int64), wl.row_ctx[live].astype(np.int64) - 1])
    return np.concatenate([rows, extra_r]), np.concatenate([toks, extra_t])


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_logits_fp8_full_size_sampled(F, orc, cfg):
    """Each workload at its real shape over a random FP8 pool, in the launch
    configuration the bench times; sampled scores against the oracle, and
    nothing written past any row's context."""
    wl = W.make(cfg, with_q=False)
    rng = np.random.default_rng([cfg, 199])
    pool = W.random_pool_fp8(rng, wl.num_pages)
    qf, qs, w = W.random_q_fp8(rng, wl.n_rows)
    say("logits_fp8", wl.name, "scores", wl.scores)
    stride = wl.max_ctx + 3
    gpu = _gpu_logits(F, qf, qs, w, wl, pool, stride=stride)
    rows, toks = _samples(rng, wl, 6000)
    f64, T, A, B = orc.logits_fp8_sampled(qf, qs, w, wl.req_row_indptr, wl.block_table, pool, rows, toks,
                                          want_b16=True)
    check_fp8(gpu[rows, toks], f64, T, A, B, f"fp8 {wl.name} (sampled)")
    cols = np.arange(stride)[None, :]
    assert np.all(np.isnan(gpu[cols >= wl.row_ctx[:, None]]))
    assert not np.any(np.isnan(gpu[cols < wl.row_ctx[:, None]]))


def test_logits_fp8_invariant_to_pages_and_batch(F, orc):
    wl = W.small(seed=31, rows=(3, 6, 1), ctxs=(500, 257, 64))
    rng = np.random.default_rng(6)
    pool = W.random_pool_fp8(rng, wl.num_pages)
    qf, qs, w = W.random_q_fp8(rng, wl.n_rows)
    base = _gpu_logits(F, qf, qs, w, wl, pool)
    perm = rng.permutation(wl.num_pages)
    inv = np.argsort(perm)
    pool2 = pool.reshape(wl.num_pages, PAGE8)[perm].reshape(-1)
    wl2 = W.small(seed=31, rows=(3, 6, 1), ctxs=(500, 257, 64))
    wl2.block_table = np.where(wl.block_table >= 0, inv[np.maximum(wl.block_table, 0)], -1).astype(np.int32)
    moved = _gpu_logits(F, qf, qs, w, wl2, pool2)
    assert np.array_equal(np.nan_to_num(base, nan=7.0).view(np.uint32), np.nan_to_num(moved, nan=7.0).view(np.uint32))
    b = 1
    r0, r1 = wl.req_row_indptr[b], wl.req_row_indptr[b + 1]
    wl3 = W.small(seed=31, rows=(3, 6, 1), ctxs=(500, 257, 64))
    wl3.req_row_indptr = np.array([0, r1 - r0], np.int32)
    wl3.row_ctx = wl.row_ctx[r0:r1].copy()
    wl3.block_table = wl.block_table[b:b + 1].copy()
    alone = _gpu_logits(F, qf[r0:r1], qs[r0:r1], w[r0:r1], wl3, pool, stride=base.shape[1])
    assert np.array_equal(np.nan_to_num(base[r0:r1], nan=7.0).view(np.uint32),
                          np.nan_to_num(alone, nan=7.0).view(np.uint32))


def _bits(x):
    return np.nan_to_num(x, nan=7.0).view(np.uint32)


@pytest.mark.parametrize("heads", [64, 128, 32])
def test_logits_fp8_same_bits_from_every_kernel(F, orc, heads):
    """A 16-row request (shared-page kernel: the FP8 pages staged in LDS,
    several page chunks) gives the same bits as its rows scored one per
    request (one-wave work-groups staging their own pages), as the same
    request next to a one-row request (a non-uniform batch: shared-page
    kernel, two rows per work-group, short chunks) and as the same request
    next to fifteen one-row requests (under three rows per request on
    average: per-wave kernel with direct operand loads, several rows per
    wave); sampled scores against the oracle."""
    rng = np.random.default_rng([23, heads])
    ctx = 20_000 if heads == 64 else 5_000  # 313 pages: many page chunks
    pages = (ctx + 63) // 64
    pool = W.random_pool_fp8(rng, pages + 3)
    qf, qs, w = W.random_q_fp8(rng, 16, heads=heads)
    table = rng.permutation(pages + 3)[:pages].astype(np.int32)[None, :]
    row_ctx = (ctx - np.arange(16)[::-1] * 7).astype(np.int32)
    row_ctx[3] = 0

    def run(q, qsc, wt, ind, cx, bt, mr):
        o = torch.full((q.shape[0], ctx), float("nan"), dtype=torch.float32, device=DEV)
        F.mqa_logits_fp8(dev(q), dev(qsc), dev(wt), dev(ind), dev(cx), dev(bt), dev(pool), mr, ctx, logits=o)
        torch.cuda.synchronize()
        return o.cpu().numpy()

    say("fp8 kernels", heads, "heads")
    a = run(qf, qs, w, np.array([0, 16], np.int32), row_ctx, table, 16)
    one = run(qf, qs, w, np.arange(17, dtype=np.int32), row_ctx, np.repeat(table, 16, axis=0), 1)
    m = run(np.concatenate([qf, qf[:1]]), np.concatenate([qs, qs[:1]]), np.concatenate([w, w[:1]]),
            np.array([0, 16, 17], np.int32), np.concatenate([row_ctx, row_ctx[:1]]), np.repeat(table, 2, axis=0),
            16)
    pick = np.concatenate([np.arange(16), np.arange(15)])
    few = run(qf[pick], qs[pick], w[pick], np.concatenate([[0], np.arange(16, 32)]).astype(np.int32), row_ctx[pick],
              np.repeat(table, 16, axis=0), 16)
    for x in (one, m[:16], few[:16]):
        assert np.array_equal(_bits(a), _bits(x))
    assert np.array_equal(_bits(a[:1]), _bits(m[16:])) and np.array_equal(_bits(a[:15]), _bits(few[16:]))
    live = np.nonzero(row_ctx > 0)[0]
    rows = live.repeat(40)
    toks = (rng.random(rows.size) * row_ctx[rows]).astype(np.int64)
    f64, T, A, B = orc.logits_fp8_sampled(qf, qs, w, np.array([0, 16], np.int32), table, pool, rows, toks,
                                          want_b16=True)
    check_fp8(a[rows, toks], f64, T, A, B, f"fp8 16-row request, {heads} heads (sampled)")
    cols = np.arange(ctx)[None, :]
    assert np.all(np.isnan(a[cols >= row_ctx[:, None]])) and not np.any(np.isnan(a[cols < row_ctx[:, None]]))


def test_logits_fp8_context_past_the_row_is_cut(F, orc):
    """A device context length beyond the logits row (a broken contract) is
    cut by the kernel to the row: the next row's entries stay untouched."""
    wl = W.small(seed=41, rows=(1, 1), ctxs=(100, 60))
    qf, qs, w, pool = _encoded_small(orc, wl)
    stride = 128
    bad = wl.row_ctx.copy()
    bad[0] = 1 << 20
    out = torch.full((wl.n_rows + 1, stride), float("nan"), dtype=torch.float32, device=DEV)
    F.mqa_logits_fp8(dev(qf), dev(qs), dev(w), dev(wl.req_row_indptr), dev(bad), dev(wl.block_table), dev(pool),
                     wl.max_rows_per_req, wl.max_ctx, logits=out[:wl.n_rows])
    torch.cuda.synchronize()
    g = out.cpu().numpy()
    _, f64, T, A, B = orc.logits_fp8(qf, qs, w, wl.req_row_indptr, wl.row_ctx, wl.block_table, pool,
                                     logits_stride=stride, want_f64=True, want_b16=True)
    c1 = wl.row_ctx[1]
    check_fp8(g[1, :c1], f64[1, :c1], T[1, :c1], A[1, :c1], B[1, :c1], "fp8 row after a broken context")
    assert np.all(np.isnan(g[1, c1:])) and np.all(np.isnan(g[2]))


# ---------------------------------------------------------------- whole FP8 path

def test_fp8_chain_write_pack_logits_topk(F, orc):
    """Writer -> Q pack -> logits -> top-k on the FP8 cache, each stage fed
    the previous GPU stage's output; bytes bit-exact, logits within the
    bound, and the top-k exact on the GPU logits and, where the oracle's
    k-th and (k+1)-th exact values are further apart than twice the bound,
    the same set the exact logits select."""
    wl = W.small(seed=12)
    tab = W.rope_table(wl.max_pos)
    pool_o = np.zeros(wl.num_pages * PAGE8, np.uint8)
    orc.write_k_fp8(wl.k_new, wl.pos_new, wl.slot_new, wl.norm_w, wl.eps, tab, pool_o)
    qo = orc.pack_q_fp8(wl.q, wl.pos_q, tab, wl.w, wl.w_scale)
    pool_g = torch.zeros(wl.num_pages * PAGE8, dtype=torch.uint8, device=DEV)
    qg = F.write_k_pack_q_fp8(bf16(wl.k_new), dev(wl.pos_new), dev(wl.slot_new), bf16(wl.norm_w), wl.eps, bf16(tab),
                              pool_g, bf16(wl.q), dev(wl.pos_q), dev(wl.w), wl.w_scale)
    logits = F.mqa_logits_fp8(qg[0], qg[1], qg[2], dev(wl.req_row_indptr), dev(wl.row_ctx), dev(wl.block_table),
                              pool_g, wl.max_rows_per_req, wl.max_ctx)
    k = 64
    idx = F.topk(logits, dev(wl.row_ctx), k, wl.max_ctx)
    torch.cuda.synchronize()
    assert np.array_equal(pool_g.cpu().numpy(), pool_o)
    for a, b in zip(qo, qg):
        assert _same(a, b.cpu().numpy())
    lg = logits.cpu().numpy()
    _, f64, T, A, B = orc.logits_fp8(*qo, wl.req_row_indptr, wl.row_ctx, wl.block_table, pool_o,
                                     logits_stride=lg.shape[1], want_f64=True, want_b16=True)
    exp_idx = orc.topk(lg, wl.row_ctx, k)
    assert np.array_equal(idx.cpu().numpy(), exp_idx)
    check_rows(lg, f64, T, A, B, wl.row_ctx, "fp8 chain (encoded K and Q)")
    for t in range(wl.n_rows):
        c = wl.row_ctx[t]
        if c > k:
            tol = fp8_bound(T[t, :c], A[t, :c], B[t, :c])
            srt = np.sort(f64[t, :c])[::-1]
            if srt[k - 1] - srt[k] > 2 * tol.max():
                exact = set(np.argsort(-f64[t, :c], kind="stable")[:k].tolist())
                assert exact == set(exp_idx[t][exp_idx[t] >= 0].tolist())
