"""GPU parity of the fused logits + top-k call (no logits written to memory).

Bar: bit-exact.  The call's indices must equal what fp4idx_mqa_logits then
fp4idx_topk write for the same inputs (same logits bit for bit, same
selection), and the oracle's top-k of those GPU logits (the selection rule);
where the oracle's exact k-th and (k+1)-th values are further apart than
twice the logits tolerance, the set must also be the one the exact logits
select.  Inputs come from the seeded generators; expected values from the
oracle or from the library's own two-call path.
"""
import numpy as np
import pytest
import torch

from bars import fp4_bound
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


def say(*a):
    print(*a, flush=True)


def _both(F, wl, qf, qs, w, pay, sc, k):
    """(fused indices, two-call indices, two-call logits) on the GPU."""
    args = (dev(qf), dev(qs), dev(w), dev(wl.req_row_indptr), dev(wl.row_ctx), dev(wl.block_table), dev(pay),
            dev(sc))
    fused = F.mqa_logits_topk(*args, k, wl.max_rows_per_req, wl.max_ctx)
    logits = F.mqa_logits(*args, max_ctx=wl.max_ctx)
    two = F.topk(logits, args[4], k, wl.max_ctx)
    torch.cuda.synchronize()
    return fused.cpu().numpy(), two.cpu().numpy(), logits.cpu().numpy()


def _encoded(orc, wl):
    tab = W.rope_table(wl.max_pos)
    pay = np.zeros(wl.num_pages * 4096, np.uint8)
    sc = np.zeros(wl.num_pages * 256, np.uint8)
    orc.write_k(wl.k_new, wl.pos_new, wl.slot_new, wl.norm_w, wl.eps, tab, pay, sc)
    qf, qs, w = orc.pack_q(wl.q, wl.pos_q, tab, wl.w, wl.w_scale)
    return qf, qs, w, pay, sc


@pytest.mark.parametrize("heads,k", [(64, 64), (16, 256), (32, 7), (64, 2048), (48, 300)])
def test_fused_equals_two_calls_small_mixed(F, orc, heads, k):
    """Single- and multi-row requests, ragged contexts, a zero-context row,
    rows shorter than k; the result against the two-call path, the oracle's
    selection of the same logits and the exact logits where the k-th gap is
    clear."""
    wl = W.small(heads=heads)
    qf, qs, w, pay, sc = _encoded(orc, wl)
    fused, two, lg = _both(F, wl, qf, qs, w, pay, sc, k)
    assert np.array_equal(fused, two)
    assert np.array_equal(fused, orc.topk(lg, wl.row_ctx, k))
    _, f64, T, A = orc.logits(qf, qs, w, wl.req_row_indptr, wl.row_ctx, wl.block_table, pay, sc,
                              logits_stride=lg.shape[1], want_f64=True)
    for t in range(wl.n_rows):
        c = wl.row_ctx[t]
        if c > k:
            tol = fp4_bound(T[t, :c], A[t, :c])
            srt = np.sort(f64[t, :c])[::-1]
            if srt[k - 1] - srt[k] > 2 * tol.max():
                exact = set(np.argsort(-f64[t, :c], kind="stable")[:k].tolist())
                assert exact == set(fused[t][fused[t] >= 0].tolist())


@pytest.mark.parametrize("ctx", [1, 700, 1024, 1025, 4096, 4100, 8192, 9000, 16384, 20000, 32768])
def test_fused_every_row_length_bucket(F, orc, ctx):
    """Rows at and across each LDS-row size the launcher picks (1k, 4k, 8k,
    16k, 32k positions), two single-row requests over a random pool."""
    rng = np.random.default_rng([ctx, 3])
    ctxs = (ctx, max(1, ctx // 3))
    wl = W.small(seed=ctx % 1000 + 5, rows=(1, 1), ctxs=ctxs)
    pay, sc = W.random_pool(rng, wl.num_pages)
    qf = rng.integers(0, 256, (wl.n_rows, 64, 64)).astype(np.uint8)
    qs = rng.integers(124, 129, (wl.n_rows, 64, 4)).astype(np.uint8)
    w = rng.uniform(0, 1, (wl.n_rows, 64)).astype(np.float32)
    for k in (1, 2048):
        fused, two, lg = _both(F, wl, qf, qs, w, pay, sc, k)
        assert np.array_equal(fused, two), (ctx, k)
        assert np.array_equal(fused, orc.topk(lg, wl.row_ctx, k)), (ctx, k)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_fused_full_size_equals_two_calls(F, orc, cfg):
    """The workloads at their real shapes (random pool and Q codes): the
    fused call writes exactly the two-call path's indices."""
    wl = W.make(cfg, with_q=False)
    rng = np.random.default_rng([cfg, 77])
    pay, sc = W.random_pool(rng, wl.num_pages)
    qf = rng.integers(0, 256, (wl.n_rows, 64, 64)).astype(np.uint8)
    qs = rng.integers(124, 129, (wl.n_rows, 64, 4)).astype(np.uint8)
    w = rng.uniform(0, 1, (wl.n_rows, 64)).astype(np.float32)
    say("fused", wl.name, "rows", wl.n_rows, "k", wl.topk)
    fused, two, lg = _both(F, wl, qf, qs, w, pay, sc, wl.topk)
    assert np.array_equal(fused, two)
    rows = np.unique(np.concatenate([np.arange(min(8, wl.n_rows)), np.linspace(0, wl.n_rows - 1, 8).astype(int)]))
    sub = orc.topk(lg[rows], wl.row_ctx[rows], wl.topk)
    assert np.array_equal(fused[rows], sub)
