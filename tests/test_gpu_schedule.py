"""GPU tests of the device-built logits schedule (fp4idx_mqa_logits_plan /
_run) through the C ABI.

The schedule is integer work: its items are read back from the workspace
and checked exactly (every (row, page) a row's context reaches is scored by
exactly one item, items stay inside their requests and the kernel's limits,
the count inside the workspace, at most 16 empty items evening out the
per-XCD lists).  The logits it drives are compared bit for
bit with the host-bounded call and against the oracle's bar (tests/bars.py).
Inputs come from the seeded generators; expected values from the oracle.
"""
import numpy as np
import pytest
import torch

from bars import check_fp4, in_context
from sparse_attention_fp4_fp4idx_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"
HDR_WORDS = 16
BLK_WORDS = 10
MAX_ITEM_PAGES = 512


def layout(n_rows, n_reqs, rows_pb):
    """(most row blocks, word offset of the items) of a plan whose kernel
    takes rows_pb rows per work-group (per-wave kernel: per wave): a 16-word
    header, the per-request list (n_reqs + 1, padded to 4 words), the
    per-block list (10 words a block, padded to 4), then the items."""
    nonempty = min(n_reqs, n_rows)
    blocks = min(n_rows, (n_rows + nonempty * (rows_pb - 1)) // rows_pb) if nonempty else 0
    return blocks, HDR_WORDS + ((n_reqs + 1 + 3) & ~3) + ((BLK_WORDS * blocks + 3) & ~3)


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from sparse_attention_fp4_fp4idx_amd import fp4idx
    fp4idx.load()
    return fp4idx


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bits(x):
    return np.nan_to_num(x, nan=7.0).view(np.uint32)


def say(*a):
    print(*a, flush=True)


def _check_schedule(ws, indptr, ctx, max_ctx, n_rows):
    """Every (row, page) below the row's context (cut to max_ctx) is covered
    by exactly one item; items lie inside their requests and limits."""
    w = ws.cpu().numpy().view(np.int32)
    n_reqs = indptr.size - 1
    n_items, rows_pb, waves, fixed = int(w[0]), int(w[4]), int(w[5]), int(w[6])
    assert (waves, rows_pb) in ((0, 1), (0, 2), (2, 4), (2, 6), (4, 8)) and n_items >= 0
    max_pages = fixed if waves == 0 else MAX_ITEM_PAGES
    # the plan lays its lists out for the shape it picked
    _, items_off = layout(n_rows, n_reqs, rows_pb)
    items = w[items_off:items_off + 4 * n_items].reshape(n_items, 4).astype(np.int64)
    empty = np.all(items == 0, axis=1)            # evens out the per-XCD lists
    assert int(empty.sum()) <= 16, int(empty.sum())
    req, row0, page0, packed = items[~empty].T
    nr, npg = packed & 0xFF, packed >> 8
    assert np.all((req >= 0) & (req < n_reqs))
    assert np.all((nr >= 1) & (nr <= rows_pb) & (npg >= 1) & (npg <= max_pages) & (page0 >= 0))
    assert np.all((indptr[req] <= row0) & (row0 + nr <= indptr[req + 1]))
    # coverage count per (row, page): +1 at an item's first page, -1 past its last, summed along pages
    need = (np.minimum(ctx.astype(np.int64), max_ctx) + 63) // 64
    width = int(max(int((page0 + npg).max(initial=0)), int(need.max(initial=0)))) + 1
    rep = np.repeat(np.arange(req.size), nr)
    rows = row0[rep] + (np.arange(rep.size) - np.repeat(np.cumsum(nr) - nr, nr))
    diff = np.zeros((max(n_rows, 1), width + 1), np.int32)
    np.add.at(diff, (rows, page0[rep]), 1)
    np.add.at(diff, (rows, page0[rep] + npg[rep]), -1)
    cover = np.cumsum(diff, axis=1)[:n_rows, :width]
    needed = np.arange(width)[None, :] < need[:, None]
    bad = np.argwhere(needed & (cover != 1))
    assert bad.size == 0, (bad[:5].tolist(), cover[tuple(bad[0])] if bad.size else None)
    # pages past a row's own context may be covered (its block's longest row reaches them), once at most
    assert cover.max(initial=0) <= 1
    return n_items, rows_pb, waves


@pytest.mark.parametrize("case", ["small", "ragged", "empty_requests", "mixed48", "prefill", "decode256x6",
                                  "decode64", "two_rows", "many_requests", "many_blocks", "blocks_1100_two_rows"])
def test_plan_covers_every_row_page_exactly_once(F, case):
    """The plan for batches of every kernel shape: near-uniform many rows
    (4 x 2), six rows (2 x 3), one to sixteen rows with contexts 8k-32k, a
    prefill of 4,096 rows, one and two rows per request (per-wave kernel),
    requests without rows and rows without context; and the plan's paths
    for large batches: over 4,096 requests (the request search outside LDS)
    and rows (context lengths read from memory), over 128 row blocks (one
    thread per block writes its items) and over 1,024 (the per-block list
    in the workspace)."""
    rng = np.random.default_rng(7)
    if case == "small":
        rows, ctxs = (1, 6, 16, 3), (130, 1000, 777, 0)
        indptr = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
        ctx = np.concatenate([[c] * r for c, r in zip(ctxs, rows)]).astype(np.int32)
    elif case == "ragged":
        R = rng.integers(1, 17, 30)
        indptr = np.concatenate([[0], np.cumsum(R)]).astype(np.int32)
        ctx = rng.integers(0, 5000, int(indptr[-1])).astype(np.int32)
    elif case == "empty_requests":
        R = np.array([0, 3, 0, 0, 9, 0, 1, 0])
        indptr = np.concatenate([[0], np.cumsum(R)]).astype(np.int32)
        ctx = rng.integers(1, 3000, int(indptr[-1])).astype(np.int32)
        ctx[2] = 0
    elif case == "two_rows":
        R = rng.integers(1, 4, 40)
        indptr = np.concatenate([[0], np.cumsum(R)]).astype(np.int32)
        ctx = rng.integers(0, 9000, int(indptr[-1])).astype(np.int32)
    elif case == "many_requests":   # 6,000 one-row requests (per-wave, one row per wave)
        indptr = np.arange(6001, dtype=np.int32)
        ctx = rng.integers(0, 3000, 6000).astype(np.int32)
    elif case == "many_blocks":     # 2,000 requests of 8 rows: 16,000 rows, 2,000 blocks of 4 x 2
        indptr = (8 * np.arange(2001)).astype(np.int32)
        ctx = rng.integers(0, 2000, 16000).astype(np.int32)
    elif case == "blocks_1100_two_rows":   # 1,100 requests of 2 rows (per-wave, two rows per wave)
        indptr = (2 * np.arange(1101)).astype(np.int32)
        ctx = rng.integers(1, 5000, 2200).astype(np.int32)
    else:
        wl = W.make({"mixed48": 4, "prefill": 3, "decode256x6": 2, "decode64": 1}[case], with_q=False)
        indptr, ctx = wl.req_row_indptr, wl.row_ctx
    n_rows, n_reqs = int(indptr[-1]), indptr.size - 1
    max_ctx = int(ctx.max(initial=0)) + 1
    for heads in (64, 128, 96):
        plan = F.LogitsPlan(heads, dev(indptr), dev(ctx), max_ctx).build()
        torch.cuda.synchronize()
        n_items, rows_pb, waves = _check_schedule(plan.workspace, indptr, ctx, max_ctx, n_rows)
        say(case, "heads", heads, "items", n_items,
            f"per-wave kernel, {rows_pb} rows per wave" if waves == 0 else f"shared-page {waves} x {rows_pb // waves}")


def test_plan_with_a_small_workspace_makes_longer_items(F, orc):
    """A workspace far below the size for the batch's contexts: the plan
    makes fewer, longer items (still every (row, page) once) and the logits
    are the same bits; a workspace too small for the row blocks' lists is
    refused."""
    wl = W.small(seed=81, rows=(5, 9, 2, 16), ctxs=(9000, 3000, 12000, 6000))
    rng = np.random.default_rng(81)
    pay, sc = W.random_pool(rng, wl.num_pages)
    qf = rng.integers(0, 256, (wl.n_rows, 64, 64)).astype(np.uint8)
    qs = rng.integers(124, 129, (wl.n_rows, 64, 4)).astype(np.uint8)
    w = rng.uniform(0, 1, (wl.n_rows, 64)).astype(np.float32)
    args = (dev(qf), dev(qs), dev(w), dev(wl.req_row_indptr), dev(wl.row_ctx), dev(wl.block_table), dev(pay), dev(sc))
    full = F.mqa_logits_workspace_bytes(wl.n_rows, wl.n_reqs, wl.max_ctx)
    ref = F.mqa_logits_bounded(*args, wl.max_rows_per_req, wl.max_ctx,
                               logits=torch.full((wl.n_rows, wl.max_ctx), float("nan"), device=DEV)).cpu().numpy()
    probe = F.LogitsPlan(64, args[3], args[4], wl.max_ctx).build()
    rows_pb = int(probe.workspace[16:20].cpu().numpy().view(np.int32)[0])
    blocks, items_off = layout(wl.n_rows, wl.n_reqs, rows_pb)
    lists = 4 * items_off
    for nbytes in (full, lists + 16 * (blocks + 3), lists + 16 * 4 * blocks):
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
        out = F.mqa_logits(*args, logits=torch.full((wl.n_rows, wl.max_ctx), float("nan"), device=DEV), workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(bits(out.cpu().numpy()), bits(ref)), nbytes
        n_items, _, _ = _check_schedule(ws, wl.req_row_indptr, wl.row_ctx, wl.max_ctx, wl.n_rows)
        say("workspace", nbytes, "of", full, "bytes:", n_items, "items")
    with pytest.raises(F.Fp4idxError, match="workspace"):   # room for fewer items than row blocks
        F.mqa_logits(*args, logits=torch.empty((wl.n_rows, wl.max_ctx), device=DEV),
                     workspace=torch.zeros(lists + 16 * (blocks - 1), dtype=torch.uint8, device=DEV))


def test_one_plan_serves_every_layer(F, orc):
    """A plan built once for a batch drives the logits of several layers
    (other Q, weights, pools and block tables over the same rows and
    contexts), each run bit-identical to the host-bounded call and within
    the oracle's bar; a run only reads the plan, so repeated runs see the
    same schedule."""
    wl = W.small(seed=82, rows=(3, 8, 1, 12), ctxs=(5000, 2200, 700, 4100))
    plan = F.LogitsPlan(64, dev(wl.req_row_indptr), dev(wl.row_ctx), wl.max_ctx).build()
    built = plan.workspace.clone()
    ind, ctx = dev(wl.req_row_indptr), dev(wl.row_ctx)
    for layer in range(3):
        rng = np.random.default_rng([82, layer])
        pay, sc = W.random_pool(rng, wl.num_pages)
        perm = rng.permutation(wl.num_pages).astype(np.int32)
        bt = np.where(wl.block_table >= 0, perm[np.maximum(wl.block_table, 0)], -1).astype(np.int32)
        qf = rng.integers(0, 256, (wl.n_rows, 64, 64)).astype(np.uint8)
        qs = rng.integers(124, 129, (wl.n_rows, 64, 4)).astype(np.uint8)
        w = rng.uniform(0, 1, (wl.n_rows, 64)).astype(np.float32)
        for rep in range(2):
            got = plan.run(dev(qf), dev(qs), dev(w), dev(bt), dev(pay), dev(sc),
                           logits=torch.full((wl.n_rows, wl.max_ctx), float("nan"), device=DEV))
            ref = F.mqa_logits_bounded(dev(qf), dev(qs), dev(w), ind, ctx, dev(bt), dev(pay), dev(sc),
                                       wl.max_rows_per_req, wl.max_ctx,
                                       logits=torch.full((wl.n_rows, wl.max_ctx), float("nan"), device=DEV))
            torch.cuda.synchronize()
            g = got.cpu().numpy()
            assert np.array_equal(bits(g), bits(ref.cpu().numpy())), (layer, rep)
        _, f64, T, A = orc.logits(qf, qs, w, wl.req_row_indptr, wl.row_ctx, bt, pay, sc, logits_stride=wl.max_ctx,
                                  want_f64=True)
        m = in_context(wl.row_ctx, wl.max_ctx)
        check_fp4(g[m], f64[m], T[m], A[m], f"plan reused, layer {layer}")
        assert np.all(np.isnan(g[~m]))
    # the runs leave the plan as it was built
    assert torch.equal(plan.workspace, built)


@pytest.mark.parametrize("rows,ctxs", [((3, 8, 1, 12), (5000, 2200, 700, 4100)),   # shared-page items
                                       ((1,) * 40, tuple(1000 + 613 * i for i in range(40))),  # per-wave
                                       ((9, 16, 5, 2, 14, 7), (30000, 9000, 17000, 4000, 26000, 12000))])
def test_a_batch_always_gets_the_same_plan(F, rows, ctxs):
    """Building the plan of one batch again, into fresh and into reused
    workspaces, gives the same workspace bytes every time: the batch's work
    (which sizes the short items) is summed in a fixed order, so nothing in
    the plan depends on the order the device happens to run its threads."""
    wl = W.small(seed=sum(rows), rows=rows, ctxs=ctxs)
    ind, ctx = dev(wl.req_row_indptr), dev(wl.row_ctx)

    def defined(ws):
        """What a plan defines: the header's words, the per-request list and
        the items up to the item count (the per-block list is the plan's
        own scratch, and the rest of a fresh workspace is never written)."""
        w = ws.cpu().numpy().view(np.int32)
        _, items_off = layout(wl.n_rows, wl.n_reqs, int(w[4]))
        req = w[HDR_WORDS:HDR_WORDS + wl.n_reqs + 1]
        return np.concatenate([w[:7], req, w[items_off:items_off + 4 * int(w[0])]])

    first = F.LogitsPlan(64, ind, ctx, wl.max_ctx).build()
    torch.cuda.synchronize()
    ref = defined(first.workspace)
    _check_schedule(first.workspace, wl.req_row_indptr, wl.row_ctx, wl.max_ctx, wl.n_rows)
    say("plan", rows[:6], "items", int(ref[0]))
    for rep in range(8):
        again = F.LogitsPlan(64, ind, ctx, wl.max_ctx).build() if rep % 2 else first.build()
        torch.cuda.synchronize()
        assert np.array_equal(defined(again.workspace), ref), rep


def test_planned_runs_interleaved_with_other_plans(F, orc):
    """Two batches, each with its own workspace, planned and run alternately
    on one stream (a serving loop with two batches in flight): each run uses
    its own plan and matches the host-bounded call."""
    wls = [W.small(seed=83, rows=(4, 4, 2), ctxs=(3000, 900, 2000)),
           W.small(seed=84, rows=(1, 16), ctxs=(6000, 1500))]
    st = []
    for i, wl in enumerate(wls):
        rng = np.random.default_rng([84, i])
        pay, sc = W.random_pool(rng, wl.num_pages)
        qf = rng.integers(0, 256, (wl.n_rows, 64, 64)).astype(np.uint8)
        qs = rng.integers(124, 129, (wl.n_rows, 64, 4)).astype(np.uint8)
        w = rng.uniform(0, 1, (wl.n_rows, 64)).astype(np.float32)
        a = (dev(qf), dev(qs), dev(w), dev(wl.req_row_indptr), dev(wl.row_ctx), dev(wl.block_table), dev(pay),
             dev(sc))
        ref = F.mqa_logits_bounded(*a, wl.max_rows_per_req, wl.max_ctx,
                                   logits=torch.full((wl.n_rows, wl.max_ctx), float("nan"), device=DEV)).cpu().numpy()
        plan = F.LogitsPlan(64, a[3], a[4], wl.max_ctx).build()
        st.append((a, ref, plan))
    for rep in range(3):
        for a, ref, plan in st:
            got = plan.run(a[0], a[1], a[2], a[5], a[6], a[7],
                           logits=torch.full(ref.shape, float("nan"), device=DEV))
            torch.cuda.synchronize()
            assert np.array_equal(bits(got.cpu().numpy()), bits(ref)), rep


@pytest.mark.parametrize("case", ["many_blocks", "many_requests"])
def test_large_batch_logits_follow_the_plan(F, orc, case):
    """Logits of batches on the plan's large-batch paths (2,000 requests of
    8 rows: 2,000 shared-page blocks, the per-block list in the workspace;
    6,000 one-row requests: the request search outside LDS), scheduled
    against the host-bounded call bit for bit, and sampled scores against
    the oracle's bar."""
    rng = np.random.default_rng(91)
    n_reqs, R = (2000, 8) if case == "many_blocks" else (6000, 1)
    n_rows = n_reqs * R
    indptr = (R * np.arange(n_reqs + 1)).astype(np.int32)
    ctx = rng.integers(0, 1500, n_rows).astype(np.int32)
    pages_per_req = 24                                         # 1,536 tokens of table per request
    num_pages = n_reqs * pages_per_req
    table = rng.permutation(num_pages).astype(np.int32).reshape(n_reqs, pages_per_req)
    pay, sc = W.random_pool(rng, num_pages)
    qf = rng.integers(0, 256, (n_rows, 64, 64)).astype(np.uint8)
    qs = rng.integers(124, 129, (n_rows, 64, 4)).astype(np.uint8)
    w = rng.uniform(0, 1, (n_rows, 64)).astype(np.float32)
    width = pages_per_req * 64
    a = (dev(qf), dev(qs), dev(w), dev(indptr), dev(ctx), dev(table), dev(pay), dev(sc))
    say(case, "rows", n_rows, "requests", n_reqs)
    got = F.mqa_logits(*a, logits=torch.full((n_rows, width), float("nan"), device=DEV))
    ref = F.mqa_logits_bounded(*a, R, width, logits=torch.full((n_rows, width), float("nan"), device=DEV))
    torch.cuda.synchronize()
    g = got.cpu().numpy()
    assert np.array_equal(bits(g), bits(ref.cpu().numpy()))
    rows = rng.integers(0, n_rows, 3000)
    rows = rows[ctx[rows] > 0]
    toks = (rng.random(rows.size) * ctx[rows]).astype(np.int64)
    f64, T, A = orc.logits_sampled(qf, qs, w, indptr, table, pay, sc, rows, toks)
    check_fp4(g[rows, toks], f64, T, A, f"{case}: {n_rows} rows (sampled)")
    cols = np.arange(width)[None, :]
    assert np.all(np.isnan(g[cols >= ctx[:, None]]))
