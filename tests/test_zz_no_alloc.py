"""fp4idx_mqa_logits_noalloc: the scheduled FP4 logits with the work
schedule in the library's own per-device scratch array instead of a caller
workspace (for callers that cannot allocate device memory).

GPU: through the C ABI, two calls in a row (the second on a smaller batch,
so the array still holds the first call's schedule when it starts), each
compared bit for bit with fp4idx_mqa_logits on a caller workspace and
against the oracle's bar (tests/bars.py).  CPU: the size limit and the
argument checks, which come before any device call.
"""
import ctypes

import numpy as np
import pytest
import torch

from bars import check_fp4, in_context
from sparse_attention_fp4_fp4idx_amd import workloads as W

DEV = "cuda"
E_INVALID, E_SCRATCH = -1, -5
SCRATCH_BYTES = 16 << 20


def test_noalloc_refuses_batches_past_its_scratch():
    """A batch whose schedule needs more than the 16 MiB array is refused
    with FP4IDX_E_SCRATCH before anything touches the device; bad arguments
    are FP4IDX_E_INVALID; an empty batch is a no-op."""
    from sparse_attention_fp4_fp4idx_amd import fp4idx as F
    lib = F.load()
    fake = ctypes.c_void_p(0x1000)
    # 65,535 requests of 16 rows with logits rows of 2^20 tokens
    big_rows, big_reqs, big_ctx = 65535 * 16, 65535, 1 << 20
    assert lib.fp4idx_mqa_logits_workspace_bytes(big_rows, big_reqs, big_ctx) > SCRATCH_BYTES
    #       q     qs    w     T         H   ind   B         ctx   bt    bts            pay   sc    P  out   ls       st
    args = [fake, fake, fake, big_rows, 64, fake, big_reqs, fake, fake, big_ctx // 64, fake, fake, 4, fake, big_ctx,
            None]
    assert lib.fp4idx_mqa_logits_noalloc(*args) == E_SCRATCH
    assert b"scratch" in lib.fp4idx_status_string(E_SCRATCH)
    # the stated example of a batch that fits
    assert lib.fp4idx_mqa_logits_workspace_bytes(16384, 64, 131072) <= SCRATCH_BYTES
    small = list(args)
    small[0] = None                                     # null Q: the host checks still run first
    assert lib.fp4idx_mqa_logits_noalloc(*small) == E_INVALID
    small = list(args)
    small[4] = 40                                       # head count (not a multiple of 16)
    assert lib.fp4idx_mqa_logits_noalloc(*small) == E_INVALID
    small = list(args)
    small[3] = 0                                        # empty batch: nothing launched
    assert lib.fp4idx_mqa_logits_noalloc(*small) == 0
    with pytest.raises(F.Fp4idxError, match="logits buffer"):
        t = torch.zeros(1)
        F.mqa_logits_noalloc(t, t, t, t, t, t, t, t, None)


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


def _batch(seed, rows, ctxs):
    wl = W.small(seed=seed, rows=rows, ctxs=ctxs)
    rng = np.random.default_rng(seed)
    pay, sc = W.random_pool(rng, wl.num_pages)
    qf = rng.integers(0, 256, (wl.n_rows, 64, 64)).astype(np.uint8)
    qs = rng.integers(124, 129, (wl.n_rows, 64, 4)).astype(np.uint8)
    w = rng.uniform(0, 1, (wl.n_rows, 64)).astype(np.float32)
    return wl, (qf, qs, w, wl.req_row_indptr, wl.row_ctx, wl.block_table, pay, sc)


@pytest.mark.gpu
def test_noalloc_matches_the_workspace_call_on_two_calls_in_a_row(F, orc):
    """Call 1: 45 rows in 5 requests (shared-page kernel), contexts to
    12,000 tokens.  Call 2, right after on the same stream: 6 one-row
    requests (per-wave kernel) with shorter contexts, so it starts from the
    first call's schedule in the array.  Each output equals
    fp4idx_mqa_logits's bits on a caller workspace and meets the oracle's
    bar; entries past each row's context are left untouched."""
    cases = [(_batch(91, (12, 9, 16, 1, 7), (12000, 3000, 9000, 500, 7000)), "larger batch"),
             (_batch(92, (1, 1, 1, 1, 1, 1), (2000, 64, 4100, 1, 300, 2500)), "smaller batch")]
    outs = [(wl, host, tuple(dev(x) for x in host), torch.full((wl.n_rows, wl.max_ctx), float("nan"), device=DEV))
            for (wl, host), _ in cases]
    torch.cuda.synchronize()
    allocated = torch.cuda.memory_allocated()
    for (wl, host, a, out), (_, what) in zip(outs, cases):
        print(what, "rows", wl.n_rows, "requests", wl.n_reqs, "max ctx", wl.max_ctx, flush=True)
        F.mqa_logits_noalloc(*a, logits=out)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == allocated   # the binding allocated nothing either
    for wl, host, a, out in outs:
        ref = F.mqa_logits(*a, logits=torch.full((wl.n_rows, wl.max_ctx), float("nan"), device=DEV))
        torch.cuda.synchronize()
        g = out.cpu().numpy()
        assert np.array_equal(bits(g), bits(ref.cpu().numpy())), wl.n_rows
        qf, qs, w, ind, ctx, bt, pay, sc = host
        _, f64, T, A = orc.logits(qf, qs, w, ind, ctx, bt, pay, sc, logits_stride=wl.max_ctx, want_f64=True)
        m = in_context(ctx, wl.max_ctx)
        check_fp4(g[m], f64[m], T[m], A[m], f"no-alloc logits, {wl.n_rows} rows")
        assert np.all(np.isnan(g[~m]))
