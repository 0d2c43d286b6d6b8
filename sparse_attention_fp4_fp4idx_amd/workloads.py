"""Seeded synthetic inputs for the FP4 lightning-indexer path.

This module only draws inputs.  It holds none of the method's arithmetic
(no normalisation, rotation, Hadamard, quantisation, scoring or selection),
so both the HIP path's tests and the CPU oracle may take their inputs from
it.  Everything is numpy (PCG64) with an explicit seed.

Shapes follow the workloads the pages describe:
  * 64 index heads of 128 dims, the first 64 dims rotary
    ("[AMD] Enable FP4 indexer for Deepseek V4", Motivation and
    Modifications);
  * 64 tokens per page in a split payload/scale pool ([P2] Motivation);
  * 68k-token inputs at compression ratio 4 (~17k compressed tokens), decode
    batches up to 256 requests with 6 draft/verify rows each
    ("dsv4.1-amd: KV cache layouts, FP4 indexer, ..." Summary), top-k 2048.
Inputs are bf16 N(0,1) for K and Q, bf16 U(0.5,1.5) for the RMSNorm weight,
fp32 U(0,1) for head weights, and a bf16 RoPE cos/sin table with
theta_j = 10000^(-j/32).  Compressed token i of a request sits at RoPE
position 4*i; a query row at raw position p sees ctx = floor((p+1)/4)
compressed tokens.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

HEADS = 64
DIM = 128
ROPE_DIMS = 64
PAGE = 64
PAYLOAD_PAGE_BYTES = 4 * 64 * 16   # [1, 4, 64, 16]
SCALE_PAGE_BYTES = 4 * 64          # [1, 4, 64]
MAX_POS = 262_144
EPS = 1e-6


def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + (((u >> 16) & 1) + np.uint32(0x7FFF))   # finite inputs only: no wrap-around
    return (u >> 16).astype(np.uint16)


def f32_from_bf16(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rope_table(max_pos: int = MAX_POS) -> np.ndarray:
    """bf16 [max_pos, 64]: cos(p*theta_j) in columns 0..31, sin in 32..63."""
    j = np.arange(ROPE_DIMS // 2, dtype=np.float64)
    theta = 10000.0 ** (-j / (ROPE_DIMS // 2))
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * theta[None, :]
    tab = np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)
    return bf16_from_f32(tab)


def bf16_normal(rng: np.random.Generator, shape) -> np.ndarray:
    return bf16_from_f32(rng.standard_normal(shape, dtype=np.float32))


def norm_weight(rng: np.random.Generator) -> np.ndarray:
    return bf16_from_f32(rng.uniform(0.5, 1.5, DIM).astype(np.float32))


def random_pool(rng: np.random.Generator, num_pages: int, scale_lo: int = 124, scale_hi: int = 128):
    """A pool filled directly with FP4 bytes: every payload byte is two
    uniform 4-bit codes, every scale byte uniform in [scale_lo, scale_hi]
    (the range an RMS-normalised, Hadamard-rotated N(0,1) row lands in)."""
    payload = rng.integers(0, 256, num_pages * PAYLOAD_PAGE_BYTES, dtype=np.uint8)
    scale = rng.integers(scale_lo, scale_hi + 1, num_pages * SCALE_PAGE_BYTES, dtype=np.uint8)
    return payload, scale


FP8_PAGE_BYTES = 8448   # 64 x 128 code bytes, then 64 fp32 scales


def _fp8_codes(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform E4M3 bytes with the two NaN codes (0x7F, 0xFF) moved to the
    neighbouring finite code."""
    c = rng.integers(0, 256, shape, dtype=np.uint8)
    return np.where((c & 0x7F) == 0x7F, c ^ 0x01, c).astype(np.uint8)


def random_pool_fp8(rng: np.random.Generator, num_pages: int, e_lo: int = -9, e_hi: int = -5) -> np.ndarray:
    """A fused FP8 pool filled directly: uniform E4M3 codes and per-token
    scales 2^e, e uniform in [e_lo, e_hi] (an RMS-normalised, rotated N(0,1)
    row has its largest element near 3.5, i.e. e near -7)."""
    pool = np.empty((num_pages, FP8_PAGE_BYTES), np.uint8)
    pool[:, :8192] = _fp8_codes(rng, (num_pages, 8192))
    pool[:, 8192:].view(np.float32)[:] = np.ldexp(np.float32(1.0), rng.integers(e_lo, e_hi + 1, (num_pages, 64)))
    return pool.reshape(-1)


def random_q_fp8(rng: np.random.Generator, n_rows: int, heads: int = 64, e_lo: int = -9, e_hi: int = -5):
    """Packed FP8 Q drawn directly: codes [T, H, 128], scales 2^e [T, H], weights U(0, 1)."""
    qf = _fp8_codes(rng, (n_rows, heads, 128))
    qs = np.ldexp(np.float32(1.0), rng.integers(e_lo, e_hi + 1, (n_rows, heads))).astype(np.float32)
    w = rng.uniform(0, 1, (n_rows, heads)).astype(np.float32)
    return qf, qs, w


@dataclass
class Workload:
    name: str
    seed: int
    topk: int
    # requests / rows
    req_row_indptr: np.ndarray          # int32 [B+1]
    row_ctx: np.ndarray                 # int32 [T]
    pos_q: np.ndarray                   # int32 [T]
    block_table: np.ndarray             # int32 [B, bt_stride]
    num_pages: int
    # K tokens written by the step (fused K writer)
    k_new: np.ndarray                   # bf16 bits [N, 128]
    pos_new: np.ndarray                 # int32 [N]
    slot_new: np.ndarray                # int32 [N]
    norm_w: np.ndarray                  # bf16 bits [128]
    eps: float = EPS
    w_scale: float = 1.0
    max_pos: int = MAX_POS
    heads: int = HEADS
    # Q side (drawn lazily: can be large)
    q: Optional[np.ndarray] = None      # bf16 bits [T, H, 128]
    w: Optional[np.ndarray] = None      # fp32 [T, H]
    # cached tokens already in the pool before the step
    cached_slots: Optional[np.ndarray] = None   # int32 [M]
    cached_pos: Optional[np.ndarray] = None     # int32 [M]
    extra: dict = field(default_factory=dict)

    @property
    def n_rows(self) -> int:
        return int(self.row_ctx.size)

    @property
    def n_reqs(self) -> int:
        return int(self.req_row_indptr.size - 1)

    @property
    def scores(self) -> int:
        return int(self.row_ctx.astype(np.int64).sum())

    @property
    def max_ctx(self) -> int:
        return int(self.row_ctx.max(initial=0))

    @property
    def max_rows_per_req(self) -> int:
        d = np.diff(self.req_row_indptr)
        return int(d.max(initial=0))

    def cached_k(self, rng_seed_offset: int = 1000):
        """bf16 K rows for the tokens already in the pool (drawn on demand)."""
        rng = np.random.default_rng([self.seed, rng_seed_offset])
        return bf16_normal(rng, (self.cached_slots.size, DIM))


def _finish(name, seed, topk, rows_per_req, pos_q, ctx, pages_per_req, rng, num_pages_extra=0,
            shared_prefix=None, k_new_tokens=None, q_heads=HEADS):
    """Common assembly: block tables from a random permutation of page ids."""
    B = len(rows_per_req)
    indptr = np.zeros(B + 1, np.int32)
    indptr[1:] = np.cumsum(rows_per_req)
    bt_stride = int(max(pages_per_req)) if B else 1
    # page ids: shared-prefix pages first, then each request's own pages
    n_shared = 0 if shared_prefix is None else shared_prefix[1]
    shared_reqs = set() if shared_prefix is None else set(shared_prefix[0])
    own = [p - (n_shared if b in shared_reqs else 0) for b, p in enumerate(pages_per_req)]
    num_pages = n_shared + int(sum(own)) + num_pages_extra
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.full((B, bt_stride), -1, np.int32)
    cur = n_shared
    for b in range(B):
        if b in shared_reqs:
            bt[b, :n_shared] = perm[:n_shared]
            bt[b, n_shared:pages_per_req[b]] = perm[cur:cur + own[b]]
        else:
            bt[b, :pages_per_req[b]] = perm[cur:cur + own[b]]
        cur += own[b]
    extra_pages = perm[cur:cur + num_pages_extra]
    return indptr, bt, num_pages, extra_pages


def make(idx: int, with_q: bool = True) -> Workload:
    """The five workloads: 0 tiny decode, 1 decode batch 64, 2 decode
    256 x 6 rows, 3 prefill 4096 rows, 4 mixed agentic batch."""
    seed = idx
    rng = np.random.default_rng(seed)
    norm_w = norm_weight(rng)
    if idx == 0:
        name, topk = "tiny decode: 1 row, 1024 tokens written into 16 pages", 256
        ctx = np.array([1024], np.int32)
        rows = [1]
        pos_q = np.array([4 * 1024 - 1], np.int32)
        pages = [16]
        indptr = np.array([0, 1], np.int32)
        bt = np.arange(16, dtype=np.int32)[None, :]
        num_pages = 16
        slot_new = np.arange(1024, dtype=np.int32)
        pos_new = (4 * np.arange(1024)).astype(np.int32)
        k_new = bf16_normal(rng, (1024, DIM))
        cached_slots = np.zeros(0, np.int32)
        cached_pos = np.zeros(0, np.int32)
    elif idx == 1:
        name, topk = "decode batch 64: 1 row each, ctx U[1024,16384]", 2048
        B = 64
        cb = rng.integers(1024, 16384 + 1, B).astype(np.int32)
        rows = [1] * B
        pos_q = (4 * cb - 1).astype(np.int32)
        ctx = cb.copy()
        pages = [int((c + PAGE - 1) // PAGE) for c in cb]
        indptr, bt, num_pages, _ = _finish(name, seed, topk, rows, pos_q, ctx, pages, rng)
        # the step writes each request's newest compressed token (index ctx-1)
        slot_new = np.array([bt[b, (cb[b] - 1) // PAGE] * PAGE + (cb[b] - 1) % PAGE for b in range(B)], np.int32)
        pos_new = (4 * (cb - 1)).astype(np.int32)
        k_new = bf16_normal(rng, (B, DIM))
        cs, cp = [], []
        for b in range(B):
            s = np.arange(cb[b] - 1)
            cs.append(bt[b, s // PAGE] * PAGE + s % PAGE)
            cp.append(4 * s)
        cached_slots = np.concatenate(cs).astype(np.int32)
        cached_pos = np.concatenate(cp).astype(np.int32)
    elif idx == 2:
        name, topk = "decode batch 256 x 6 rows, 17408 cached tokens each", 2048
        B, R, C = 256, 6, 17408
        rows = [R] * B
        p = np.arange(69626, 69632, dtype=np.int64)
        pos_q = np.tile(p, B).astype(np.int32)
        ctx = ((pos_q.astype(np.int64) + 1) // 4).astype(np.int32)
        pages = [C // PAGE] * B
        indptr, bt, num_pages, _ = _finish(name, seed, topk, rows, pos_q, ctx, pages, rng)
        # compressed tokens 17406 and 17407 are completed by this step's rows
        new_idx = np.array([17406, 17407])
        slot_new = (bt[:, new_idx // PAGE] * PAGE + new_idx % PAGE).reshape(-1).astype(np.int32)
        pos_new = np.tile(4 * new_idx, B).astype(np.int32)
        k_new = bf16_normal(rng, (slot_new.size, DIM))
        s = np.arange(17406)
        cached_slots = (bt[:, s // PAGE] * PAGE + s % PAGE).reshape(-1).astype(np.int32)
        cached_pos = np.tile(4 * s, B).astype(np.int32)
    elif idx == 3:
        name, topk = "prefill: 4096 rows over 16384 cached + 1024 new tokens", 2048
        T, C0, N = 4096, 16384, 1024
        rows = [T]
        pos_q = (4 * C0 + np.arange(T)).astype(np.int32)
        ctx = ((pos_q.astype(np.int64) + 1) // 4).astype(np.int32)
        pages = [(C0 + N) // PAGE]
        indptr, bt, num_pages, _ = _finish(name, seed, topk, rows, pos_q, ctx, pages, rng)
        new_idx = np.arange(C0, C0 + N)
        slot_new = (bt[0, new_idx // PAGE] * PAGE + new_idx % PAGE).astype(np.int32)
        pos_new = (4 * new_idx).astype(np.int32)
        k_new = bf16_normal(rng, (N, DIM))
        s = np.arange(C0)
        cached_slots = (bt[0, s // PAGE] * PAGE + s % PAGE).astype(np.int32)
        cached_pos = (4 * s).astype(np.int32)
    elif idx == 4:
        name, topk = "mixed agentic: 48 requests, ctx U[8192,32768], 1-16 rows, 40% shared prefix", 2048
        B = 48
        Cb = rng.integers(8192, 32768 + 1, B).astype(np.int64)
        Rb = rng.integers(1, 16 + 1, B).astype(np.int64)
        shared = sorted(rng.choice(B, 19, replace=False).tolist())
        rows = Rb.tolist()
        pos_q = np.concatenate([4 * Cb[b] - Rb[b] + np.arange(Rb[b]) for b in range(B)]).astype(np.int32)
        ctx = ((pos_q.astype(np.int64) + 1) // 4).astype(np.int32)
        pages = [int((c + PAGE - 1) // PAGE) for c in Cb]
        indptr, bt, num_pages, extra = _finish(name, seed, topk, rows, pos_q, ctx, pages, rng,
                                               num_pages_extra=1024, shared_prefix=(shared, 128))
        # bulk write: 65,536 new tokens into 1,024 fresh pages (a prefill not scored in this step)
        t = np.arange(65536)
        slot_new = (extra[t // PAGE].astype(np.int64) * PAGE + t % PAGE).astype(np.int32)
        pos_new = (4 * t).astype(np.int32)
        k_new = bf16_normal(rng, (65536, DIM))
        cs, cp, seen = [], [], set()
        for b in range(B):
            s = np.arange(Cb[b])
            if b in shared:
                if seen:
                    s = s[s >= 128 * PAGE]   # shared pages are listed once
                seen.add(b)
            cs.append(bt[b, s // PAGE] * PAGE + s % PAGE)
            cp.append(4 * s)
        cached_slots = np.concatenate(cs).astype(np.int32)
        cached_pos = np.concatenate(cp).astype(np.int32)
    else:
        raise ValueError(idx)
    T = int(ctx.size)
    wl = Workload(name=name, seed=seed, topk=topk, req_row_indptr=indptr.astype(np.int32),
                  row_ctx=ctx.astype(np.int32), pos_q=pos_q.astype(np.int32), block_table=bt.astype(np.int32),
                  num_pages=int(num_pages), k_new=k_new, pos_new=pos_new.astype(np.int32),
                  slot_new=slot_new.astype(np.int32), norm_w=norm_w, cached_slots=cached_slots,
                  cached_pos=cached_pos)
    if with_q:
        rq = np.random.default_rng([seed, 7])
        wl.q = bf16_normal(rq, (T, HEADS, DIM))
        wl.w = rq.uniform(0.0, 1.0, (T, HEADS)).astype(np.float32)
    return wl


def small(seed: int = 11, rows=(1, 6, 16, 3), ctxs=(130, 1000, 777, 0), heads: int = HEADS,
          topk: int = 256, shuffle_pages: bool = True) -> Workload:
    """A small mixed problem the oracle finishes in a second: several
    requests with different row counts, ragged contexts (not multiples of
    16 or 64), a padded row with ctx 0 and permuted pages."""
    rng = np.random.default_rng(seed)
    B = len(rows)
    indptr = np.zeros(B + 1, np.int32)
    indptr[1:] = np.cumsum(rows)
    ctx_rows, pos_rows = [], []
    for b in range(B):
        C = ctxs[b]
        for r in range(rows[b]):
            c = max(0, C - (rows[b] - 1 - r) // 4) if C > 0 else 0
            ctx_rows.append(c)
            pos_rows.append(max(0, 4 * c - 1))
    ctx = np.array(ctx_rows, np.int32)
    pos_q = np.array(pos_rows, np.int32)
    pages = [max(1, (c + PAGE - 1) // PAGE) for c in ctxs]
    num_pages = int(sum(pages)) + 2
    perm = rng.permutation(num_pages).astype(np.int32) if shuffle_pages else np.arange(num_pages, dtype=np.int32)
    bt = np.full((B, max(pages) + 1), -1, np.int32)
    cur = 0
    for b in range(B):
        bt[b, :pages[b]] = perm[cur:cur + pages[b]]
        cur += pages[b]
    slots, poss = [], []
    for b in range(B):
        s = np.arange(ctxs[b])
        slots.append(bt[b, s // PAGE] * PAGE + s % PAGE)
        poss.append(4 * s)
    slot_all = np.concatenate(slots).astype(np.int32)
    pos_all = np.concatenate(poss).astype(np.int32)
    k = bf16_normal(rng, (slot_all.size, DIM))
    T = ctx.size
    wl = Workload(name="small mixed", seed=seed, topk=topk, req_row_indptr=indptr, row_ctx=ctx, pos_q=pos_q,
                  block_table=bt, num_pages=num_pages, k_new=k, pos_new=pos_all, slot_new=slot_all,
                  norm_w=norm_weight(rng), max_pos=1 << 16, heads=heads,
                  cached_slots=np.zeros(0, np.int32), cached_pos=np.zeros(0, np.int32))
    wl.q = bf16_normal(rng, (T, heads, DIM))
    wl.w = rng.uniform(0.0, 1.0, (T, heads)).astype(np.float32)
    return wl
