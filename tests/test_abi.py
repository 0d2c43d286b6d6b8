"""C ABI checks that need no GPU: the built library loads, exports every
symbol include/fp4idx.h declares, and rejects bad host arguments with a
negative status before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4idx.h")


@pytest.fixture(scope="module")
def F():
    from sparse_attention_fp4_fp4idx_amd import fp4idx
    if not os.path.exists(fp4idx.lib_path()):
        pytest.fail("libfp4idx.so is not built; run __graft_entry__.build() first")
    fp4idx.load()
    return fp4idx


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4idx_\w+)\s*\(", text)))


def test_header_declares_the_four_path_calls():
    names = declared_functions()
    for n in ("fp4idx_write_k", "fp4idx_pack_q", "fp4idx_mqa_logits", "fp4idx_topk"):
        assert n in names


def test_every_declared_symbol_is_exported(F):
    lib = ctypes.CDLL(F.lib_path())
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(F.EXPORTS) <= set(declared_functions())


def test_status_strings_and_version(F):
    assert F.status_string(0) == "ok"
    for code in (-1, -2, -3, -4):
        assert F.status_string(code) != "unknown status"
    assert F.status_string(-99) == "unknown status"
    assert F.version() >= 100


def test_host_validation_rejects_before_any_launch(F):
    lib = F.load()
    E = -1
    fake = ctypes.c_void_p(0x1000)
    # write_k: nulls, bad stride, unaligned row pointer, negative eps
    assert lib.fp4idx_write_k(None, 5, 128, None, None, None, 1e-6, None, 10, None, None, 1, None) == E
    assert lib.fp4idx_write_k(fake, 5, 100, fake, fake, fake, 1e-6, fake, 10, fake, fake, 1, None) == E
    assert lib.fp4idx_write_k(ctypes.c_void_p(0x1002), 5, 128, fake, fake, fake, 1e-6, fake, 10, fake, fake, 1,
                              None) == E
    assert lib.fp4idx_write_k(fake, 5, 128, fake, fake, fake, -1.0, fake, 10, fake, fake, 1, None) == E
    assert lib.fp4idx_write_k(fake, -1, 128, fake, fake, fake, 1e-6, fake, 10, fake, fake, 1, None) == E
    assert lib.fp4idx_write_k(None, 0, 128, None, None, None, 1e-6, None, 10, None, None, 0, None) == 0
    # pack_q: unsupported head counts, short stride
    for h in (0, 8, 40, 144, 256):
        assert lib.fp4idx_pack_q(fake, 2, h, 128 * 64, fake, fake, 10, fake, 1.0, fake, fake, fake, None) == E
    assert lib.fp4idx_pack_q(fake, 2, 64, 100, fake, fake, 10, fake, 1.0, fake, fake, fake, None) == E
    # logits: ctx bound beyond the block table or the logits row
    assert lib.fp4idx_mqa_logits_bounded(fake, fake, fake, 4, 64, fake, 1, fake, fake, 2, fake, fake, 4, fake, 4096,
                                         4, 129, None) == E
    assert lib.fp4idx_mqa_logits_bounded(fake, fake, fake, 4, 64, fake, 1, fake, fake, 2, fake, fake, 4, fake, 100,
                                         4, 128, None) == E
    assert lib.fp4idx_mqa_logits_bounded(fake, fake, fake, 4, 64, fake, 1, fake, fake, 2, fake, fake, 4, fake, 128,
                                         5, 128, None) == E
    assert lib.fp4idx_mqa_logits_bounded(fake, fake, fake, 4, 40, fake, 1, fake, fake, 2, fake, fake, 4, fake, 128,
                                         4, 128, None) == E
    # top-k: k out of range, ctx bound beyond the row
    for k in (0, -3, 2049):
        assert lib.fp4idx_topk(fake, 1, 100, fake, k, fake, None) == E
        assert lib.fp4idx_topk_bounded(fake, 1, 100, fake, k, fake, 10, None) == E
    assert lib.fp4idx_topk_bounded(fake, 1, 100, fake, 16, fake, 101, None) == E
    assert lib.fp4idx_topk(fake, 1, -1, fake, 16, fake, None) == E
    # write_k_pack_q: each half is checked as its own call would check it
    wk = [fake, 5, 128, fake, fake, fake, 1e-6, fake, 10, fake, fake, 1]
    pq = [fake, 2, 64, 128 * 64, fake, fake, 1.0, fake, fake, fake]
    assert lib.fp4idx_write_k_pack_q(*wk[:2], 100, *wk[3:], *pq, None) == E          # K row stride
    assert lib.fp4idx_write_k_pack_q(*wk, fake, 2, 40, *pq[3:], None) == E           # head count
    assert lib.fp4idx_write_k_pack_q(*wk, None, 2, 64, *pq[3:], None) == E           # null Q
    assert lib.fp4idx_write_k_pack_q(None, 0, 128, None, None, None, 1e-6, None, 10, None, None, 0,
                                     None, 0, 64, 128 * 64, None, None, 1.0, None, None, None, None) == 0
    # timing events armed before a rejected call are dropped with it (no launch, events untouched)
    assert lib.fp4idx_time_next_call(None, None) == 0
    assert lib.fp4idx_time_next_call(fake, fake) == 0
    assert lib.fp4idx_topk_bounded(fake, 1, 100, fake, 0, fake, 10, None) == E
    # empty problems are a successful no-op
    assert lib.fp4idx_topk(None, 0, 100, None, 16, None, None) == 0
    assert lib.fp4idx_topk_bounded(None, 0, 100, None, 16, None, 10, None) == 0
    assert lib.fp4idx_mqa_logits_bounded(None, None, None, 0, 64, None, 0, None, None, 0, None, None, 0, None, 0, 0,
                                         0, None) == 0


def test_scheduled_logits_validate_workspace_and_arguments(F):
    """fp4idx_mqa_logits / _plan / _run: a missing, unaligned or too small
    workspace is FP4IDX_E_WORKSPACE; bad scalars FP4IDX_E_INVALID; an empty
    batch is a no-op; the workspace size grows with rows, requests and
    contexts and is 0 for an empty batch."""
    lib = F.load()
    E, EW = -1, -4
    fake = ctypes.c_void_p(0x1000)
    need = lib.fp4idx_mqa_logits_workspace_bytes(4, 1, 128)
    assert need > 0
    assert lib.fp4idx_mqa_logits_workspace_bytes(0, 1, 128) == 0
    assert lib.fp4idx_mqa_logits_workspace_bytes(4, 0, 128) == 0
    assert lib.fp4idx_mqa_logits_workspace_bytes(8, 1, 128) >= need
    assert lib.fp4idx_mqa_logits_workspace_bytes(64, 64, 128) > need
    assert lib.fp4idx_mqa_logits_workspace_bytes(4, 1, 4096) > need
    assert lib.fp4idx_mqa_logits_workspace_bytes(4, 4, 128) > need
    #          q     qs    w     T  H   ind   B  ctx   bt    bts pay   sc    P  out   ls   ws    wsb   stream
    base = [fake, fake, fake, 4, 64, fake, 1, fake, fake, 2, fake, fake, 4, fake, 128, fake, need, None]

    def call(fn, **kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return fn(*a)
    for fn in (lib.fp4idx_mqa_logits, lib.fp4idx_mqa_logits_run):
        assert call(fn, a15=None) == EW                       # no workspace
        assert call(fn, a15=ctypes.c_void_p(0x1008)) == EW    # not 16-byte aligned
        assert call(fn, a16=64) == EW                         # too small for the batch's row blocks
        assert call(fn, a4=48 + 8) == E
        assert call(fn, a4=144) == E
        assert call(fn, a3=-1) == E
        assert call(fn, a12=0) == E                           # rows but no pool
        assert call(fn, a0=None) == E
        assert call(fn, a13=None) == E
        assert call(fn, a0=ctypes.c_void_p(0x1004)) == E      # unaligned Q codes
        assert call(fn, a3=0, a15=None) == 0                  # empty batch: nothing launched
        assert call(fn, a6=0, a15=None) == 0
    #             T  H   ind   B  ctx  max_ctx ws    wsb  stream
    pbase = [4, 64, fake, 1, fake, 128, fake, need, None]
    assert lib.fp4idx_mqa_logits_plan(*pbase[:6], None, need, None) == EW
    assert lib.fp4idx_mqa_logits_plan(*pbase[:6], fake, 32, None) == EW
    assert lib.fp4idx_mqa_logits_plan(4, 40, *pbase[2:]) == E
    assert lib.fp4idx_mqa_logits_plan(4, 64, None, *pbase[3:]) == E
    assert lib.fp4idx_mqa_logits_plan(4, 64, fake, 1, fake, -1, fake, need, None) == E
    assert lib.fp4idx_mqa_logits_plan(0, 64, None, 1, None, 128, None, 0, None) == 0


def test_fp8_calls_validate_like_their_fp4_twins(F):
    lib = F.load()
    E = -1
    fake = ctypes.c_void_p(0x1000)
    # write_k_fp8: nulls, bad stride, unaligned pool, negative eps; empty batch is a no-op
    assert lib.fp4idx_write_k_fp8(None, 5, 128, None, None, None, 1e-6, None, 10, None, 1, None) == E
    assert lib.fp4idx_write_k_fp8(fake, 5, 120, fake, fake, fake, 1e-6, fake, 10, fake, 1, None) == E
    assert lib.fp4idx_write_k_fp8(fake, 5, 128, fake, fake, fake, 1e-6, fake, 10, ctypes.c_void_p(0x1008), 1,
                                  None) == E
    assert lib.fp4idx_write_k_fp8(fake, 5, 128, fake, fake, fake, -1.0, fake, 10, fake, 1, None) == E
    assert lib.fp4idx_write_k_fp8(None, 0, 128, None, None, None, 1e-6, None, 10, None, 0, None) == 0
    # pack_q_fp8: head counts, stride, unaligned code output
    for h in (0, 8, 40, 144, 256):
        assert lib.fp4idx_pack_q_fp8(fake, 2, h, 128 * 64, fake, fake, 10, fake, 1.0, fake, fake, fake, None) == E
    assert lib.fp4idx_pack_q_fp8(fake, 2, 64, 100, fake, fake, 10, fake, 1.0, fake, fake, fake, None) == E
    assert lib.fp4idx_pack_q_fp8(fake, 2, 64, 128 * 64, fake, fake, 10, fake, 1.0, ctypes.c_void_p(0x1004), fake,
                                 fake, None) == E
    # one-launch pair: each half checked as its own call
    wk = [fake, 5, 128, fake, fake, fake, 1e-6, fake, 10, fake, 1]
    pq = [fake, 2, 64, 128 * 64, fake, fake, 1.0, fake, fake, fake]
    assert lib.fp4idx_write_k_pack_q_fp8(*wk[:2], 100, *wk[3:], *pq, None) == E
    assert lib.fp4idx_write_k_pack_q_fp8(*wk, fake, 2, 40, *pq[3:], None) == E
    assert lib.fp4idx_write_k_pack_q_fp8(None, 0, 128, None, None, None, 1e-6, None, 10, None, 0,
                                         None, 0, 64, 128 * 64, None, None, 1.0, None, None, None, None) == 0
    # logits_fp8: ctx bound beyond the table / the row, head count, unaligned scale, empty pool
    args = [fake, fake, fake, 4, 64, fake, 1, fake, fake, 2, fake, 4, fake, 4096, 4, 128, None]
    a = list(args); a[15] = 129
    assert lib.fp4idx_mqa_logits_fp8(*a) == E
    a = list(args); a[13] = 100
    assert lib.fp4idx_mqa_logits_fp8(*a) == E
    a = list(args); a[4] = 40
    assert lib.fp4idx_mqa_logits_fp8(*a) == E
    a = list(args); a[1] = ctypes.c_void_p(0x1002)
    assert lib.fp4idx_mqa_logits_fp8(*a) == E
    a = list(args); a[11] = 0
    assert lib.fp4idx_mqa_logits_fp8(*a) == E
    assert lib.fp4idx_mqa_logits_fp8(None, None, None, 0, 64, None, 0, None, None, 0, None, 0, None, 0, 0, 0,
                                     None) == 0


def test_fused_logits_topk_validates_its_host_arguments(F):
    lib = F.load()
    E = -1
    fake = ctypes.c_void_p(0x1000)
    #          q     qs    w     T  H   ind   B  ctx   bt    bts pay   sc    P  k   out   mr  mc   stream
    base = [fake, fake, fake, 4, 64, fake, 1, fake, fake, 2, fake, fake, 4, 16, fake, 4, 128, None]

    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.fp4idx_mqa_logits_topk(*a)
    assert call(a4=128) == E            # more than 64 heads: not served by the fused call
    assert call(a4=80) == E
    assert call(a4=40) == E
    for k in (0, -1, 2049):
        assert call(a13=k) == E
    assert call(a16=129) == E           # ctx bound beyond the block table
    assert call(a9=1024, a16=32769) == E  # beyond the fused row
    assert call(a15=0) == E             # rows exist but no row per request
    assert call(a15=5) == E             # more rows per request than rows
    assert call(a0=ctypes.c_void_p(0x1004)) == E
    assert call(a14=None) == E
    assert call(a3=0, a15=0) == 0 and call(a6=0) == 0   # empty batch: nothing launched


def test_peak_microbenchmarks_validate_their_arguments(F):
    lib = F.load()
    fake = ctypes.c_void_p(0x1000)
    assert lib.fp4idx_peak_mfma_fp4(0, fake, None) == -1
    assert lib.fp4idx_peak_mfma_fp4(8, None, None) == -1
    assert lib.fp4idx_peak_valu_fp32(0, fake, None) == -1
    assert lib.fp4idx_peak_valu_fp32(8, None, None) == -1
    assert lib.fp4idx_peak_mfma_valu(3, 8, fake, None) == -1
    assert lib.fp4idx_peak_mfma_valu(-1, 8, fake, None) == -1
    assert lib.fp4idx_peak_mfma_valu(2, 0, fake, None) == -1
    assert lib.fp4idx_peak_mfma_valu(0, 8, None, None) == -1
    assert lib.fp4idx_peak_read(fake, 100, fake, None) == -1          # not a multiple of 16
    assert lib.fp4idx_peak_read(fake, 0, fake, None) == -1
    assert lib.fp4idx_peak_read(ctypes.c_void_p(0x1008), 4096, fake, None) == -1
    assert lib.fp4idx_peak_read(None, 4096, fake, None) == -1


def test_binding_imports_no_oracle():
    import sparse_attention_fp4_fp4idx_amd.fp4idx as m
    src = open(m.__file__).read()
    assert "oracle" not in src.replace("no fallback", "")
    for f in os.listdir(os.path.join(ROOT, "sparse_attention_fp4_fp4idx_amd", "csrc")):
        assert "oracle" not in open(os.path.join(ROOT, "sparse_attention_fp4_fp4idx_amd", "csrc", f)).read().lower()


def _logits_inputs(T=3, H=64, B=2, max_ctx=200, code=64, fp8=False):
    import torch
    q = torch.zeros((T, H, code), dtype=torch.uint8)
    qs = torch.zeros((T, H), dtype=torch.float32) if fp8 else torch.zeros((T, H, 4), dtype=torch.uint8)
    return dict(q=q, qs=qs, w=torch.zeros((T, H)), ind=torch.zeros(B + 1, dtype=torch.int32),
                ctx=torch.zeros(T, dtype=torch.int32), bt=torch.zeros((B, (max_ctx + 63) // 64), dtype=torch.int32),
                pay=torch.zeros(5 * 4096, dtype=torch.uint8), sc=torch.zeros(5 * 256, dtype=torch.uint8),
                pool=torch.zeros(5 * 8448, dtype=torch.uint8), out=torch.zeros((T, max_ctx)),
                idx=torch.zeros((T, 16), dtype=torch.int32))


def _raises(F, fn, *words):
    with pytest.raises(F.Fp4idxError) as e:
        fn()
    for w in words:
        assert w in str(e.value), (w, str(e.value))


def test_binding_checks_buffer_sizes_before_any_call(F):
    """Every buffer the kernels index by T, H, k, n_reqs or num_pages is
    checked against those sizes in the binding: a mismatch raises
    Fp4idxError naming the buffer (host tensors: with every size right the
    binding gets as far as asking for device memory)."""
    import torch
    d = _logits_inputs()

    def logits(**kw):
        a = dict(d, **kw)
        return lambda: F.mqa_logits_bounded(a["q"], a["qs"], a["w"], a["ind"], a["ctx"], a["bt"], a["pay"], a["sc"],
                                            2, 200, logits=a["out"])

    def planned(**kw):
        a = dict(d, **kw)
        return lambda: F.mqa_logits(a["q"], a["qs"], a["w"], a["ind"], a["ctx"], a["bt"], a["pay"], a["sc"],
                                    logits=a["out"], workspace=a.get("ws", torch.zeros(64, dtype=torch.uint8)))
    _raises(F, planned(), "device tensor")
    _raises(F, planned(ctx=torch.zeros(2, dtype=torch.int32)), "row_ctx")
    _raises(F, planned(out=torch.zeros((2, 200))), "output")
    _raises(F, planned(sc=torch.zeros(4 * 256, dtype=torch.uint8)), "pool sizes")
    _raises(F, planned(ws=torch.zeros(64, dtype=torch.int32)), "workspace")
    _raises(F, logits(), "device tensor")
    _raises(F, logits(out=torch.zeros((2, 200))), "output")                 # fewer rows than T
    _raises(F, logits(out=torch.zeros((3, 150))), "output")                 # rows shorter than max_ctx
    _raises(F, logits(ctx=torch.zeros(2, dtype=torch.int32)), "row_ctx")
    _raises(F, logits(bt=torch.zeros((1, 4), dtype=torch.int32)), "block_table")
    _raises(F, logits(bt=torch.zeros((2, 3), dtype=torch.int32)), "block_table")  # 3 pages < 200 tokens
    _raises(F, logits(w=torch.zeros((3, 32))), "w")
    _raises(F, logits(qs=torch.zeros((3, 64, 3), dtype=torch.uint8)), "q_scale")
    _raises(F, logits(q=torch.zeros((3, 64, 32), dtype=torch.uint8)), "Q codes")
    _raises(F, logits(sc=torch.zeros(4 * 256, dtype=torch.uint8)), "pool sizes")

    def fused(**kw):
        a = dict(d, **kw)
        return lambda: F.mqa_logits_topk(a["q"], a["qs"], a["w"], a["ind"], a["ctx"], a["bt"], a["pay"], a["sc"], 16,
                                         2, 200, out_idx=a["idx"])
    _raises(F, fused(), "device tensor")
    _raises(F, fused(idx=torch.zeros((3, 8), dtype=torch.int32)), "out_idx")
    _raises(F, fused(ctx=torch.zeros(4, dtype=torch.int32)), "row_ctx")

    def topk(**kw):
        a = dict(d, **kw)
        return lambda: F.topk(a["out"], a["ctx"], 16, a.get("mc", 200), out_idx=a["idx"])
    _raises(F, topk(), "device tensor")
    _raises(F, topk(idx=torch.zeros((2, 16), dtype=torch.int32)), "out_idx")
    _raises(F, topk(ctx=torch.zeros(5, dtype=torch.int32)), "row_ctx")
    _raises(F, topk(mc=201), "max_ctx")

    d8 = _logits_inputs(code=128, fp8=True)

    def logits8(**kw):
        a = dict(d8, **kw)
        return lambda: F.mqa_logits_fp8(a["q"], a["qs"], a["w"], a["ind"], a["ctx"], a["bt"], a["pool"], 2, 200,
                                        logits=a["out"])
    _raises(F, logits8(), "device tensor")
    _raises(F, logits8(qs=torch.zeros((3, 64, 4), dtype=torch.uint8)), "q_scale")
    _raises(F, logits8(pool=torch.zeros(5 * 8448 + 1, dtype=torch.uint8)), "8448")
    _raises(F, logits8(out=torch.zeros((3, 199))), "output")

    # the encoders
    q = torch.zeros((3, 64, 128), dtype=torch.bfloat16)
    tab = torch.zeros((10, 64), dtype=torch.bfloat16)
    pos = torch.zeros(3, dtype=torch.int32)
    w = torch.zeros((3, 64))
    _raises(F, lambda: F.pack_q(q, pos, tab, w), "device tensor")
    _raises(F, lambda: F.pack_q(q, pos[:2], tab, w), "pos")
    _raises(F, lambda: F.pack_q(q, pos, tab, w[:, :32]), "w_in")
    _raises(F, lambda: F.pack_q(q, pos, tab, w, 1.0, torch.zeros((3, 64, 32), dtype=torch.uint8)), "q codes")
    _raises(F, lambda: F.pack_q(q, pos, tab, w, 1.0, None, torch.zeros((3, 64), dtype=torch.uint8)), "q_scale")
    _raises(F, lambda: F.pack_q(q, pos, tab, w, 1.0, None, None, torch.zeros((2, 64))), "w_out")
    _raises(F, lambda: F.pack_q(q, pos, torch.zeros((10, 32), dtype=torch.bfloat16), w), "cos_sin")
    _raises(F, lambda: F.pack_q_fp8(q, pos, tab, w, 1.0, None, torch.zeros((3, 64, 4), dtype=torch.float32)),
            "q_scale")
    k = torch.zeros((4, 128), dtype=torch.bfloat16)
    kp, ks = torch.zeros(4, dtype=torch.int32), torch.zeros(4, dtype=torch.int32)
    nw = torch.zeros(128, dtype=torch.bfloat16)
    _raises(F, lambda: F.write_k(k, kp, ks, nw, 1e-6, tab, d["pay"], d["sc"]), "device tensor")
    _raises(F, lambda: F.write_k(k, kp, ks, nw[:64], 1e-6, tab, d["pay"], d["sc"]), "norm_w")
    _raises(F, lambda: F.write_k(k[:, :100], kp, ks, nw, 1e-6, tab, d["pay"], d["sc"]), "k must be")
    _raises(F, lambda: F.write_k(k, kp[:3], ks, nw, 1e-6, tab, d["pay"], d["sc"]), "pos/slot")
    _raises(F, lambda: F.read_k(d["pay"], d["sc"], ks, out=torch.zeros((3, 128))), "out must be")
