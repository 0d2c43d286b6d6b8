"""Thin Python binding of ``libfp4idx.so`` (C ABI in ``include/fp4idx.h``).

Argument marshalling only: torch tensors provide device memory and the
current stream; every step of the path runs in the library's HIP kernels.
There is no fallback: if the library is missing or the device is not gfx950
the calls raise.

Functions carry the C names (``fp4idx_write_k`` ...) and short aliases
(``write_k`` ...).
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp4idx.so")
_lib = None

FP4IDX_OK = 0
HEAD_DIM = 128
ROPE_DIM = 64
PAGE_TOKENS = 64
PAYLOAD_PAGE_BYTES = 4096
SCALE_PAGE_BYTES = 256
FP8_PAGE_BYTES = 8448
MAX_TOPK = 2048
FUSED_MAX_CTX = 32768

_CALLS = ("fp4idx_write_k", "fp4idx_pack_q", "fp4idx_write_k_pack_q", "fp4idx_mqa_logits", "fp4idx_mqa_logits_plan",
          "fp4idx_mqa_logits_run", "fp4idx_mqa_logits_bounded", "fp4idx_mqa_logits_noalloc", "fp4idx_topk",
          "fp4idx_topk_bounded",
          "fp4idx_mqa_logits_topk", "fp4idx_read_k", "fp4idx_write_k_fp8", "fp4idx_pack_q_fp8", "fp4idx_write_k_pack_q_fp8",
          "fp4idx_mqa_logits_fp8", "fp4idx_peak_mfma_fp4", "fp4idx_peak_valu_fp32", "fp4idx_peak_mfma_valu",
          "fp4idx_peak_read")
EXPORTS = _CALLS + ("fp4idx_mqa_logits_workspace_bytes", "fp4idx_time_next_call", "fp4idx_status_string",
                    "fp4idx_version")


class Fp4idxError(RuntimeError):
    pass


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load the shared library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise Fp4idxError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "or python -m sparse_attention_fp4_fp4idx_amd.build")
    lib = ctypes.CDLL(_LIB_PATH)
    P, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    lib.fp4idx_write_k.argtypes = [P, i64, i64, P, P, P, f32, P, i32, P, P, i64, P]
    lib.fp4idx_pack_q.argtypes = [P, i64, i32, i64, P, P, i32, P, f32, P, P, P, P]
    lib.fp4idx_write_k_pack_q.argtypes = [P, i64, i64, P, P, P, f32, P, i32, P, P, i64,
                                          P, i64, i32, i64, P, P, f32, P, P, P, P]
    sz = ctypes.c_size_t
    lib.fp4idx_mqa_logits.argtypes = [P, P, P, i64, i32, P, i32, P, P, i32, P, P, i64, P, i64, P, sz, P]
    lib.fp4idx_mqa_logits_run.argtypes = [P, P, P, i64, i32, P, i32, P, P, i32, P, P, i64, P, i64, P, sz, P]
    lib.fp4idx_mqa_logits_plan.argtypes = [i64, i32, P, i32, P, i64, P, sz, P]
    lib.fp4idx_mqa_logits_noalloc.argtypes = [P, P, P, i64, i32, P, i32, P, P, i32, P, P, i64, P, i64, P]
    lib.fp4idx_mqa_logits_bounded.argtypes = [P, P, P, i64, i32, P, i32, P, P, i32, P, P, i64, P, i64, i32, i64, P]
    lib.fp4idx_mqa_logits_workspace_bytes.argtypes = [i64, i32, i64]
    lib.fp4idx_mqa_logits_workspace_bytes.restype = ctypes.c_size_t
    lib.fp4idx_topk.argtypes = [P, i64, i64, P, i32, P, P]
    lib.fp4idx_topk_bounded.argtypes = [P, i64, i64, P, i32, P, i64, P]
    lib.fp4idx_read_k.argtypes = [P, P, i64, P, i64, P, i64, P]
    lib.fp4idx_peak_mfma_fp4.argtypes = [i32, P, P]
    lib.fp4idx_peak_valu_fp32.argtypes = [i32, P, P]
    lib.fp4idx_peak_mfma_valu.argtypes = [i32, i32, P, P]
    lib.fp4idx_peak_read.argtypes = [P, i64, P, P]
    lib.fp4idx_mqa_logits_topk.argtypes = [P, P, P, i64, i32, P, i32, P, P, i32, P, P, i64, i32, P, i32, i64, P]
    lib.fp4idx_write_k_fp8.argtypes = [P, i64, i64, P, P, P, f32, P, i32, P, i64, P]
    lib.fp4idx_pack_q_fp8.argtypes = [P, i64, i32, i64, P, P, i32, P, f32, P, P, P, P]
    lib.fp4idx_write_k_pack_q_fp8.argtypes = [P, i64, i64, P, P, P, f32, P, i32, P, i64,
                                              P, i64, i32, i64, P, P, f32, P, P, P, P]
    lib.fp4idx_mqa_logits_fp8.argtypes = [P, P, P, i64, i32, P, i32, P, P, i32, P, i64, P, i64, i32, i64, P]
    for name in _CALLS:
        getattr(lib, name).restype = ctypes.c_int
    lib.fp4idx_time_next_call.argtypes = [P, P]
    lib.fp4idx_time_next_call.restype = ctypes.c_int
    lib.fp4idx_status_string.argtypes = [ctypes.c_int]
    lib.fp4idx_status_string.restype = ctypes.c_char_p
    lib.fp4idx_version.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().fp4idx_status_string(int(code)).decode()


def version() -> int:
    return int(load().fp4idx_version())


def _check(rc: int, what: str):
    if rc != FP4IDX_OK:
        raise Fp4idxError(f"{what}: {status_string(rc)} (status {rc})")


def _run(name: str, args) -> None:
    _check(getattr(load(), name)(*args), name)


class Prepared:
    """One library call with its arguments marshalled once (device pointers,
    sizes, stream): calling it issues the same call again with a single ctypes
    call.  For loops that run the same step over the same buffers (a serving
    loop's decode step, a benchmark).  It holds references to the tensors it
    was prepared from; they must keep their storage (no resize_ / set_)."""

    __slots__ = ("_fn", "_args", "_name", "_keep")

    def __init__(self, name: str, args, keep=()):
        self._name = name
        self._fn = getattr(load(), name)
        self._args = tuple(args)
        self._keep = tuple(keep)

    def __call__(self) -> None:
        rc = self._fn(*self._args)
        if rc != FP4IDX_OK:
            _check(rc, self._name)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t: torch.Tensor, dtypes, name: str):
    if not t.is_cuda:
        raise Fp4idxError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise Fp4idxError(f"{name}: dtype {t.dtype} not in {dtypes}")
    return ctypes.c_void_p(t.data_ptr())


_BF16 = (torch.bfloat16, torch.int16, torch.uint16) if hasattr(torch, "uint16") else (torch.bfloat16, torch.int16)
_I32 = (torch.int32,)
_U8 = (torch.uint8,)
_F32 = (torch.float32,)


def _need(ok: bool, what: str, msg: str) -> None:
    if not ok:
        raise Fp4idxError(f"{what}: {msg}")


def _shape(t: torch.Tensor, shape, what: str, name: str) -> None:
    """t must have exactly this shape (a buffer the kernels index by these sizes)."""
    _need(tuple(t.shape) == tuple(int(x) for x in shape), what,
          f"{name} has shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")


def _pitch(t: torch.Tensor) -> int:
    """Elements between consecutive rows (dim 0).  With a single row any
    stride is valid for dim 0 (numpy and torch may report 0 for an inserted
    axis), so the row's own length is passed instead."""
    if t.shape[0] == 1:
        n = 1
        for d in t.shape[1:]:
            n *= int(d)
        return n
    return int(t.stride(0))


def _rowstride(t: torch.Tensor, name: str) -> int:
    if t.dim() < 2 or t.stride(-1) != 1:
        raise Fp4idxError(f"{name} must be 2-D (or more) with unit last stride")
    return _pitch(t)


def _write_k_args(k, pos, slot, norm_w, eps, cos_sin, payload, scale):
    if not (pos.is_contiguous() and slot.is_contiguous() and payload.is_contiguous() and scale.is_contiguous()
            and cos_sin.is_contiguous() and norm_w.is_contiguous()):
        raise Fp4idxError("write_k: pos, slot, norm_w, cos_sin and the pools must be contiguous")
    n = int(k.shape[0])
    _need(k.dim() == 2 and (n == 0 or k.shape[1] >= HEAD_DIM), "write_k", "k must be [N, >=128]")
    if pos.numel() != n or slot.numel() != n:
        raise Fp4idxError("write_k: pos/slot length must equal the number of K rows")
    _need(norm_w.numel() == HEAD_DIM, "write_k", "norm_w must hold 128 values")
    num_pages = payload.numel() // PAYLOAD_PAGE_BYTES
    if payload.numel() != num_pages * PAYLOAD_PAGE_BYTES or scale.numel() != num_pages * SCALE_PAGE_BYTES:
        raise Fp4idxError("write_k: pool sizes must be num_pages*4096 and num_pages*256 bytes")
    if cos_sin.dim() != 2 or cos_sin.shape[1] != ROPE_DIM:
        raise Fp4idxError("write_k: cos_sin must be [max_pos, 64]")
    return [_ptr(k, _BF16, "k"), n, _rowstride(k, "k") if n else HEAD_DIM, _ptr(pos, _I32, "pos"),
            _ptr(slot, _I32, "slot"), _ptr(norm_w, _BF16, "norm_w"), ctypes.c_float(eps),
            _ptr(cos_sin, _BF16, "cos_sin"), int(cos_sin.shape[0]), _ptr(payload, _U8, "payload"),
            _ptr(scale, _U8, "scale"), num_pages]


def _write_k_fp8_args(k, pos, slot, norm_w, eps, cos_sin, pool):
    if not (pos.is_contiguous() and slot.is_contiguous() and pool.is_contiguous() and cos_sin.is_contiguous()
            and norm_w.is_contiguous()):
        raise Fp4idxError("write_k_fp8: pos, slot, norm_w, cos_sin and the pool must be contiguous")
    n = int(k.shape[0])
    _need(k.dim() == 2 and (n == 0 or k.shape[1] >= HEAD_DIM), "write_k_fp8", "k must be [N, >=128]")
    if pos.numel() != n or slot.numel() != n:
        raise Fp4idxError("write_k_fp8: pos/slot length must equal the number of K rows")
    _need(norm_w.numel() == HEAD_DIM, "write_k_fp8", "norm_w must hold 128 values")
    num_pages = pool.numel() // FP8_PAGE_BYTES
    if pool.numel() != num_pages * FP8_PAGE_BYTES:
        raise Fp4idxError("write_k_fp8: the pool must be num_pages*8448 bytes")
    if cos_sin.dim() != 2 or cos_sin.shape[1] != ROPE_DIM:
        raise Fp4idxError("write_k_fp8: cos_sin must be [max_pos, 64]")
    return [_ptr(k, _BF16, "k"), n, _rowstride(k, "k") if n else HEAD_DIM, _ptr(pos, _I32, "pos"),
            _ptr(slot, _I32, "slot"), _ptr(norm_w, _BF16, "norm_w"), ctypes.c_float(eps),
            _ptr(cos_sin, _BF16, "cos_sin"), int(cos_sin.shape[0]), _ptr(pool, _U8, "pool"), num_pages]


def fp4idx_write_k(k: torch.Tensor, pos: torch.Tensor, slot: torch.Tensor, norm_w: torch.Tensor, eps: float,
                   cos_sin: torch.Tensor, payload: torch.Tensor, scale: torch.Tensor, stream=None) -> None:
    """Encode K rows [N, >=128] bf16 and scatter them into the split pool."""
    _run("fp4idx_write_k", _write_k_args(k, pos, slot, norm_w, eps, cos_sin, payload, scale) + [_stream(stream)])


def prepare_write_k(k, pos, slot, norm_w, eps, cos_sin, payload, scale, stream=None) -> "Prepared":
    """fp4idx_write_k with its arguments marshalled once (see Prepared)."""
    return Prepared("fp4idx_write_k", _write_k_args(k, pos, slot, norm_w, eps, cos_sin, payload, scale)
                    + [_stream(stream)], keep=(k, pos, slot, norm_w, cos_sin, payload, scale))


def _pack_q_args(q, pos, cos_sin, w_in, w_scale, q_out, q_scale, w_out, with_table=True, fp8=False):
    what = "pack_q_fp8" if fp8 else "pack_q"
    T, H = int(q.shape[0]), int(q.shape[1])
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or (T and (q.stride(2) != 1 or q.stride(1) != HEAD_DIM)):
        raise Fp4idxError(f"{what}: q must be [T, H, 128] with heads packed inside a row")
    dev = q.device
    code_shape = (T, H, HEAD_DIM) if fp8 else (T, H, 64)
    scale_shape = (T, H) if fp8 else (T, H, 4)
    _need(pos.numel() == T, what, f"pos must hold one position per row ({T})")
    _shape(w_in, (T, H), what, "w_in")
    if with_table:
        _need(cos_sin.dim() == 2 and cos_sin.shape[1] == ROPE_DIM, what, "cos_sin must be [max_pos, 64]")
    for t, shp, name in ((q_out, code_shape, "q codes"), (q_scale, scale_shape, "q_scale"), (w_out, (T, H), "w_out")):
        if t is not None:
            _shape(t, shp, what, name)
    q_out = q_out if q_out is not None else torch.empty(code_shape, dtype=torch.uint8, device=dev)
    q_scale = q_scale if q_scale is not None else torch.empty(
        scale_shape, dtype=torch.float32 if fp8 else torch.uint8, device=dev)
    w_out = w_out if w_out is not None else torch.empty((T, H), dtype=torch.float32, device=dev)
    for t, name in ((pos, "pos"), (w_in, "w_in"), (q_out, "q codes"), (q_scale, "q_scale"), (w_out, "w_out"),
                    (cos_sin, "cos_sin")):
        if not t.is_contiguous():
            raise Fp4idxError(f"{what}: {name} must be contiguous")
    head = [_ptr(q, _BF16, "q"), T, H, _pitch(q) if T else H * HEAD_DIM, _ptr(pos, _I32, "pos")]
    table = [_ptr(cos_sin, _BF16, "cos_sin"), int(cos_sin.shape[0])] if with_table else []
    tail = [_ptr(w_in, _F32, "w_in"), ctypes.c_float(w_scale), _ptr(q_out, _U8, "q codes"),
            _ptr(q_scale, _F32 if fp8 else _U8, "q_scale"), _ptr(w_out, _F32, "w_out")]
    return head + table + tail, (q_out, q_scale, w_out)


def fp4idx_pack_q(q: torch.Tensor, pos: torch.Tensor, cos_sin: torch.Tensor, w_in: torch.Tensor,
                  w_scale: float = 1.0, q_fp4: torch.Tensor = None, q_scale: torch.Tensor = None,
                  w_out: torch.Tensor = None, stream=None):
    """q: [T, H, 128] bf16 (rows may be strided) -> (q_fp4 [T,H,64] u8, q_scale [T,H,4] u8, w [T,H] f32)."""
    args, outs = _pack_q_args(q, pos, cos_sin, w_in, w_scale, q_fp4, q_scale, w_out)
    _run("fp4idx_pack_q", args + [_stream(stream)])
    return outs


def prepare_pack_q(q, pos, cos_sin, w_in, w_scale=1.0, q_fp4=None, q_scale=None, w_out=None, stream=None):
    """fp4idx_pack_q with its arguments marshalled once: (Prepared, outputs)."""
    args, outs = _pack_q_args(q, pos, cos_sin, w_in, w_scale, q_fp4, q_scale, w_out)
    return Prepared("fp4idx_pack_q", args + [_stream(stream)], keep=(q, pos, cos_sin, w_in) + outs), outs


def _write_k_pack_q_args(k, pos_k, slot, norm_w, eps, cos_sin, payload, scale, q, pos_q, w_in, w_scale, q_fp4,
                         q_scale, w_out, stream):
    kargs = _write_k_args(k, pos_k, slot, norm_w, eps, cos_sin, payload, scale)
    qargs, outs = _pack_q_args(q, pos_q, cos_sin, w_in, w_scale, q_fp4, q_scale, w_out, with_table=False)
    return kargs + qargs + [_stream(stream)], outs


def fp4idx_write_k_pack_q(k: torch.Tensor, pos_k: torch.Tensor, slot: torch.Tensor, norm_w: torch.Tensor,
                          eps: float, cos_sin: torch.Tensor, payload: torch.Tensor, scale: torch.Tensor,
                          q: torch.Tensor, pos_q: torch.Tensor, w_in: torch.Tensor, w_scale: float = 1.0,
                          q_fp4: torch.Tensor = None, q_scale: torch.Tensor = None, w_out: torch.Tensor = None,
                          stream=None):
    """write_k and pack_q in one launch; returns pack_q's (q_fp4, q_scale, w_out)."""
    args, outs = _write_k_pack_q_args(k, pos_k, slot, norm_w, eps, cos_sin, payload, scale, q, pos_q, w_in, w_scale,
                                      q_fp4, q_scale, w_out, stream)
    _run("fp4idx_write_k_pack_q", args)
    return outs


def prepare_write_k_pack_q(k, pos_k, slot, norm_w, eps, cos_sin, payload, scale, q, pos_q, w_in, w_scale=1.0,
                           q_fp4=None, q_scale=None, w_out=None, stream=None):
    """fp4idx_write_k_pack_q with its arguments marshalled once: (Prepared, outputs)."""
    args, outs = _write_k_pack_q_args(k, pos_k, slot, norm_w, eps, cos_sin, payload, scale, q, pos_q, w_in, w_scale,
                                      q_fp4, q_scale, w_out, stream)
    keep = (k, pos_k, slot, norm_w, cos_sin, payload, scale, q, pos_q, w_in) + outs
    return Prepared("fp4idx_write_k_pack_q", args, keep=keep), outs


def _check_logits_shapes(what, q, q_scale, w, indptr, row_ctx, block_table, max_ctx, out, code_bytes, scale_tail):
    """Sizes the logits kernels index by: Q codes [T, H, code_bytes], Q scales
    [T, H, *scale_tail], w [T, H], indptr [n_reqs + 1], row_ctx [T], a block
    table of at least n_reqs rows and ceil(max_ctx / 64) columns, and (when
    given) an output of at least T rows and max_ctx columns."""
    _need(q.dim() == 3 and q.shape[2] == code_bytes, what, f"Q codes must be [T, H, {code_bytes}]")
    T, H = int(q.shape[0]), int(q.shape[1])
    _shape(q_scale, (T, H) + tuple(scale_tail), what, "q_scale")
    _shape(w, (T, H), what, "w")
    _need(indptr.dim() == 1 and indptr.numel() >= 1, what, "req_row_indptr must be [n_reqs + 1]")
    n_reqs = int(indptr.numel()) - 1
    _need(row_ctx.numel() == T, what, f"row_ctx must hold one context length per row ({T})")
    _need(block_table.dim() == 2 and block_table.shape[0] >= n_reqs, what,
          f"block_table must be [n_reqs, stride] with at least {n_reqs} rows")
    _need(int(max_ctx) >= 0 and block_table.shape[1] * PAGE_TOKENS >= int(max_ctx), what,
          f"block_table has {block_table.shape[1]} columns, max_ctx {max_ctx} needs {(int(max_ctx) + 63) // 64}")
    if out is not None:
        _need(out.dim() == 2 and out.shape[0] >= T and out.shape[1] >= int(max_ctx), what,
              f"the output must be [>= {T}, >= {max_ctx}], got {tuple(out.shape)}")


def _split_pool_pages(what, payload, scale) -> int:
    num_pages = payload.numel() // PAYLOAD_PAGE_BYTES
    _need(payload.numel() == num_pages * PAYLOAD_PAGE_BYTES and scale.numel() == num_pages * SCALE_PAGE_BYTES,
          what, "pool sizes must be num_pages*4096 and num_pages*256 bytes")
    return num_pages


def _mqa_logits_args(q_fp4, q_scale, w, req_row_indptr, row_ctx, block_table, payload, scale, max_rows_per_req,
                     max_ctx, logits, stream):
    """Arguments of fp4idx_mqa_logits_bounded (host bounds max_rows_per_req, max_ctx)."""
    _check_logits_shapes("mqa_logits", q_fp4, q_scale, w, req_row_indptr, row_ctx, block_table, max_ctx, logits,
                         64, (4,))
    T, H = int(q_fp4.shape[0]), int(q_fp4.shape[1])
    n_reqs = int(req_row_indptr.numel()) - 1
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise Fp4idxError("mqa_logits: block_table must be [n_reqs, stride] with unit inner stride")
    if logits is None:
        logits = torch.empty((T, max(1, int(max_ctx))), dtype=torch.float32, device=q_fp4.device)
    if logits.stride(-1) != 1:
        raise Fp4idxError("mqa_logits: logits must have unit inner stride")
    for t, name in ((q_fp4, "q_fp4"), (q_scale, "q_scale"), (w, "w"), (req_row_indptr, "indptr"),
                    (row_ctx, "row_ctx"), (payload, "payload"), (scale, "scale")):
        if not t.is_contiguous():
            raise Fp4idxError(f"mqa_logits: {name} must be contiguous")
    num_pages = _split_pool_pages("mqa_logits", payload, scale)
    args = [_ptr(q_fp4, _U8, "q_fp4"), _ptr(q_scale, _U8, "q_scale"), _ptr(w, _F32, "w"), T, H,
            _ptr(req_row_indptr, _I32, "req_row_indptr"), n_reqs, _ptr(row_ctx, _I32, "row_ctx"),
            _ptr(block_table, _I32, "block_table"), _pitch(block_table), _ptr(payload, _U8, "payload"),
            _ptr(scale, _U8, "scale"), num_pages, _ptr(logits, _F32, "logits"), _pitch(logits),
            int(max_rows_per_req), int(max_ctx), _stream(stream)]
    return args, logits


def fp4idx_mqa_logits_workspace_bytes(n_rows: int, n_reqs: int, max_ctx: int) -> int:
    """Workspace bytes of fp4idx_mqa_logits / fp4idx_mqa_logits_plan for the batch sizes."""
    return int(load().fp4idx_mqa_logits_workspace_bytes(int(n_rows), int(n_reqs), int(max_ctx)))


def new_workspace(n_rows: int, n_reqs: int, max_ctx: int, device=None) -> torch.Tensor:
    """A device workspace (uint8, 16-byte aligned) sized for the batch."""
    n = max(16, fp4idx_mqa_logits_workspace_bytes(n_rows, n_reqs, max_ctx))
    return torch.empty(n, dtype=torch.uint8, device=device if device is not None else "cuda")


def _workspace_arg(ws: torch.Tensor):
    _need(ws.is_contiguous() and ws.dtype == torch.uint8, "mqa_logits", "workspace must be a contiguous uint8 tensor")
    return [_ptr(ws, _U8, "workspace"), int(ws.numel())]


_NO_WORKSPACE = object()  # _planned_args for the call that takes none


def _planned_args(q_fp4, q_scale, w, req_row_indptr, row_ctx, block_table, payload, scale, logits, workspace,
                  max_ctx, stream, what="mqa_logits"):
    """Arguments of fp4idx_mqa_logits / fp4idx_mqa_logits_run.  Without
    logits, an output of max_ctx columns is allocated; without a workspace,
    one sized for contexts up to the output's width."""
    if logits is None:
        _need(max_ctx is not None, what, "give the logits buffer or max_ctx")
        logits = torch.empty((int(q_fp4.shape[0]), max(1, int(max_ctx))), dtype=torch.float32, device=q_fp4.device)
    width = int(logits.shape[1]) if logits.dim() == 2 else 0
    _check_logits_shapes(what, q_fp4, q_scale, w, req_row_indptr, row_ctx, block_table, 0, logits, 64, (4,))
    T, H = int(q_fp4.shape[0]), int(q_fp4.shape[1])
    n_reqs = int(req_row_indptr.numel()) - 1
    _need(block_table.stride(1) == 1, what, "block_table must have unit inner stride")
    _need(logits.stride(-1) == 1, what, "logits must have unit inner stride")
    for t, name in ((q_fp4, "q_fp4"), (q_scale, "q_scale"), (w, "w"), (req_row_indptr, "indptr"),
                    (row_ctx, "row_ctx"), (payload, "payload"), (scale, "scale")):
        _need(t.is_contiguous(), what, f"{name} must be contiguous")
    num_pages = _split_pool_pages(what, payload, scale)
    if workspace is _NO_WORKSPACE:
        ws_args = [None, 0]
    else:
        if workspace is None:
            bound = min(width, int(block_table.shape[1]) * PAGE_TOKENS)
            workspace = new_workspace(T, n_reqs, bound, q_fp4.device)
        _need(workspace.is_contiguous() and workspace.dtype == torch.uint8, what,
              "workspace must be a contiguous uint8 tensor")
        ws_args = _workspace_arg(workspace)
    args = [_ptr(q_fp4, _U8, "q_fp4"), _ptr(q_scale, _U8, "q_scale"), _ptr(w, _F32, "w"), T, H,
            _ptr(req_row_indptr, _I32, "req_row_indptr"), n_reqs, _ptr(row_ctx, _I32, "row_ctx"),
            _ptr(block_table, _I32, "block_table"), _pitch(block_table), _ptr(payload, _U8, "payload"),
            _ptr(scale, _U8, "scale"), num_pages, _ptr(logits, _F32, "logits"), _pitch(logits)]
    return args + ws_args + [_stream(stream)], logits, workspace


def fp4idx_mqa_logits(q_fp4: torch.Tensor, q_scale: torch.Tensor, w: torch.Tensor, req_row_indptr: torch.Tensor,
                      row_ctx: torch.Tensor, block_table: torch.Tensor, payload: torch.Tensor, scale: torch.Tensor,
                      logits: torch.Tensor = None, workspace: torch.Tensor = None, max_ctx: int = None,
                      stream=None) -> torch.Tensor:
    """Paged FP4 logits [T, stride] fp32 (only [0, ctx[t]) of each row is
    written): the device schedule (plan) and the scheduled kernel (run) in
    two launches.  workspace: a uint8 device tensor of
    fp4idx_mqa_logits_workspace_bytes() bytes (allocated when omitted)."""
    args, logits, _ = _planned_args(q_fp4, q_scale, w, req_row_indptr, row_ctx, block_table, payload, scale, logits,
                                    workspace, max_ctx, stream)
    _run("fp4idx_mqa_logits", args)
    return logits


def fp4idx_mqa_logits_noalloc(q_fp4: torch.Tensor, q_scale: torch.Tensor, w: torch.Tensor,
                              req_row_indptr: torch.Tensor, row_ctx: torch.Tensor, block_table: torch.Tensor,
                              payload: torch.Tensor, scale: torch.Tensor, logits: torch.Tensor,
                              stream=None) -> torch.Tensor:
    """fp4idx_mqa_logits with the schedule in the library's per-device
    scratch array (no workspace, no device allocation: the caller passes the
    logits buffer).  Calls that overlap on one device race."""
    _need(logits is not None, "mqa_logits_noalloc", "give the logits buffer (this call allocates nothing)")
    args, logits, _ = _planned_args(q_fp4, q_scale, w, req_row_indptr, row_ctx, block_table, payload, scale, logits,
                                    _NO_WORKSPACE, None, stream, what="mqa_logits_noalloc")
    _run("fp4idx_mqa_logits_noalloc", args[:-3] + args[-1:])
    return logits


def prepare_mqa_logits(q_fp4, q_scale, w, req_row_indptr, row_ctx, block_table, payload, scale, logits=None,
                       workspace=None, max_ctx=None, stream=None):
    """fp4idx_mqa_logits with its arguments marshalled once: (Prepared, logits)."""
    args, logits, workspace = _planned_args(q_fp4, q_scale, w, req_row_indptr, row_ctx, block_table, payload, scale,
                                            logits, workspace, max_ctx, stream)
    keep = (q_fp4, q_scale, w, req_row_indptr, row_ctx, block_table, payload, scale, logits, workspace)
    return Prepared("fp4idx_mqa_logits", args, keep=keep), logits


class LogitsPlan:
    """The work schedule of one batch, kept in a device workspace for reuse.

    The schedule depends only on the batch: the rows of each request
    (req_row_indptr), their context lengths (row_ctx) and the head count.
    build() issues fp4idx_mqa_logits_plan; run() issues fp4idx_mqa_logits_run
    for any Q, weights, pool and block table of that batch, so one plan serves
    every compressed-attention layer of a step and every replay of a captured
    step (re-build when the batch changes; the tensors are read at build and
    at run time, so in-place updates of row_ctx need a new build).  max_ctx
    bounds the contexts the schedule covers (the logits width)."""

    def __init__(self, n_heads: int, req_row_indptr: torch.Tensor, row_ctx: torch.Tensor, max_ctx: int,
                 workspace: torch.Tensor = None, stream=None):
        _need(req_row_indptr.dim() == 1 and req_row_indptr.numel() >= 1 and req_row_indptr.is_contiguous(),
              "LogitsPlan", "req_row_indptr must be a contiguous [n_reqs + 1] tensor")
        _need(row_ctx.dim() == 1 and row_ctx.is_contiguous(), "LogitsPlan", "row_ctx must be a contiguous [T] tensor")
        self.n_heads = int(n_heads)
        self.indptr, self.row_ctx, self.max_ctx = req_row_indptr, row_ctx, int(max_ctx)
        self.n_rows, self.n_reqs = int(row_ctx.numel()), int(req_row_indptr.numel()) - 1
        self.workspace = workspace if workspace is not None else new_workspace(
            self.n_rows, self.n_reqs, self.max_ctx, row_ctx.device)
        self._plan = Prepared("fp4idx_mqa_logits_plan", [
            self.n_rows, self.n_heads, _ptr(req_row_indptr, _I32, "req_row_indptr"), self.n_reqs,
            _ptr(row_ctx, _I32, "row_ctx"), self.max_ctx] + _workspace_arg(self.workspace) + [_stream(stream)],
            keep=(req_row_indptr, row_ctx, self.workspace))

    def build(self) -> "LogitsPlan":
        self._plan()
        return self

    def prepare_build(self) -> Prepared:
        return self._plan

    def _run_args(self, q_fp4, q_scale, w, block_table, payload, scale, logits, stream):
        _need(int(q_fp4.shape[0]) == self.n_rows and int(q_fp4.shape[1]) == self.n_heads, "LogitsPlan.run",
              f"Q must be [{self.n_rows}, {self.n_heads}, 64] for this plan")
        if logits is None:
            logits = torch.empty((self.n_rows, max(1, self.max_ctx)), dtype=torch.float32, device=q_fp4.device)
        args, logits, _ = _planned_args(q_fp4, q_scale, w, self.indptr, self.row_ctx, block_table, payload, scale,
                                        logits, self.workspace, None, stream, what="mqa_logits_run")
        return args, logits

    def run(self, q_fp4, q_scale, w, block_table, payload, scale, logits=None, stream=None) -> torch.Tensor:
        args, logits = self._run_args(q_fp4, q_scale, w, block_table, payload, scale, logits, stream)
        _run("fp4idx_mqa_logits_run", args)
        return logits

    def prepare_run(self, q_fp4, q_scale, w, block_table, payload, scale, logits=None, stream=None):
        """fp4idx_mqa_logits_run with its arguments marshalled once: (Prepared, logits)."""
        args, logits = self._run_args(q_fp4, q_scale, w, block_table, payload, scale, logits, stream)
        keep = (q_fp4, q_scale, w, self.indptr, self.row_ctx, block_table, payload, scale, logits, self.workspace)
        return Prepared("fp4idx_mqa_logits_run", args, keep=keep), logits


def fp4idx_mqa_logits_bounded(q_fp4: torch.Tensor, q_scale: torch.Tensor, w: torch.Tensor,
                              req_row_indptr: torch.Tensor, row_ctx: torch.Tensor, block_table: torch.Tensor,
                              payload: torch.Tensor, scale: torch.Tensor, max_rows_per_req: int, max_ctx: int,
                              logits: torch.Tensor = None, stream=None) -> torch.Tensor:
    """The same logits without a workspace, the grid sized from host bounds."""
    args, logits = _mqa_logits_args(q_fp4, q_scale, w, req_row_indptr, row_ctx, block_table, payload, scale,
                                    max_rows_per_req, max_ctx, logits, stream)
    _run("fp4idx_mqa_logits_bounded", args)
    return logits


def prepare_mqa_logits_bounded(q_fp4, q_scale, w, req_row_indptr, row_ctx, block_table, payload, scale,
                               max_rows_per_req, max_ctx, logits=None, stream=None):
    """fp4idx_mqa_logits_bounded with its arguments marshalled once: (Prepared, logits)."""
    args, logits = _mqa_logits_args(q_fp4, q_scale, w, req_row_indptr, row_ctx, block_table, payload, scale,
                                    max_rows_per_req, max_ctx, logits, stream)
    keep = (q_fp4, q_scale, w, req_row_indptr, row_ctx, block_table, payload, scale, logits)
    return Prepared("fp4idx_mqa_logits_bounded", args, keep=keep), logits


def _mqa_logits_topk_args(q_fp4, q_scale, w, req_row_indptr, row_ctx, block_table, payload, scale, k,
                          max_rows_per_req, max_ctx, out_idx, stream):
    _check_logits_shapes("mqa_logits_topk", q_fp4, q_scale, w, req_row_indptr, row_ctx, block_table, max_ctx, None,
                         64, (4,))
    T, H = int(q_fp4.shape[0]), int(q_fp4.shape[1])
    n_reqs = int(req_row_indptr.numel()) - 1
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise Fp4idxError("mqa_logits_topk: block_table must be [n_reqs, stride] with unit inner stride")
    if out_idx is not None:
        _shape(out_idx, (T, int(k)), "mqa_logits_topk", "out_idx")
    if out_idx is None:
        out_idx = torch.empty((T, int(k)), dtype=torch.int32, device=q_fp4.device)
    for t, name in ((q_fp4, "q_fp4"), (q_scale, "q_scale"), (w, "w"), (req_row_indptr, "indptr"),
                    (row_ctx, "row_ctx"), (payload, "payload"), (scale, "scale"), (out_idx, "out_idx")):
        if not t.is_contiguous():
            raise Fp4idxError(f"mqa_logits_topk: {name} must be contiguous")
    num_pages = _split_pool_pages("mqa_logits_topk", payload, scale)
    args = [_ptr(q_fp4, _U8, "q_fp4"), _ptr(q_scale, _U8, "q_scale"), _ptr(w, _F32, "w"), T, H,
            _ptr(req_row_indptr, _I32, "req_row_indptr"), n_reqs, _ptr(row_ctx, _I32, "row_ctx"),
            _ptr(block_table, _I32, "block_table"), _pitch(block_table), _ptr(payload, _U8, "payload"),
            _ptr(scale, _U8, "scale"), num_pages, int(k), _ptr(out_idx, _I32, "out_idx"), int(max_rows_per_req),
            int(max_ctx), _stream(stream)]
    return args, out_idx


def fp4idx_mqa_logits_topk(q_fp4: torch.Tensor, q_scale: torch.Tensor, w: torch.Tensor,
                           req_row_indptr: torch.Tensor, row_ctx: torch.Tensor, block_table: torch.Tensor,
                           payload: torch.Tensor, scale: torch.Tensor, k: int, max_rows_per_req: int, max_ctx: int,
                           out_idx: torch.Tensor = None, stream=None) -> torch.Tensor:
    """[T, k] int32: the top-k positions of every row (as mqa_logits then topk), logits never written."""
    args, out_idx = _mqa_logits_topk_args(q_fp4, q_scale, w, req_row_indptr, row_ctx, block_table, payload, scale,
                                          k, max_rows_per_req, max_ctx, out_idx, stream)
    _run("fp4idx_mqa_logits_topk", args)
    return out_idx


def prepare_mqa_logits_topk(q_fp4, q_scale, w, req_row_indptr, row_ctx, block_table, payload, scale, k,
                            max_rows_per_req, max_ctx, out_idx=None, stream=None):
    """fp4idx_mqa_logits_topk with its arguments marshalled once: (Prepared, out_idx)."""
    args, out_idx = _mqa_logits_topk_args(q_fp4, q_scale, w, req_row_indptr, row_ctx, block_table, payload, scale,
                                          k, max_rows_per_req, max_ctx, out_idx, stream)
    keep = (q_fp4, q_scale, w, req_row_indptr, row_ctx, block_table, payload, scale, out_idx)
    return Prepared("fp4idx_mqa_logits_topk", args, keep=keep), out_idx


def _topk_args(logits, row_ctx, k, max_ctx, out_idx, stream):
    """Arguments of fp4idx_topk (max_ctx None) or fp4idx_topk_bounded: (name, args, out_idx)."""
    _need(logits.dim() == 2, "topk", "logits must be [T, stride]")
    T = int(logits.shape[0])
    if logits.stride(-1) != 1:
        raise Fp4idxError("topk: logits must have unit inner stride")
    _need(row_ctx.numel() == T, "topk", f"row_ctx must hold one context length per row ({T})")
    if max_ctx is not None:
        _need(0 <= int(max_ctx) <= logits.shape[1], "topk",
              f"max_ctx {max_ctx} exceeds the logits rows ({logits.shape[1]})")
    if out_idx is not None:
        _shape(out_idx, (T, int(k)), "topk", "out_idx")
    if out_idx is None:
        out_idx = torch.empty((T, int(k)), dtype=torch.int32, device=logits.device)
    if not out_idx.is_contiguous() or not row_ctx.is_contiguous():
        raise Fp4idxError("topk: out_idx and row_ctx must be contiguous")
    args = [_ptr(logits, _F32, "logits"), T, _pitch(logits), _ptr(row_ctx, _I32, "row_ctx"), int(k),
            _ptr(out_idx, _I32, "out_idx")]
    if max_ctx is None:
        return "fp4idx_topk", args + [_stream(stream)], out_idx
    return "fp4idx_topk_bounded", args + [int(max_ctx), _stream(stream)], out_idx


def fp4idx_topk(logits: torch.Tensor, row_ctx: torch.Tensor, k: int, max_ctx: int = None,
                out_idx: torch.Tensor = None, stream=None) -> torch.Tensor:
    """[T, k] int32: top-k positions per row, ascending, then -1.  With
    max_ctx (a host bound on the contexts) fp4idx_topk_bounded runs."""
    name, args, out_idx = _topk_args(logits, row_ctx, k, max_ctx, out_idx, stream)
    _run(name, args)
    return out_idx


def fp4idx_topk_bounded(logits: torch.Tensor, row_ctx: torch.Tensor, k: int, max_ctx: int,
                        out_idx: torch.Tensor = None, stream=None) -> torch.Tensor:
    """fp4idx_topk with the host bound max_ctx on the contexts."""
    return fp4idx_topk(logits, row_ctx, k, max_ctx, out_idx, stream)


def prepare_topk(logits, row_ctx, k, max_ctx=None, out_idx=None, stream=None):
    """fp4idx_topk (or _bounded) with its arguments marshalled once: (Prepared, out_idx)."""
    name, args, out_idx = _topk_args(logits, row_ctx, k, max_ctx, out_idx, stream)
    return Prepared(name, args, keep=(logits, row_ctx, out_idx)), out_idx


def fp4idx_read_k(payload: torch.Tensor, scale: torch.Tensor, slot: torch.Tensor, out: torch.Tensor = None,
                  stream=None) -> torch.Tensor:
    """Pool tokens at `slot` back to fp32 [N, 128] (a slot outside the pool gives a zero row)."""
    n = int(slot.numel())
    if not (payload.is_contiguous() and scale.is_contiguous() and slot.is_contiguous()):
        raise Fp4idxError("read_k: payload, scale and slot must be contiguous")
    num_pages = payload.numel() // PAYLOAD_PAGE_BYTES
    if payload.numel() != num_pages * PAYLOAD_PAGE_BYTES or scale.numel() != num_pages * SCALE_PAGE_BYTES:
        raise Fp4idxError("read_k: pool sizes must be num_pages*4096 and num_pages*256 bytes")
    if out is not None:
        _need(out.dim() == 2 and out.shape[0] == n and out.shape[1] >= HEAD_DIM, "read_k",
              f"out must be [{n}, >=128], got {tuple(out.shape)}")
    if out is None:
        out = torch.empty((n, HEAD_DIM), dtype=torch.float32, device=payload.device)
    _run("fp4idx_read_k", [_ptr(payload, _U8, "payload"), _ptr(scale, _U8, "scale"), num_pages,
                           _ptr(slot, _I32, "slot"), n, _ptr(out, _F32, "out"),
                           _rowstride(out, "out") if n else HEAD_DIM, _stream(stream)])
    return out


PEAK_MFMA_WAVES = 4096


def fp4idx_peak_mfma_fp4(iterations: int, sink: torch.Tensor, stream=None) -> int:
    """Launch the FP4 MFMA peak microbenchmark; returns the flop it performs."""
    _run("fp4idx_peak_mfma_fp4", [int(iterations), _ptr(sink, _F32, "sink"), _stream(stream)])
    return PEAK_MFMA_WAVES * 4 * int(iterations) * 65536


def fp4idx_peak_valu_fp32(iterations: int, sink: torch.Tensor, stream=None) -> int:
    """Launch the fp32 VALU FMA peak microbenchmark; returns the FMA lane-ops it performs."""
    _run("fp4idx_peak_valu_fp32", [int(iterations), _ptr(sink, _F32, "sink"), _stream(stream)])
    return PEAK_MFMA_WAVES * 64 * 16 * int(iterations)


def fp4idx_peak_mfma_valu(mode: int, iterations: int, sink: torch.Tensor, stream=None) -> None:
    """Launch the MFMA / VALU co-execution microbenchmark (mode 0: MFMAs, 1: FMAs, 2: both)."""
    _run("fp4idx_peak_mfma_valu", [int(mode), int(iterations), _ptr(sink, _F32, "sink"), _stream(stream)])


def fp4idx_peak_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> int:
    """Launch the streaming-read microbenchmark over buf (uint8, contiguous); returns the bytes it reads."""
    if not buf.is_contiguous():
        raise Fp4idxError("peak_read: buf must be contiguous")
    n = buf.numel() // 16 * 16
    _run("fp4idx_peak_read", [_ptr(buf, _U8, "buf"), n, _ptr(sink, (torch.int32,), "sink"), _stream(stream)])
    return n


def _event_handle(ev):
    if ev is None:
        return None
    h = int(getattr(ev, "cuda_event", ev) or 0)
    if h == 0:
        raise Fp4idxError("time_next_call: the event has no HIP event yet (record it once first)")
    return ctypes.c_void_p(h)


def fp4idx_time_next_call(start_event, stop_event) -> None:
    """Arm two timing events (torch.cuda.Event with enable_timing=True, already
    recorded once so that the HIP event exists, or raw hipEvent_t handles) for
    this thread's next library call (each launches one kernel): they receive
    that call's kernel start and end timestamps."""
    _check(load().fp4idx_time_next_call(_event_handle(start_event), _event_handle(stop_event)),
           "fp4idx_time_next_call")


# ---- FP8 cache (132-byte fused tokens) ----------------------------------------

def fp4idx_write_k_fp8(k: torch.Tensor, pos: torch.Tensor, slot: torch.Tensor, norm_w: torch.Tensor, eps: float,
                       cos_sin: torch.Tensor, pool: torch.Tensor, stream=None) -> None:
    """Encode K rows [N, >=128] bf16 into the fused FP8 pool [num_pages * 8448] u8."""
    _run("fp4idx_write_k_fp8", _write_k_fp8_args(k, pos, slot, norm_w, eps, cos_sin, pool) + [_stream(stream)])


def prepare_write_k_fp8(k, pos, slot, norm_w, eps, cos_sin, pool, stream=None) -> "Prepared":
    """fp4idx_write_k_fp8 with its arguments marshalled once (see Prepared)."""
    return Prepared("fp4idx_write_k_fp8", _write_k_fp8_args(k, pos, slot, norm_w, eps, cos_sin, pool)
                    + [_stream(stream)], keep=(k, pos, slot, norm_w, cos_sin, pool))


def fp4idx_pack_q_fp8(q: torch.Tensor, pos: torch.Tensor, cos_sin: torch.Tensor, w_in: torch.Tensor,
                      w_scale: float = 1.0, q_fp8: torch.Tensor = None, q_scale: torch.Tensor = None,
                      w_out: torch.Tensor = None, stream=None):
    """q: [T, H, 128] bf16 -> (q_fp8 [T,H,128] u8, q_scale [T,H] f32, w [T,H] f32)."""
    args, outs = _pack_q_args(q, pos, cos_sin, w_in, w_scale, q_fp8, q_scale, w_out, fp8=True)
    _run("fp4idx_pack_q_fp8", args + [_stream(stream)])
    return outs


def prepare_pack_q_fp8(q, pos, cos_sin, w_in, w_scale=1.0, q_fp8=None, q_scale=None, w_out=None, stream=None):
    """fp4idx_pack_q_fp8 with its arguments marshalled once: (Prepared, outputs)."""
    args, outs = _pack_q_args(q, pos, cos_sin, w_in, w_scale, q_fp8, q_scale, w_out, fp8=True)
    return Prepared("fp4idx_pack_q_fp8", args + [_stream(stream)], keep=(q, pos, cos_sin, w_in) + outs), outs


def _write_k_pack_q_fp8_args(k, pos_k, slot, norm_w, eps, cos_sin, pool, q, pos_q, w_in, w_scale, q_fp8, q_scale,
                             w_out, stream):
    kargs = _write_k_fp8_args(k, pos_k, slot, norm_w, eps, cos_sin, pool)
    qargs, outs = _pack_q_args(q, pos_q, cos_sin, w_in, w_scale, q_fp8, q_scale, w_out, with_table=False, fp8=True)
    return kargs + qargs + [_stream(stream)], outs


def fp4idx_write_k_pack_q_fp8(k, pos_k, slot, norm_w, eps, cos_sin, pool, q, pos_q, w_in, w_scale=1.0, q_fp8=None,
                              q_scale=None, w_out=None, stream=None):
    """write_k_fp8 and pack_q_fp8 in one launch; returns (q_fp8, q_scale, w_out)."""
    args, outs = _write_k_pack_q_fp8_args(k, pos_k, slot, norm_w, eps, cos_sin, pool, q, pos_q, w_in, w_scale,
                                          q_fp8, q_scale, w_out, stream)
    _run("fp4idx_write_k_pack_q_fp8", args)
    return outs


def prepare_write_k_pack_q_fp8(k, pos_k, slot, norm_w, eps, cos_sin, pool, q, pos_q, w_in, w_scale=1.0,
                               q_fp8=None, q_scale=None, w_out=None, stream=None):
    """fp4idx_write_k_pack_q_fp8 with its arguments marshalled once: (Prepared, outputs)."""
    args, outs = _write_k_pack_q_fp8_args(k, pos_k, slot, norm_w, eps, cos_sin, pool, q, pos_q, w_in, w_scale,
                                          q_fp8, q_scale, w_out, stream)
    keep = (k, pos_k, slot, norm_w, cos_sin, pool, q, pos_q, w_in) + outs
    return Prepared("fp4idx_write_k_pack_q_fp8", args, keep=keep), outs


def _mqa_logits_fp8_args(q_fp8, q_scale, w, req_row_indptr, row_ctx, block_table, pool, max_rows_per_req, max_ctx,
                         logits, stream):
    _check_logits_shapes("mqa_logits_fp8", q_fp8, q_scale, w, req_row_indptr, row_ctx, block_table, max_ctx, logits,
                         HEAD_DIM, ())
    T, H = int(q_fp8.shape[0]), int(q_fp8.shape[1])
    n_reqs = int(req_row_indptr.numel()) - 1
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise Fp4idxError("mqa_logits_fp8: block_table must be [n_reqs, stride] with unit inner stride")
    if logits is None:
        logits = torch.empty((T, max(1, int(max_ctx))), dtype=torch.float32, device=q_fp8.device)
    if logits.stride(-1) != 1:
        raise Fp4idxError("mqa_logits_fp8: logits must have unit inner stride")
    for t, name in ((q_fp8, "q_fp8"), (q_scale, "q_scale"), (w, "w"), (req_row_indptr, "indptr"),
                    (row_ctx, "row_ctx"), (pool, "pool")):
        if not t.is_contiguous():
            raise Fp4idxError(f"mqa_logits_fp8: {name} must be contiguous")
    num_pages = pool.numel() // FP8_PAGE_BYTES
    _need(pool.numel() == num_pages * FP8_PAGE_BYTES, "mqa_logits_fp8", "the pool must be num_pages*8448 bytes")
    args = [_ptr(q_fp8, _U8, "q_fp8"), _ptr(q_scale, _F32, "q_scale"), _ptr(w, _F32, "w"), T, H,
            _ptr(req_row_indptr, _I32, "req_row_indptr"), n_reqs, _ptr(row_ctx, _I32, "row_ctx"),
            _ptr(block_table, _I32, "block_table"), _pitch(block_table), _ptr(pool, _U8, "pool"), num_pages,
            _ptr(logits, _F32, "logits"), _pitch(logits), int(max_rows_per_req), int(max_ctx),
            _stream(stream)]
    return args, logits


def fp4idx_mqa_logits_fp8(q_fp8: torch.Tensor, q_scale: torch.Tensor, w: torch.Tensor,
                          req_row_indptr: torch.Tensor, row_ctx: torch.Tensor, block_table: torch.Tensor,
                          pool: torch.Tensor, max_rows_per_req: int, max_ctx: int, logits: torch.Tensor = None,
                          stream=None) -> torch.Tensor:
    """Paged logits over the FP8 pool [T, stride] fp32; only [0, ctx[t]) of each row is written."""
    args, logits = _mqa_logits_fp8_args(q_fp8, q_scale, w, req_row_indptr, row_ctx, block_table, pool,
                                        max_rows_per_req, max_ctx, logits, stream)
    _run("fp4idx_mqa_logits_fp8", args)
    return logits


def prepare_mqa_logits_fp8(q_fp8, q_scale, w, req_row_indptr, row_ctx, block_table, pool, max_rows_per_req,
                           max_ctx, logits=None, stream=None):
    """fp4idx_mqa_logits_fp8 with its arguments marshalled once: (Prepared, logits)."""
    args, logits = _mqa_logits_fp8_args(q_fp8, q_scale, w, req_row_indptr, row_ctx, block_table, pool,
                                        max_rows_per_req, max_ctx, logits, stream)
    keep = (q_fp8, q_scale, w, req_row_indptr, row_ctx, block_table, pool, logits)
    return Prepared("fp4idx_mqa_logits_fp8", args, keep=keep), logits


write_k = fp4idx_write_k
pack_q = fp4idx_pack_q
mqa_logits = fp4idx_mqa_logits
mqa_logits_bounded = fp4idx_mqa_logits_bounded
mqa_logits_noalloc = fp4idx_mqa_logits_noalloc
mqa_logits_workspace_bytes = fp4idx_mqa_logits_workspace_bytes
topk = fp4idx_topk
topk_bounded = fp4idx_topk_bounded
write_k_pack_q = fp4idx_write_k_pack_q
read_k = fp4idx_read_k
time_next_call = fp4idx_time_next_call
write_k_fp8 = fp4idx_write_k_fp8
pack_q_fp8 = fp4idx_pack_q_fp8
write_k_pack_q_fp8 = fp4idx_write_k_pack_q_fp8
mqa_logits_fp8 = fp4idx_mqa_logits_fp8
mqa_logits_topk = fp4idx_mqa_logits_topk
peak_mfma_fp4 = fp4idx_peak_mfma_fp4
peak_valu_fp32 = fp4idx_peak_valu_fp32
peak_mfma_valu = fp4idx_peak_mfma_valu
peak_read = fp4idx_peak_read
