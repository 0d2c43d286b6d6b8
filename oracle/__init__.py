"""CPU oracle for the FP4 lightning-indexer hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
path (the HIP library and its Python binding) never imports it and shares no
code with it.

The arithmetic lives in ``fp4idx_oracle.c`` (plain C, compiled with gcc,
``-ffp-contract=off``, no fast-math); this module compiles it on demand and
wraps it for numpy arrays.  ``brute.py`` holds an exact rational brute force
for tiny inputs, used to pin this oracle.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp4idx_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

D = 128
PAGE = 64


def build(force: bool = False) -> str:
    """Compile the C oracle into ``oracle/liboracle.so`` (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        lib.orc_set_threads.argtypes = [ctypes.c_int]
        lib.orc_get_threads.restype = ctypes.c_int
        lib.orc_rmsnorm128.argtypes = [P, P, f32, P]
        lib.orc_rope64.argtypes = [P, P]
        lib.orc_fwht128.argtypes = [P]
        lib.orc_hadamard_scale.restype = f32
        lib.orc_block_exponent.argtypes = [f32]
        lib.orc_block_exponent.restype = ctypes.c_int
        lib.orc_e2m1_code.argtypes = [f32, ctypes.c_int]
        lib.orc_e2m1_code.restype = ctypes.c_int
        lib.orc_e2m1_codes.argtypes = [P, i64, ctypes.c_int, P]
        lib.orc_quant128.argtypes = [P, P, P]
        lib.orc_dequant128.argtypes = [P, P, P]
        lib.orc_encode_k_token.argtypes = [P, P, f32, P, P, P]
        lib.orc_encode_q_head.argtypes = [P, P, P, P]
        lib.orc_write_k.argtypes = [P, i64, i64, P, P, P, f32, P, i32, P, P, i64]
        lib.orc_pack_q.argtypes = [P, i64, i32, i64, P, P, i32, P, f32, P, P, P]
        lib.orc_logits.argtypes = [P, P, P, i64, i32, P, i32, P, P, i32, P, P, i64, P, i64, P, P, P]
        lib.orc_logits_sampled.argtypes = [P, P, P, i32, P, i32, P, i32, P, P, i64, i64, P, P, P, P, P]
        lib.orc_topk.argtypes = [P, i64, i64, P, i32, P]
        lib.orc_read_k.argtypes = [P, P, i64, P, i64, P]
        lib.orc_fp8_exponent.argtypes = [f32]
        lib.orc_fp8_exponent.restype = ctypes.c_int
        lib.orc_e4m3_value.argtypes = [ctypes.c_int]
        lib.orc_e4m3_value.restype = ctypes.c_double
        lib.orc_e4m3_code.argtypes = [f32, ctypes.c_int]
        lib.orc_e4m3_code.restype = ctypes.c_int
        lib.orc_quant_fp8_128.argtypes = [P, P, P]
        lib.orc_dequant_fp8_128.argtypes = [P, f32, P]
        lib.orc_encode_k_token_fp8.argtypes = [P, P, f32, P, P, P]
        lib.orc_encode_q_head_fp8.argtypes = [P, P, P, P]
        lib.orc_write_k_fp8.argtypes = [P, i64, i64, P, P, P, f32, P, i32, P, i64]
        lib.orc_pack_q_fp8.argtypes = [P, i64, i32, i64, P, P, i32, P, f32, P, P, P]
        lib.orc_logits_fp8.argtypes = [P, P, P, i64, i32, P, i32, P, P, i32, P, i64, P, i64, P, P, P, P]
        lib.orc_logits_fp8_sampled.argtypes = [P, P, P, i32, P, i32, P, i32, P, i64, i64, P, P, P, P, P, P]
        for name in ("orc_write_k", "orc_pack_q", "orc_logits", "orc_logits_sampled", "orc_topk", "orc_read_k",
                     "orc_write_k_fp8", "orc_pack_q_fp8", "orc_logits_fp8", "orc_logits_fp8_sampled"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what}: oracle rejected the arguments (rc={rc})")


def set_threads(n: int) -> None:
    _load().orc_set_threads(int(n))


def get_threads() -> int:
    return int(_load().orc_get_threads())


# ---- step-level entry points (used by the pins) ---------------------------

def rmsnorm128(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    x = _c(x, np.float32); g = _c(g, np.float32)
    y = np.empty(D, np.float32)
    _load().orc_rmsnorm128(_p(x), _p(g), ctypes.c_float(eps), _p(y))
    return y


def rope64(y: np.ndarray, cs: np.ndarray) -> np.ndarray:
    y = _c(y, np.float32).copy(); cs = _c(cs, np.float32)
    _load().orc_rope64(_p(y), _p(cs))
    return y


def fwht128(z: np.ndarray) -> np.ndarray:
    z = _c(z, np.float32).copy()
    _load().orc_fwht128(_p(z))
    return z


def hadamard_scale() -> np.float32:
    return np.float32(_load().orc_hadamard_scale())


def block_exponent(amax: float) -> int:
    return int(_load().orc_block_exponent(ctypes.c_float(amax)))


def e2m1_code(z: float, e: int) -> int:
    return int(_load().orc_e2m1_code(ctypes.c_float(z), int(e)))


def e2m1_codes(z: np.ndarray, e: int) -> np.ndarray:
    z = _c(z, np.float32)
    out = np.empty(z.size, np.uint8)
    _load().orc_e2m1_codes(_p(z), z.size, int(e), _p(out))
    return out.reshape(z.shape)


def quant128(z: np.ndarray):
    z = _c(z, np.float32)
    codes = np.empty(64, np.uint8); sc = np.empty(4, np.uint8)
    _load().orc_quant128(_p(z), _p(codes), _p(sc))
    return codes, sc


def dequant128(codes: np.ndarray, sc: np.ndarray) -> np.ndarray:
    codes = _c(codes, np.uint8); sc = _c(sc, np.uint8)
    out = np.empty(D, np.float64)
    _load().orc_dequant128(_p(codes), _p(sc), _p(out))
    return out


def encode_k_token(k_row, norm_w, eps, cs_row):
    k_row = _c(k_row, np.uint16); norm_w = _c(norm_w, np.uint16); cs_row = _c(cs_row, np.uint16)
    codes = np.empty(64, np.uint8); sc = np.empty(4, np.uint8)
    _load().orc_encode_k_token(_p(k_row), _p(norm_w), ctypes.c_float(eps), _p(cs_row), _p(codes), _p(sc))
    return codes, sc


def encode_q_head(q_row, cs_row):
    q_row = _c(q_row, np.uint16); cs_row = _c(cs_row, np.uint16)
    codes = np.empty(64, np.uint8); sc = np.empty(4, np.uint8)
    _load().orc_encode_q_head(_p(q_row), _p(cs_row), _p(codes), _p(sc))
    return codes, sc


# ---- the four path calls ---------------------------------------------------

def write_k(k, pos, slot, norm_w, eps, cos_sin, payload, scale):
    """Encode K rows and scatter them into the split pools (in place)."""
    k = _c(k, np.uint16); pos = _c(pos, np.int32); slot = _c(slot, np.int32)
    norm_w = _c(norm_w, np.uint16); cos_sin = _c(cos_sin, np.uint16)
    assert payload.dtype == np.uint8 and payload.flags.c_contiguous
    assert scale.dtype == np.uint8 and scale.flags.c_contiguous
    num_pages = payload.size // (PAGE * D // 2)
    assert scale.size == num_pages * PAGE * 4
    n = k.shape[0]
    rc = _load().orc_write_k(_p(k), n, k.shape[1] if n else D, _p(pos), _p(slot), _p(norm_w),
                             ctypes.c_float(eps), _p(cos_sin), cos_sin.shape[0], _p(payload), _p(scale),
                             num_pages)
    _check(rc, "write_k")


def pack_q(q, pos, cos_sin, w_in, w_scale=1.0):
    """q: uint16 [T, H, 128] -> (q_fp4 [T,H,64] u8, q_scale [T,H,4] u8, w_out [T,H] f32)."""
    q = _c(q, np.uint16); pos = _c(pos, np.int32); cos_sin = _c(cos_sin, np.uint16)
    w_in = _c(w_in, np.float32)
    T, H = q.shape[0], q.shape[1]
    q_fp4 = np.empty((T, H, 64), np.uint8); q_scale = np.empty((T, H, 4), np.uint8)
    w_out = np.empty((T, H), np.float32)
    rc = _load().orc_pack_q(_p(q), T, H, H * D, _p(pos), _p(cos_sin), cos_sin.shape[0], _p(w_in),
                            ctypes.c_float(w_scale), _p(q_fp4), _p(q_scale), _p(w_out))
    _check(rc, "pack_q")
    return q_fp4, q_scale, w_out


def logits(q_fp4, q_scale, w, indptr, row_ctx, block_table, payload, scale, logits_stride=None,
           want_f64=False):
    """Full logits [T, stride] (fp32; entries >= ctx stay NaN).  With want_f64
    also returns the fp64 values, T = sum |w| max(d,0) and A = sum |w| sum |q k|."""
    q_fp4 = _c(q_fp4, np.uint8); q_scale = _c(q_scale, np.uint8); w = _c(w, np.float32)
    indptr = _c(indptr, np.int32); row_ctx = _c(row_ctx, np.int32); bt = _c(block_table, np.int32)
    T, H = q_fp4.shape[0], q_fp4.shape[1]
    stride = int(logits_stride if logits_stride is not None else max(1, int(row_ctx.max(initial=0))))
    num_pages = payload.size // (PAGE * D // 2)
    out = np.full((T, stride), np.nan, np.float32)
    f64 = np.full((T, stride), np.nan, np.float64) if want_f64 else None
    tol = np.full((T, stride), np.nan, np.float64) if want_f64 else None
    absr = np.full((T, stride), np.nan, np.float64) if want_f64 else None
    rc = _load().orc_logits(_p(q_fp4), _p(q_scale), _p(w), T, H, _p(indptr), len(indptr) - 1, _p(row_ctx),
                            _p(bt), bt.shape[1] if bt.ndim == 2 else bt.size, _p(payload), _p(scale), num_pages,
                            _p(out), stride, _p(f64) if want_f64 else None, _p(tol) if want_f64 else None,
                            _p(absr) if want_f64 else None)
    _check(rc, "logits")
    return (out, f64, tol, absr) if want_f64 else out


def logits_sampled(q_fp4, q_scale, w, indptr, block_table, payload, scale, rows, toks):
    """fp64 logits at (rows[i], toks[i]) with their T and A tolerance scales."""
    q_fp4 = _c(q_fp4, np.uint8); q_scale = _c(q_scale, np.uint8); w = _c(w, np.float32)
    indptr = _c(indptr, np.int32); bt = _c(block_table, np.int32)
    rows = _c(rows, np.int64); toks = _c(toks, np.int64)
    H = q_fp4.shape[1]
    num_pages = payload.size // (PAGE * D // 2)
    out = np.empty(rows.size, np.float64); tol = np.empty(rows.size, np.float64)
    absr = np.empty(rows.size, np.float64)
    rc = _load().orc_logits_sampled(_p(q_fp4), _p(q_scale), _p(w), H, _p(indptr), len(indptr) - 1, _p(bt),
                                    bt.shape[1], _p(payload), _p(scale), num_pages, rows.size, _p(rows),
                                    _p(toks), _p(out), _p(tol), _p(absr))
    _check(rc, "logits_sampled")
    return out, tol, absr


def topk(logits_arr, row_ctx, k):
    logits_arr = _c(logits_arr, np.float32); row_ctx = _c(row_ctx, np.int32)
    T = logits_arr.shape[0]
    out = np.empty((T, k), np.int32)
    rc = _load().orc_topk(_p(logits_arr), T, logits_arr.shape[1], _p(row_ctx), int(k), _p(out))
    _check(rc, "topk")
    return out


def read_k(payload, scale, slots) -> np.ndarray:
    """Pool tokens at `slots` back to their exact values, fp64 [N, 128]; a
    slot outside the pool reads as zeros."""
    payload = _c(payload, np.uint8); scale = _c(scale, np.uint8); slots = _c(slots, np.int32)
    num_pages = payload.size // 4096
    out = np.empty((slots.size, D), np.float64)
    _check(_load().orc_read_k(_p(payload), _p(scale), num_pages, _p(slots), slots.size, _p(out)), "orc_read_k")
    return out


# ---- FP8 indexer variant ------------------------------------------------------

FP8_PAGE_BYTES = PAGE * (D + 4)   # 64 tokens x (128 codes + fp32 scale)


def fp8_exponent(amax: float) -> int:
    return int(_load().orc_fp8_exponent(ctypes.c_float(amax)))


def e4m3_value(code: int) -> float:
    return float(_load().orc_e4m3_value(int(code)))


def e4m3_code(z: float, e: int) -> int:
    return int(_load().orc_e4m3_code(ctypes.c_float(z), int(e)))


def quant_fp8_128(z: np.ndarray):
    z = _c(z, np.float32)
    codes = np.empty(D, np.uint8); sc = np.empty(1, np.float32)
    _load().orc_quant_fp8_128(_p(z), _p(codes), _p(sc))
    return codes, np.float32(sc[0])


def dequant_fp8_128(codes, scale) -> np.ndarray:
    codes = _c(codes, np.uint8)
    out = np.empty(D, np.float64)
    _load().orc_dequant_fp8_128(_p(codes), ctypes.c_float(float(scale)), _p(out))
    return out


def encode_k_token_fp8(k_row, norm_w, eps, cs_row):
    k_row = _c(k_row, np.uint16); norm_w = _c(norm_w, np.uint16); cs_row = _c(cs_row, np.uint16)
    codes = np.empty(D, np.uint8); sc = np.empty(1, np.float32)
    _load().orc_encode_k_token_fp8(_p(k_row), _p(norm_w), ctypes.c_float(eps), _p(cs_row), _p(codes), _p(sc))
    return codes, np.float32(sc[0])


def encode_q_head_fp8(q_row, cs_row):
    q_row = _c(q_row, np.uint16); cs_row = _c(cs_row, np.uint16)
    codes = np.empty(D, np.uint8); sc = np.empty(1, np.float32)
    _load().orc_encode_q_head_fp8(_p(q_row), _p(cs_row), _p(codes), _p(sc))
    return codes, np.float32(sc[0])


def write_k_fp8(k, pos, slot, norm_w, eps, cos_sin, pool):
    """Encode K rows into the fused FP8 pool (num_pages * 8448 bytes, in place)."""
    k = _c(k, np.uint16); pos = _c(pos, np.int32); slot = _c(slot, np.int32)
    norm_w = _c(norm_w, np.uint16); cos_sin = _c(cos_sin, np.uint16)
    assert pool.dtype == np.uint8 and pool.flags.c_contiguous and pool.size % FP8_PAGE_BYTES == 0
    n = k.shape[0]
    rc = _load().orc_write_k_fp8(_p(k), n, k.shape[1] if n else D, _p(pos), _p(slot), _p(norm_w),
                                 ctypes.c_float(eps), _p(cos_sin), cos_sin.shape[0], _p(pool),
                                 pool.size // FP8_PAGE_BYTES)
    _check(rc, "write_k_fp8")


def pack_q_fp8(q, pos, cos_sin, w_in, w_scale=1.0):
    """q: uint16 [T, H, 128] -> (q_fp8 [T,H,128] u8, q_scale [T,H] f32, w_out [T,H] f32)."""
    q = _c(q, np.uint16); pos = _c(pos, np.int32); cos_sin = _c(cos_sin, np.uint16)
    w_in = _c(w_in, np.float32)
    T, H = q.shape[0], q.shape[1]
    q_fp8 = np.empty((T, H, D), np.uint8); q_scale = np.empty((T, H), np.float32)
    w_out = np.empty((T, H), np.float32)
    rc = _load().orc_pack_q_fp8(_p(q), T, H, H * D, _p(pos), _p(cos_sin), cos_sin.shape[0], _p(w_in),
                                ctypes.c_float(w_scale), _p(q_fp8), _p(q_scale), _p(w_out))
    _check(rc, "pack_q_fp8")
    return q_fp8, q_scale, w_out


def logits_fp8(q_fp8, q_scale, w, indptr, row_ctx, block_table, pool, logits_stride=None, want_f64=False,
               want_b16=False):
    """FP8-variant logits [T, stride] (fp32; entries >= ctx stay NaN); with
    want_f64 also the fp64 values and the T, A tolerance scales, and with
    want_b16 as well B16 = sum_h |w_h| (sum of the 16 largest |q_hi k_i|)."""
    q_fp8 = _c(q_fp8, np.uint8); q_scale = _c(q_scale, np.float32); w = _c(w, np.float32)
    indptr = _c(indptr, np.int32); row_ctx = _c(row_ctx, np.int32); bt = _c(block_table, np.int32)
    T, H = q_fp8.shape[0], q_fp8.shape[1]
    stride = int(logits_stride if logits_stride is not None else max(1, int(row_ctx.max(initial=0))))
    out = np.full((T, stride), np.nan, np.float32)
    f64 = np.full((T, stride), np.nan, np.float64) if want_f64 else None
    tol = np.full((T, stride), np.nan, np.float64) if want_f64 else None
    absr = np.full((T, stride), np.nan, np.float64) if want_f64 else None
    b16 = np.full((T, stride), np.nan, np.float64) if (want_f64 and want_b16) else None
    rc = _load().orc_logits_fp8(_p(q_fp8), _p(q_scale), _p(w), T, H, _p(indptr), len(indptr) - 1, _p(row_ctx),
                                _p(bt), bt.shape[1], _p(pool), pool.size // FP8_PAGE_BYTES, _p(out), stride,
                                _p(f64) if want_f64 else None, _p(tol) if want_f64 else None,
                                _p(absr) if want_f64 else None, _p(b16) if b16 is not None else None)
    _check(rc, "logits_fp8")
    if not want_f64:
        return out
    return (out, f64, tol, absr, b16) if want_b16 else (out, f64, tol, absr)


def logits_fp8_sampled(q_fp8, q_scale, w, indptr, block_table, pool, rows, toks, want_b16=False):
    """fp64 FP8-variant logits at (rows[i], toks[i]) with their T and A scales
    (and B16, see logits_fp8, with want_b16)."""
    q_fp8 = _c(q_fp8, np.uint8); q_scale = _c(q_scale, np.float32); w = _c(w, np.float32)
    indptr = _c(indptr, np.int32); bt = _c(block_table, np.int32)
    rows = _c(rows, np.int64); toks = _c(toks, np.int64)
    H = q_fp8.shape[1]
    out = np.empty(rows.size, np.float64); tol = np.empty(rows.size, np.float64)
    absr = np.empty(rows.size, np.float64)
    b16 = np.empty(rows.size, np.float64) if want_b16 else None
    rc = _load().orc_logits_fp8_sampled(_p(q_fp8), _p(q_scale), _p(w), H, _p(indptr), len(indptr) - 1, _p(bt),
                                        bt.shape[1], _p(pool), pool.size // FP8_PAGE_BYTES, rows.size, _p(rows),
                                        _p(toks), _p(out), _p(tol), _p(absr), _p(b16) if want_b16 else None)
    _check(rc, "logits_fp8_sampled")
    return (out, tol, absr, b16) if want_b16 else (out, tol, absr)
