"""ctypes wrapper of the CPU oracle (idx_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU product path.

Functions take plain numpy arrays (or any object with the attributes of a
workload: q, w, pool, block_size, block_table, q_req, chunk_ids, n_chunks,
limits, n_cols) and return numpy arrays in double precision.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "idx_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_c_i32p = ctypes.POINTER(ctypes.c_int32)
_c_u8p = ctypes.POINTER(ctypes.c_uint8)
_c_u16p = ctypes.POINTER(ctypes.c_uint16)
_c_f32p = ctypes.POINTER(ctypes.c_float)
_c_f64p = ctypes.POINTER(ctypes.c_double)

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C99, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fopenmp",
               "-shared", "-fPIC", _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_scale_value.restype = ctypes.c_double
    lib.oracle_scale_value.argtypes = [_c_u8p, ctypes.c_int32]
    lib.oracle_logit.restype = ctypes.c_double
    lib.oracle_logit.argtypes = [_c_u16p, _c_f32p, ctypes.c_int32, ctypes.c_int32, _c_u8p]
    lib.oracle_sigmoid.restype = ctypes.c_double
    lib.oracle_sigmoid.argtypes = [ctypes.c_double]
    lib.oracle_sigmoid_array.restype = None
    lib.oracle_sigmoid_array.argtypes = [_c_f64p, ctypes.c_int64, _c_f64p]
    lib.oracle_score.restype = ctypes.c_int
    lib.oracle_score.argtypes = [
        _c_u16p, _c_f32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        _c_u8p, ctypes.c_int64, ctypes.c_int32,
        _c_i32p, ctypes.c_int32, ctypes.c_int32, _c_i32p,
        _c_i32p, _c_i32p, ctypes.c_int32, _c_i32p, ctypes.c_int32,
        _c_f64p, ctypes.c_int32]
    lib.oracle_score_q8.restype = ctypes.c_int
    lib.oracle_score_q8.argtypes = [_c_u8p] + lib.oracle_score.argtypes[1:]
    lib.oracle_score_mxfp4.restype = ctypes.c_int
    lib.oracle_score_mxfp4.argtypes = lib.oracle_score.argtypes
    lib.oracle_e2m1_round.restype = ctypes.c_double
    lib.oracle_e2m1_round.argtypes = [ctypes.c_double]
    lib.oracle_mxfp4_exponent.restype = ctypes.c_int
    lib.oracle_mxfp4_exponent.argtypes = [ctypes.c_double]
    lib.oracle_mxfp4_round.restype = None
    lib.oracle_mxfp4_round.argtypes = [_c_f64p, ctypes.c_int32, _c_f64p]
    lib.oracle_topk.restype = ctypes.c_int
    lib.oracle_topk.argtypes = [_c_f64p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                ctypes.c_int32, _c_i32p, _c_f64p, ctypes.c_int32]
    lib.oracle_cols_to_entries.restype = ctypes.c_int
    lib.oracle_cols_to_entries.argtypes = [_c_i32p, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, _c_i32p, ctypes.c_int32, _c_i32p]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_quantize_row.restype = None
    lib.oracle_quantize_row.argtypes = [_c_u16p, ctypes.c_int32, _c_u8p]
    lib.oracle_write_keys.restype = ctypes.c_int64
    lib.oracle_write_keys.argtypes = [_c_u16p, ctypes.c_int64, ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_int64), _c_u8p, ctypes.c_int64]
    lib.oracle_level1_select.restype = ctypes.c_int
    lib.oracle_level1_select.argtypes = [_c_f32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int64, _c_i32p, ctypes.c_int32, ctypes.c_float,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _c_i32p, _c_i32p]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    _lib = lib
    return lib


def _ptr(a, ctype):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def e4m3_value(u: int) -> float:
    """Value of one float8_e4m3fn byte (closed form)."""
    return float(_load().oracle_e4m3_value(ctypes.c_uint8(int(u) & 0xFF)))


def scale_value(row: np.ndarray, head_dim: int) -> float:
    row = np.ascontiguousarray(row, dtype=np.uint8)
    return float(_load().oracle_scale_value(_ptr(row, ctypes.c_uint8), head_dim))


def logit(q_row: np.ndarray, w_row: np.ndarray, key_row: np.ndarray) -> float:
    """One logit: q_row uint16 [H, D] (bf16 bits), w_row float32 [H], key_row uint8 [D+4]."""
    q_row = np.ascontiguousarray(q_row, dtype=np.uint16)
    w_row = np.ascontiguousarray(w_row, dtype=np.float32)
    key_row = np.ascontiguousarray(key_row, dtype=np.uint8)
    H, D = q_row.shape
    assert key_row.shape == (D + 4,) and w_row.shape == (H,)
    return float(_load().oracle_logit(_ptr(q_row, ctypes.c_uint16), _ptr(w_row, ctypes.c_float),
                                      H, D, _ptr(key_row, ctypes.c_uint8)))


def sigmoid(x) -> np.ndarray:
    """The oracle's sigmoid of each logit (double); -inf gives 0."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    _load().oracle_sigmoid_array(_ptr(x.reshape(-1), ctypes.c_double), x.size,
                                 _ptr(out.reshape(-1), ctypes.c_double))
    return out


def sigmoid_scalar(x: float) -> float:
    """The oracle's scalar sigmoid (the function the array form applies)."""
    return float(_load().oracle_sigmoid(float(x)))


def e2m1_round(x: float) -> float:
    """The E2M1 value nearest x (ties to the even code, saturating at 6)."""
    return float(_load().oracle_e2m1_round(float(x)))


def mxfp4_exponent(amax: float) -> int:
    """MXFP4 block exponent for a block whose largest magnitude is amax > 0."""
    return int(_load().oracle_mxfp4_exponent(float(amax)))


def mxfp4_round(v) -> np.ndarray:
    """v (length a multiple of 32) rounded to MXFP4 block by block."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    assert v.size % 32 == 0
    out = np.empty_like(v)
    _load().oracle_mxfp4_round(_ptr(v.reshape(-1), ctypes.c_double), v.size,
                               _ptr(out.reshape(-1), ctypes.c_double))
    return out


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def score(wl, rows=None, n_threads: int = 0, q8=None, mxfp4: bool = False) -> np.ndarray:
    """Double logits [B, n_cols] (or [len(rows), n_cols] for a row subset);
    unscored columns are -inf.  With q8 (uint8 [B, H, D + 4] quantised query
    rows, see quantize_q) the query is q8's dequantised values instead of
    wl.q.  With mxfp4, query heads and keys are rounded to MXFP4 blocks of
    32 first (the MXFP4 variant)."""
    q = np.ascontiguousarray(wl.q, dtype=np.uint16)
    if q8 is not None:
        q8 = np.ascontiguousarray(q8, dtype=np.uint8)
        if rows is not None:
            q8 = np.ascontiguousarray(q8[np.asarray(rows, dtype=np.int64)])
    w = np.ascontiguousarray(wl.w, dtype=np.float32)
    limits = _i32(wl.limits)
    q_req = _i32(wl.q_req)
    chunk_ids = _i32(wl.chunk_ids)
    n_chunks = _i32(wl.n_chunks)
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        q = np.ascontiguousarray(q[rows])
        w = np.ascontiguousarray(w[rows])
        limits = np.ascontiguousarray(limits[rows])
        if q_req is None:
            q_req = rows.astype(np.int32)      # keep each row's own request
        else:
            q_req = np.ascontiguousarray(q_req[rows])
        if chunk_ids is not None:
            chunk_ids = np.ascontiguousarray(chunk_ids[rows])
            n_chunks = np.ascontiguousarray(n_chunks[rows])
    B, H, D = q.shape
    table = _i32(wl.block_table)
    n_req = 0 if table is None else table.shape[0]
    max_blocks = 0 if table is None else table.shape[1]
    max_chunks = 0 if chunk_ids is None else chunk_ids.shape[1]
    pool = np.ascontiguousarray(wl.pool, dtype=np.uint8)
    assert pool.shape[1] == D + 4
    out = np.empty((B, wl.n_cols), dtype=np.float64)
    assert not (mxfp4 and q8 is not None)
    if q8 is not None:
        fn, qp = _load().oracle_score_q8, _ptr(q8, ctypes.c_uint8)
    else:
        fn = _load().oracle_score_mxfp4 if mxfp4 else _load().oracle_score
        qp = _ptr(q, ctypes.c_uint16)
    rc = fn(
        qp, _ptr(w, ctypes.c_float), B, H, D,
        _ptr(pool, ctypes.c_uint8), pool.shape[0], wl.block_size,
        _ptr(table, ctypes.c_int32), n_req, max_blocks, _ptr(q_req, ctypes.c_int32),
        _ptr(chunk_ids, ctypes.c_int32), _ptr(n_chunks, ctypes.c_int32), max_chunks,
        _ptr(limits, ctypes.c_int32), wl.n_cols, _ptr(out, ctypes.c_double), n_threads)
    if rc != 0:
        raise RuntimeError(f"oracle_score failed ({rc})")
    return out


def topk(vals: np.ndarray, k: int, n_threads: int = 0):
    """Top-k columns per row of vals [B, n] (desc value, ties -> lower column;
    -inf and NaN never selected; -1 padding).  Returns (cols int32, vals f64)."""
    vals = np.ascontiguousarray(vals, dtype=np.float64)
    B, n = vals.shape
    cols = np.empty((B, k), dtype=np.int32)
    out_v = np.empty((B, k), dtype=np.float64)
    rc = _load().oracle_topk(_ptr(vals, ctypes.c_double), B, n, n, k,
                             _ptr(cols, ctypes.c_int32), _ptr(out_v, ctypes.c_double),
                             n_threads)
    if rc != 0:
        raise RuntimeError(f"oracle_topk failed ({rc})")
    return cols, out_v


def cols_to_entries(wl, cols: np.ndarray, rows=None) -> np.ndarray:
    """Map selected columns to logical entry ids (chunk lists resolved)."""
    cols = np.ascontiguousarray(cols, dtype=np.int32)
    B, k = cols.shape
    chunk_ids = _i32(wl.chunk_ids)
    if chunk_ids is not None and rows is not None:
        chunk_ids = np.ascontiguousarray(chunk_ids[np.asarray(rows)])
    max_chunks = 0 if chunk_ids is None else chunk_ids.shape[1]
    out = np.empty_like(cols)
    _load().oracle_cols_to_entries(_ptr(cols, ctypes.c_int32), B, k, wl.block_size,
                                   _ptr(chunk_ids, ctypes.c_int32), max_chunks,
                                   _ptr(out, ctypes.c_int32))
    return out


def score_topk(wl, rows=None, n_threads: int = 0, mxfp4: bool = False):
    """Oracle of the whole path: (entry ids [B,k], their logits [B,k], logits
    [B,n_cols]); with mxfp4, of the MXFP4 variant."""
    lg = score(wl, rows=rows, n_threads=n_threads, mxfp4=mxfp4)
    cols, vals = topk(lg, wl.k, n_threads=n_threads)
    return cols_to_entries(wl, cols, rows=rows), vals, lg


def e4m3_encode(y) -> np.ndarray:
    """float8_e4m3fn byte of each float32 value: nearest value, ties to the
    even code, saturating at +-448 (the writer's rounding)."""
    lib = _load()
    y = np.asarray(y, dtype=np.float32)
    flat = y.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for i, v in enumerate(flat.tolist()):
        out[i] = lib.oracle_e4m3_encode(ctypes.c_float(v))
    return out.reshape(y.shape)


def quantize_row(k_row: np.ndarray) -> np.ndarray:
    """One pool row (uint8 [D + 4]) from a key of D bf16 bit patterns."""
    k_row = np.ascontiguousarray(k_row, dtype=np.uint16)
    (D,) = k_row.shape
    row = np.empty(D + 4, dtype=np.uint8)
    _load().oracle_quantize_row(_ptr(k_row, ctypes.c_uint16), D, _ptr(row, ctypes.c_uint8))
    return row


def write_keys(k: np.ndarray, slots: np.ndarray, pool: np.ndarray) -> int:
    """Quantise keys k (uint16 [n, D], bf16 bits) into pool rows slots[i]
    (int64 [n]; -1 = none) in place.  Returns the count of slots outside the
    pool (those write nothing)."""
    k = np.ascontiguousarray(k, dtype=np.uint16)
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    assert pool.flags["C_CONTIGUOUS"] and pool.dtype == np.uint8
    n, D = k.shape
    assert slots.shape == (n,) and pool.shape[1] == D + 4
    return int(_load().oracle_write_keys(_ptr(k, ctypes.c_uint16), n, D,
                                         _ptr(slots, ctypes.c_int64),
                                         _ptr(pool, ctypes.c_uint8), pool.shape[0]))


ENSEMBLE_MAX, ENSEMBLE_MEAN = 0, 1


def level1_select(scores: np.ndarray, limits, ensemble: int, threshold: float, n_sink: int,
                  n_recent: int, kmax: int):
    """Level-1 resident pages from per-layer binary32 sigmoid scores
    [L, B, n_cols]: (pages int32 [B, kmax] ascending, -1 padded; count [B])."""
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    L, B, n = scores.shape
    limits = np.ascontiguousarray(limits, dtype=np.int32)
    pages = np.empty((B, kmax), dtype=np.int32)
    count = np.empty(B, dtype=np.int32)
    rc = _load().oracle_level1_select(_ptr(scores, ctypes.c_float), L, B, n, n,
                                      _ptr(limits, ctypes.c_int32), ensemble,
                                      ctypes.c_float(threshold), n_sink, n_recent, kmax,
                                      _ptr(pages, ctypes.c_int32), _ptr(count, ctypes.c_int32))
    if rc != 0:
        raise RuntimeError(f"oracle_level1_select failed ({rc})")
    return pages, count


def level1_scores(layers, rows=None, n_threads: int = 0) -> np.ndarray:
    """The oracle's own per-layer scores [L, B, n_cols]: sigmoid of the double
    logits of each layer's workload, rounded to binary32 (0 where unscored)."""
    out = []
    for wl in layers:
        lg = score(wl, rows=rows, n_threads=n_threads)
        with np.errstate(over="ignore"):
            s = 1.0 / (1.0 + np.exp(-lg))
        out.append(s.astype(np.float32))
    return np.stack(out)


def quantize_q(q: np.ndarray) -> np.ndarray:
    """Quantised query rows uint8 [B, H, D + 4] from q (bf16 bits [B, H, D]):
    each head through the index-plane writer's rule (amax / 448 scale)."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    B, H, D = q.shape
    out = np.zeros((B * H, D + 4), dtype=np.uint8)
    write_keys(q.reshape(B * H, D), np.arange(B * H, dtype=np.int64), out)
    return out.reshape(B, H, D + 4)
