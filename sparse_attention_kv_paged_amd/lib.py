"""ctypes binding of libidx.so (argument marshalling only).

Every function has the name of the C entry point it calls (include/idx.h);
all computation runs in the library's HIP kernels.  PyTorch supplies device
memory and the current stream.  There is no CPU fallback: if the library is
missing the call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libidx.so")

IDX_OK, IDX_E_ARG, IDX_E_SHAPE, IDX_E_ALIGN, IDX_E_WORKSPACE, IDX_E_HIP = range(6)
IDX_OP_SCORE, IDX_OP_TOPK, IDX_OP_SCORE_TOPK = range(3)
STATUS_LIMIT_CLAMPED, STATUS_BAD_BLOCK, STATUS_BAD_REQUEST, STATUS_BAD_CHUNK = 1, 2, 4, 8
STATUS_BAD_SLOT = 16
ENSEMBLE_MAX, ENSEMBLE_MEAN = 0, 1
MAX_LAYERS = 8
MAX_COLS = 1 << 27                # IDX_MAX_COLS
STATIC_SCRATCH_BYTES = 16 << 20   # IDX_STATIC_SCRATCH_BYTES

EXPORTS = ("idx_score", "idx_topk", "idx_score_topk", "idx_score_topk_noalloc", "idx_score_q8", "idx_score_topk_q8",
           "idx_score_fp8q", "idx_score_topk_fp8q", "idx_score_mxfp4", "idx_score_topk_mxfp4",
           "idx_write_keys", "idx_select_resident",
           "idx_resident_workspace_bytes", "idx_workspace_bytes",
           "idx_error_string", "idx_last_error", "idx_profile_events", "idx_abi_version")


class IdxKeys(ctypes.Structure):
    """Mirror of `struct idx_keys`."""
    _fields_ = [
        ("pool", ctypes.c_void_p),
        ("n_pool_rows", ctypes.c_int64),
        ("block_size", ctypes.c_int32),
        ("n_req", ctypes.c_int32),
        ("block_table", ctypes.c_void_p),
        ("max_blocks", ctypes.c_int32),
        ("max_chunks", ctypes.c_int32),
        ("q_req", ctypes.c_void_p),
        ("chunk_ids", ctypes.c_void_p),
        ("n_chunks", ctypes.c_void_p),
        ("limits", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
    ]


class ResidentCfg(ctypes.Structure):
    """Mirror of `struct idx_resident_cfg`."""
    _fields_ = [
        ("ensemble", ctypes.c_int32),
        ("threshold", ctypes.c_float),
        ("n_sink", ctypes.c_int32),
        ("n_recent", ctypes.c_int32),
        ("kmax", ctypes.c_int32),
    ]


class IdxError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"idx error {code}: {msg}")
        self.code = code


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libidx.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m sparse_attention_kv_paged_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    kp = ctypes.POINTER(IdxKeys)
    lib.idx_score.argtypes = [vp, vp, i32, i32, i32, kp, i32, vp, vp, vp]
    lib.idx_score.restype = ctypes.c_int
    lib.idx_topk.argtypes = [vp, i32, i32, i64, i32, vp, vp, vp, sz, vp]
    lib.idx_topk.restype = ctypes.c_int
    lib.idx_score_topk.argtypes = [vp, vp, i32, i32, i32, kp, i32, i32, vp, vp, vp, sz, vp]
    lib.idx_score_topk.restype = ctypes.c_int
    lib.idx_score_topk_noalloc.argtypes = [vp, vp, i32, i32, i32, kp, i32, i32, vp, vp, vp]
    lib.idx_score_topk_noalloc.restype = ctypes.c_int
    lib.idx_score_fp8q.argtypes = [vp, vp, i32, i32, i32, kp, i32, vp, vp, vp]
    lib.idx_score_fp8q.restype = ctypes.c_int
    lib.idx_score_topk_fp8q.argtypes = [vp, vp, i32, i32, i32, kp, i32, i32, vp, vp, vp, sz, vp]
    lib.idx_score_topk_fp8q.restype = ctypes.c_int
    lib.idx_score_mxfp4.argtypes = [vp, vp, i32, i32, i32, kp, i32, vp, vp, vp]
    lib.idx_score_mxfp4.restype = ctypes.c_int
    lib.idx_score_topk_mxfp4.argtypes = [vp, vp, i32, i32, i32, kp, i32, i32, vp, vp, vp, sz, vp]
    lib.idx_score_topk_mxfp4.restype = ctypes.c_int
    lib.idx_score_q8.argtypes = [vp, vp, i32, i32, i32, kp, i32, vp, vp, vp]
    lib.idx_score_q8.restype = ctypes.c_int
    lib.idx_score_topk_q8.argtypes = [vp, vp, i32, i32, i32, kp, i32, i32, vp, vp, vp, sz, vp]
    lib.idx_score_topk_q8.restype = ctypes.c_int
    lib.idx_write_keys.argtypes = [vp, i64, i32, vp, vp, i64, vp, vp]
    lib.idx_write_keys.restype = ctypes.c_int
    lib.idx_select_resident.argtypes = [i32, vp, vp, i32, i32, i32, kp, i32, ctypes.POINTER(ResidentCfg),
                                        vp, vp, vp, sz, vp]
    lib.idx_select_resident.restype = ctypes.c_int
    lib.idx_resident_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.idx_resident_workspace_bytes.restype = sz
    lib.idx_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.idx_workspace_bytes.restype = sz
    lib.idx_error_string.argtypes = [i32]
    lib.idx_error_string.restype = ctypes.c_char_p
    lib.idx_last_error.argtypes = []
    lib.idx_last_error.restype = ctypes.c_char_p
    lib.idx_profile_events.argtypes = [vp, vp]
    lib.idx_profile_events.restype = ctypes.c_int
    lib.idx_abi_version.argtypes = []
    lib.idx_abi_version.restype = i32
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(rc: int):
    if rc != IDX_OK:
        lib = load()
        raise IdxError(rc, f"{lib.idx_error_string(rc).decode()}: {lib.idx_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: Optional[torch.Tensor], dtype, name: str):
    if t is None:
        return None
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous CUDA {dtype} tensor")
    return t


@dataclass
class Keys:
    """Device tensors of the paged index plane and the per-row tile lists
    (fields as in `struct idx_keys`)."""
    pool: torch.Tensor                          # uint8 [n_pool_rows, 132]
    limits: torch.Tensor                        # int32 [B]
    block_table: Optional[torch.Tensor] = None  # int32 [n_req, max_blocks]
    q_req: Optional[torch.Tensor] = None        # int32 [B]
    chunk_ids: Optional[torch.Tensor] = None    # int32 [B, max_chunks]
    n_chunks: Optional[torch.Tensor] = None     # int32 [B]
    status: Optional[torch.Tensor] = None       # int32 [1] (bits OR-ed in)
    block_size: int = 64                        # rows per pool block: 64 or 16

    def struct(self, B: int) -> IdxKeys:
        """The C struct for a call over B query rows.  Every per-row tensor
        must hold at least B rows: the kernels read rows 0 .. B - 1, so a
        short one is rejected here instead of being read past its end."""
        pool = _dev(self.pool, torch.uint8, "pool")
        bt = _dev(self.block_table, torch.int32, "block_table")
        ci = _dev(self.chunk_ids, torch.int32, "chunk_ids")
        limits = _dev(self.limits, torch.int32, "limits")
        q_req = _dev(self.q_req, torch.int32, "q_req")
        n_chunks = _dev(self.n_chunks, torch.int32, "n_chunks")
        status = _dev(self.status, torch.int32, "status")
        if pool.dim() != 2:
            raise ValueError("pool must be [n_pool_rows, D + 4]")
        for name, t in (("limits", limits), ("q_req", q_req), ("n_chunks", n_chunks)):
            if t is not None and (t.dim() != 1 or t.shape[0] < B):
                raise ValueError(f"{name} must hold one int32 per query row ({B}), got shape {tuple(t.shape)}")
        if bt is not None and bt.dim() != 2:
            raise ValueError("block_table must be [n_req, max_blocks]")
        if ci is not None:
            if ci.dim() != 2 or ci.shape[0] < B:
                raise ValueError(f"chunk_ids must be [{B}, max_chunks], got shape {tuple(ci.shape)}")
            if n_chunks is None:
                raise ValueError("n_chunks is required with chunk_ids")
        if status is not None and status.numel() < 1:
            raise ValueError("status must hold at least one int32")
        k = IdxKeys()
        k.pool = pool.data_ptr()
        k.n_pool_rows = pool.shape[0]
        k.block_size = self.block_size
        k.n_req = 0 if bt is None else bt.shape[0]
        k.block_table = None if bt is None else bt.data_ptr()
        k.max_blocks = 0 if bt is None else bt.shape[1]
        k.max_chunks = 0 if ci is None else ci.shape[1]
        k.q_req = None if q_req is None else q_req.data_ptr()
        k.chunk_ids = None if ci is None else ci.data_ptr()
        k.n_chunks = None if n_chunks is None else n_chunks.data_ptr()
        k.limits = limits.data_ptr()
        k.status = None if status is None else status.data_ptr()
        return k


def idx_profile_events(before, after) -> None:
    """Record hipEvents (torch.cuda.Event objects, or None to stop) around
    every later score-kernel or writer-kernel launch on this thread."""
    bp = None if before is None else ctypes.c_void_p(before.cuda_event)
    ap = None if after is None else ctypes.c_void_p(after.cuda_event)
    _check(load().idx_profile_events(bp, ap))


def workspace_bytes(op: int, B: int, n_cols: int, k: int) -> int:
    n = load().idx_workspace_bytes(op, B, n_cols, k)
    if n == ctypes.c_size_t(-1).value:
        raise IdxError(IDX_E_ARG, "invalid workspace request")
    return int(n)


def idx_workspace_bytes(op: int, B: int, n_cols: int, k: int) -> int:
    return workspace_bytes(op, B, n_cols, k)


def new_workspace(n: int, device="cuda") -> torch.Tensor:
    """A device workspace of n bytes, zeroed (the library's per-row arrival
    counters must read zero on a workspace's first use; every call leaves
    them zero)."""
    return torch.zeros(max(n, 1), dtype=torch.uint8, device=device)


def _workspace(n: int, device) -> torch.Tensor:
    return new_workspace(n, device)


def _qw(q, w):
    if q.dtype == torch.bfloat16:
        q = q.view(torch.int16)
    q = _dev(q, torch.int16, "q (bf16 bits)")
    w = _dev(w, torch.float32, "w")
    if q.dim() != 3 or w.dim() != 2 or w.shape != q.shape[:2]:
        raise ValueError("q must be [B, H, D] and w [B, H]")
    return q, w


def idx_score(q, w, keys: Keys, n_cols: int, with_scores: bool = False,
              logits: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None,
              stream=None):
    """Logits [B, n_cols] (fp32, -inf where unscored) and optionally scores."""
    q, w = _qw(q, w)
    B, H, D = q.shape
    if logits is None:
        logits = torch.empty((B, n_cols), dtype=torch.float32, device=q.device)
    if with_scores and scores is None:
        scores = torch.empty((B, n_cols), dtype=torch.float32, device=q.device)
    _dev(logits, torch.float32, "logits")
    _dev(scores, torch.float32, "scores")
    ks = keys.struct(B)
    _check(load().idx_score(_ptr(q), _ptr(w), B, H, D, ctypes.byref(ks), n_cols,
                            _ptr(logits), _ptr(scores), _stream(stream)))
    return (logits, scores) if with_scores else logits


def idx_topk(logits: torch.Tensor, k: int, n_cols: Optional[int] = None,
             out_col=None, out_val=None, workspace=None, stream=None):
    """Top-k columns [B, k] (int32) and values [B, k] of each logits row."""
    if logits.dim() != 2 or logits.dtype != torch.float32 or not logits.is_cuda or logits.stride(1) != 1:
        raise ValueError("logits must be a CUDA float32 [B, ld] tensor with unit column stride")
    B = logits.shape[0]
    n_cols = logits.shape[1] if n_cols is None else n_cols
    ld = logits.stride(0) if B > 1 else max(n_cols, logits.shape[1])
    if out_col is None:
        out_col = torch.empty((B, k), dtype=torch.int32, device=logits.device)
    if out_val is None:
        out_val = torch.empty((B, k), dtype=torch.float32, device=logits.device)
    need = workspace_bytes(IDX_OP_TOPK, B, n_cols, k)
    if workspace is None:
        workspace = _workspace(need, logits.device)
    _check(load().idx_topk(_ptr(logits), B, n_cols, ld, k, _ptr(out_col), _ptr(out_val),
                           _ptr(workspace), workspace.numel(), _stream(stream)))
    return out_col, out_val


def idx_score_topk(q, w, keys: Keys, n_cols: int, k: int, out_idx=None, out_val=None,
                   workspace=None, stream=None):
    """Top-k logical entry ids [B, k] (int32, -1 padded) and their logits."""
    q, w = _qw(q, w)
    B, H, D = q.shape
    if out_idx is None:
        out_idx = torch.empty((B, k), dtype=torch.int32, device=q.device)
    if out_val is None:
        out_val = torch.empty((B, k), dtype=torch.float32, device=q.device)
    need = workspace_bytes(IDX_OP_SCORE_TOPK, B, n_cols, k)
    if workspace is None:
        workspace = _workspace(need, q.device)
    ks = keys.struct(B)
    _check(load().idx_score_topk(_ptr(q), _ptr(w), B, H, D, ctypes.byref(ks), n_cols, k,
                                 _ptr(out_idx), _ptr(out_val), _ptr(workspace),
                                 workspace.numel(), _stream(stream)))
    return out_idx, out_val


def idx_score_topk_noalloc(q, w, keys: Keys, n_cols: int, k: int, out_idx=None, out_val=None, stream=None):
    """idx_score_topk on the library's static device scratch (no workspace;
    the call allocates nothing when out_idx and out_val are passed in)."""
    q, w = _qw(q, w)
    B, H, D = q.shape
    if out_idx is None:
        out_idx = torch.empty((B, k), dtype=torch.int32, device=q.device)
    if out_val is None:
        out_val = torch.empty((B, k), dtype=torch.float32, device=q.device)
    _dev(out_idx, torch.int32, "out_idx")
    _dev(out_val, torch.float32, "out_val")
    ks = keys.struct(B)
    _check(load().idx_score_topk_noalloc(_ptr(q), _ptr(w), B, H, D, ctypes.byref(ks), n_cols, k,
                                         _ptr(out_idx), _ptr(out_val), _stream(stream)))
    return out_idx, out_val


def _score_quantised(fn, q, w, keys: Keys, n_cols: int, with_scores, logits, scores, stream):
    q, w = _qw(q, w)
    B, H, D = q.shape
    if logits is None:
        logits = torch.empty((B, n_cols), dtype=torch.float32, device=q.device)
    if with_scores and scores is None:
        scores = torch.empty((B, n_cols), dtype=torch.float32, device=q.device)
    _dev(logits, torch.float32, "logits")
    _dev(scores, torch.float32, "scores")
    ks = keys.struct(B)
    _check(fn(_ptr(q), _ptr(w), B, H, D, ctypes.byref(ks), n_cols, _ptr(logits), _ptr(scores), _stream(stream)))
    return (logits, scores) if with_scores else logits


def _score_topk_quantised(fn, q, w, keys: Keys, n_cols: int, k: int, out_idx, out_val, workspace, stream):
    q, w = _qw(q, w)
    B, H, D = q.shape
    if out_idx is None:
        out_idx = torch.empty((B, k), dtype=torch.int32, device=q.device)
    if out_val is None:
        out_val = torch.empty((B, k), dtype=torch.float32, device=q.device)
    need = workspace_bytes(IDX_OP_SCORE_TOPK, B, n_cols, k)
    if workspace is None:
        workspace = _workspace(need, q.device)
    ks = keys.struct(B)
    _check(fn(_ptr(q), _ptr(w), B, H, D, ctypes.byref(ks), n_cols, k, _ptr(out_idx), _ptr(out_val),
              _ptr(workspace), workspace.numel(), _stream(stream)))
    return out_idx, out_val


def idx_score_fp8q(q, w, keys: Keys, n_cols: int, with_scores: bool = False,
                   logits: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None, stream=None):
    """idx_score with the query quantised inside the score kernel (the
    writer's rule per head; equal to quantize_q followed by idx_score_q8)."""
    return _score_quantised(load().idx_score_fp8q, q, w, keys, n_cols, with_scores, logits, scores, stream)


def idx_score_topk_fp8q(q, w, keys: Keys, n_cols: int, k: int, out_idx=None, out_val=None,
                        workspace=None, stream=None):
    """idx_score_topk with the query quantised inside the score kernel."""
    return _score_topk_quantised(load().idx_score_topk_fp8q, q, w, keys, n_cols, k, out_idx, out_val, workspace,
                                 stream)


def idx_score_mxfp4(q, w, keys: Keys, n_cols: int, with_scores: bool = False,
                    logits: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None, stream=None):
    """idx_score with query heads and keys rounded to MXFP4 blocks of 32
    inside the score kernel (the contraction on e2m1 MFMA)."""
    return _score_quantised(load().idx_score_mxfp4, q, w, keys, n_cols, with_scores, logits, scores, stream)


def idx_score_topk_mxfp4(q, w, keys: Keys, n_cols: int, k: int, out_idx=None, out_val=None,
                         workspace=None, stream=None):
    """idx_score_topk of the MXFP4 variant."""
    return _score_topk_quantised(load().idx_score_topk_mxfp4, q, w, keys, n_cols, k, out_idx, out_val, workspace,
                                 stream)


def quantize_q(q: torch.Tensor, out: Optional[torch.Tensor] = None, slots: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """Quantised query rows [B, H, D + 4] (uint8) from q [B, H, D] (bf16):
    each head quantised by idx_write_keys (amax / 448 scale).  out and slots
    (arange(B * H), int64) may be passed in to avoid allocations."""
    B, H, D = q.shape
    q8 = torch.empty((B * H, D + 4), dtype=torch.uint8, device=q.device) if out is None else out.view(B * H, D + 4)
    if slots is None:
        slots = torch.arange(B * H, dtype=torch.int64, device=q.device)
    idx_write_keys(q.reshape(B * H, D), slots, q8, stream=stream)
    return q8.view(B, H, D + 4)


def _q8w(q8, w):
    q8 = _dev(q8, torch.uint8, "q8")
    w = _dev(w, torch.float32, "w")
    if q8.dim() != 3 or w.dim() != 2 or w.shape != q8.shape[:2]:
        raise ValueError("q8 must be [B, H, D + 4] and w [B, H]")
    return q8, w


def idx_score_q8(q8, w, keys: Keys, n_cols: int, with_scores: bool = False,
                 logits: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None, stream=None):
    """idx_score with quantised query rows (see quantize_q)."""
    q8, w = _q8w(q8, w)
    B, H, D4 = q8.shape
    if logits is None:
        logits = torch.empty((B, n_cols), dtype=torch.float32, device=q8.device)
    if with_scores and scores is None:
        scores = torch.empty((B, n_cols), dtype=torch.float32, device=q8.device)
    _dev(logits, torch.float32, "logits")
    _dev(scores, torch.float32, "scores")
    ks = keys.struct(B)
    _check(load().idx_score_q8(_ptr(q8), _ptr(w), B, H, D4 - 4, ctypes.byref(ks), n_cols,
                               _ptr(logits), _ptr(scores), _stream(stream)))
    return (logits, scores) if with_scores else logits


def idx_score_topk_q8(q8, w, keys: Keys, n_cols: int, k: int, out_idx=None, out_val=None,
                      workspace=None, stream=None):
    """idx_score_topk with quantised query rows (see quantize_q)."""
    q8, w = _q8w(q8, w)
    B, H, D4 = q8.shape
    if out_idx is None:
        out_idx = torch.empty((B, k), dtype=torch.int32, device=q8.device)
    if out_val is None:
        out_val = torch.empty((B, k), dtype=torch.float32, device=q8.device)
    need = workspace_bytes(IDX_OP_SCORE_TOPK, B, n_cols, k)
    if workspace is None:
        workspace = _workspace(need, q8.device)
    ks = keys.struct(B)
    _check(load().idx_score_topk_q8(_ptr(q8), _ptr(w), B, H, D4 - 4, ctypes.byref(ks), n_cols, k,
                                    _ptr(out_idx), _ptr(out_val), _ptr(workspace), workspace.numel(),
                                    _stream(stream)))
    return out_idx, out_val


def idx_write_keys(k: torch.Tensor, slots: torch.Tensor, pool: torch.Tensor,
                   status: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Quantise keys k [n, 128] (bf16) into pool rows slots[i] (int64 [n],
    -1 = none) of pool (uint8 [n_pool_rows, 132]) in place; returns pool."""
    if k.dtype == torch.bfloat16:
        k = k.view(torch.int16)
    k = _dev(k, torch.int16, "k (bf16 bits)")
    slots = _dev(slots, torch.int64, "slots")
    pool = _dev(pool, torch.uint8, "pool")
    _dev(status, torch.int32, "status")
    if k.dim() != 2 or slots.shape != (k.shape[0],) or pool.dim() != 2 or pool.shape[1] != k.shape[1] + 4:
        raise ValueError("k must be [n, D], slots [n] and pool [n_pool_rows, D + 4]")
    _check(load().idx_write_keys(_ptr(k), k.shape[0], k.shape[1], _ptr(slots), _ptr(pool),
                                 pool.shape[0], _ptr(status), _stream(stream)))
    return pool


def resident_workspace_bytes(n_layers: int, B: int, n_cols: int, kmax: int) -> int:
    n = load().idx_resident_workspace_bytes(n_layers, B, n_cols, kmax)
    if n == ctypes.c_size_t(-1).value:
        raise IdxError(IDX_E_ARG, "invalid workspace request")
    return int(n)


def idx_resident_workspace_bytes(n_layers: int, B: int, n_cols: int, kmax: int) -> int:
    return resident_workspace_bytes(n_layers, B, n_cols, kmax)


def idx_select_resident(qs, ws, keys_list, n_cols: int, kmax: int, ensemble: int = ENSEMBLE_MAX,
                        threshold: float = 0.5, n_sink: int = 1, n_recent: int = 1, out_pages=None,
                        out_count=None, workspace=None, stream=None):
    """Level-1 resident pages [B, kmax] (int32, ascending, -1 padded) and
    their count [B] from per-layer q, w and Keys (lists of equal length)."""
    L = len(qs)
    if not (len(ws) == len(keys_list) == L) or L < 1 or L > MAX_LAYERS:
        raise ValueError(f"need 1..{MAX_LAYERS} layers with one q, w and Keys each")
    pairs = [_qw(q, w) for q, w in zip(qs, ws)]
    B, H, D = pairs[0][0].shape
    if any(q.shape != (B, H, D) for q, _ in pairs):
        raise ValueError("every layer's q must have the same shape")
    dev = pairs[0][0].device
    if out_pages is None:
        out_pages = torch.empty((B, kmax), dtype=torch.int32, device=dev)
    if out_count is None:
        out_count = torch.empty(B, dtype=torch.int32, device=dev)
    _dev(out_pages, torch.int32, "out_pages")
    _dev(out_count, torch.int32, "out_count")
    need = resident_workspace_bytes(L, B, n_cols, kmax)
    if workspace is None:
        workspace = _workspace(need, dev)
    qa = (ctypes.c_void_p * L)(*[q.data_ptr() for q, _ in pairs])
    wa = (ctypes.c_void_p * L)(*[w.data_ptr() for _, w in pairs])
    ka = (IdxKeys * L)(*[k.struct(B) for k in keys_list])
    cfg = ResidentCfg(ensemble, threshold, n_sink, n_recent, kmax)
    _check(load().idx_select_resident(L, qa, wa, B, H, D, ka, n_cols, ctypes.byref(cfg), _ptr(out_pages),
                                      _ptr(out_count), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out_pages, out_count


# ---------------------------------------------------------------------------
# host workload -> device tensors

@dataclass
class DeviceInputs:
    q: torch.Tensor
    w: torch.Tensor
    keys: Keys
    n_cols: int
    k: int


def to_device(wl, device="cuda", status: bool = False) -> DeviceInputs:
    """Copy a host workload (numpy arrays) to device tensors."""
    def t(a, dtype=None):
        if a is None:
            return None
        x = torch.from_numpy(np.ascontiguousarray(a))
        if dtype is not None:
            x = x.view(dtype)
        return x.to(device)
    q = t(wl.q.view(np.int16)).view(torch.bfloat16)
    keys = Keys(pool=t(wl.pool), limits=t(wl.limits), block_table=t(wl.block_table),
                q_req=t(wl.q_req), chunk_ids=t(wl.chunk_ids), n_chunks=t(wl.n_chunks),
                status=torch.zeros(1, dtype=torch.int32, device=device) if status else None,
                block_size=wl.block_size)
    return DeviceInputs(q=q, w=t(wl.w), keys=keys, n_cols=wl.n_cols, k=wl.k)
