"""C-ABI checks that need no GPU: the library loads, exports every function
include/idx.h declares, and rejects bad host-side arguments before launching
anything (so these calls never touch a device)."""
import ctypes
import os
import re

import pytest

from sparse_attention_kv_paged_amd import lib as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "idx.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(idx_[a-z_0-9]+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return L.load()


def test_header_declares_the_entry_points():
    assert _declared_functions() == sorted(L.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_error_strings(lib):
    assert lib.idx_abi_version() == 1
    assert lib.idx_error_string(0) == b"ok"
    for code in range(1, 6):
        assert lib.idx_error_string(code) not in (b"ok", b"unknown error")
    assert lib.idx_error_string(99) == b"unknown error"


def test_keys_struct_layout_matches_header():
    # pointer/int64 fields are 8-byte aligned; the struct is 80 bytes on x86-64
    assert ctypes.sizeof(L.IdxKeys) == 80
    assert L.IdxKeys.block_table.offset == 24 and L.IdxKeys.status.offset == 72


def test_workspace_bytes(lib):
    assert L.workspace_bytes(L.IDX_OP_SCORE, 4, 1000, 512) == 0
    # rows that fit one top-k workgroup need no scratch of their own
    assert L.workspace_bytes(L.IDX_OP_TOPK, 4, 1000, 512) == 0
    # score_topk holds the logits (4 rows x 1024 padded columns x 4 B) and
    # per-row column counts and merge counters, each piece 256-byte aligned
    assert L.workspace_bytes(L.IDX_OP_SCORE_TOPK, 4, 1000, 512) == 4 * 1024 * 4 + 2 * 256
    # more than 512 rows (the per-row split): also room for one request's key
    # blocks rounded to MXFP4 ahead of the score launch, 4608 B per 64 columns
    assert L.workspace_bytes(L.IDX_OP_SCORE_TOPK, 600, 1000, 512) == 600 * 1024 * 4 + 2 * 2560 + 16 * 4608
    assert L.workspace_bytes(L.IDX_OP_SCORE_TOPK, 512, 1000, 512) == 512 * 1024 * 4 + 2 * 2048
    # one flag per workgroup when long segments (at least 8192 columns) select
    # through a sampled threshold first (k up to 640)
    assert L.workspace_bytes(L.IDX_OP_TOPK, 4096, 17408, 512) == 4096 * 4
    assert L.workspace_bytes(L.IDX_OP_TOPK, 4096, 17408, 640) == 4096 * 4
    assert L.workspace_bytes(L.IDX_OP_TOPK, 4096, 17408, 641) == 0
    assert L.workspace_bytes(L.IDX_OP_TOPK, 4096, 4000, 512) == 0
    # long rows: per-part (key, column) lists of k items and their counts
    parts = -(-262144 // 32768)
    need = L.workspace_bytes(L.IDX_OP_TOPK, 8, 262144, 512)
    assert need >= 8 * parts * 512 * 8 + 8 * 512 * 8
    assert lib.idx_workspace_bytes(L.IDX_OP_TOPK, 1, 10, 0) == ctypes.c_size_t(-1).value
    assert lib.idx_workspace_bytes(L.IDX_OP_TOPK, 1, 10, 2049) == ctypes.c_size_t(-1).value
    assert lib.idx_workspace_bytes(7, 1, 10, 1) == ctypes.c_size_t(-1).value


def _keys(**kw):
    k = L.IdxKeys()
    k.pool = kw.get("pool", 0x1000)
    k.n_pool_rows = kw.get("n_pool_rows", 64)
    k.block_size = kw.get("block_size", 64)
    k.limits = kw.get("limits", 0x2000)
    k.block_table = kw.get("block_table", None)
    k.n_req = kw.get("n_req", 0)
    k.max_blocks = kw.get("max_blocks", 0)
    k.chunk_ids = kw.get("chunk_ids", None)
    k.n_chunks = kw.get("n_chunks", None)
    k.max_chunks = kw.get("max_chunks", 0)
    return k


def _score(lib, q=0x1000, w=0x1000, B=1, H=64, D=128, keys=None, n_cols=64, logits=0x3000):
    keys = _keys() if keys is None else keys
    return lib.idx_score(q, w, B, H, D, ctypes.byref(keys), n_cols, logits, None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(H=32), L.IDX_E_SHAPE),
    (dict(D=64), L.IDX_E_SHAPE),
    (dict(B=-1), L.IDX_E_ARG),
    (dict(n_cols=0), L.IDX_E_SHAPE),
    (dict(n_cols=L.MAX_COLS + 1), L.IDX_E_SHAPE),
    (dict(n_cols=-5), L.IDX_E_SHAPE),
    (dict(q=None), L.IDX_E_ARG),
    (dict(q=0x1004), L.IDX_E_ALIGN),
    (dict(w=0x1008), L.IDX_E_ALIGN),
    (dict(logits=None), L.IDX_E_ARG),
    (dict(logits=0x3004), L.IDX_E_ALIGN),
    (dict(keys=_keys(block_size=32)), L.IDX_E_SHAPE),
    (dict(keys=_keys(block_size=0)), L.IDX_E_SHAPE),
    (dict(keys=_keys(block_size=16, block_table=0x4000, n_req=1, max_blocks=4, n_pool_rows=40)), L.IDX_E_SHAPE),
    (dict(keys=_keys(pool=0x1001)), L.IDX_E_ALIGN),
    (dict(keys=_keys(limits=None)), L.IDX_E_ARG),
    (dict(keys=_keys(block_table=0x4000, n_req=0, max_blocks=4)), L.IDX_E_SHAPE),
    (dict(keys=_keys(block_table=0x4000, n_req=1, max_blocks=4, n_pool_rows=100)), L.IDX_E_SHAPE),
    (dict(keys=_keys(chunk_ids=0x5000, max_chunks=4)), L.IDX_E_ARG),
    (dict(keys=_keys(chunk_ids=0x5000, n_chunks=0x6000, max_chunks=0)), L.IDX_E_SHAPE),
])
def test_score_rejects_bad_arguments(lib, kw, code):
    assert _score(lib, **kw) == code
    assert lib.idx_last_error() != b""


def test_score_with_no_rows_is_a_no_op(lib):
    assert _score(lib, B=0, q=None, w=None, logits=None) == L.IDX_OK


def test_topk_rejects_bad_arguments(lib):
    need = L.workspace_bytes(L.IDX_OP_TOPK, 2, 100, 8)
    ok = dict(logits=0x1000, B=2, n_cols=100, ld=100, k=8, out_col=0x2000, out_val=None,
              ws=0x10000, ws_bytes=need)

    def call(**kw):
        a = {**ok, **kw}
        return lib.idx_topk(a["logits"], a["B"], a["n_cols"], a["ld"], a["k"], a["out_col"],
                            a["out_val"], a["ws"], a["ws_bytes"], None)
    assert call(k=0) == L.IDX_E_SHAPE
    assert call(k=2049) == L.IDX_E_SHAPE
    assert call(ld=99) == L.IDX_E_SHAPE
    assert call(n_cols=0) == L.IDX_E_SHAPE
    assert need == 0
    need = L.workspace_bytes(L.IDX_OP_TOPK, 2, 100000, 8)
    ok.update(n_cols=100000, ld=100000, ws_bytes=need)
    assert call(ws_bytes=need - 1) == L.IDX_E_WORKSPACE
    assert call(ws=None) == L.IDX_E_WORKSPACE
    assert call(ws=0x10010) == L.IDX_E_ALIGN
    assert call(out_col=None) == L.IDX_E_ARG
    assert call(B=0) == L.IDX_OK


def test_score_topk_rejects_small_workspace(lib):
    keys = _keys()
    need = L.workspace_bytes(L.IDX_OP_SCORE_TOPK, 1, 64, 16)
    rc = lib.idx_score_topk(0x1000, 0x1000, 1, 64, 128, ctypes.byref(keys), 64, 16, 0x2000, None,
                            0x10000, need - 256, None)
    assert rc == L.IDX_E_WORKSPACE
    rc = lib.idx_score_topk(0x1000, 0x1000, 1, 64, 128, ctypes.byref(keys), 64, 4096, 0x2000, None,
                            0x10000, need, None)
    assert rc == L.IDX_E_SHAPE


@pytest.mark.parametrize("kw,code", [
    (dict(D=64), L.IDX_E_SHAPE),
    (dict(n=-1), L.IDX_E_ARG),
    (dict(n_pool_rows=-1), L.IDX_E_ARG),
    (dict(k=None), L.IDX_E_ARG),
    (dict(slots=None), L.IDX_E_ARG),
    (dict(pool=None), L.IDX_E_ARG),
    (dict(k=0x1008), L.IDX_E_ALIGN),
    (dict(slots=0x2004), L.IDX_E_ALIGN),
    (dict(pool=0x3002), L.IDX_E_ALIGN),
    (dict(status=0x4001), L.IDX_E_ALIGN),
    (dict(n=(1 << 31) * 16), L.IDX_E_SHAPE),
])
def test_write_keys_rejects_bad_arguments(lib, kw, code):
    a = dict(k=0x1000, n=10, D=128, slots=0x2000, pool=0x3000, n_pool_rows=64, status=None)
    a.update(kw)
    rc = lib.idx_write_keys(a["k"], a["n"], a["D"], a["slots"], a["pool"], a["n_pool_rows"],
                            a["status"], None)
    assert rc == code
    assert lib.idx_last_error() != b""


def test_write_keys_with_no_keys_is_a_no_op(lib):
    assert lib.idx_write_keys(None, 0, 128, None, None, 0, None, None) == L.IDX_OK


def _resident(lib, n_layers=3, B=2, n_cols=640, cfg=None, out_pages=0x7000, ws=0x10000, ws_bytes=None,
              keys=None, q=0x1000):
    cfg = cfg or L.ResidentCfg(L.ENSEMBLE_MAX, 0.7, 1, 1, 8)
    need = L.resident_workspace_bytes(max(n_layers, 1), max(B, 0), max(n_cols, 1), max(cfg.kmax, 1)) \
        if 1 <= n_layers <= L.MAX_LAYERS and 1 <= cfg.kmax <= 2048 and n_cols >= 1 else 0
    ws_bytes = need if ws_bytes is None else ws_bytes
    n = max(n_layers, 1)
    qa = (ctypes.c_void_p * n)(*([q] * n))
    wa = (ctypes.c_void_p * n)(*([0x2000] * n))
    ka = (L.IdxKeys * n)(*([keys or _keys()] * n))
    return lib.idx_select_resident(n_layers, qa, wa, B, 64, 128, ka, n_cols, ctypes.byref(cfg), out_pages,
                                   None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n_layers=0), L.IDX_E_SHAPE),
    (dict(n_layers=9), L.IDX_E_SHAPE),
    (dict(n_cols=0), L.IDX_E_SHAPE),
    (dict(cfg=L.ResidentCfg(7, 0.7, 1, 1, 8)), L.IDX_E_ARG),
    (dict(cfg=L.ResidentCfg(0, float("nan"), 1, 1, 8)), L.IDX_E_ARG),
    (dict(cfg=L.ResidentCfg(0, 0.7, 1, 1, 0)), L.IDX_E_SHAPE),
    (dict(cfg=L.ResidentCfg(0, 0.7, 1, 1, 2049)), L.IDX_E_SHAPE),
    (dict(cfg=L.ResidentCfg(0, 0.7, 5, 4, 8)), L.IDX_E_SHAPE),
    (dict(cfg=L.ResidentCfg(0, 0.7, -1, 0, 8)), L.IDX_E_SHAPE),
    (dict(q=0x1008), L.IDX_E_ALIGN),
    (dict(keys=_keys(chunk_ids=0x5000, n_chunks=0x6000, max_chunks=4)), L.IDX_E_ARG),
    (dict(out_pages=None), L.IDX_E_ARG),
    (dict(ws_bytes=256), L.IDX_E_WORKSPACE),
    (dict(ws=0x10010), L.IDX_E_ALIGN),
])
def test_select_resident_rejects_bad_arguments(lib, kw, code):
    assert _resident(lib, **kw) == code
    assert lib.idx_last_error() != b""


def test_resident_workspace_bytes(lib):
    # logits [B, ld] + scores [L, B, ld] + page keys [B, ldp] (ld = n_cols rounded to 64,
    # ldp = pages rounded to 64), each piece 256-byte aligned, no top-k lists for short rows
    n = L.resident_workspace_bytes(3, 2, 640, 8)
    assert n == 2 * 640 * 4 + 3 * 2 * 640 * 4 + 2 * 64 * 4 + 256
    assert lib.idx_resident_workspace_bytes(0, 2, 640, 8) == ctypes.c_size_t(-1).value
    assert lib.idx_resident_workspace_bytes(3, 2, 640, 0) == ctypes.c_size_t(-1).value
    assert _resident(lib, B=0, out_pages=None) == L.IDX_OK


@pytest.mark.parametrize("kw,code", [
    (dict(H=32), L.IDX_E_SHAPE),
    (dict(D=64), L.IDX_E_SHAPE),
    (dict(B=-1), L.IDX_E_ARG),
    (dict(q8=None), L.IDX_E_ARG),
    (dict(w=None), L.IDX_E_ARG),
    (dict(q8=0x1002), L.IDX_E_ALIGN),
    (dict(w=0x2004), L.IDX_E_ALIGN),
    (dict(n_cols=0), L.IDX_E_SHAPE),
    (dict(logits=None), L.IDX_E_ARG),
])
def test_score_q8_rejects_bad_arguments(lib, kw, code):
    a = dict(q8=0x1004, w=0x2000, B=1, H=64, D=128, n_cols=64, logits=0x3000)   # q8 needs only 4-byte alignment
    a.update(kw)
    keys = _keys()
    rc = lib.idx_score_q8(a["q8"], a["w"], a["B"], a["H"], a["D"], ctypes.byref(keys), a["n_cols"], a["logits"],
                          None, None)
    assert rc == code
    assert lib.idx_last_error() != b""


def test_score_topk_q8_rejects_bad_arguments_and_accepts_empty(lib):
    keys = _keys()
    need = L.workspace_bytes(L.IDX_OP_SCORE_TOPK, 1, 64, 16)
    assert lib.idx_score_topk_q8(0x1004, 0x2000, 1, 64, 128, ctypes.byref(keys), 64, 4096, 0x3000, None,
                                 0x10000, need, None) == L.IDX_E_SHAPE
    assert lib.idx_score_topk_q8(0x1004, 0x2000, 1, 64, 128, ctypes.byref(keys), 64, 16, 0x3000, None,
                                 0x10000, need - 256, None) == L.IDX_E_WORKSPACE
    assert lib.idx_score_topk_q8(None, None, 0, 64, 128, ctypes.byref(keys), 64, 16, None, None,
                                 None, 0, None) == L.IDX_OK


def test_h128_accepted_for_bf16_rejected_for_q8(lib):
    keys = _keys()
    # 96 heads: rejected on every path; 128: rejected for the quantised query only
    assert _score(lib, H=96) == L.IDX_E_SHAPE
    assert lib.idx_score_q8(0x1004, 0x2000, 1, 128, 128, ctypes.byref(keys), 64, 0x3000, None, None) == L.IDX_E_SHAPE
    # 128 heads pass every host check (B = 0 returns before any launch)
    assert _score(lib, H=128, B=0, q=None, w=None, logits=None) == L.IDX_OK
    # the query quantised in the kernel: bf16 q as for idx_score, 64 heads
    assert lib.idx_score_fp8q(0x1000, 0x2000, 1, 128, 128, ctypes.byref(keys), 64, 0x3000, None, None) == L.IDX_E_SHAPE
    assert lib.idx_score_fp8q(0x1004, 0x2000, 1, 64, 128, ctypes.byref(keys), 64, 0x3000, None, None) == L.IDX_E_ALIGN
    assert lib.idx_score_fp8q(None, None, 1, 64, 128, ctypes.byref(keys), 64, 0x3000, None, None) == L.IDX_E_ARG
    assert lib.idx_score_fp8q(None, None, 0, 64, 128, ctypes.byref(keys), 64, None, None, None) == L.IDX_OK
    need = L.workspace_bytes(L.IDX_OP_SCORE_TOPK, 1, 64, 16)
    assert lib.idx_score_topk_fp8q(0x1000, 0x2000, 1, 128, 128, ctypes.byref(keys), 64, 16, 0x3000, None,
                                   0x10000, need, None) == L.IDX_E_SHAPE
    assert need > 0
    assert lib.idx_score_topk_fp8q(0x1000, 0x2000, 1, 64, 128, ctypes.byref(keys), 64, 16, 0x3000, None,
                                   0x10000, need - 1, None) == L.IDX_E_WORKSPACE


def test_column_limit(lib):
    """n_cols above IDX_MAX_COLS (2^27: column byte offsets and the work index
    stay within 32 bits) is refused by every entry point, before anything is
    launched; the limit itself is accepted by the workspace query."""
    assert L.MAX_COLS == 1 << 27
    big = L.MAX_COLS + 1
    keys = _keys()
    assert lib.idx_score_topk(0x1000, 0x1000, 1, 64, 128, ctypes.byref(keys), big, 16, 0x2000, None,
                              0x10000, 1 << 40, None) == L.IDX_E_SHAPE
    assert lib.idx_score_q8(0x1000, 0x1000, 1, 64, 128, ctypes.byref(keys), big, 0x3000, None, None) == L.IDX_E_SHAPE
    assert lib.idx_topk(0x1000, 1, big, big, 16, 0x2000, None, 0x10000, 1 << 40, None) == L.IDX_E_SHAPE
    assert lib.idx_workspace_bytes(L.IDX_OP_SCORE_TOPK, 1, big, 16) == ctypes.c_size_t(-1).value
    assert lib.idx_workspace_bytes(L.IDX_OP_TOPK, 1, L.MAX_COLS, 16) != ctypes.c_size_t(-1).value
    assert lib.idx_resident_workspace_bytes(1, 1, big, 16) == ctypes.c_size_t(-1).value
    qa = (ctypes.c_void_p * 1)(0x1000)
    wa = (ctypes.c_void_p * 1)(0x1000)
    ka = (L.IdxKeys * 1)(keys)
    cfg = L.ResidentCfg(0, 0.5, 0, 0, 16)
    assert lib.idx_select_resident(1, qa, wa, 1, 64, 128, ka, big, ctypes.byref(cfg), 0x2000, None,
                                   0x10000, 1 << 40, None) == L.IDX_E_SHAPE


def test_noalloc_rejects_calls_beyond_the_static_scratch(lib):
    """The allocation-free entry point refuses, before touching a device, a
    call whose workspace exceeds the static scratch (a 4096-row prefill), and
    checks its arguments like idx_score_topk."""
    assert L.STATIC_SCRATCH_BYTES == 16 << 20
    keys = _keys(n_pool_rows=64 * 272, block_table=0x4000, n_req=1, max_blocks=272)
    assert L.workspace_bytes(L.IDX_OP_SCORE_TOPK, 4096, 17408, 512) > L.STATIC_SCRATCH_BYTES
    rc = lib.idx_score_topk_noalloc(0x1000, 0x1000, 4096, 64, 128, ctypes.byref(keys), 17408, 512, 0x2000, None, None)
    assert rc == L.IDX_E_WORKSPACE and b"static scratch" in lib.idx_last_error()
    rc = lib.idx_score_topk_noalloc(0x1000, 0x1000, 1, 64, 128, ctypes.byref(_keys()), 64, 4096, 0x2000, None, None)
    assert rc == L.IDX_E_SHAPE
    rc = lib.idx_score_topk_noalloc(0x1000, 0x1000, 1, 32, 128, ctypes.byref(_keys()), 64, 16, 0x2000, None, None)
    assert rc == L.IDX_E_SHAPE
    rc = lib.idx_score_topk_noalloc(0x1000, 0x1000, 1, 64, 128, ctypes.byref(_keys()), 64, 16, None, None, None)
    assert rc == L.IDX_E_ARG
    assert lib.idx_score_topk_noalloc(None, None, 0, 64, 128, ctypes.byref(_keys()), 64, 16, None, None, None) == L.IDX_OK
    # the decode shapes fit
    for B, n in [(32, 32768), (8, 262144), (40, 24576)]:
        assert L.workspace_bytes(L.IDX_OP_SCORE_TOPK, B, n, 512) <= L.STATIC_SCRATCH_BYTES


def test_mxfp4_entry_points_reject_bad_arguments(lib):
    """The MXFP4 variant: bf16 q as for idx_score, 64 heads only."""
    keys = _keys()
    assert lib.idx_score_mxfp4(0x1000, 0x2000, 1, 128, 128, ctypes.byref(keys), 64, 0x3000, None, None) == L.IDX_E_SHAPE
    assert lib.idx_score_mxfp4(0x1000, 0x2000, 1, 64, 96, ctypes.byref(keys), 64, 0x3000, None, None) == L.IDX_E_SHAPE
    assert lib.idx_score_mxfp4(0x1004, 0x2000, 1, 64, 128, ctypes.byref(keys), 64, 0x3000, None, None) == L.IDX_E_ALIGN
    assert lib.idx_score_mxfp4(None, None, 1, 64, 128, ctypes.byref(keys), 64, 0x3000, None, None) == L.IDX_E_ARG
    assert lib.idx_score_mxfp4(None, None, 0, 64, 128, ctypes.byref(keys), 64, None, None, None) == L.IDX_OK
    assert lib.idx_score_mxfp4(0x1000, 0x2000, 1, 64, 128, ctypes.byref(keys), 0, 0x3000, None, None) == L.IDX_E_SHAPE
    need = L.workspace_bytes(L.IDX_OP_SCORE_TOPK, 1, 64, 16)
    assert lib.idx_score_topk_mxfp4(0x1000, 0x2000, 1, 128, 128, ctypes.byref(keys), 64, 16, 0x3000, None,
                                    0x10000, need, None) == L.IDX_E_SHAPE
    assert lib.idx_score_topk_mxfp4(0x1000, 0x2000, 1, 64, 128, ctypes.byref(keys), 64, 16, 0x3000, None,
                                    0x10000, need - 1, None) == L.IDX_E_WORKSPACE
    assert lib.idx_score_topk_mxfp4(0x1000, 0x2000, 1, 64, 128, ctypes.byref(keys), 64, 0, 0x3000, None,
                                    0x10000, need, None) == L.IDX_E_SHAPE
