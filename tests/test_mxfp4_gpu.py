"""GPU parity of the MXFP4 variant (idx_score_mxfp4 / idx_score_topk_mxfp4)
against the oracle's MXFP4 scoring, through the C ABI.

Query heads and keys are rounded to MXFP4 blocks of 32 inside the score
kernel; the rounding is decided in exact arithmetic on both sides (bf16 and
e4m3 values divided by a power of two), so the e2m1 codes agree and only the
fp32 accumulation differs: logits must be within |g - o| <= 1e-4 + 2e-3 |o|
of the oracle's MXFP4 logits, top-k exact on the GPU's own logits and
near-tie-exact against the oracle's.
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from sparse_attention_kv_paged_amd import lib as L
from sparse_attention_kv_paged_amd import workloads as W
from tests.parity import assert_logits_close, assert_topk_near_tie, column_order

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def _log(msg):
    print(msg, flush=True)


def _check_mx(wl, rows=None, tag=""):
    _log(f"[mxfp4] {tag} {wl.name}: {wl.description} rows={'all' if rows is None else len(rows)}")
    d = L.to_device(wl)
    lg, sc = L.idx_score_mxfp4(d.q, d.w, d.keys, d.n_cols, with_scores=True)
    lg_only = L.idx_score_mxfp4(d.q, d.w, d.keys, d.n_cols)
    g_idx, g_val = L.idx_score_topk_mxfp4(d.q, d.w, d.keys, d.n_cols, wl.k)
    torch.cuda.synchronize()
    g_logits, g_scores = lg.cpu().numpy(), sc.cpu().numpy()
    assert np.array_equal(lg_only.cpu().numpy(), g_logits), f"{tag}: logits-only launch differs"
    sel = slice(None) if rows is None else np.asarray(rows)
    ref = oracle.score(wl, rows=rows, mxfp4=True)
    assert_logits_close(g_logits[sel], ref, f"{tag} mxfp4 logits")
    ref_sc = oracle.sigmoid(ref)
    err = np.abs(g_scores[sel] - ref_sc)
    assert np.all(err <= 1e-4 + 2e-3 * ref_sc), f"{tag} mxfp4 scores: worst {err.max():.3e}"
    g_idx, g_val = g_idx.cpu().numpy(), g_val.cpu().numpy()
    own_cols, own_vals = column_order(*oracle.topk(g_logits.astype(np.float64), wl.k))
    own_ids = oracle.cols_to_entries(wl, own_cols)
    assert np.array_equal(g_idx, own_ids), f"{tag}: mxfp4 score_topk != top-k of its own logits"
    ok = own_cols >= 0
    assert np.array_equal(g_val[ok], own_vals[ok].astype(np.float32))
    ref_cols, _ = oracle.topk(ref, wl.k)
    ref_ids = oracle.cols_to_entries(wl, ref_cols, rows=rows)

    def logit_of(b, ids):
        ids = np.asarray(ids, dtype=np.int64)
        if wl.chunk_ids is None:
            return ref[b, ids]
        row = b if rows is None else rows[b]
        bs = wl.block_size
        pos = {int(c): j for j, c in enumerate(wl.chunk_ids[row][:wl.n_chunks[row]])}
        return ref[b, np.array([pos[int(e) // bs] * bs + int(e) % bs for e in ids], dtype=np.int64)]
    assert_topk_near_tie(g_idx[sel], ref_ids, logit_of, wl.k, f"{tag} mxfp4")
    return g_logits


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_mxfp4_small_workloads(cfg):
    _check_mx(W.small_config(cfg), tag=f"small{cfg}")


def test_mxfp4_full_size_decode_batch():
    """The flattened split at full size: rows staged per workgroup and rows
    that waves start outside their workgroup's staged rows."""
    _check_mx(W.config(1), tag="full1")


def test_mxfp4_full_size_resident_subset():
    _check_mx(W.config(4), tag="full4")


def test_mxfp4_full_size_prefill_sampled_rows():
    """Chunked prefill at full size (per-row path), 64 rows against the oracle
    (the first and last, block-boundary rows and random ones)."""
    wl = W.config(3)
    rng = np.random.default_rng(71)
    rows = sorted(set([0, 1, 63, 64, 255, 256, 4095] + list(rng.choice(4096, 57, replace=False))))
    _check_mx(wl, rows=rows, tag="full3")


def test_mxfp4_full_size_prefill_all_rows():
    """Chunked prefill at full size: every one of the 4096 rows' logits,
    scores and top-512 against the oracle's MXFP4 scoring."""
    _check_mx(W.config(3), tag="full3-all")


def test_mxfp4_per_row_path_and_16_row_blocks():
    _check_mx(W.prefill(8192, 603, seed=72, name="mx-rows"), tag="per-row")
    _check_mx(W.reblock(W.small_config(4), seed=73), tag="b16-chunks")


def test_mxfp4_zero_tiny_and_huge_heads_negative_scales_padding():
    """Zero heads, heads of bf16 values below 2^-124 (block exponent clamped
    to -127), a head scaled by 2^100, keys with negative and zero scales, an
    absent block and a padding row."""
    wl = W.paged_decode([700, 64, 1, 129, 2048], seed=74, max_blocks=40, k=64, name="mx-edge")
    q = wl.q.copy().view(np.uint16)
    rng = np.random.default_rng(75)
    q[0, 3:9] = 0
    q[1, 10:14] = W.bf16_bits((rng.standard_normal((4, 128)) * 2.0 ** -128).astype(np.float32))
    q[1, 20] = W.bf16_bits((rng.standard_normal(128) * 2.0 ** -124).astype(np.float32))
    q[2, 30:33] = W.bf16_bits((rng.standard_normal((3, 128)) * 2.0 ** 100).astype(np.float32))
    wl.q = q
    sc = wl.pool[:, 128:].copy().view("<f4")
    sc[rng.random(len(sc)) < 0.3] *= -1
    sc[rng.random(len(sc)) < 0.05] = 0.0
    wl.pool = wl.pool.copy()
    wl.pool[:, 128:] = sc.view(np.uint8)
    wl.block_table = wl.block_table.copy()
    wl.block_table[4, 3] = -1
    wl.q_req = np.arange(wl.B, dtype=np.int32)
    wl.q_req[3] = -1
    _check_mx(wl, tag="edge")


def test_mxfp4_keys_rounded_ahead_edge_cases():
    """Many rows of one request (the per-row split) take keys rounded once
    ahead of the score launch in idx_score_topk_mxfp4, while idx_score_mxfp4
    rounds them in the tile loop: the two must agree bit for bit (the check
    compares score_topk with the top-k of the score-only logits) and with the
    oracle, here with negative and zero key scales, absent and out-of-range
    block ids, padding rows and a zero bound."""
    wl = W.prefill(8192, 600, seed=76, k=64, name="mx-ahead-edge")
    rng = np.random.default_rng(77)
    sc = wl.pool[:, 128:].copy().view("<f4")
    sc[rng.random(len(sc)) < 0.3] *= -1
    sc[rng.random(len(sc)) < 0.05] = 0.0
    wl.pool = wl.pool.copy()
    wl.pool[:, 128:] = sc.view(np.uint8)
    wl.block_table = wl.block_table.copy()
    wl.block_table[0, 3] = -1
    wl.block_table[0, 7] = 1 << 20                            # past the pool: absent, flagged
    wl.q_req = wl.q_req.copy()
    wl.q_req[[5, 300]] = -1
    wl.limits = wl.limits.copy()
    wl.limits[11] = 0
    _check_mx(wl, tag="ahead-edge")


def _grid_values(rng, shape, e):
    g = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])[rng.integers(0, 8, size=shape)]
    g = g * np.where(rng.random(shape) < 0.5, -1.0, 1.0)
    blocks = g.reshape(-1, 32)
    blocks[np.arange(len(blocks)), rng.integers(0, 32, size=len(blocks))] = 6.0
    return blocks.reshape(shape) * 2.0 ** e


@pytest.mark.parametrize("seed", [0, 1])
def test_mxfp4_grid_case_matches_the_plain_path(seed):
    """Query and key values already on MXFP4 grids with block scale 1 and
    power-of-two weights and row scales: rounding changes nothing, so the
    MXFP4 logits equal the oracle's plain logits (bit for bit on the oracle
    side).  Every product, dot product and partial head sum is a multiple of
    1/4 below 2^22 (dots below 4608, weights 1, 2 or 4, row scales 1 or 2),
    so exact in binary32: the GPU's logits must be exact as well."""
    rng = np.random.default_rng(100 + seed)
    wl = W.small_config(1, seed=seed)
    wl.q = W.bf16_bits(_grid_values(rng, wl.q.shape, 0).astype(np.float32))
    wl.w = (2.0 ** rng.integers(0, 3, size=wl.w.shape)).astype(np.float32)
    n = wl.pool.shape[0]
    vals = _grid_values(rng, (n, wl.D), 0)
    codes = np.array([oracle.e4m3_encode(float(x)) for x in vals.reshape(-1)], np.uint8).reshape(n, wl.D)
    wl.pool = wl.pool.copy()
    wl.pool[:, :wl.D] = codes
    wl.pool[:, wl.D:] = (2.0 ** rng.integers(0, 2, size=(n, 1))).astype("<f4").view(np.uint8)
    ref = oracle.score(wl, mxfp4=True)
    assert np.array_equal(ref, oracle.score(wl))
    d = L.to_device(wl)
    g = L.idx_score_mxfp4(d.q, d.w, d.keys, d.n_cols).cpu().numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(g == -np.inf, ~fin)
    assert np.array_equal(g[fin].astype(np.float64), ref[fin])
