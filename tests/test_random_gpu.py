"""Randomised GPU parity (through the C ABI) against the oracle.

Each seed draws one configuration: paged rows of ragged lengths (empty rows
included), a contiguous pool with per-row bounds, resident chunk lists, or
more than 512 rows (the per-row path); k from 1 to 2048; 64-row or 16-row
pool blocks; negative and zero key scales; padding rows; 64 or 128 heads;
and one of the three query paths (bf16, the query quantised to e4m3 inside
the score kernel, MXFP4).  Logits must be within |g - o| <= 1e-4 + 2e-3 |o| of
the oracle's (exactly -inf where unscored), score_topk must equal the top-k
of the GPU's own logits exactly, and differ from the oracle's only at
near-ties.  The draws are seeded, so every case is reproducible.
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


def _case(seed):
    rng = np.random.default_rng(5000 + seed)
    kind = int(rng.integers(0, 4))
    k = int(rng.choice([1, 7, 64, 300, 512, 513, 2048]))
    path = str(rng.choice(["bf16", "fp8q", "mxfp4"]))
    H = 128 if path == "bf16" and rng.random() < 0.2 else 64
    if kind == 0:
        B = int(rng.integers(1, 40))
        entries = rng.integers(0, 6000, size=B)
        entries[rng.random(B) < 0.1] = 0
        entries[0] = max(int(entries[0]), 1)
        mb = -(-int(entries.max()) // 64) + int(rng.integers(0, 3))
        wl = W.paged_decode(entries, seed=seed, k=k, max_blocks=mb, H=H, name=f"random{seed}-paged")
    elif kind == 1:
        n = int(rng.integers(1, 5000))
        B = int(rng.integers(1, 8))
        wl = W.contiguous(n, B=B, seed=seed, k=k, H=H, name=f"random{seed}-contiguous")
        wl.limits = rng.integers(0, n + 1, size=B).astype(np.int32)
    elif kind == 2:
        B = int(rng.integers(1, 30))
        cpr = int(rng.integers(64, 512))
        wl = W.resident(B=B, chunks_per_req=cpr, n_resident=int(rng.integers(1, 40)), seed=seed, k=k, H=H,
                        name=f"random{seed}-resident")
    else:
        B = int(rng.integers(513, 700))
        entries = rng.integers(0, 1500, size=B)
        entries[0] = max(int(entries[0]), 1)
        wl = W.paged_decode(entries, seed=seed, k=k, H=H, name=f"random{seed}-rows")
    if wl.block_table is not None and rng.random() < 0.3:
        wl = W.reblock(wl, seed=seed)
    if rng.random() < 0.5:
        sc = wl.pool[:, -4:].copy().view("<f4")
        sc[rng.random(len(sc)) < 0.2] *= -1
        sc[rng.random(len(sc)) < 0.05] = 0.0
        wl.pool = wl.pool.copy()
        wl.pool[:, -4:] = sc.view(np.uint8)
    if rng.random() < 0.3 and wl.B > 1:
        wl.q_req = (np.arange(wl.B, dtype=np.int32) if wl.q_req is None else wl.q_req.copy())
        wl.q_req[rng.integers(0, wl.B)] = -1
    return wl, path


@pytest.mark.parametrize("seed", range(48))
def test_random_configuration(seed):
    wl, path = _case(seed)
    print(f"[random] seed {seed}: {wl.name} {wl.description} H={wl.H} k={wl.k} block={wl.block_size} "
          f"path={path}", flush=True)
    d = L.to_device(wl)
    if path == "bf16":
        lg = L.idx_score(d.q, d.w, d.keys, d.n_cols)
        idx, val = L.idx_score_topk(d.q, d.w, d.keys, d.n_cols, wl.k)
        ref = oracle.score(wl)
    elif path == "fp8q":
        lg = L.idx_score_fp8q(d.q, d.w, d.keys, d.n_cols)
        idx, val = L.idx_score_topk_fp8q(d.q, d.w, d.keys, d.n_cols, wl.k)
        ref = oracle.score(wl, q8=oracle.quantize_q(wl.q))
    else:
        lg = L.idx_score_mxfp4(d.q, d.w, d.keys, d.n_cols)
        idx, val = L.idx_score_topk_mxfp4(d.q, d.w, d.keys, d.n_cols, wl.k)
        ref = oracle.score(wl, mxfp4=True)
    torch.cuda.synchronize()
    g = lg.cpu().numpy()
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    assert_logits_close(g, ref, f"random {seed} {path}")
    own_cols, own_vals = column_order(*oracle.topk(g.astype(np.float64), wl.k))
    assert np.array_equal(idx, oracle.cols_to_entries(wl, own_cols)), f"seed {seed}: top-k != top-k of own logits"
    ok = own_cols >= 0
    assert np.array_equal(val[ok], own_vals[ok].astype(np.float32))
    ref_cols, _ = oracle.topk(ref, wl.k)
    ref_ids = oracle.cols_to_entries(wl, ref_cols)

    def logit_of(b, ids):
        ids = np.asarray(ids, dtype=np.int64)
        if wl.chunk_ids is None:
            return ref[b, ids]
        bs = wl.block_size
        pos = {int(c): j for j, c in enumerate(wl.chunk_ids[b][:wl.n_chunks[b]])}
        return ref[b, np.array([pos[int(e) // bs] * bs + int(e) % bs for e in ids], dtype=np.int64)]
    assert_topk_near_tie(idx, ref_ids, logit_of, wl.k, f"random {seed} {path}")


@pytest.mark.parametrize("seed", range(12))
def test_random_shared_request_rows(seed):
    """Many query rows of one request (chunked prefill: the per-row split, and
    for MXFP4 the request's keys rounded once per call) with a random prefix,
    row count, k, path and masked table entries."""
    rng = np.random.default_rng(9000 + seed)
    prefix = int(rng.integers(1, 40)) * 1024
    rows = int(rng.integers(513, 700))
    k = int(rng.choice([7, 64, 512, 1000]))
    path = str(rng.choice(["bf16", "fp8q", "mxfp4"]))
    wl = W.prefill(prefix, rows, seed=9000 + seed, k=k, name=f"random{seed}-shared")
    if rng.random() < 0.5:
        wl.block_table = wl.block_table.copy()
        wl.block_table[0, rng.integers(0, wl.block_table.shape[1])] = -1
    if rng.random() < 0.5:
        sc = wl.pool[:, -4:].copy().view("<f4")
        sc[rng.random(len(sc)) < 0.2] *= -1
        wl.pool = wl.pool.copy()
        wl.pool[:, -4:] = sc.view(np.uint8)
    print(f"[random] shared {seed}: {wl.description} rows={rows} k={k} path={path}", flush=True)
    d = L.to_device(wl)
    if path == "bf16":
        lg = L.idx_score(d.q, d.w, d.keys, d.n_cols)
        idx, val = L.idx_score_topk(d.q, d.w, d.keys, d.n_cols, wl.k)
        ref = oracle.score(wl)
    elif path == "fp8q":
        lg = L.idx_score_fp8q(d.q, d.w, d.keys, d.n_cols)
        idx, val = L.idx_score_topk_fp8q(d.q, d.w, d.keys, d.n_cols, wl.k)
        ref = oracle.score(wl, q8=oracle.quantize_q(wl.q))
    else:
        lg = L.idx_score_mxfp4(d.q, d.w, d.keys, d.n_cols)
        idx, val = L.idx_score_topk_mxfp4(d.q, d.w, d.keys, d.n_cols, wl.k)
        ref = oracle.score(wl, mxfp4=True)
    torch.cuda.synchronize()
    g = lg.cpu().numpy()
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    assert_logits_close(g, ref, f"shared {seed} {path}")
    own_cols, own_vals = column_order(*oracle.topk(g.astype(np.float64), wl.k))
    assert np.array_equal(idx, oracle.cols_to_entries(wl, own_cols)), f"seed {seed}: top-k != top-k of own logits"
    ok = own_cols >= 0
    assert np.array_equal(val[ok], own_vals[ok].astype(np.float32))
    ref_ids = oracle.cols_to_entries(wl, oracle.topk(ref, wl.k)[0])
    assert_topk_near_tie(idx, ref_ids, lambda b, ids: ref[b, np.asarray(ids, dtype=np.int64)], wl.k,
                         f"shared {seed} {path}")


@pytest.mark.parametrize("seed", range(16))
def test_random_long_segment_topk(seed):
    """Standalone top-k over many rows of one long segment each -- the
    sampled-threshold path and its re-run -- with a random row length
    (every segment size), k up to 640 and a random value distribution per
    row: normal, exponential, uniform, heavy ties, a shift on the sampled
    columns (thread t's first column) up or down, rows shorter than k, and
    NaN / +-inf sprinkled in.  The result must equal the oracle's top-k
    exactly (columns and values)."""
    rng = np.random.default_rng(11000 + seed)
    n = int(rng.choice([6000, 8192, 12000, 16384, 17408, 20480, 24000, 30000]))
    k = int(rng.choice([1, 7, 64, 300, 512, 640]))
    B = 256
    per = {8192: 16, 16384: 32, 20480: 40, 24576: 48}.get(next(c for c in (8192, 16384, 20480, 24576, 32768) if n <= c), 32)
    vals = np.empty((B, n), np.float32)
    kinds = rng.integers(0, 8, size=B)
    for r in range(B):
        kind = int(kinds[r])
        if kind == 0:
            v = rng.standard_normal(n) * rng.uniform(0.1, 10)
        elif kind == 1:
            v = rng.exponential(size=n)
        elif kind == 2:
            v = rng.random(n)
        elif kind == 3:
            v = np.round(rng.standard_normal(n) * 2) / 2            # heavy ties
        elif kind == 4:
            v = rng.standard_normal(n)
            v[::per] += rng.choice([-1000.0, 1000.0])                 # the samples mislead
        elif kind == 5:
            v = np.full(n, -np.inf)
            m = int(rng.integers(0, 2 * k + 2))
            v[rng.choice(n, min(m, n), replace=False)] = rng.standard_normal(min(m, n))   # short rows
        elif kind == 6:
            v = rng.standard_normal(n)
            v[rng.random(n) < 0.02] = np.nan
            v[rng.random(n) < 0.01] = np.inf
            v[rng.random(n) < 0.2] = -np.inf
        else:
            v = np.full(n, float(rng.standard_normal()))              # one value
        vals[r] = v.astype(np.float32)
    print(f"[random] long segments {seed}: n={n} k={k} kinds={np.bincount(kinds, minlength=8).tolist()}", flush=True)
    cols, v = L.idx_topk(torch.from_numpy(vals).cuda(), k)
    torch.cuda.synchronize()
    ref_cols, ref_v = column_order(*oracle.topk(vals.astype(np.float64), k))
    got = cols.cpu().numpy()
    bad = np.nonzero((got != ref_cols).any(axis=1))[0]
    assert bad.size == 0, f"seed {seed}: rows {bad[:8].tolist()} (kinds {kinds[bad[:8]].tolist()}) differ"
    ok = ref_cols >= 0
    assert np.array_equal(v.cpu().numpy()[ok], ref_v[ok].astype(np.float32))
