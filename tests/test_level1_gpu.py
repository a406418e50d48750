"""GPU parity of the Level-1 resident-set selection (idx_select_resident,
through the C ABI) against the CPU oracle.

The selection is integer work decided by binary32 comparisons, so it is
checked two ways:
  * exactly, in the scorer's precision: the oracle's selection applied to the
    GPU's own binary32 per-layer scores (idx_score, the same kernel the entry
    point runs) must give the same pages and counts;
  * against the oracle's own double scores: the scores agree within the
    path's tolerance, and every page's density differs from the oracle's by
    no more than its entries whose oracle score lies within that tolerance of
    the threshold.
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from sparse_attention_kv_paged_amd import lib as L
from sparse_attention_kv_paged_amd import workloads as W
from tests.parity import ATOL, RTOL, assert_logits_close, assert_topk_near_tie

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def _log(msg):
    print(msg, flush=True)


def _device_layers(rl):
    return [L.to_device(wl) for wl in rl.layers]


def _gpu_scores(dls, n_cols):
    """Per-layer binary32 sigmoid scores [L, B, n_cols] from idx_score."""
    out = []
    for d in dls:
        _, sc = L.idx_score(d.q, d.w, d.keys, n_cols, with_scores=True)
        out.append(sc)
    torch.cuda.synchronize()
    return torch.stack(out).cpu().numpy()


def _select(rl, dls, **over):
    cfg = dict(kmax=rl.kmax, ensemble=rl.ensemble, threshold=rl.threshold, n_sink=rl.n_sink,
               n_recent=rl.n_recent)
    cfg.update(over)
    pages, count = L.idx_select_resident([d.q for d in dls], [d.w for d in dls], [d.keys for d in dls],
                                         rl.n_cols, **cfg)
    torch.cuda.synchronize()
    return pages.cpu().numpy(), count.cpu().numpy(), cfg


def _stacked(dls):
    """The layers' q and w stacked into one [L, B, H, D] / [L, B, H] tensor
    each (the layout for which one score launch covers every layer), as
    per-layer views."""
    q = torch.stack([d.q for d in dls])
    w = torch.stack([d.w for d in dls])
    return [q[l] for l in range(len(dls))], [w[l] for l in range(len(dls))]


def _select_stacked(rl, dls, **over):
    cfg = dict(kmax=rl.kmax, ensemble=rl.ensemble, threshold=rl.threshold, n_sink=rl.n_sink,
               n_recent=rl.n_recent)
    cfg.update(over)
    qs, ws = _stacked(dls)
    pages, count = L.idx_select_resident(qs, ws, [d.keys for d in dls], rl.n_cols, **cfg)
    torch.cuda.synchronize()
    return pages.cpu().numpy(), count.cpu().numpy(), cfg


def _densities(s, limits, ens, tau):
    """[B, pages] densities of per-layer scores s [L, B, n] (binary32)."""
    Ly, B, n = s.shape
    P = -(-n // 64)
    out = np.zeros((B, P), np.int64)
    for b in range(B):
        hist = int(min(max(limits[b], 0), n))
        if ens == L.ENSEMBLE_MAX:
            e = s[:, b, :hist].max(axis=0)
        else:
            e = s[0, b, :hist].copy()
            for l in range(1, Ly):
                e = (e + s[l, b, :hist]).astype(np.float32)
            e = (e / np.float32(Ly)).astype(np.float32)
        sel = (e >= np.float32(tau)).astype(np.int64)
        out[b, :-(-hist // 64)] = np.add.reduceat(sel, np.arange(0, hist, 64)) if hist else []
    return out


def _check(rl, dls, g_scores, ref_scores, **over):
    pages, count, cfg = _select(rl, dls, **over)
    want_p, want_c = oracle.level1_select(g_scores, rl.limits, cfg["ensemble"], cfg["threshold"],
                                          cfg["n_sink"], cfg["n_recent"], cfg["kmax"])
    assert np.array_equal(count, want_c), (cfg, count, want_c)
    assert np.array_equal(pages, want_p), cfg
    if ref_scores is not None:
        # densities from the oracle's double scores: differences only where an
        # entry's score is within tolerance of the threshold
        tau = cfg["threshold"]
        dg = _densities(g_scores, rl.limits, cfg["ensemble"], tau)
        do = _densities(ref_scores, rl.limits, cfg["ensemble"], tau)
        near = np.zeros_like(do)
        Ly, B, n = ref_scores.shape
        for b in range(B):
            hist = int(min(max(rl.limits[b], 0), n))
            if cfg["ensemble"] == L.ENSEMBLE_MAX:
                e = ref_scores[:, b, :hist].astype(np.float64).max(axis=0)
            else:
                e = ref_scores[:, b, :hist].astype(np.float64).mean(axis=0)
            # twice the tolerance: the ensemble's own binary32 rounding on top
            amb = (np.abs(e - tau) <= 2 * (ATOL + RTOL * abs(tau))).astype(np.int64)
            if hist:
                near[b, :-(-hist // 64)] = np.add.reduceat(amb, np.arange(0, hist, 64))
        assert np.all(np.abs(dg - do) <= near), cfg
    return pages, count


@pytest.mark.parametrize("ens", [L.ENSEMBLE_MAX, L.ENSEMBLE_MEAN])
def test_resident_selection_matches_oracle(ens):
    """Four ragged rows (a partial last page, a row shorter than one page),
    three layers: exact pages given the GPU's scores, densities consistent
    with the oracle's double scores, for several settings."""
    rl = W.memory_indexer(entries=[16384, 9001, 700, 40], n_layers=3, seed=40 + ens, kmax=32,
                          threshold=0.72, ensemble=ens, name="memory-indexer-small")
    _log(f"[level1] {rl.description}")
    dls = _device_layers(rl)
    g = _gpu_scores(dls, rl.n_cols)
    ref = oracle.level1_scores(rl.layers)
    for l in range(3):
        assert_logits_close(g[l], ref[l], f"layer {l} scores")
    for over in [dict(), dict(threshold=0.8, kmax=8), dict(threshold=0.6, n_sink=2, n_recent=3, kmax=40),
                 dict(threshold=2.0), dict(kmax=1, n_sink=1, n_recent=0), dict(kmax=2048, threshold=0.7),
                 dict(kmax=5, n_sink=0, n_recent=0, threshold=0.75)]:
        _check(rl, dls, g, ref, **over)


def test_resident_forced_pages_and_counts():
    """A threshold nothing passes leaves exactly the sink and recent pages;
    a threshold everything passes gives the first pages by density ties."""
    rl = W.memory_indexer(entries=[6400, 129, 64, 0], n_layers=2, seed=50, kmax=16, name="memory-indexer-edge")
    dls = _device_layers(rl)
    g = _gpu_scores(dls, rl.n_cols)
    pages, count = _check(rl, dls, g, None, threshold=2.0, n_sink=2, n_recent=3)
    assert count.tolist() == [5, 3, 1, 0]
    assert pages[0, :5].tolist() == [0, 1, 97, 98, 99] and (pages[0, 5:] == -1).all()
    pages, count = _check(rl, dls, g, None, threshold=0.0, n_sink=0, n_recent=0, kmax=4)
    assert pages.tolist()[0] == [0, 1, 2, 3] and count.tolist() == [4, 3, 1, 0]


def test_resident_pages_feed_level2():
    """Level 1's pages and counts, used as the chunk list of Level 2 (the
    resident-subset scoring), give the oracle's logits and top-512 for that
    chunk list."""
    rl = W.memory_indexer(entries=[32768, 20000, 12345], n_layers=3, seed=60, kmax=64, threshold=0.72,
                          name="memory-indexer-chain")
    dls = _device_layers(rl)
    pages, count, _ = _select(rl, dls)
    lvl2 = rl.layers[0]
    wl = W.Workload(name="level2-on-resident", q=lvl2.q, w=lvl2.w, pool=lvl2.pool, limits=lvl2.limits,
                    n_cols=rl.kmax * 64, k=512, block_table=lvl2.block_table, chunk_ids=pages,
                    n_chunks=count, description="Level 2 over the Level-1 pages")
    d = L.to_device(wl)
    logits = L.idx_score(d.q, d.w, d.keys, d.n_cols)
    idx, _ = L.idx_score_topk(d.q, d.w, d.keys, d.n_cols, wl.k)
    torch.cuda.synchronize()
    ref = oracle.score(wl)
    assert_logits_close(logits.cpu().numpy(), ref, "level-2 logits on resident pages")
    ref_cols, _ = oracle.topk(ref, wl.k)
    ref_ids = oracle.cols_to_entries(wl, ref_cols)

    def logit_of(b, ids):
        pos = {int(c): j for j, c in enumerate(pages[b])}
        cols = np.array([pos[int(e) // 64] * 64 + int(e) % 64 for e in ids])
        return ref[b, cols]
    assert_topk_near_tie(idx.cpu().numpy(), ref_ids, logit_of, wl.k, "level-2 top-512 on resident pages")
    # every selected entry lies in a resident page
    sel = idx.cpu().numpy()
    for b in range(wl.B):
        ok = sel[b][sel[b] >= 0] // 64
        assert set(ok.tolist()) <= set(pages[b][pages[b] >= 0].tolist())


def test_resident_full_size_sampled_rows():
    """The benchmark's shape (8 requests at 1M tokens, 3 layers, KMAX 384):
    every row's pages equal the oracle's selection on the GPU's scores; two
    rows are also checked against the oracle's own double scores."""
    rl = W.memory_indexer()
    _log(f"[level1] full size: {rl.description}")
    dls = _device_layers(rl)
    g = _gpu_scores(dls, rl.n_cols)
    pages, count, cfg = _select(rl, dls)
    want_p, want_c = oracle.level1_select(g, rl.limits, cfg["ensemble"], cfg["threshold"], cfg["n_sink"],
                                          cfg["n_recent"], cfg["kmax"])
    assert np.array_equal(count, want_c) and np.array_equal(pages, want_p)
    assert (count == rl.kmax).all()
    rows = [0, 5]
    ref = oracle.level1_scores(rl.layers, rows=rows)
    for l in range(3):
        assert_logits_close(g[l][rows], ref[l], f"full-size layer {l} scores (rows {rows})")
    tau = cfg["threshold"]
    dg = _densities(g[:, rows], rl.limits[rows], cfg["ensemble"], tau)
    do = _densities(ref, rl.limits[rows], cfg["ensemble"], tau)
    e = ref.astype(np.float64).max(axis=0)
    amb = (np.abs(e - tau) <= 2 * (ATOL + RTOL * tau)).astype(np.int64)
    near = np.add.reduceat(amb, np.arange(0, e.shape[1], 64), axis=1)
    assert np.all(np.abs(dg - do) <= near)


def test_resident_rows_beyond_the_exact_key_range():
    """A row of more than 2^17 pages (8.4M entries; one layer over a
    contiguous pool) takes the other page-key form: the pages still equal
    the oracle's selection on the GPU's scores."""
    rng = np.random.default_rng(70)
    n = (1 << 17) * 64 + 640
    pool = np.empty((n, 132), np.uint8)
    # any finite e4m3 byte (0x00..0x7E with either sign), fp32 scales as in the other workloads
    pool[:, :128] = rng.integers(0, 0x7F, size=(n, 128), dtype=np.uint8) | \
        (rng.integers(0, 2, size=(n, 128), dtype=np.uint8) << 7)
    pool[:, 128:] = rng.uniform(0.005, 0.05, n).astype("<f4").view(np.uint8).reshape(n, 4)
    q = W.bf16_bits(rng.standard_normal((1, 64, 128), dtype=np.float32))
    w = (rng.standard_normal((1, 64), dtype=np.float32) * np.float32(128 ** -0.5 * 64 ** -0.5)).astype(np.float32)
    wl = W.Workload(name="huge-row", q=q, w=w, pool=pool, limits=np.array([n - 5], np.int32), n_cols=n,
                    description="one row of 8.4M entries, contiguous pool")
    rl = W.ResidentLoad(name="huge-row", layers=[wl], kmax=300, threshold=0.6, n_sink=2, n_recent=2)
    _log(f"[level1] {n} entries in one row ({-(-n // 64)} pages)")
    dls = _device_layers(rl)
    g = _gpu_scores(dls, rl.n_cols)
    pages, count = _check(rl, dls, g, None)
    assert count.tolist() == [300]
    del dls
    torch.cuda.empty_cache()


def test_resident_selection_with_128_head_layers():
    """The trained retriever's 128 heads: every layer scored as two head
    halves; pages exact given the GPU's scores and densities consistent with
    the oracle's."""
    rl = W.memory_indexer(entries=[12000, 5000, 300], n_layers=3, seed=75, kmax=24, threshold=0.76, H=128,
                          name="memory-indexer-h128")
    _log(f"[level1] {rl.description} H=128")
    dls = _device_layers(rl)
    g = _gpu_scores(dls, rl.n_cols)
    ref = oracle.level1_scores(rl.layers)
    for l in range(3):
        assert_logits_close(g[l], ref[l], f"h128 layer {l} scores")
    for over in [dict(), dict(ensemble=L.ENSEMBLE_MEAN, threshold=0.6), dict(kmax=4, n_sink=1, n_recent=2)]:
        _check(rl, dls, g, ref, **over)


def test_one_launch_over_stacked_layers():
    """Stacked queries and weights, max ensemble: one score launch over every
    (layer, row) writes selection bits instead of scores.  Its pages and
    counts equal the oracle's selection on the per-layer binary32 scores
    (and so the per-layer launches' result) for several settings, including
    thresholds at or below 0 that select masked entries' score 0."""
    rl = W.memory_indexer(entries=[16384, 9001, 700, 40], n_layers=3, seed=80, kmax=32, threshold=0.72,
                          ensemble=L.ENSEMBLE_MAX, name="memory-indexer-stacked")
    _log(f"[level1] {rl.description} (stacked layers)")
    dls = _device_layers(rl)
    g = _gpu_scores(dls, rl.n_cols)
    for over in [dict(), dict(threshold=0.8, kmax=8), dict(threshold=0.6, n_sink=2, n_recent=3, kmax=40),
                 dict(threshold=2.0), dict(threshold=0.0, kmax=12), dict(threshold=-1.0, kmax=7, n_sink=0),
                 dict(kmax=1, n_sink=1, n_recent=0), dict(kmax=2048, threshold=0.7)]:
        pages, count, cfg = _select_stacked(rl, dls, **over)
        want_p, want_c = oracle.level1_select(g, rl.limits, cfg["ensemble"], cfg["threshold"], cfg["n_sink"],
                                              cfg["n_recent"], cfg["kmax"])
        assert np.array_equal(count, want_c), (cfg, count, want_c)
        assert np.array_equal(pages, want_p), cfg
        p2, c2, _ = _select(rl, dls, **over)
        assert np.array_equal(pages, p2) and np.array_equal(count, c2), cfg


def test_one_launch_over_stacked_layers_two_and_eight_layers():
    """Two layers, and eight layers (the most one launch takes), of ragged
    rows with different block tables per layer."""
    for n_layers, entries in ((2, [5000, 64, 1, 3333]), (8, [4096, 777, 129])):
        rl = W.memory_indexer(entries=entries, n_layers=n_layers, seed=81 + n_layers, kmax=16, threshold=0.7,
                              ensemble=L.ENSEMBLE_MAX, name=f"memory-indexer-{n_layers}-layers")
        _log(f"[level1] {rl.description}")
        dls = _device_layers(rl)
        g = _gpu_scores(dls, rl.n_cols)
        pages, count, cfg = _select_stacked(rl, dls)
        want_p, want_c = oracle.level1_select(g, rl.limits, cfg["ensemble"], cfg["threshold"], cfg["n_sink"],
                                              cfg["n_recent"], cfg["kmax"])
        assert np.array_equal(count, want_c) and np.array_equal(pages, want_p), n_layers


def test_one_launch_over_stacked_layers_full_size():
    """The benchmark's shape through one launch: every row's pages equal the
    oracle's selection on the GPU's per-layer scores."""
    rl = W.memory_indexer()
    _log(f"[level1] full size, stacked layers: {rl.description}")
    dls = _device_layers(rl)
    g = _gpu_scores(dls, rl.n_cols)
    pages, count, cfg = _select_stacked(rl, dls)
    want_p, want_c = oracle.level1_select(g, rl.limits, cfg["ensemble"], cfg["threshold"], cfg["n_sink"],
                                          cfg["n_recent"], cfg["kmax"])
    assert np.array_equal(count, want_c) and np.array_equal(pages, want_p)


def test_one_launch_over_stacked_layers_rows_beyond_the_rank_cache():
    """Two stacked layers of one row of 16,400 pages (more than the 16,384
    page ranks the selection keeps in LDS, so its second pass recomputes
    them): the pages equal the oracle's selection on the GPU's scores."""
    n = 16400 * 64 - 17
    rl = W.memory_indexer(entries=[n], n_layers=2, seed=88, kmax=500, threshold=0.75, n_sink=3, n_recent=2,
                          ensemble=L.ENSEMBLE_MAX, name="memory-indexer-long-row")
    _log(f"[level1] {rl.description}")
    dls = _device_layers(rl)
    g = _gpu_scores(dls, rl.n_cols)
    for over in [dict(), dict(kmax=2048, threshold=0.7)]:
        pages, count, cfg = _select_stacked(rl, dls, **over)
        want_p, want_c = oracle.level1_select(g, rl.limits, cfg["ensemble"], cfg["threshold"], cfg["n_sink"],
                                              cfg["n_recent"], cfg["kmax"])
        assert np.array_equal(count, want_c) and np.array_equal(pages, want_p), cfg
    del dls
    torch.cuda.empty_cache()
