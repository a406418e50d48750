"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Inputs are the seeded synthetic workloads; expected values come only from
the oracle.  Logits must match to |g - o| <= 1e-4 + 2e-3 |o| (exactly -inf
where unscored); integer-exact inputs must match bit for bit; top-k index
work must be exact given the same fp32 values, and against the oracle's
double logits may differ only at near-ties.
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


def _entry_logit_fn(wl, ref_logits, rows=None):
    """(b, entry ids) -> oracle logits, resolving chunk lists to columns."""
    def f(b, ids):
        ids = np.asarray(ids, dtype=np.int64)
        if wl.chunk_ids is None:
            cols = ids
        else:
            row = b if rows is None else rows[b]
            bs = wl.block_size
            pos = {int(c): j for j, c in enumerate(wl.chunk_ids[row][:wl.n_chunks[row]])}
            cols = np.array([pos[int(e) // bs] * bs + int(e) % bs for e in ids], dtype=np.int64)
        return ref_logits[b, cols]
    return f


def _gpu_logits(d, with_scores=False):
    out = L.idx_score(d.q, d.w, d.keys, d.n_cols, with_scores=with_scores)
    torch.cuda.synchronize()
    if with_scores:
        return out[0].cpu().numpy(), out[1].cpu().numpy()
    return out.cpu().numpy()


def _check_workload(wl, rows=None, check_topk=True, tag=""):
    """Full comparison on all rows (or oracle on a row subset)."""
    _log(f"[parity] {tag} {wl.name}: {wl.description} rows={'all' if rows is None else len(rows)}")
    d = L.to_device(wl)
    g_logits, g_scores = _gpu_logits(d, with_scores=True)
    ref = oracle.score(wl, rows=rows)
    sel = slice(None) if rows is None else np.asarray(rows)
    assert_logits_close(g_logits[sel], ref, f"{wl.name} logits")
    # sigmoid scores: 0 where unscored, else close to the oracle's
    ref_sc = oracle.sigmoid(ref)
    err = np.abs(g_scores[sel] - ref_sc)
    assert np.all(err <= 1e-4 + 2e-3 * ref_sc), f"{wl.name} scores: worst {err.max():.3e}"
    if not check_topk:
        return
    g_idx, g_val = L.idx_score_topk(d.q, d.w, d.keys, d.n_cols, wl.k)
    torch.cuda.synchronize()
    g_idx, g_val = g_idx.cpu().numpy(), g_val.cpu().numpy()
    # (1) same precision as the kernel: exact top-k of the GPU's own logits
    own_cols, own_vals = column_order(*oracle.topk(g_logits.astype(np.float64), wl.k))
    own_ids = oracle.cols_to_entries(wl, own_cols)
    assert np.array_equal(g_idx, own_ids), f"{wl.name}: score_topk != top-k of its own logits"
    ok = own_cols >= 0
    assert np.array_equal(g_val[ok], own_vals[ok].astype(np.float32))
    # (2) idx_topk on the same logits: columns, bit-exact
    t_cols, t_vals = L.idx_topk(torch.from_numpy(g_logits).cuda(), wl.k)
    torch.cuda.synchronize()
    assert np.array_equal(t_cols.cpu().numpy(), own_cols), f"{wl.name}: idx_topk columns differ"
    # (3) against the oracle's double logits: equal up to near-ties
    ref_cols, _ = oracle.topk(ref, wl.k)
    ref_ids = oracle.cols_to_entries(wl, ref_cols, rows=rows)
    assert_topk_near_tie(g_idx[sel], ref_ids, _entry_logit_fn(wl, ref, rows), wl.k, wl.name)


# --------------------------------------------------------------- exactness

def test_fp8_decode_table_on_device():
    """Each of the 254 finite e4m3fn bytes decodes exactly: row r holds byte r
    at d = 0; q[:, 0] = 1, w = e_0, so logit = relu(s * e4m3(r)); scales +1
    and -1 recover positive and negative values."""
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    q = np.zeros((1, 64, 128), dtype=np.float32)
    q[0, :, 0] = 1.0
    w = np.zeros((1, 64), dtype=np.float32)
    w[0, 0] = 1.0
    got = {}
    for s in (1.0, -1.0):
        f8 = np.zeros((256, 128), dtype=np.uint8)
        f8[:, 0] = np.arange(256)
        pool = np.zeros((256, 132), dtype=np.uint8)
        pool[:, :128] = f8
        pool[:, 128:] = np.array([s], "<f4").view(np.uint8)
        wl = W.Workload(name="fp8", q=W.bf16_bits(q), w=w, pool=pool,
                        limits=np.array([256], np.int32), n_cols=256)
        got[s] = _gpu_logits(L.to_device(wl))[0]
    fin = ~np.isnan(ref)
    dec = np.where(ref > 0, got[1.0], -got[-1.0])
    assert np.array_equal(dec[fin & (ref != 0)], ref[fin & (ref != 0)])
    assert np.all(got[1.0][ref == 0] == 0) and np.all(got[-1.0][ref == 0] == 0)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_integer_case_is_bit_exact(seed):
    """Small-integer keys, bf16 integer queries, power-of-two weights and
    scales: every partial sum is exact, so GPU == oracle bit for bit."""
    rng = np.random.default_rng(seed)
    n, B = 64 * 5 + 17, 3
    kv = rng.integers(-4, 5, size=(n, 128)).astype(np.float32)
    scales = np.ldexp(1.0, rng.integers(-2, 3, size=n)).astype(np.float32)
    scales[rng.random(n) < 0.2] *= -1                       # negative scales too
    pool = np.zeros((n, 132), dtype=np.uint8)
    pool[:, :128] = W.e4m3_bytes(kv)
    pool[:, 128:] = scales.astype("<f4").view(np.uint8).reshape(n, 4)
    q = rng.integers(-2, 3, size=(B, 64, 128)).astype(np.float32)
    w = (rng.choice([-1.0, 1.0], size=(B, 64)) * np.ldexp(1.0, rng.integers(-3, 4, size=(B, 64)))).astype(np.float32)
    wl = W.Workload(name="int", q=W.bf16_bits(q), w=w, pool=pool,
                    limits=np.array([n, n - 40, 70], np.int32), n_cols=n + 30)
    g = _gpu_logits(L.to_device(wl))
    ref = oracle.score(wl)
    assert np.array_equal(g.astype(np.float64), ref)


# --------------------------------------------------------------- workloads

@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_small_workloads(cfg):
    _check_workload(W.small_config(cfg), tag=f"small{cfg}")


@pytest.mark.parametrize("cfg", [0, 1, 2, 4])
def test_full_size_workloads(cfg):
    _check_workload(W.config(cfg), tag=f"full{cfg}")


def test_full_size_prefill_all_rows():
    """4096-row chunked prefill at full size: every row's logits, scores and
    top-512 against the oracle (causal bounds (65537 + i) // 4 over 272
    shuffled blocks)."""
    _check_workload(W.config(3), tag="full3")


def test_many_rows_sharing_a_request():
    """More than 512 rows of one request take the per-row path (one
    workgroup per row, its four waves splitting the row's blocks); a padding
    row and an out-of-range request id among them."""
    wl = W.prefill(8192, 603, seed=13, name="shared-rows")
    wl.q_req = wl.q_req.copy()
    wl.q_req[301] = -1                                         # padding row inside a group
    wl.q_req[450] = 5                                          # no such request: absent, flagged
    _check_workload(wl, tag="shared-rows")


@pytest.mark.parametrize("n_req,draft", [(16, 4), (130, 4)])
def test_speculative_draft_rows(n_req, draft):
    """Several query rows per request in one call, each with its own bound
    (draft tokens of speculative decoding): 64 rows take the flattened split,
    520 rows (130 requests) the per-row path."""
    wl = W.speculative_decode(n_req=n_req, draft=draft, seed=80 + n_req)
    _check_workload(wl, tag="speculative")


# ------------------------------------------------------------ 128 heads

@pytest.mark.parametrize("seed", [0, 1])
def test_h128_integer_case_is_bit_exact(seed):
    """128 heads (two launches over the head halves, the second adding to the
    first's logits): integer data keeps every partial sum exact, so the GPU
    equals the oracle bit for bit."""
    rng = np.random.default_rng(60 + seed)
    n, B = 64 * 5 + 17, 3
    kv = rng.integers(-4, 5, size=(n, 128)).astype(np.float32)
    scales = np.ldexp(1.0, rng.integers(-2, 3, size=n)).astype(np.float32)
    scales[rng.random(n) < 0.2] *= -1
    pool = np.zeros((n, 132), dtype=np.uint8)
    pool[:, :128] = W.e4m3_bytes(kv)
    pool[:, 128:] = scales.astype("<f4").view(np.uint8).reshape(n, 4)
    q = rng.integers(-2, 3, size=(B, 128, 128)).astype(np.float32)
    w = (rng.choice([-1.0, 1.0], size=(B, 128)) * np.ldexp(1.0, rng.integers(-3, 4, size=(B, 128)))).astype(np.float32)
    wl = W.Workload(name="int-h128", q=W.bf16_bits(q), w=w, pool=pool,
                    limits=np.array([n, n - 40, 70], np.int32), n_cols=n + 30)
    g = _gpu_logits(L.to_device(wl))
    ref = oracle.score(wl)
    assert np.array_equal(g.astype(np.float64), ref)


def test_h128_paged_rows():
    """128 heads on the flattened split: ragged paged rows, scores, top-k."""
    wl = W.paged_decode([9000, 64, 1, 4097, 16384], seed=61, max_blocks=256, H=128, k=512, name="h128-paged")
    _check_workload(wl, tag="h128")


def test_h128_chunk_lists():
    wl = W.resident(5, 256, 24, seed=62, H=128, name="h128-resident")
    _check_workload(wl, tag="h128-chunks")


def test_h128_per_row_path():
    """More than 512 rows of one request with 128 heads (per-row path)."""
    wl = W.prefill(4096, 520, seed=63, H=128, name="h128-rows")
    _check_workload(wl, tag="h128-rows")


# --------------------------------------------------------------- edge cases

def _small_paged(seed=7, entries=(700, 64, 1, 129, 2048)):
    return W.paged_decode(list(entries), seed=seed, max_blocks=40, k=512, name="edge")


def test_ragged_rows_fewer_entries_than_k():
    wl = _small_paged()
    _check_workload(wl, tag="edge-ragged")
    d = L.to_device(wl)
    idx, _ = L.idx_score_topk(d.q, d.w, d.keys, d.n_cols, wl.k)
    idx = idx.cpu().numpy()
    assert np.all(idx[1, 64:] == -1) and np.all(idx[2, 1:] == -1)      # 64 and 1 entries


def test_padding_rows_holes_and_status_bits():
    wl = _small_paged()
    wl.q_req = np.arange(wl.B, dtype=np.int32)
    wl.q_req[3] = -1                                           # padding row
    wl.block_table = wl.block_table.copy()
    wl.block_table[0, 2] = -1                                  # hole
    _check_workload(wl, tag="edge-padding")
    # out-of-range ids are absent and flagged
    wl2 = _small_paged()
    wl2.block_table = wl2.block_table.copy()
    wl2.block_table[4, 5] = 10 ** 6                            # past the pool
    wl2.limits = wl2.limits.copy()
    wl2.limits[1] = 10 ** 7            # above capacity (row 1 holds one full block)
    wl2.q_req = np.arange(wl2.B, dtype=np.int32)
    wl2.q_req[3] = 99                                          # no such request
    d = L.to_device(wl2, status=True)
    g = L.idx_score(d.q, d.w, d.keys, d.n_cols).cpu().numpy()
    st = int(d.keys.status.cpu().item())
    assert st & L.STATUS_BAD_BLOCK and st & L.STATUS_LIMIT_CLAMPED and st & L.STATUS_BAD_REQUEST
    wl2.block_table[4, 5] = -1                                 # what "absent" means
    wl2.q_req[3] = -1
    assert_logits_close(g, oracle.score(wl2), "status case")


def test_zero_limits_and_unaligned_columns():
    wl = _small_paged(entries=(0, 5, 191))
    wl.n_cols = 200                                            # not a multiple of 64
    _check_workload(wl, tag="edge-limits")


def test_degenerate_all_equal_logits_ties_go_to_low_columns():
    """w = 0 makes every scored logit 0: the top-k is the k lowest scored
    columns (ties resolved by column)."""
    wl = W.small_config(2)
    wl.w = np.zeros_like(wl.w)
    _check_workload(wl, tag="edge-ties")
    d = L.to_device(wl)
    idx, val = L.idx_score_topk(d.q, d.w, d.keys, d.n_cols, 512)
    assert np.array_equal(idx.cpu().numpy(), np.tile(np.arange(512, dtype=np.int32), (wl.B, 1)))
    assert np.all(val.cpu().numpy() == 0)


@pytest.mark.parametrize("k", [1, 7, 512, 2048])
def test_k_values(k):
    wl = W.small_config(1)
    wl.k = k
    _check_workload(wl, tag=f"k{k}")


@pytest.mark.parametrize("k", [1, 7, 512, 1500, 2048])
def test_multi_part_rows_k_values(k):
    """Rows of up to 20000 entries, each split over 5 top-k workgroups: for
    k <= 1638 the row's last part merges the parts' lists in the same launch,
    k = 2048 takes a separate merge launch."""
    wl = W.paged_decode([20000, 9000, 300, 16000], seed=11, k=k, name="multi-part")
    _check_workload(wl, tag=f"multipart-k{k}")


@pytest.mark.parametrize("k", [1, 512, 1024, 2048])
def test_few_long_rows_sixteen_parts(k):
    """Three rows of ~250000 entries: 16 top-k parts of up to 16384 columns
    per row, merged by the row's last part in the same launch while the lists
    fit one segment (k <= 1024), else by a separate merge launch."""
    wl = W.paged_decode([250000, 180001, 249999], seed=27, k=k, name="long-rows")
    _check_workload(wl, tag=f"long-rows-k{k}")


@pytest.mark.parametrize("k", [7, 512])
def test_multi_part_rows_with_chunk_lists(k):
    """Chunk-list rows over 4 top-k parts: the in-launch merge resolves the
    winners' columns to logical entries."""
    wl = W.resident(3, 512, 200, seed=12, k=k, name="multi-part-chunks")
    _check_workload(wl, tag=f"multipart-chunks-k{k}")


def test_negative_and_zero_scales():
    wl = W.small_config(0)
    sc = wl.pool[:, 128:].copy().view("<f4")
    rng = np.random.default_rng(5)
    sc[rng.random(len(sc)) < 0.3] *= -1
    sc[rng.random(len(sc)) < 0.05] = 0.0
    wl.pool[:, 128:] = sc.view(np.uint8)
    _check_workload(wl, tag="edge-scales")


@pytest.mark.parametrize("B", [601, 602, 603, 300])
def test_no_writes_past_the_last_row(B):
    """The last workgroup of the per-row path may hold fewer than four rows;
    nothing may be written below row B of the logits or scores."""
    wl = W.prefill(4096, B, seed=25, name="tail-rows")
    d = L.to_device(wl)
    guard = 8
    big_l = torch.full((B + guard, d.n_cols), 7.0, dtype=torch.float32, device="cuda")
    big_s = torch.full((B + guard, d.n_cols), 7.0, dtype=torch.float32, device="cuda")
    L.idx_score(d.q, d.w, d.keys, d.n_cols, with_scores=True, logits=big_l[:B], scores=big_s[:B])
    torch.cuda.synchronize()
    assert torch.all(big_l[B:] == 7.0) and torch.all(big_s[B:] == 7.0)
    assert bool(torch.all(big_l[:B] != 7.0))


def _flip_some_scales(wl, seed):
    sc = wl.pool[:, 128:].copy().view("<f4")
    rng = np.random.default_rng(seed)
    sc[rng.random(len(sc)) < 0.3] *= -1
    sc[rng.random(len(sc)) < 0.05] = 0.0
    wl.pool[:, 128:] = sc.view(np.uint8)


def test_per_row_path_negative_and_zero_scales():
    """Over 512 rows (one workgroup per row): negative and zero scales reach
    the sign flip inside the pipelined tile loop; logits, scores and top-k."""
    wl = W.prefill(4096, 600, seed=21, name="per-row-edge-scales")
    _flip_some_scales(wl, 22)
    _check_workload(wl, tag="per-row-edge-scales")


def test_per_row_path_chunk_lists_negative_scales():
    """Over 512 rows with chunk lists (per-row path, chunked kernel)."""
    wl = W.resident(B=520, chunks_per_req=64, n_resident=20, seed=23, name="per-row-chunks")
    _flip_some_scales(wl, 24)
    _check_workload(wl, tag="per-row-chunks")


def test_contiguous_chunk_list():
    """Chunk lists over a contiguous pool (no block table)."""
    base = W.contiguous(64 * 20, B=3, seed=9)
    rng = np.random.default_rng(9)
    chunk_ids = np.stack([rng.choice(20, 6, replace=False) for _ in range(3)]).astype(np.int32)
    chunk_ids[1, 4] = -1                                       # absent chunk
    wl = W.Workload(name="contig-chunks", q=base.q, w=base.w, pool=base.pool,
                    limits=np.array([64 * 20, 64 * 10, 64 * 20 - 3], np.int32), n_cols=6 * 64,
                    k=100, chunk_ids=chunk_ids, n_chunks=np.array([6, 5, 6], np.int32))
    _check_workload(wl, tag="edge-contig-chunks")


def test_topk_standalone_exact_with_ties_nan_and_signed_zero():
    rng = np.random.default_rng(1)
    B, n, k = 5, 70000, 512
    vals = rng.integers(-50, 50, size=(B, n)).astype(np.float32) / 8    # heavy ties
    vals[rng.random((B, n)) < 0.1] = -np.inf
    vals[rng.random((B, n)) < 0.01] = np.nan
    vals[0, :100] = -0.0
    vals[1] = -np.inf
    vals[1, [5, 9]] = [1.0, 1.0]
    vals[2] = rng.standard_normal(n).astype(np.float32)
    cols, v = L.idx_topk(torch.from_numpy(vals).cuda(), k)
    torch.cuda.synchronize()
    ref_cols, ref_v = column_order(*oracle.topk(vals.astype(np.float64), k))
    assert np.array_equal(cols.cpu().numpy(), ref_cols)
    ok = ref_cols >= 0
    assert np.array_equal(v.cpu().numpy()[ok], ref_v[ok].astype(np.float32))


def test_repeat_runs_are_bitwise_identical():
    wl = W.small_config(4)
    d = L.to_device(wl)
    first = [x.cpu().numpy() for x in L.idx_score_topk(d.q, d.w, d.keys, d.n_cols, wl.k)]
    lg0 = L.idx_score(d.q, d.w, d.keys, d.n_cols).cpu().numpy()
    for _ in range(20):
        again = [x.cpu().numpy() for x in L.idx_score_topk(d.q, d.w, d.keys, d.n_cols, wl.k)]
        assert all(np.array_equal(a, b) for a, b in zip(first, again))
        assert np.array_equal(L.idx_score(d.q, d.w, d.keys, d.n_cols).cpu().numpy(), lg0)


def test_empty_batch():
    wl = W.small_config(0)
    d = L.to_device(wl)
    L.idx_score(d.q[:0], d.w[:0], d.keys, d.n_cols)
    idx, _ = L.idx_score_topk(d.q[:0], d.w[:0], d.keys, d.n_cols, 16)
    assert idx.shape == (0, 16)


@pytest.mark.parametrize("n,k", [(300000, 2048), (100000, 7), (40000, 512), (4096, 4096 // 8)])
def test_topk_standalone_multilevel(n, k):
    """Rows longer than one top-k workgroup: per-part lists merged over one or
    more further launches (300000 columns at k=2048 needs three levels)."""
    rng = np.random.default_rng(n + k)
    B = 3
    vals = rng.standard_normal((B, n)).astype(np.float32)
    vals[1, ::3] = -np.inf
    vals[2, :] = np.round(vals[2, :] * 4) / 4                 # many exact ties
    cols, v = L.idx_topk(torch.from_numpy(vals).cuda(), k)
    torch.cuda.synchronize()
    ref_cols, ref_v = column_order(*oracle.topk(vals.astype(np.float64), k))
    assert np.array_equal(cols.cpu().numpy(), ref_cols)
    assert np.array_equal(v.cpu().numpy(), ref_v.astype(np.float32))

@pytest.mark.gpu
@pytest.mark.parametrize("n,k", [(6000, 512), (8192, 1000), (12000, 300), (17408, 512), (20000, 512), (24000, 2048),
                                 (24576, 7), (30000, 640)])
def test_topk_standalone_one_segment_per_row(n, k):
    """Many rows (one top-k workgroup per row) whose segment sizes are not a
    multiple of the write-out's 8-slot groups (20 and 24 slots per thread);
    every segment size, through the sampled threshold (k <= 640) or not."""
    rng = np.random.default_rng(n + 7 * k)
    B = 256
    vals = rng.standard_normal((B, n)).astype(np.float32)
    vals[1, ::3] = -np.inf
    vals[2, :] = np.round(vals[2, :] * 4) / 4                 # many exact ties
    vals[3, n // 2:] = -np.inf                                # half the row not selectable
    cols, v = L.idx_topk(torch.from_numpy(vals).cuda(), k)
    torch.cuda.synchronize()
    ref_cols, ref_v = column_order(*oracle.topk(vals.astype(np.float64), k))
    assert np.array_equal(cols.cpu().numpy(), ref_cols)
    assert np.array_equal(v.cpu().numpy(), ref_v.astype(np.float32))



@pytest.mark.parametrize("B,n,k", [(32, 160000, 512), (32, 190000, 7), (32, 150000, 2048), (16, 200000, 2048),
                                   (64, 90000, 512)])
def test_topk_long_segments_writing_lists(B, n, k):
    """Rows split into parts of 16384-24576 columns that are not merged in the
    same launch: each part (candidates compacted in LDS, or the register path
    past 1024 candidates) writes a (key, column) list that a further launch
    merges.  Some rows are mostly masked so that parts hold fewer selectable
    items than k, or none."""
    rng = np.random.default_rng(B + n + k)
    vals = rng.standard_normal((B, n)).astype(np.float32)
    vals[0, : n - 300] = -np.inf                              # 300 selectable, all in the last part
    vals[1] = -np.inf                                         # none
    vals[2, ::2] = -np.inf
    vals[3] = np.round(vals[3] * 4) / 4                       # many exact ties
    vals[4, rng.random(n) < 0.01] = np.nan
    cols, v = L.idx_topk(torch.from_numpy(vals).cuda(), k)
    torch.cuda.synchronize()
    ref_cols, ref_v = column_order(*oracle.topk(vals.astype(np.float64), k))
    got = cols.cpu().numpy()
    for r in range(5):
        assert np.array_equal(got[r], ref_cols[r]), f"row {r}"
    assert np.array_equal(got, ref_cols)
    ok = ref_cols >= 0
    assert np.array_equal(v.cpu().numpy()[ok], ref_v[ok].astype(np.float32))


@pytest.mark.parametrize("k", [512, 1000])
def test_topk_one_segment_compaction_boundaries(k):
    """Rows of one long segment each (256 rows of 20000 columns): after the
    histogram the items that can still win are compacted when they number at
    most 1024, else the selection stays on every slot.  Rows at and around
    that bound and the degenerate cases: nothing selectable, fewer selectable
    items than k, NaN with signed zeros, exactly 1024 and 1025 tied items in
    the top bin, one value everywhere, half the row masked."""
    rng = np.random.default_rng(k)
    B, n = 256, 20000
    vals = rng.standard_normal((B, n)).astype(np.float32)
    vals[0] = -np.inf                                         # nothing selectable
    vals[1] = -np.inf
    vals[1, rng.choice(n, 300, replace=False)] = rng.standard_normal(300)   # fewer than k
    vals[2, rng.random(n) < 0.01] = np.nan
    vals[2, :50] = -0.0
    vals[2, 50:100] = 0.0
    vals[3, rng.choice(n, 1024, replace=False)] = 100.0      # 1024 tied in the top bin
    vals[4, rng.choice(n, 1025, replace=False)] = 100.0      # one past the compaction bound
    vals[5] = 0.5                                             # one value everywhere
    vals[6, n // 2:] = -np.inf
    vals[7, : k - 3] = 7.0                                    # k - 3 clear winners, then the cut
    cols, v = L.idx_topk(torch.from_numpy(vals).cuda(), k)
    torch.cuda.synchronize()
    ref_cols, ref_v = column_order(*oracle.topk(vals.astype(np.float64), k))
    got = cols.cpu().numpy()
    for r in range(8):
        assert np.array_equal(got[r], ref_cols[r]), f"row {r}"
    assert np.array_equal(got, ref_cols)
    ok = ref_cols >= 0
    assert np.array_equal(v.cpu().numpy()[ok], ref_v[ok].astype(np.float32))
    assert (got[0] == -1).all() and (got[1] >= 0).sum() == 300


@pytest.mark.parametrize("k", [1, 7, 300, 512, 640, 641])
def test_topk_one_segment_sampled_threshold(k):
    """Rows of one long segment each (256 rows of 20000 columns, 40 columns
    per thread, the first of each thread's run sampled): for k up to 640 a
    threshold from the samples picks the items to compact when at least k and
    at most 2048 reach it, else the histogram path runs.  Rows whose samples
    overstate the row (the sampled columns far above the rest: too few items
    reach the threshold), understate it (far below: too many), one value
    almost everywhere (too many ties at the threshold), fewer selectable
    samples than the threshold's rank, NaN and +-inf with signed zeros, and
    the sampled columns alone being the row's largest."""
    rng = np.random.default_rng(100 + k)
    B, n = 256, 20000
    vals = rng.standard_normal((B, n)).astype(np.float32)
    sampled = np.arange(0, n, 40)
    vals[0, sampled] += 1000.0                                # samples overstate the row
    vals[1, sampled] -= 1000.0                                # samples understate it
    vals[2] = 1.0
    vals[2, rng.choice(n, 100, replace=False)] = rng.random(100).astype(np.float32) + 2.0    # ties at T
    vals[3] = -np.inf
    keep = rng.choice(n, 300, replace=False)
    vals[3, keep] = rng.standard_normal(300)                  # few selectable samples
    vals[4, rng.random(n) < 0.05] = np.nan
    vals[4, rng.random(n) < 0.05] = np.inf
    vals[4, rng.random(n) < 0.3] = -np.inf
    vals[4, :40] = -0.0
    vals[4, 40:80] = 0.0
    vals[5] = -np.inf
    vals[5, sampled] = rng.standard_normal(len(sampled))     # only the sampled columns selectable
    vals[6, sampled[: k]] = 50.0                              # k tied winners, all sampled
    vals[7] = np.round(vals[7] * 4) / 4                       # many ties everywhere
    cols, v = L.idx_topk(torch.from_numpy(vals).cuda(), k)
    torch.cuda.synchronize()
    ref_cols, ref_v = column_order(*oracle.topk(vals.astype(np.float64), k))
    got = cols.cpu().numpy()
    for r in range(8):
        assert np.array_equal(got[r], ref_cols[r]), f"row {r}"
    assert np.array_equal(got, ref_cols)
    ok = ref_cols >= 0
    assert np.array_equal(v.cpu().numpy()[ok], ref_v[ok].astype(np.float32))


@pytest.mark.parametrize("n,k", [(100, 4), (4096, 384), (70000, 512)])
def test_topk_standalone_values_far_from_zero_in_a_narrow_range(n, k):
    """Values whose magnitude is large against their spread (|min| / range
    well past 8192): the histogram's bin offset rounds by more than one bin,
    and the lowest values must still rank lowest.  Distinct integers near
    2^23, near -2^23, and fractions just above 1e6, with ties at the cut."""
    rng = np.random.default_rng(n + k + 5)
    B = 4
    base = np.arange(n, dtype=np.float64)
    vals = np.empty((B, n), np.float32)
    vals[0] = (2.0 ** 23 + 131071 - base).astype(np.float32)          # decreasing: the first k win
    vals[1] = (-(2.0 ** 23) + rng.permutation(n)).astype(np.float32)
    vals[2] = (1.0e6 + np.round(rng.random(n) * 64) / 64).astype(np.float32)
    vals[3] = (3.0e7 + rng.integers(0, 3, n) * 2.0).astype(np.float32)  # three values, heavy ties
    cols, v = L.idx_topk(torch.from_numpy(vals).cuda(), k)
    torch.cuda.synchronize()
    ref_cols, ref_v = column_order(*oracle.topk(vals.astype(np.float64), k))
    assert np.array_equal(cols.cpu().numpy(), ref_cols)
    assert np.array_equal(v.cpu().numpy(), ref_v.astype(np.float32))
    assert cols.cpu().numpy()[0].tolist() == list(range(k))
