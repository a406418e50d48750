"""GPU parity of the index-plane writer (idx_write_keys, through the C ABI)
against the CPU oracle's writer.

Writing is byte work decided by fp32 arithmetic (the binary32 divisions and
the e4m3 rounding), taken in the same precision on both sides, so every byte
of the pool must match the oracle exactly: written rows, and untouched rows
left as they were.
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from sparse_attention_kv_paged_amd import lib as L
from sparse_attention_kv_paged_amd import workloads as W
from tests.parity import assert_logits_close, assert_topk_near_tie

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def _log(msg):
    print(msg, flush=True)


def _gpu_write(k, slots, pool, status=False):
    """Run the writer on device copies; returns (pool after, status word)."""
    kd = torch.from_numpy(np.ascontiguousarray(k).view(np.int16)).cuda()
    sd = torch.from_numpy(np.ascontiguousarray(slots, dtype=np.int64)).cuda()
    pd = torch.from_numpy(np.ascontiguousarray(pool)).cuda()
    st = torch.zeros(1, dtype=torch.int32, device="cuda") if status else None
    L.idx_write_keys(kd, sd, pd, status=st)
    torch.cuda.synchronize()
    return pd.cpu().numpy(), (None if st is None else int(st.item()))


def _oracle_write(k, slots, pool):
    out = pool.copy()
    bad = oracle.write_keys(k, np.asarray(slots, dtype=np.int64), out)
    return out, bad


def _assert_pools_equal(got, want, tag):
    diff = np.nonzero((got != want).any(axis=1))[0]
    assert diff.size == 0, (f"{tag}: {diff.size} rows differ, first {diff[:8].tolist()}; "
                            f"row {diff[0]}: gpu {got[diff[0]].tolist()} oracle {want[diff[0]].tolist()}")


@pytest.mark.parametrize("seed", range(3))
def test_write_keys_matches_oracle_bytewise(seed):
    """Ragged n, shuffled slots with padding (-1) and out-of-range ones, keys
    spanning 60 binades: the whole pool equals the oracle's, byte for byte."""
    rng = np.random.default_rng(1000 + seed)
    n, rows = 1000 + 37 * seed, 2560
    _log(f"[writer] seed {seed}: n={n}, pool rows {rows}")
    x = rng.standard_normal((n, 128)).astype(np.float32)
    x *= np.exp2(rng.uniform(-30, 30, size=(n, 1))).astype(np.float32)
    k = W.bf16_bits(x)
    slots = rng.permutation(rows)[:n].astype(np.int64)
    slots[rng.choice(n, 20, replace=False)] = -1
    bad_at = rng.choice(np.nonzero(slots >= 0)[0], 3, replace=False)
    slots[bad_at] = [rows, -7, 1 << 40]
    pool = rng.integers(0, 256, size=(rows, 132), dtype=np.uint8)
    got, status = _gpu_write(k, slots, pool, status=True)
    want, bad = _oracle_write(k, slots, pool)
    assert bad == 3
    _assert_pools_equal(got, want, f"seed {seed}")
    assert status == L.STATUS_BAD_SLOT


def _special_rows():
    """Keys at the edges of the rounding: ties, saturation, zeros of both
    signs, subnormal codes, binary32-subnormal scales, the largest bf16."""
    v = np.arange(0x7F, dtype=np.int32).astype(np.uint8)
    mags = torch.from_numpy(v).view(torch.float8_e4m3fn).float().numpy()     # 127 finite values
    mids = ((mags[:-1].astype(np.float64) + mags[1:]) / 2).astype(np.float32)
    rows = []
    # amax exactly 448: scale 1, every quotient exact, so ties to even decide
    r = np.zeros(128, np.float32)
    r[0] = 448.0
    r[1:1 + 126] = mids
    r[127] = -mids[60]
    rows.append(r)
    # the same at scale 2^j (the quotients stay exact)
    for j in (-40, -3, 17, 100):
        rows.append(r * np.float32(2.0 ** j))
    # subnormal bf16 values: amax 7 * 2^-133 gives the binary32-subnormal
    # scale 2^-139 and exact quotients 448, 384, ..., 64
    t = np.zeros(128, np.float32)
    t[:8] = np.array([7, 6, 5, 4, 3, 2, 1, -7], np.float32) * np.float32(2.0 ** -133)
    rows.append(t)
    rows.append(np.zeros(128, np.float32))                    # zeros: bytes 0, scale 0
    rows.append(-np.zeros(128, np.float32))                   # negative zeros: same
    z = np.zeros(128, np.float32)
    z[5] = -3.0                                               # one nonzero element
    rows.append(z)
    rows.append(np.full(128, 1.5, np.float32))                # all equal: all 448
    big = np.linspace(-3.3e38, 3.3e38, 128).astype(np.float32)
    rows.append(big)                                          # near the bf16 maximum
    spread = np.exp2(np.linspace(-40, 10, 128)).astype(np.float32) * np.where(np.arange(128) % 3, 1, -1)
    rows.append(spread.astype(np.float32))                    # most elements far below amax
    return W.bf16_bits(np.stack(rows))


def test_write_keys_special_rows_match_oracle():
    k = _special_rows()
    n = k.shape[0]
    _log(f"[writer] {n} special rows")
    slots = np.arange(n, dtype=np.int64)[::-1].copy()
    pool = np.full((n + 3, 132), 0x5A, dtype=np.uint8)
    got, status = _gpu_write(k, slots, pool, status=True)
    want, bad = _oracle_write(k, slots, pool)
    assert bad == 0 and status == 0
    _assert_pools_equal(got, want, "special rows")
    # the scale-1 row stores 448 as 0x7E and leaves the last three rows alone
    assert got[n - 1, 0] == 0x7E and list(got[n - 1, 128:]) == [0, 0, 0x80, 0x3F]
    assert (got[n:] == 0x5A).all()


def _every_value_keys(amax_bits):
    """For each bf16 amax (bit pattern), keys holding amax at element 0 and
    then every bf16 value v with |v| <= amax, 127 per key (the last key
    padded with zeros)."""
    keys = []
    mags = np.arange(0x8000, dtype=np.uint32)
    for ha in amax_bits:
        vals = mags[mags <= ha]
        vals = np.concatenate([vals, vals[1:] | 0x8000]).astype(np.uint16)   # both signs, -0 once
        vals = np.concatenate([vals, [0x8000]]).astype(np.uint16)
        m = -(-len(vals) // 127)
        block = np.zeros((m, 128), np.uint16)
        block[:, 0] = ha
        flat = np.zeros(m * 127, np.uint16)
        flat[:len(vals)] = vals
        block[:, 1:] = flat.reshape(m, 127)
        keys.append(block)
    return np.concatenate(keys)


def test_write_keys_every_bf16_value_at_sampled_scales():
    """Every bf16 value up to amax, for 40 amax values across the whole
    range (subnormal, around 2^-100, ordinary, 448, the largest finite):
    each key's scale and every code equal the oracle's.  This covers the
    rounding of every quotient magnitude the writer can meet at those
    scales, ties included."""
    rng = np.random.default_rng(31)
    fixed = [0x0001, 0x0040, 0x0080, 0x0C80, 0x0D00, 0x0D80, 0x3F80, 0x3FC0, 0x43E0,
             0x43DF, 0x4400, 0x7F00, 0x7F7F]          # 2^-133 .. 2^-126, ~2^-101..2^-99, 1, 1.5, 448 .. max
    amax_bits = sorted(set(fixed) | set(int(x) for x in rng.integers(1, 0x7F80, 27)))
    k = _every_value_keys(amax_bits)
    n = k.shape[0]
    _log(f"[writer] every bf16 value at {len(amax_bits)} scales: {n} keys")
    slots = rng.permutation(n).astype(np.int64)
    pool = np.zeros((n, 132), np.uint8)
    got, status = _gpu_write(k, slots, pool, status=True)
    want, bad = _oracle_write(k, slots, pool)
    assert bad == 0 and status == 0
    _assert_pools_equal(got, want, "every bf16 value")


def test_write_keys_empty_and_single():
    pool = np.full((64, 132), 0x11, dtype=np.uint8)
    k = W.bf16_bits(np.zeros((0, 128), np.float32))
    got, status = _gpu_write(k, np.zeros(0, np.int64), pool, status=True)
    assert (got == pool).all() and status == 0
    k1 = W.bf16_bits(np.linspace(-2, 1, 128, dtype=np.float32)[None])
    got, _ = _gpu_write(k1, np.array([63]), pool)
    want, _ = _oracle_write(k1, np.array([63]), pool)
    _assert_pools_equal(got, want, "single key")


def test_write_keys_overwrites_and_repeats_bitwise():
    """A second write to the same slots replaces the rows; the same write
    twice gives the same bytes."""
    rng = np.random.default_rng(77)
    n = 300
    slots = rng.permutation(512)[:n].astype(np.int64)
    k1 = W.bf16_bits(rng.standard_normal((n, 128)).astype(np.float32))
    k2 = W.bf16_bits(rng.standard_normal((n, 128)).astype(np.float32) * 5)
    pool = np.zeros((512, 132), np.uint8)
    kd1 = torch.from_numpy(k1.view(np.int16)).cuda()
    kd2 = torch.from_numpy(k2.view(np.int16)).cuda()
    sd = torch.from_numpy(slots).cuda()
    pd = torch.from_numpy(pool).cuda()
    L.idx_write_keys(kd1, sd, pd)
    L.idx_write_keys(kd2, sd, pd)
    torch.cuda.synchronize()
    first = pd.cpu().numpy()
    L.idx_write_keys(kd2, sd, pd)
    torch.cuda.synchronize()
    assert np.array_equal(first, pd.cpu().numpy())
    want, _ = _oracle_write(k2, slots, pool)
    _assert_pools_equal(first, want, "overwrite")


def test_written_pool_scores_like_the_oracle():
    """Write a request's keys into a shuffled paged pool on the GPU, then
    score and select on that pool: the pool equals the oracle writer's, and
    the logits and top-512 of the written rows match the oracle's."""
    wr = W.index_fill(n_keys=8000, seed=21)
    _log(f"[writer] write-then-score: {wr.description}")
    got, status = _gpu_write(wr.k, wr.slots, wr.pool, status=True)
    want, bad = _oracle_write(wr.k, wr.slots, wr.pool)
    assert bad == 0 and status == 0
    _assert_pools_equal(got, want, "index-fill small")
    rng = np.random.default_rng(22)
    B = 3
    q = W.bf16_bits(rng.standard_normal((B, 64, 128), dtype=np.float32))
    w = (rng.standard_normal((B, 64), dtype=np.float32) * np.float32(128 ** -0.5 * 64 ** -0.5)).astype(np.float32)
    limits = np.array([8000, 5000, 63], np.int32)
    nblk = wr.block_table.shape[1]
    wl = W.Workload(name="written-pool", q=q, w=w, pool=got, limits=limits, n_cols=nblk * 64,
                    k=512, block_table=wr.block_table, q_req=np.zeros(B, np.int32),
                    description="rows written by idx_write_keys")
    d = L.to_device(wl)
    logits = L.idx_score(d.q, d.w, d.keys, d.n_cols)
    idx, _ = L.idx_score_topk(d.q, d.w, d.keys, d.n_cols, wl.k)
    torch.cuda.synchronize()
    ref = oracle.score(wl)
    assert_logits_close(logits.cpu().numpy(), ref, "written pool logits")
    ref_cols, _ = oracle.topk(ref, wl.k)
    ref_ids = oracle.cols_to_entries(wl, ref_cols)
    assert_topk_near_tie(idx.cpu().numpy(), ref_ids, lambda b, e: ref[b, np.asarray(e)], wl.k,
                         "written pool top-k")


def test_write_keys_full_size_index_fill():
    """The full index-fill workload (262,144 keys, 4096 shuffled blocks) in
    the launch shape the benchmark times: 4096 sampled keys (every 64th)
    equal the oracle's rows, every row not written keeps its poison bytes."""
    wr = W.index_fill()
    _log(f"[writer] full size: {wr.description}")
    kd = torch.from_numpy(wr.k.view(np.int16)).cuda()
    sd = torch.from_numpy(wr.slots).cuda()
    pd = torch.from_numpy(wr.pool).cuda()
    before = pd.clone()
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    L.idx_write_keys(kd, sd, pd, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    written = torch.zeros(pd.shape[0], dtype=torch.bool, device="cuda")
    written[sd] = True
    assert torch.equal(pd[~written], before[~written])
    sample = np.arange(0, wr.n, 64)
    got = pd[sd[torch.from_numpy(sample).cuda()]].cpu().numpy()
    want = np.stack([oracle.quantize_row(wr.k[i]) for i in sample])
    _assert_pools_equal(got, want, "index-fill sample")
