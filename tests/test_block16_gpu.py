"""GPU parity of 16-row pool blocks (through the C ABI) against the CPU oracle.

"DeepSeek-V4.1 native paged runtime" names 16 index rows per block id.  The
kernel keeps its 64-column slots and reads each slot's four small blocks
through their own table entries.  Every test here re-lays a 64-row workload
into independently placed 16-row blocks (workloads.reblock), so besides the
oracle the 64-row run of the same keys is a second reference: per entry the
arithmetic is the same, so its logits must come back bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from sparse_attention_kv_paged_amd import lib as L
from sparse_attention_kv_paged_amd import workloads as W
from tests.parity import assert_logits_close
from tests.test_parity_gpu import _check_workload
from tests.test_q8_gpu import _check_q8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def _log(msg):
    print(msg, flush=True)


def _logits(wl):
    d = L.to_device(wl)
    out = L.idx_score(d.q, d.w, d.keys, d.n_cols)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_b16_small_workloads(cfg):
    _check_workload(W.reblock(W.small_config(cfg), seed=30 + cfg), tag=f"b16-small{cfg}")


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_b16_logits_equal_64_row_blocks_bit_for_bit(cfg):
    wl = W.small_config(cfg)
    wl16 = W.reblock(wl, seed=40 + cfg)
    _log(f"[b16] bitwise {wl16.name}")
    a, b = _logits(wl), _logits(wl16)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("cfg", [1, 4])
def test_b16_full_size_workloads(cfg):
    _check_workload(W.reblock(W.config(cfg), seed=50 + cfg), tag=f"b16-full{cfg}")


def test_b16_full_size_prefill_all_rows():
    """Chunked prefill over 16-row blocks at full size, every one of the 4096 rows."""
    _check_workload(W.reblock(W.config(3), seed=53), tag="b16-full3")


def test_b16_per_row_path():
    """More than 512 rows of one request (a workgroup per row)."""
    _check_workload(W.reblock(W.prefill(4096, 603, seed=55, name="b16-rows"), seed=56), tag="b16-rows")


def test_b16_h128_and_quantised_query():
    wl = W.reblock(W.paged_decode([9000, 64, 1, 4097, 16384], seed=57, max_blocks=256, H=128, k=512,
                                  name="b16-h128"), seed=58)
    _check_workload(wl, tag="b16-h128")
    _check_q8(W.reblock(W.small_config(1), seed=59), tag="b16-q8")
    _check_q8(W.reblock(W.small_config(4), seed=60), tag="b16-q8-chunks")


def test_b16_holes_padding_bad_ids_and_status_bits():
    """A missing small block inside a slot, a padding row, a negative chunk
    id, out-of-range ids (absent and flagged), a clamped bound and a chunk
    count above the list's capacity."""
    wl = W.reblock(W.paged_decode([700, 64, 1, 129, 2048], seed=61, max_blocks=40, k=512, name="b16-edge"),
                   seed=62)
    wl.q_req = np.arange(wl.B, dtype=np.int32)
    wl.q_req[3] = -1                                           # padding row
    wl.block_table = wl.block_table.copy()
    wl.block_table[0, 5] = -1                                  # second small block of slot 1
    wl.block_table[4, 9] = -1
    _check_workload(wl, tag="b16-holes")

    wl2 = W.reblock(W.paged_decode([700, 64, 1, 129, 2048], seed=61, max_blocks=40, k=512, name="b16-edge"),
                    seed=62)
    wl2.block_table = wl2.block_table.copy()
    wl2.block_table[4, 6] = 10 ** 6                            # past the pool
    wl2.limits = wl2.limits.copy()
    wl2.limits[1] = 10 ** 7                                    # above capacity
    d = L.to_device(wl2, status=True)
    g = L.idx_score(d.q, d.w, d.keys, d.n_cols).cpu().numpy()
    st = int(d.keys.status.cpu().item())
    assert st & L.STATUS_BAD_BLOCK and st & L.STATUS_LIMIT_CLAMPED
    wl2.block_table[4, 6] = -1
    assert_logits_close(g, oracle.score(wl2), "b16 status case")

    wl3 = W.reblock(W.resident(5, 256, 24, seed=63, name="b16-chunk-edge"), seed=64)
    wl3.chunk_ids = wl3.chunk_ids.copy()
    wl3.n_chunks = wl3.n_chunks.copy()
    wl3.chunk_ids[0, 5] = -1                                   # a listed hole
    wl3.n_chunks[2] = wl3.max_chunks + 9                       # clamped to the list
    absent = int(np.flatnonzero(wl3.block_table[2] < 0)[0])    # a small block row 2 does not hold
    wl3.chunk_ids[2, :] = np.where(wl3.chunk_ids[2] < 0, absent, wl3.chunk_ids[2])
    d = L.to_device(wl3, status=True)
    g = L.idx_score(d.q, d.w, d.keys, d.n_cols).cpu().numpy()
    st = int(d.keys.status.cpu().item())
    assert st & L.STATUS_BAD_CHUNK
    wl3.n_chunks[2] = wl3.max_chunks
    assert_logits_close(g, oracle.score(wl3), "b16 chunk edge")
    _check_workload(wl3, tag="b16-chunk-edge")


def test_b16_level1_pages_equal_64_row_blocks():
    """Level 1 over 16-row blocks: pages stay 64 entries, and with logits
    equal bit for bit the chosen pages are the same."""
    rl = W.memory_indexer(entries=[20000, 9000, 64, 40000], n_layers=3, kmax=96, seed=65)
    outs = []
    for layers in (rl.layers, [W.reblock(x, seed=66 + i) for i, x in enumerate(rl.layers)]):
        dl = [L.to_device(x) for x in layers]
        pages, count = L.idx_select_resident([d.q for d in dl], [d.w for d in dl], [d.keys for d in dl],
                                             rl.n_cols, rl.kmax, threshold=rl.threshold, n_sink=1, n_recent=1)
        torch.cuda.synchronize()
        outs.append((pages.cpu().numpy(), count.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


def test_b16_repeat_runs_are_bitwise_identical():
    wl = W.reblock(W.small_config(4), seed=67)
    d = L.to_device(wl)
    a = L.idx_score_topk(d.q, d.w, d.keys, d.n_cols, wl.k)
    b = L.idx_score_topk(d.q, d.w, d.keys, d.n_cols, wl.k)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


def test_b16_contiguous_pool_chunk_lists_and_unaligned_columns():
    """Chunk lists of 16-row blocks over a contiguous pool (no block table):
    21 listed blocks make 336 columns, not a multiple of a 64-column slot;
    a shorter list, an empty one and a bound inside a listed block."""
    wl = W.reblock(W.contiguous(2048, B=3, seed=75, name="b16-contig"), seed=76)
    rng = np.random.default_rng(77)
    wl.chunk_ids = np.stack([rng.choice(128, 21, replace=False) for _ in range(3)]).astype(np.int32)
    wl.n_chunks = np.array([21, 17, 0], np.int32)
    wl.chunk_ids[1, 17:] = -1
    wl.limits = np.array([2048, 1000, 2048], np.int32)
    wl.n_cols = 21 * 16
    wl.k = 64
    _check_workload(wl, tag="b16-contig-chunks")


@pytest.mark.parametrize("k", [1, 2048])
def test_b16_k_extremes(k):
    wl = W.reblock(W.small_config(1), seed=78)
    wl.k = k
    _check_workload(wl, tag=f"b16-k{k}")
