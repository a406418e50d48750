"""GPU parity of the per-row path at 2048 rows and more (through the C ABI).

The flattened split covers up to 512 rows; above that every row gets its
own workgroups.  These cases check that path where many rows share a
request (prefill chunks, draft rows of many requests, the same rows
reordered so that neighbours belong to different requests), across rows
that need several 64-slot groups of table reads, padding rows and unknown
requests, negative and zero scales, absent blocks, status bits and the
last rows of the grid; expected values come only from the oracle.
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from sparse_attention_kv_paged_amd import lib as L
from sparse_attention_kv_paged_amd import workloads as W
from tests.parity import assert_logits_close
from tests.test_parity_gpu import _check_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def _log(msg):
    print(msg, flush=True)


def _flip_some_scales(wl, seed):
    sc = wl.pool[:, 128:].copy().view("<f4")
    rng = np.random.default_rng(seed)
    sc[rng.random(len(sc)) < 0.3] *= -1
    sc[rng.random(len(sc)) < 0.05] = 0.0
    wl.pool[:, 128:] = sc.view(np.uint8)


def _roll_rows(wl, shift):
    """The same rows in another order (every per-row array rolled alike)."""
    wl.q = np.roll(wl.q, shift, axis=0)
    wl.w = np.roll(wl.w, shift, axis=0)
    wl.limits = np.roll(wl.limits, shift)
    wl.q_req = np.roll(wl.q_req, shift)


def _logits_only(wl, tag):
    """The logits-only launch (no scores, every column) against the oracle."""
    d = L.to_device(wl)
    g = L.idx_score(d.q, d.w, d.keys, d.n_cols).cpu().numpy()
    assert_logits_close(g, oracle.score(wl), f"{tag} logits only")


def test_one_request_causal_rows():
    """2048 prefill rows of one request (24 slots), causal bounds: logits,
    scores, top-512, logits only."""
    wl = W.prefill(4096, 2048, seed=41, name="rows-prefill")
    _check_workload(wl, tag="rows-prefill")
    _logits_only(wl, "rows-prefill")


def test_rows_over_several_slot_groups_negative_scales_holes():
    """88 slots per row (two 64-slot groups of table reads), negative and
    zero scales, an absent block, a padding row and an unknown request."""
    wl = W.prefill(20480, 2048, seed=42, name="rows-long")
    _flip_some_scales(wl, 43)
    wl.block_table = wl.block_table.copy()
    wl.block_table[0, 70] = -1                                 # hole in the second slot group
    wl.q_req = wl.q_req.copy()
    wl.q_req[5] = -1                                           # padding row
    wl.q_req[1030] = 3                                         # no such request: absent, flagged
    _check_workload(wl, tag="rows-long")


def test_status_bits_among_many_rows():
    """Out-of-range block id and request id among 2048 rows set their status
    bits and score as absent."""
    wl = W.prefill(4096, 2048, seed=44, name="rows-status")
    wl.block_table = wl.block_table.copy()
    wl.block_table[0, 7] = 10 ** 6                             # past the pool
    wl.q_req = wl.q_req.copy()
    wl.q_req[9] = 2                                            # no such request
    d = L.to_device(wl, status=True)
    g = L.idx_score(d.q, d.w, d.keys, d.n_cols).cpu().numpy()
    st = int(d.keys.status.cpu().item())
    assert st & L.STATUS_BAD_BLOCK and st & L.STATUS_BAD_REQUEST
    wl.block_table[0, 7] = -1                                  # what "absent" means
    wl.q_req[9] = -1
    assert_logits_close(g, oracle.score(wl), "rows status case")


def test_many_requests_adjacent_rows():
    """512 requests x 4 draft rows, each request's rows adjacent."""
    wl = W.speculative_decode(n_req=512, draft=4, seed=45, name="rows-aligned")
    _check_workload(wl, tag="rows-aligned")


def test_neighbouring_rows_of_different_requests():
    """The same rows rolled by two: neighbouring rows of different requests,
    negative and zero scales."""
    wl = W.speculative_decode(n_req=512, draft=4, seed=46, name="rows-mixed")
    _roll_rows(wl, 2)
    _flip_some_scales(wl, 47)
    _check_workload(wl, tag="rows-mixed")
    _logits_only(wl, "rows-mixed")


@pytest.mark.parametrize("B", [2049, 2050, 2051])
def test_no_writes_past_the_last_of_many_rows(B):
    """Nothing is written below row B, whatever B is modulo four."""
    wl = W.prefill(4096, B, seed=48, name="rows-tail")
    d = L.to_device(wl)
    guard = 8
    big_l = torch.full((B + guard, d.n_cols), 7.0, dtype=torch.float32, device="cuda")
    big_s = torch.full((B + guard, d.n_cols), 7.0, dtype=torch.float32, device="cuda")
    L.idx_score(d.q, d.w, d.keys, d.n_cols, with_scores=True, logits=big_l[:B], scores=big_s[:B])
    torch.cuda.synchronize()
    assert torch.all(big_l[B:] == 7.0) and torch.all(big_s[B:] == 7.0)
    assert bool(torch.all(big_l[:B] != 7.0))
    rows = [0, 1, 2047, 2048, B - 1]
    assert_logits_close(big_l[:B].cpu().numpy()[rows], oracle.score(wl, rows=rows), f"rows tail {B}")
