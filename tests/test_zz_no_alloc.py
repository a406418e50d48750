"""The allocation-free entry point (idx_score_topk_noalloc, through the C ABI)
against idx_score_topk with a caller-owned workspace.

Both run the same kernels on the same inputs, so the selected ids and their
logits must be identical (index work: bit-exact).  Two calls in a row on the
static scratch, the second with a smaller input, then the largest decode
shape; and a call beyond the scratch is refused."""
import numpy as np
import pytest
import torch

from oracle import oracle
from sparse_attention_kv_paged_amd import lib as L
from sparse_attention_kv_paged_amd import workloads as W
from tests.parity import assert_topk_near_tie

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def _reference(wl):
    d = L.to_device(wl)
    idx, val = L.idx_score_topk(d.q, d.w, d.keys, d.n_cols, wl.k)
    torch.cuda.synchronize()
    return d, idx.cpu().numpy(), val.cpu().numpy()


def test_noalloc_equals_workspace_entry_point_on_consecutive_calls():
    big = W.config(1)                     # decode-batch: 32 rows, up to 32768 columns
    small = W.small_config(4)             # a smaller chunk-list workload afterwards
    print(f"[noalloc] {big.name}: {big.description}; then {small.name}: {small.description}", flush=True)
    d_big, ref_big, val_big = _reference(big)
    d_small, ref_small, val_small = _reference(small)
    out_big = L.idx_score_topk_noalloc(d_big.q, d_big.w, d_big.keys, d_big.n_cols, big.k)
    out_small = L.idx_score_topk_noalloc(d_small.q, d_small.w, d_small.keys, d_small.n_cols, small.k)
    torch.cuda.synchronize()
    for name, (idx, val), ref, rval in (("first", out_big, ref_big, val_big),
                                        ("second", out_small, ref_small, val_small)):
        assert np.array_equal(idx.cpu().numpy(), ref), f"{name} call: ids differ"
        assert np.array_equal(val.cpu().numpy().view(np.uint32), rval.view(np.uint32)), f"{name} call: values differ"
    # and the smaller call against the oracle, near-ties allowed
    lg = oracle.score(small)
    cols, _ = oracle.topk(lg, small.k)
    ref_ids = oracle.cols_to_entries(small, cols)

    def logit_of(b, ids):
        ids = np.asarray(ids, dtype=np.int64)
        bs = small.block_size
        pos = {int(c): j for j, c in enumerate(small.chunk_ids[b][:small.n_chunks[b]])}
        return lg[b, np.array([pos[int(e) // bs] * bs + int(e) % bs for e in ids], dtype=np.int64)]
    assert_topk_near_tie(out_small[0].cpu().numpy(), ref_ids, logit_of, small.k, "noalloc small")


def test_noalloc_long_decode_then_tiny():
    """The largest decode shape (8 rows x 262,144 entries, 16 top-k parts per
    row merged in the same launch), then a one-row call on the same scratch."""
    for wl in (W.config(2), W.config(0)):
        print(f"[noalloc] {wl.name}: {wl.description}", flush=True)
        d, ref, rval = _reference(wl)
        idx, val = L.idx_score_topk_noalloc(d.q, d.w, d.keys, d.n_cols, wl.k)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), ref), wl.name
        assert np.array_equal(val.cpu().numpy().view(np.uint32), rval.view(np.uint32)), wl.name


def test_noalloc_refuses_a_call_beyond_its_scratch():
    wl = W.config(3)                      # 4096-row prefill: its workspace is ~285 MB
    d = L.to_device(wl)
    with pytest.raises(L.IdxError) as e:
        L.idx_score_topk_noalloc(d.q, d.w, d.keys, d.n_cols, wl.k)
    assert e.value.code == L.IDX_E_WORKSPACE
