"""HIP-graph capture of every entry point (through the C ABI).

Bounds, tables and chunk lists stay on the device and the library neither
allocates nor synchronises, so each call can be captured once and replayed
("DeepSeek-V4.1 native paged runtime", "Current execution scope": calls are
graph-capturable).  Each case runs the call eagerly for the expected
outputs, captures it, and replays the graph several times; before every
replay the outputs are overwritten and other eager calls (on other inputs,
sharing the workspace) run and are waited for.  Every replay must give the
eager outputs bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from sparse_attention_kv_paged_amd import lib as L
from sparse_attention_kv_paged_amd import workloads as W
from tests.parity import column_order

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def _replay_check(tag, call, outs, between=None, n_replays=3, reset=None):
    print(f"[graph] {tag}", flush=True)
    call()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i in range(n_replays):
        if reset is None:
            for o in outs:
                o.fill_(7)
        else:
            reset()
        if between is not None:
            between()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(_bits(o), _bits(r)), f"{tag}: replay {i} differs from the eager result"


def _other_q(d, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn(d.q.shape, generator=g).to(torch.bfloat16).to(d.q.device)


@pytest.mark.parametrize("name,wl", [
    ("decode", lambda: W.small_config(1)),
    ("long-rows", lambda: W.small_config(2)),
    ("chunks", lambda: W.small_config(4)),
    ("chunks-b16", lambda: W.reblock(W.small_config(4), seed=70)),
    ("per-row", lambda: W.prefill(4096, 600, seed=71, name="graph-rows")),
])
def test_score_topk_replays(name, wl):
    wl = wl()
    d = L.to_device(wl)
    out_idx = torch.empty((wl.B, wl.k), dtype=torch.int32, device="cuda")
    out_val = torch.empty((wl.B, wl.k), dtype=torch.float32, device="cuda")
    ws = L.new_workspace(L.workspace_bytes(L.IDX_OP_SCORE_TOPK, wl.B, wl.n_cols, wl.k), "cuda")
    q2 = _other_q(d, 1)
    o2 = (torch.empty_like(out_idx), torch.empty_like(out_val))

    def call():
        L.idx_score_topk(d.q, d.w, d.keys, wl.n_cols, wl.k, out_idx=out_idx, out_val=out_val, workspace=ws)

    def between():
        L.idx_score_topk(q2, d.w, d.keys, wl.n_cols, wl.k, out_idx=o2[0], out_val=o2[1], workspace=ws)

    _replay_check(f"score_topk {name}", call, [out_idx, out_val], between)


def test_score_with_scores_replays():
    wl = W.small_config(2)
    d = L.to_device(wl)
    lg = torch.empty((wl.B, wl.n_cols), dtype=torch.float32, device="cuda")
    sc = torch.empty_like(lg)
    q2 = _other_q(d, 2)

    def call():
        L.idx_score(d.q, d.w, d.keys, wl.n_cols, with_scores=True, logits=lg, scores=sc)

    _replay_check("score", call, [lg, sc],
                  lambda: L.idx_score(q2, d.w, d.keys, wl.n_cols, with_scores=True))


@pytest.mark.parametrize("B,n,k", [(3, 300000, 2048), (3, 40000, 512), (256, 20000, 512)])
def test_topk_replays(B, n, k):
    """Rows longer than one merge (separate list-merge launches), and many
    rows of one long segment each (candidates compacted in LDS, two
    workgroups per CU)."""
    rng = np.random.default_rng(72)
    lg = torch.from_numpy(rng.standard_normal((B, n), dtype=np.float32)).cuda()
    oc = torch.empty((B, k), dtype=torch.int32, device="cuda")
    ov = torch.empty((B, k), dtype=torch.float32, device="cuda")
    ws = L.new_workspace(max(L.workspace_bytes(L.IDX_OP_TOPK, B, n, k), 1), "cuda")
    lg2 = -lg

    def call():
        L.idx_topk(lg, k, out_col=oc, out_val=ov, workspace=ws)

    _replay_check(f"topk {n} {k}", call, [oc, ov], lambda: L.idx_topk(lg2, k, workspace=ws))


def test_topk_sampled_threshold_rerun_replays():
    """Many rows of one long segment each with k <= 640 select through a
    threshold sampled from the first value of every thread's 40 columns; the
    rows whose samples misrepresent them (every 7th row: the sampled columns
    far above the rest) are re-run by a second launch that reads the first
    launch's flags.  The calls between the replays negate the logits, so other
    rows (the sampled columns now far below) are flagged: each launch must
    rewrite every flag."""
    rng = np.random.default_rng(73)
    B, n, k = 256, 20000, 512
    vals = rng.standard_normal((B, n), dtype=np.float32)
    vals[::7, ::40] += 1000.0
    lg = torch.from_numpy(vals).cuda()
    oc = torch.empty((B, k), dtype=torch.int32, device="cuda")
    ov = torch.empty((B, k), dtype=torch.float32, device="cuda")
    ws = L.new_workspace(max(L.workspace_bytes(L.IDX_OP_TOPK, B, n, k), 1), "cuda")
    lg2 = -lg

    def call():
        L.idx_topk(lg, k, out_col=oc, out_val=ov, workspace=ws)

    _replay_check("topk sampled threshold", call, [oc, ov], lambda: L.idx_topk(lg2, k, workspace=ws))
    ref_cols, ref_v = column_order(*oracle.topk(vals.astype(np.float64), k))
    assert np.array_equal(oc.cpu().numpy(), ref_cols)
    assert np.array_equal(ov.cpu().numpy(), ref_v.astype(np.float32))


def test_quantised_query_replays():
    wl = W.small_config(1)
    d = L.to_device(wl)
    q8 = torch.empty((wl.B, wl.H, wl.D + 4), dtype=torch.uint8, device="cuda")
    slots = torch.arange(wl.B * wl.H, dtype=torch.int64, device="cuda")
    out_idx = torch.empty((wl.B, wl.k), dtype=torch.int32, device="cuda")
    out_val = torch.empty((wl.B, wl.k), dtype=torch.float32, device="cuda")
    ws = L.new_workspace(L.workspace_bytes(L.IDX_OP_SCORE_TOPK, wl.B, wl.n_cols, wl.k), "cuda")
    q2 = _other_q(d, 3)

    def call():
        L.quantize_q(d.q, out=q8, slots=slots)
        L.idx_score_topk_q8(q8, d.w, d.keys, wl.n_cols, wl.k, out_idx=out_idx, out_val=out_val, workspace=ws)

    def between():
        L.idx_score_topk_q8(L.quantize_q(q2), d.w, d.keys, wl.n_cols, wl.k, workspace=ws)

    _replay_check("quantised query", call, [q8, out_idx, out_val], between)


def test_query_quantised_in_kernel_replays():
    wl = W.small_config(1)
    d = L.to_device(wl)
    out_idx = torch.empty((wl.B, wl.k), dtype=torch.int32, device="cuda")
    out_val = torch.empty((wl.B, wl.k), dtype=torch.float32, device="cuda")
    ws = L.new_workspace(L.workspace_bytes(L.IDX_OP_SCORE_TOPK, wl.B, wl.n_cols, wl.k), "cuda")
    q2 = _other_q(d, 4)

    def call():
        L.idx_score_topk_fp8q(d.q, d.w, d.keys, wl.n_cols, wl.k, out_idx=out_idx, out_val=out_val, workspace=ws)

    def between():
        L.idx_score_topk_fp8q(q2, d.w, d.keys, wl.n_cols, wl.k, workspace=ws)

    _replay_check("query quantised in the kernel", call, [out_idx, out_val], between)


def test_select_resident_replays():
    rl = W.memory_indexer(entries=[20000, 9000, 64, 40000], n_layers=3, kmax=96, seed=73)
    dl = [L.to_device(x) for x in rl.layers]
    pages = torch.empty((rl.B, rl.kmax), dtype=torch.int32, device="cuda")
    count = torch.empty(rl.B, dtype=torch.int32, device="cuda")
    ws = L.new_workspace(L.resident_workspace_bytes(3, rl.B, rl.n_cols, rl.kmax), "cuda")
    q2 = [_other_q(d, 10 + i) for i, d in enumerate(dl)]

    def run(qs, p, c):
        L.idx_select_resident(qs, [d.w for d in dl], [d.keys for d in dl], rl.n_cols, rl.kmax,
                              threshold=rl.threshold, n_sink=1, n_recent=1, out_pages=p, out_count=c, workspace=ws)

    _replay_check("select_resident", lambda: run([d.q for d in dl], pages, count), [pages, count],
                  lambda: run(q2, None, None))


def test_mxfp4_replays():
    wl = W.small_config(4)
    d = L.to_device(wl)
    out_idx = torch.empty((wl.B, wl.k), dtype=torch.int32, device="cuda")
    out_val = torch.empty((wl.B, wl.k), dtype=torch.float32, device="cuda")
    ws = L.new_workspace(L.workspace_bytes(L.IDX_OP_SCORE_TOPK, wl.B, wl.n_cols, wl.k), "cuda")
    q2 = _other_q(d, 5)

    def call():
        L.idx_score_topk_mxfp4(d.q, d.w, d.keys, wl.n_cols, wl.k, out_idx=out_idx, out_val=out_val, workspace=ws)

    def between():
        L.idx_score_topk_mxfp4(q2, d.w, d.keys, wl.n_cols, wl.k, workspace=ws)

    _replay_check("mxfp4", call, [out_idx, out_val], between)


def test_select_resident_stacked_layers_replays():
    """The one-launch Level 1 (stacked layers, selection bits, counting
    selection) under capture."""
    rl = W.memory_indexer(entries=[20000, 9000, 64, 40000], n_layers=3, kmax=96, seed=74)
    dl = [L.to_device(x) for x in rl.layers]
    q_all = torch.stack([d.q for d in dl])
    w_all = torch.stack([d.w for d in dl])
    q_oth = torch.stack([_other_q(d, 20 + i) for i, d in enumerate(dl)])
    pages = torch.empty((rl.B, rl.kmax), dtype=torch.int32, device="cuda")
    count = torch.empty(rl.B, dtype=torch.int32, device="cuda")
    ws = L.new_workspace(L.resident_workspace_bytes(3, rl.B, rl.n_cols, rl.kmax), "cuda")

    def run(q, p, c):
        L.idx_select_resident([q[l] for l in range(3)], [w_all[l] for l in range(3)], [d.keys for d in dl],
                              rl.n_cols, rl.kmax, threshold=rl.threshold, n_sink=1, n_recent=1, out_pages=p,
                              out_count=c, workspace=ws)

    _replay_check("select_resident, stacked layers", lambda: run(q_all, pages, count), [pages, count],
                  lambda: run(q_oth, None, None))


def test_write_keys_replays():
    wk = W.index_fill(n_keys=5000, seed=74)
    k = torch.from_numpy(wk.k.view(np.int16)).cuda()
    slots = torch.from_numpy(wk.slots).cuda()
    pool0 = torch.from_numpy(wk.pool).cuda()
    pool = pool0.clone()
    other = torch.zeros_like(pool)

    def call():
        L.idx_write_keys(k, slots, pool)

    # rows no slot names keep what they held, so each replay starts from
    # the poisoned pool again
    _replay_check("write_keys", call, [pool], lambda: L.idx_write_keys(k, slots, other),
                  reset=lambda: pool.copy_(pool0))
