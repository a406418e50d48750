"""Comparison rules shared by the GPU parity tests.

Tolerance (fp32 accumulation vs the double oracle): a scored column passes if
|gpu - oracle| <= ATOL + RTOL * |oracle|; an unscored column must be exactly
-inf on both sides.  Top-k sets may differ only at near-ties: every entry in
the symmetric difference of the GPU and oracle sets must have an oracle logit
within the same tolerance of the oracle's k-th value.
"""
import numpy as np

ATOL = 1e-4
RTOL = 2e-3


def assert_logits_close(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    masked = ref == -np.inf
    assert np.array_equal(gpu == -np.inf, masked), f"{what}: -inf pattern differs"
    g, r = gpu[~masked], ref[~masked]
    assert np.all(np.isfinite(g)), f"{what}: non-finite logit at a scored column"
    err = np.abs(g - r)
    bound = ATOL + RTOL * np.abs(r)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} logits out of tolerance; "
                           f"worst err {err.max():.3e} (bound there {bound[np.argmax(err)]:.3e})")
    # how much of the tolerance the worst logit uses (printed for the record)
    used = float((err / bound).max()) if err.size else 0.0
    print(f"[tol] {what}: {err.size} logits, worst err/bound {used:.4f}, "
          f"median err {float(np.median(err)) if err.size else 0.0:.3e}", flush=True)
    return used


def assert_topk_near_tie(gpu_idx, ref_idx, ref_logit_of_entry, k, what=""):
    """gpu_idx/ref_idx: [B, k] logical entry ids (-1 padded);
    ref_logit_of_entry(b, ids) -> oracle logits of those entries (double)."""
    gpu_idx = np.asarray(gpu_idx)
    ref_idx = np.asarray(ref_idx)
    for b in range(ref_idx.shape[0]):
        ref_set = ref_idx[b][ref_idx[b] >= 0]
        gpu_set = gpu_idx[b][gpu_idx[b] >= 0]
        assert len(np.unique(gpu_set)) == len(gpu_set), f"{what} row {b}: duplicate ids"
        assert len(gpu_set) == len(ref_set), f"{what} row {b}: {len(gpu_set)} vs {len(ref_set)} selected"
        if len(ref_set) == 0:
            continue
        assert np.all(gpu_idx[b][len(gpu_set):] == -1), f"{what} row {b}: padding not at the end"
        diff = np.setxor1d(gpu_set, ref_set)
        if len(diff) == 0:
            continue
        if len(ref_set) < k:
            raise AssertionError(f"{what} row {b}: sets differ although all entries fit")
        lg = ref_logit_of_entry(b, diff)
        t = ref_logit_of_entry(b, ref_set[-1:])[0]     # oracle's k-th value
        tol = ATOL + RTOL * abs(t)
        far = np.abs(lg - t) > tol
        assert not far.any(), (f"{what} row {b}: {far.sum()} differing ids are not near-ties "
                               f"(k-th {t:.6g}, offending {lg[far][:4]})")


def column_order(cols, vals=None):
    """Reorder each row's selected columns ascending (-1 padding last), the
    order the GPU top-k writes; the oracle lists them by value."""
    cols = np.asarray(cols)
    out_c = np.full_like(cols, -1)
    out_v = None if vals is None else np.full(np.shape(vals), -np.inf, dtype=np.asarray(vals).dtype)
    for b in range(cols.shape[0]):
        sel = np.nonzero(cols[b] >= 0)[0]
        order = sel[np.argsort(cols[b][sel], kind="stable")]
        out_c[b, :len(order)] = cols[b][order]
        if vals is not None:
            out_v[b, :len(order)] = np.asarray(vals)[b][order]
    return (out_c, out_v) if vals is not None else out_c
