"""Element-by-element comparison of GPU logits with the oracle.

The bar: every entry the oracle masks must be exactly -inf (bit pattern
0xFF800000); every other entry must be finite and within the oracle's
per-entry bound |gpu - oracle| <= 2e-3 * sum_h |w_h| |scale_t q_h.k_t| + 1e-6.
No NaN anywhere.
"""
import numpy as np

NEG_INF_BITS = np.uint32(0xFF800000)


def check(gpu, ref, label=""):
    """gpu: float32 [rows, M]; ref: oracle dict with 'logits' and 'tol'."""
    gpu = np.asarray(gpu, dtype=np.float32)
    want = ref["logits"]
    tol = ref["tol"]
    assert gpu.shape == want.shape, (label, gpu.shape, want.shape)
    assert not np.isnan(gpu).any(), f"{label}: NaN in GPU output"
    masked = np.isneginf(want)
    gbits = gpu.view(np.uint32)
    bad_mask = masked & (gbits != NEG_INF_BITS)
    assert not bad_mask.any(), (f"{label}: {int(bad_mask.sum())} masked entries not -inf, "
                                f"first at {np.argwhere(bad_mask)[:5].tolist()}")
    unmasked = ~masked
    assert np.isfinite(gpu[unmasked]).all(), (
        f"{label}: non-finite unmasked entries at {np.argwhere(unmasked & ~np.isfinite(gpu))[:5].tolist()}")
    with np.errstate(invalid="ignore"):
        err = np.abs(gpu.astype(np.float64) - want.astype(np.float64))
    over = unmasked & (err > tol)
    if over.any():
        idx = np.argwhere(over)[:5]
        details = [(int(i), int(j), float(gpu[i, j]), float(want[i, j]), float(tol[i, j]))
                   for i, j in idx]
        raise AssertionError(f"{label}: {int(over.sum())} entries outside tolerance: {details}")
    ratio = float((err[unmasked] / tol[unmasked]).max()) if unmasked.any() else 0.0
    return {"masked": int(masked.sum()), "checked": int(unmasked.sum()), "max_err_over_tol": ratio}


def check_topk(idx, val, ref, n_rows, k, label=""):
    """Top-k of GPU rows against the fp64 oracle.

    idx, val: GPU output [rows, k]; ref: oracle dict of those rows (logits,
    tol); n_rows: candidate count per row.  Checks the layout (ascending
    columns below n, then -1 / -inf), each value within tolerance of the
    oracle, and that the selection is one a tie-aware reader of the oracle
    could make: no unselected candidate exceeds a selected one by more than
    their two tolerances."""
    want, tol = ref["logits"], ref["tol"]
    for r in range(idx.shape[0]):
        n = int(n_rows[r])
        cnt = min(k, n)
        sel = idx[r, :cnt].astype(np.int64)
        assert np.all(idx[r, cnt:] == -1) and np.all(np.isneginf(val[r, cnt:])), (label, r)
        assert np.all(np.diff(sel) > 0) and (cnt == 0 or (sel[0] >= 0 and sel[-1] < n)), \
            (label, r)
        if cnt == 0:
            continue
        assert np.all(np.abs(val[r, :cnt].astype(np.float64) - want[r, sel]) <= tol[r, sel]), \
            (label, r)
        if cnt < n:
            mask = np.ones(n, bool)
            mask[sel] = False
            lo = np.min(want[r, sel] + tol[r, sel])
            hi = np.max(want[r, :n][mask] - tol[r, :n][mask])
            assert hi <= lo, (label, r, hi, lo)
