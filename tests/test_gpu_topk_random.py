"""select_topk against the oracle on seeded random cases: row counts,
widths, k, value distributions (normal, heavy ties, signed zeros, -inf
padding, equal rows), lengths and output offsets drawn together, so that
every selection path (copy, wavefront, workgroup listing, digit passes)
meets shapes the targeted tests do not name.  Batches of at most two rows
per compute unit give every row of more than k candidates a workgroup, so
the wavefront path is drawn with more rows than that."""
import numpy as np
import pytest
import torch

from gpu_util import announce
from oracle import topk as otk

pytestmark = pytest.mark.gpu
pmqa = pytest.importorskip("paged_mqa_logits_amd")


def _case(seed, many=False):
    rng = np.random.default_rng(seed)
    if many:   # more rows than two per compute unit, mostly wavefront rows
        rows = int(rng.integers(513, 1100))
        M = int(rng.choice([300, 2100, 4097, 6143, 6144, 6145, 9000]))
    else:
        rows = int(rng.integers(1, 160))
        M = int(rng.choice([7, 300, 2100, 6143, 6145, 9000, 20000, 70000]))
    k = int(rng.choice([1, 3, 64, 255, 256, 257, 1000, 2047, 2048, 3001]))
    kind = seed % 5
    if kind == 0:
        x = rng.standard_normal((rows, M)).astype(np.float32)
    elif kind == 1:  # heavy ties
        x = np.round(rng.standard_normal((rows, M)), 1).astype(np.float32)
    elif kind == 2:  # signed zeros, infinities and a few values
        pool = np.array([-np.inf, -1.0, -0.0, 0.0, 0.25, 1.0, np.inf], np.float32)
        x = rng.choice(pool, size=(rows, M)).astype(np.float32)
    elif kind == 3:  # finite values then -inf (a length past the context)
        x = np.full((rows, M), -np.inf, np.float32)
        fin = rng.integers(0, M + 1, size=rows)
        for r in range(rows):
            x[r, :fin[r]] = rng.standard_normal(fin[r]).astype(np.float32)
    else:  # scaled logits with some equal rows
        x = (rng.standard_normal((rows, M)) * 30 + 5).astype(np.float32)
        x[::4] = np.float32(2.5)
    n = rng.integers(0, M + 1, size=rows).astype(np.int32)
    if rows > 2:
        n[0], n[1] = M, min(M, k)
    off = int(rng.integers(0, 4))
    return x, n, k, off


def _run(seed, many):
    x, n, k, off = _case(seed, many)
    rows, M = x.shape
    announce(f"select_topk random seed {seed} many={many}: rows {rows} M {M} k {k} offset {off}")
    ib = torch.full((rows, k + 4), -7, dtype=torch.int32, device="cuda")
    vb = torch.full((rows, k + 4), 7.0, dtype=torch.float32, device="cuda")
    ld = (M + 3) // 4 * 4                            # row stride: a multiple of 4 columns
    buf = torch.full((rows, ld), float("nan"), device="cuda")
    buf[:, :M] = torch.from_numpy(x).cuda()          # NaN past the width: never read
    idx, val = pmqa.select_topk(buf[:, :M], torch.from_numpy(n).cuda(), k,
                                indices=ib[:, off:off + k], values=vb[:, off:off + k],
                                select_workspace=None)
    gi, gv = idx.cpu().numpy(), val.cpu().numpy()
    for r in range(rows):
        wi, wv = otk.select_topk(x[r], int(n[r]), k)
        assert np.array_equal(gi[r], wi), (seed, r)
        assert np.array_equal(gv[r].view(np.uint32), wv.view(np.uint32)), (seed, r)


@pytest.mark.parametrize("seed", range(40))
def test_select_topk_random_cases(seed):
    _run(seed, False)


@pytest.mark.parametrize("seed", range(100, 112))
def test_select_topk_random_many_rows(seed):
    _run(seed, True)
