"""select_topk_noalloc: the selection with its split workspace in the
library's static scratch, called through the C ABI, against select_topk (a
caller's workspace, and none) bit for bit, and against the top-k oracle, on
two calls in a row, the second with a smaller input."""
import numpy as np
import pytest
import torch

from gpu_util import announce
from oracle import topk as otk

pytestmark = pytest.mark.gpu
pmqa = pytest.importorskip("paged_mqa_logits_amd")


def _rows(seed, rows, M, k):
    """Logits with ties and signed zeros, and candidate counts covering
    n <= k, rows kept in LDS and rows long enough to be split."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, M)).astype(np.float32)
    x[:, ::7] = np.round(x[:, ::7], 1)             # ties
    x[:, 3::11] = 0.0
    x[:, 5::13] = -0.0
    n = rng.integers(M // 3, M + 1, size=rows).astype(np.int32)
    n[0] = k // 2                                   # fewer candidates than k
    n[1] = min(M, 7000)                             # kept in LDS
    n[2] = M                                        # the longest
    return x, n


def _check(x, n, k, label):
    rows, M = x.shape
    ld = (M + 3) // 4 * 4
    buf = torch.zeros((rows, ld), dtype=torch.float32, device="cuda")
    buf[:, :M] = torch.from_numpy(x).cuda()
    lg = buf[:, :M]
    lens = torch.from_numpy(n).cuda()
    idx = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    val = torch.full((rows, k), 7.0, dtype=torch.float32, device="cuda")
    i0, v0 = pmqa.select_topk_noalloc(lg, lens, k, indices=idx, values=val)
    i1, v1 = pmqa.select_topk(lg, lens, k, select_workspace="auto")
    i2, v2 = pmqa.select_topk(lg, lens, k, select_workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(i0, i1) and torch.equal(v0.view(torch.int32), v1.view(torch.int32)), label
    assert torch.equal(i0, i2) and torch.equal(v0.view(torch.int32), v2.view(torch.int32)), label
    gi, gv = i0.cpu().numpy(), v0.cpu().numpy()
    for r in range(rows):
        wi, wv = otk.select_topk(x[r], int(n[r]), k)
        assert np.array_equal(gi[r], wi), (label, r)
        assert np.array_equal(gv[r].view(np.uint32), wv.view(np.uint32)), (label, r)


def test_noalloc_matches_select_topk_on_two_calls():
    k = 2048
    announce("select_topk_noalloc call 1: 24 rows x 600000")
    assert pmqa.select_workspace_bytes(24, 600000, k) > 0    # the split path runs
    x, n = _rows(90, 24, 600000, k)
    _check(x, n, k, "call 1")
    announce("select_topk_noalloc call 2: 9 rows x 530001")
    assert pmqa.select_workspace_bytes(9, 530001, k) > 0
    x, n = _rows(91, 9, 530001, k)
    _check(x, n, k, "call 2")


def test_noalloc_without_split_rows():
    """More rows than are ever split, and rows all short enough for LDS:
    the scratch is not used, the result is the same."""
    announce("select_topk_noalloc: 600 rows x 9000, 5 rows x 3000")
    x, n = _rows(92, 600, 9000, 300)
    _check(x, n, 300, "600 rows")
    x, n = _rows(93, 5, 3000, 300)
    _check(x, n, 300, "5 rows")
