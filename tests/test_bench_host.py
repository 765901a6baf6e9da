"""Host-side logic of bench.py: the algorithmic byte count and scored-token
count the reported figures divide by, and the readers of the committed
counter summaries (no GPU)."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_algorithmic_bytes_fp8_by_hand():
    # two rows: 100 tokens (2 pages) and 0; next_n 1, 64 heads, D 128, M 256
    ctx = np.array([100, 0], np.int32)
    got = bench.algorithmic_bytes(ctx, 1, 256, 64, 128, 64, sched_bytes=40)
    k = 132 * 100                       # 128 E4M3 + 4-byte scale per token
    table = 4 * 2                       # block-table entries of the used pages
    qw = 2 * 64 * (128 + 4)             # q + weight per head per row
    out = 4 * 2 * 256                   # every logit, -inf included
    assert got == k + table + qw + 4 * 2 + out + 40


def test_algorithmic_bytes_fp4_next_n_and_truncation():
    # one row of 300 tokens, output width 200: only 200 tokens are read
    ctx = np.array([300], np.int32)
    got = bench.algorithmic_bytes(ctx, 2, 200, 16, 128, 64, sched_bytes=0, variant="fp4")
    k = 68 * 200                        # 64 packed + 4 E8M0 per token
    table = 4 * 4                       # ceil(200 / 64) pages
    qw = 1 * 2 * 16 * (64 + 4 + 4)      # packed q + its scales + weight per head
    out = 4 * 2 * 200
    assert got == k + table + qw + 4 + out


def test_scored_tokens_causal_offset_and_truncation():
    ctx = np.array([10, 1, 0, 500], np.int32)
    # next_n 2: rows score ctx - 1 + j tokens, clipped to [0, 300]
    want = (9 + 10) + (0 + 1) + (0 + 0) + (300 + 300)
    assert bench.scored_tokens(ctx, 2, 300) == want
    assert bench.scored_tokens(ctx, 1, 300) == 10 + 1 + 0 + 300


def test_strip_comments_keeps_code():
    src = "int a; // one\n/* two\nlines */ int b;\n\n  // three\nint c;\n"
    assert bench.strip_comments(src) == "int a;\n int b;\nint c;"
    assert bench.strip_comments("x = 1  # no\n# gone\ny = 2\n", python=True) == "x = 1  # no\ny = 2"


def test_summary_readers_follow_the_hash(tmp_path, monkeypatch):
    traffic = tmp_path / "traffic.txt"
    traffic.write_text("# header\nkernel_source_hash = abc\nhbm_bytes_per_launch = 1234\n")
    mfma = tmp_path / "mfma.txt"
    mfma.write_text("# kernel source hash (bench.py kernel_source_hash): abc\n"
                    "workload, kernel, dispatches, MfmaUtil_pct\nlarge_fp8, k, 3, 15.5\n")
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(traffic))
    monkeypatch.setattr(bench, "MFMA_SUMMARY", str(mfma))
    assert bench.read_traffic("abc", 0) == 1234.0
    assert bench.read_traffic("other", 0) is None
    assert bench.read_mfma_busy("abc", "large_fp8") == 15.5
    assert bench.read_mfma_busy("abc", "mxfp4") is None
    assert bench.read_mfma_busy("other", "large_fp8") is None


def test_pages_read_by_hand():
    """The ceiling gather's page list: the first ceil(min(ctx, M)/64) entries
    of each row, in row order."""
    bt = np.array([[7, 8, 9, 10], [3, 4, 5, 6], [1, 2, 11, 12]], np.int32)
    ctx = np.array([65, 0, 300], np.int32)
    got = bench.pages_read(ctx, bt, 200, 64)           # row 2 truncated to 200 -> 4 pages
    assert got.tolist() == [7, 8, 1, 2, 11, 12]
    assert got.dtype == np.int32 and got.flags["C_CONTIGUOUS"]
