"""The oracle's pins must catch plausible slips.

Each case plants one mistake in a private copy of oracle/reference.py (on the
CPU; the real module is untouched) and checks that the hand-derived fixtures
and the rational brute force reject the mutant: its logits, and the per-entry
parity bound 2e-3 * sum_h |w_h| |X_h| + 1e-6 that every GPU comparison uses.
"""
import importlib.util
import os
import sys
import types

import numpy as np
import pytest

import golden_fixtures as gf
from oracle import exact
from workloads import make_fp4, make_fp8

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "reference.py")

MUTANTS = {
    "scale dropped": ("x = s[:lim, None] * sd", "x = sd"),
    "relu before scale": ("o64 = np.maximum(x, 0.0) @ w",
                          "o64 = (s[:lim, None] * np.maximum(sd, 0.0)) @ w"),
    "relu sign flipped": ("np.maximum(x, 0.0) @ w", "np.minimum(x, 0.0) @ w"),
    "causal offset off by one": ("return min(ctx - next_n + 1 + j, max_context_len)",
                                 "return min(ctx - next_n + j, max_context_len)"),
    "weights of the batch row": ("w = weights[r].astype(np.float64)",
                                 "w = weights[b].astype(np.float64)"),
    "query row swapped": ("sd = k[:lim] @ qd[b, j].T", "sd = k[:lim] @ qd[b, next_n - 1 - j].T"),
    "pages in table order of wrong row": ("block_table[b, :npg]", "block_table[0, :npg]"),
    "fp4 nibble order": ("out[..., 0::2] = lo", "out[..., 0::2] = hi"),
    "fp4 block scale stride": ("np.repeat(scl, 32, axis=1)", "np.tile(scl, (1, 32))"),
    # the per-entry parity bound 2e-3 * sum_h |w_h| |X_h| + 1e-6
    "bound factor 10x looser": ("2e-3 * (np.abs(x) @ np.abs(w))", "2e-2 * (np.abs(x) @ np.abs(w))"),
    "bound without the token scale": ("np.abs(x) @ np.abs(w)", "np.abs(sd) @ np.abs(w)"),
    "bound with signed weights": ("np.abs(x) @ np.abs(w)", "np.abs(x) @ w"),
    "bound of the rectified scores": ("np.abs(x) @ np.abs(w)", "np.maximum(x, 0.0) @ np.abs(w)"),
    "bound of the summed score": ("np.abs(x) @ np.abs(w)", "np.abs(x @ w)"),
    "bound floor dropped": ("(np.abs(x) @ np.abs(w)) + 1e-6", "(np.abs(x) @ np.abs(w))"),
}


def _load_mutant(old, new):
    with open(SRC) as f:
        code = f.read()
    fmt_path = os.path.join(os.path.dirname(SRC), "formats.py")
    with open(fmt_path) as f:
        fcode = f.read()
    if old in code:
        code = code.replace(old, new)
    else:
        assert old in fcode, old
        fcode = fcode.replace(old, new)
    pkg = types.ModuleType("mutant_oracle")
    pkg.__path__ = []
    fm = types.ModuleType("mutant_oracle.formats")
    exec(compile(fcode, "formats_mutant", "exec"), fm.__dict__)
    sys.modules["mutant_oracle"] = pkg
    sys.modules["mutant_oracle.formats"] = fm
    pkg.formats = fm
    rm = types.ModuleType("mutant_oracle.reference")
    rm.__package__ = "mutant_oracle"
    exec(compile(code, "reference_mutant", "exec"), rm.__dict__)
    return rm


def _tol_ok(tol, bound_rows):
    """tol against 2e-3 * bound + 1e-6 (exact or hand-derived bounds; None or
    a masked entry: 0)."""
    for i, row in enumerate(bound_rows):
        for t, v in enumerate(row):
            want = 0.0 if v is None else 2e-3 * float(v) + 1e-6
            if abs(tol[i, t] - want) > 1e-12 * want:
                return False
    return True


def _pins_pass(ref):
    """True when every pin used here accepts the implementation `ref`."""
    for case in range(2):
        f = gf.load_fp8(case)
        r = ref.paged_mqa_logits_fp8(f["q"], f["kv_cache"], f["weights"], f["context_lens"],
                                     f["block_table"], f["max_context_len"],
                                     page_size=f["page_size"], want_tol=True)
        if not np.array_equal(r["logits"].astype(np.float64), f["expected"]):
            return False
        hand = [[None if np.isneginf(e) else b for e, b in zip(f["expected"][0], f["bound"][0])]]
        if not _tol_ok(r["tol"], hand):
            return False
    f = gf.load_fp4()
    r = ref.paged_mqa_logits_fp4(f["q"], f["q_scale"], f["kv_cache"], f["weights"],
                                 f["context_lens"], f["block_table"], f["max_context_len"],
                                 page_size=f["page_size"], want_tol=True)
    if not np.array_equal(r["logits"].astype(np.float64), f["expected"]):
        return False
    hand = [[None if np.isneginf(e) else b for e, b in zip(f["expected"][0], f["bound"][0])]]
    if not _tol_ok(r["tol"], hand):
        return False
    d = make_fp8([3, 6, 2], next_n=2, max_context_len=7, seed=1, num_heads=3, head_dim=8,
                 page_size=2, negative_scales=True)
    r = ref.paged_mqa_logits_fp8(d["q"], d["kv_cache"], d["weights"], d["context_lens"],
                                 d["block_table"], d["max_context_len"], page_size=2,
                                 want_tol=True)
    ent = exact.entries_fp8(d["q"], d["kv_cache"], d["weights"], d["context_lens"],
                            d["block_table"], d["max_context_len"], page_size=2)
    for i, row in enumerate(ent):
        for t, e in enumerate(row):
            want = -np.inf if e is None else np.float32(float(e[0]))
            if r["logits"][i, t] != want:
                return False
    if not _tol_ok(r["tol"], [[None if e is None else e[1] for e in row] for row in ent]):
        return False
    d = make_fp4([5, 3], max_context_len=6, seed=2, num_heads=2, head_dim=64, page_size=2)
    r = ref.paged_mqa_logits_fp4(d["q"], d["q_scale"], d["kv_cache"], d["weights"],
                                 d["context_lens"], d["block_table"], d["max_context_len"],
                                 page_size=2, want_tol=True)
    ent = exact.entries_fp4(d["q"], d["q_scale"], d["kv_cache"], d["weights"],
                            d["context_lens"], d["block_table"], d["max_context_len"],
                            page_size=2)
    for i, row in enumerate(ent):
        for t, e in enumerate(row):
            want = -np.inf if e is None else np.float32(float(e[0]))
            if r["logits"][i, t] != want:
                return False
    return _tol_ok(r["tol"], [[None if e is None else e[1] for e in row] for row in ent])


def test_unmutated_oracle_passes_pins():
    assert _pins_pass(_load_mutant("", ""))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    assert not _pins_pass(_load_mutant(old, new)), name
