"""Reference top-k token selection over rows of logits.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Page "[flashinfer] ... Paged MQA Logits ...", introduction: the logits feed
the indexer, which selects KV tokens by them.  The page gives neither k nor
an order, so the reading here (the plainest one):

* a row's candidates are its first n columns (n = its number of scored
  tokens);
* the selection is the k largest candidates under the total order of fp32
  values in which -0 < +0 (no NaN), equal values ordered by token index,
  lower first;
* the selected token indices are returned in ascending order, with their
  values; when n < k every candidate is selected and the remaining k - n
  entries are index -1, value -inf.

For the fused indexer path a row r = b * next_n + j has
n = min(causal limit, 256 * c_b, max_context_len), c_b the row's unit count
in the schedule (the columns a scheduled unit covers), or 0 when the schedule
does not belong to the call.

Pins: ``tests/test_oracle_topk.py`` (brute force over all subsets of tiny
rows, a library sort, hand cases with ties and signed zeros).
"""
import numpy as np


def order_key(values):
    """uint64 keys ordering fp32 values as described above (-0 < +0)."""
    v = np.asarray(values, dtype=np.float32)
    if np.isnan(v).any():
        raise ValueError("NaN has no place in the order")
    b = v.view(np.uint32).astype(np.uint64)
    neg = (b >> np.uint64(31)) == 1
    return np.where(neg, np.uint64(0xFFFFFFFF) - b, b + np.uint64(0x80000000))


def select_topk(values, n, k):
    """(indices int32 [k], values float32 [k]) of the top k of values[:n]."""
    row = np.asarray(values, dtype=np.float32)[:n]
    idx = np.full(k, -1, dtype=np.int32)
    val = np.full(k, -np.inf, dtype=np.float32)
    if n <= 0:
        return idx, val
    key = order_key(row)
    # primary: descending key (ascending bitwise complement); secondary:
    # ascending index
    order = np.lexsort((np.arange(len(row)), ~key))
    take = np.sort(order[:min(k, len(row))])
    idx[:len(take)] = take
    val[:len(take)] = row[take]
    return idx, val


def fused_row_length(ctx_b, next_n, j, max_context_len, units_b):
    """Candidates of output row (b, j) on the fused indexer path."""
    lim = int(ctx_b) - next_n + 1 + j
    return max(0, min(lim, 256 * int(units_b), int(max_context_len)))
