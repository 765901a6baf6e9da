"""Reference partition of work units over persistent workers.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: page "[flashinfer] ... Paged MQA Logits ...", sections 1-2 and the
general lessons.  The work of one call is cut into 256-token units of one
row (the lessons state that schedule metadata stays valid only while every
ceil(context_len / 256) is unchanged), rows of length zero contribute no
unit and are skipped by the task iterator (section 1, first bullet), and each
persistent worker's share is found by searching the prefix sum of per-row unit
counts: a linear scan before the change, a binary search after it (section 1,
third bullet).

Reading of the partition rule (the pages give no formula): with c_b units in
row b, T = sum_b c_b and W workers, worker w takes global unit indices
[floor(w*T/W), floor((w+1)*T/W)).  Global index g lies in row b when
S[b] <= g < S[b+1] (S the exclusive prefix sum of c), at unit u = g - S[b].
Worker W's start is the terminal pair (B, 0).

Both searches are written here so that they pin each other and a brute-force
enumeration; the GPU schedule must equal them exactly.
"""
from bisect import bisect_right

UNIT_TOKENS = 256


def units_per_row(context_lens, unit=UNIT_TOKENS):
    """c_b = ceil(ctx_b / unit); negative lengths are rejected."""
    out = []
    for b, L in enumerate(context_lens):
        L = int(L)
        if L < 0:
            raise ValueError(f"context_lens[{b}] = {L} < 0")
        out.append(-(-L // unit))
    return out


def worker_boundary(w, total, num_workers):
    """Global index of worker w's first unit: floor(w*T/W) in exact integers."""
    return (w * total) // num_workers


def starts_linear(c, num_workers):
    """Start (row, unit) of every worker 0..W by linear scan over rows."""
    B = len(c)
    T = sum(c)
    starts = []
    for w in range(num_workers + 1):
        g = worker_boundary(w, T, num_workers)
        acc = 0
        found = (B, 0)
        for b in range(B):
            if acc <= g < acc + c[b]:
                found = (b, g - acc)
                break
            acc += c[b]
        starts.append(found)
    return starts


def starts_binary(c, num_workers):
    """Start (row, unit) of every worker 0..W by binary search of prefix sums."""
    B = len(c)
    S = [0]
    for x in c:
        S.append(S[-1] + x)
    T = S[-1]
    starts = []
    for w in range(num_workers + 1):
        g = worker_boundary(w, T, num_workers)
        b = bisect_right(S, g) - 1          # last b with S[b] <= g
        starts.append((b, g - S[b]))
    return starts


def prefix_sums(c):
    """Exclusive prefix sum S[0..B] of the unit counts."""
    S = [0]
    for x in c:
        S.append(S[-1] + x)
    return S


def enumerate_units(c):
    """Every (row, unit) pair in row-major order: the global unit sequence."""
    return [(b, u) for b in range(len(c)) for u in range(c[b])]


def worker_units_bruteforce(c, num_workers):
    """Units of each worker by slicing the enumerated sequence."""
    seq = enumerate_units(c)
    T = len(seq)
    return [seq[worker_boundary(w, T, num_workers):worker_boundary(w + 1, T, num_workers)]
            for w in range(num_workers)]


def advance(c, b, u):
    """Task iterator step: next unit after (b, u), skipping rows with no unit."""
    B = len(c)
    u += 1
    if u < c[b]:
        return b, u
    b += 1
    while b < B and c[b] == 0:
        b += 1
    return b, 0


def walk(c, start, end):
    """Units visited by a worker that iterates from start up to (not incl.) end."""
    B = len(c)
    b, u = start
    out = []
    while b < B and (b, u) < end:
        out.append((b, u))
        b, u = advance(c, b, u)
    return out
