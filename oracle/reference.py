"""fp64 reference for paged MQA logits (fp8 and MXFP4 variants).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Definition followed
-------------------
Page "[flashinfer] Blackwell 아키텍처를 위한 고성능 Paged MQA Logits 커널 도입",
introduction: the sparse-attention indexer chooses KV tokens by a score that
passes each head's query-key product through ReLU, weights it per head and
sums over heads; an fp8 and an fp4 kernel compute it over a paged KV cache.
Written out (the plain reading of that description, with a per-token K
scale):

    S[r, h, t]  = sum_d q[r, h, d] * k[t, d]                 (exact in fp64)
    X[r, h, t]  = scale_t * S[r, h, t]
    logit[r, t] = sum_h w[r, h] * max(X[r, h, t], 0)          t <  lim_r
    logit[r, t] = -inf                                        t >= lim_r

Output row r = b * next_n + j is query j of batch row b.  Its causal limit is
lim_r = min(ctx_b - next_n + 1 + j, max_context_len); for next_n = 1 this is
the row's context length.  A row whose limit is <= 0 is all -inf.

Byte layouts (the pages give none; these are the readings this library uses):

* fp8 page (page_size tokens, head_dim D): ``page_size*D`` E4M3fn bytes,
  token-major, followed by ``page_size`` little-endian fp32 per-token scales.
  For 64 tokens x 128 that is 8192 + 256 = 8448 bytes.
* fp4 page: ``page_size*D/2`` packed E2M1 bytes, token-major (element 2i in
  the low nibble of byte i), followed by ``page_size*D/32`` E8M0 bytes, one per
  32 consecutive elements of a token, token-major.  For 64 x 128 that is
  4096 + 256 = 4352 bytes.  There is no per-token fp32 scale (scale_t = 1).
* q fp8: E4M3fn [B, next_n, H, D].  q fp4: packed E2M1 [B, next_n, H, D/2]
  plus E8M0 [B, next_n, H, D/32].
* weights fp32 [B*next_n, H]; context_lens int32 [B];
  block_table int32 [B, stride], logical page i of row b is physical page
  block_table[b, i]; only the first ceil(ctx_b/page_size) entries are used.

Exactness: every finite E4M3 value is a multiple of 2^-9 below 2^9, so a
product is a multiple of 2^-18 below 2^18 and a sum of 128 products an
integer below 2^43 in units of 2^-18: fp64 holds it exactly, in any summation
order.  For E2M1 x E2M1 with power-of-two block scales the same holds.  The
only roundings are scale_t * S (one fp64 rounding), the fp64 head sum and the
final fp32 round-to-nearest-even.

Pins: tests/test_oracle_exact.py (rational brute force), tests/
test_oracle_invariants.py (mask, permutations, one-hot head, constant closed
forms, linearity, next_n reduction) and the hand-derived fixtures in
tests/golden/.
"""
import numpy as np

from . import formats


def fp8_page_bytes(page_size: int, head_dim: int) -> int:
    """Bytes of one fp8 K page: values then fp32 scales."""
    return page_size * head_dim + 4 * page_size


def fp4_page_bytes(page_size: int, head_dim: int) -> int:
    """Bytes of one MXFP4 K page: packed values then E8M0 block scales."""
    return page_size * head_dim // 2 + page_size * head_dim // 32


def causal_limit(ctx: int, next_n: int, j: int, max_context_len: int) -> int:
    """Number of scored tokens of query j of a row with context ctx."""
    return min(ctx - next_n + 1 + j, max_context_len)


def gather_fp8_tokens(kv_cache, pages, n_tokens, page_size, head_dim):
    """Decode the first n_tokens of a row's pages: (K fp64 [n, D], scale fp64 [n])."""
    vbytes = page_size * head_dim
    ks, ss = [], []
    for pid in pages:
        page = kv_cache[int(pid)]
        ks.append(formats.decode_e4m3fn(page[:vbytes].reshape(page_size, head_dim)))
        sc = np.frombuffer(page[vbytes:vbytes + 4 * page_size].tobytes(), dtype="<f4")
        ss.append(sc.astype(np.float64))
    k = np.concatenate(ks, axis=0)[:n_tokens]
    s = np.concatenate(ss, axis=0)[:n_tokens]
    return k, s


def gather_fp4_tokens(kv_cache, pages, n_tokens, page_size, head_dim):
    """Decode the first n_tokens of a row's MXFP4 pages: K fp64 [n, D]."""
    vbytes = page_size * head_dim // 2
    nblk = head_dim // 32
    ks = []
    for pid in pages:
        page = kv_cache[int(pid)]
        vals = formats.decode_e2m1_packed(page[:vbytes].reshape(page_size, head_dim // 2))
        scl = formats.decode_e8m0(page[vbytes:vbytes + page_size * nblk].reshape(page_size, nblk))
        ks.append(vals * np.repeat(scl, 32, axis=1))
    return np.concatenate(ks, axis=0)[:n_tokens]


def _score_rows(kfun, qd, weights, context_lens, block_table, max_context_len,
                page_size, next_n, rows, want_tol, want_fp64):
    """Shared row loop: kfun(b, L) -> (K fp64 [L, D], scale fp64 [L])."""
    B = len(context_lens)
    M = int(max_context_len)
    if rows is None:
        rows = range(B * next_n)
    rows = [int(r) for r in rows]
    out = np.full((len(rows), M), -np.inf, dtype=np.float32)
    tol = np.zeros((len(rows), M), dtype=np.float64) if want_tol else None
    ex = np.full((len(rows), M), -np.inf, dtype=np.float64) if want_fp64 else None
    cache = {}
    for i, r in enumerate(rows):
        b, j = divmod(r, next_n)
        L = int(context_lens[b])
        if L < 0:
            raise ValueError(f"context_lens[{b}] = {L} < 0")
        lim = causal_limit(L, next_n, j, M)
        if lim <= 0:
            continue
        if b not in cache:
            npg = -(-L // page_size)
            cache = {b: kfun(b, npg, L)}
        k, s = cache[b]
        sd = k[:lim] @ qd[b, j].T                     # [lim, H], exact
        x = s[:lim, None] * sd                        # scale inside the ReLU
        w = weights[r].astype(np.float64)
        o64 = np.maximum(x, 0.0) @ w                  # weighted head sum
        out[i, :lim] = o64.astype(np.float32)
        if want_tol:
            tol[i, :lim] = 2e-3 * (np.abs(x) @ np.abs(w)) + 1e-6
        if want_fp64:
            ex[i, :lim] = o64
    res = {"logits": out, "rows": np.asarray(rows, dtype=np.int64)}
    if want_tol:
        res["tol"] = tol
    if want_fp64:
        res["fp64"] = ex
    return res


def paged_mqa_logits_fp8(q, kv_cache, weights, context_lens, block_table,
                         max_context_len, page_size=64, rows=None,
                         want_tol=False, want_fp64=False):
    """fp8 variant: E4M3fn q and K, per-token fp32 K scale.

    q: uint8 [B, next_n, H, D]; kv_cache: uint8 [num_pages, page bytes];
    weights: float32 [B*next_n, H]; context_lens: int [B];
    block_table: int [B, stride].  rows: optional subset of output rows.

    Returns a dict with ``logits`` fp32 [len(rows), M] and, on request,
    ``tol`` (the per-entry parity bound 2e-3*sum_h|w||X| + 1e-6, zero where
    masked) and ``fp64`` (the pre-rounding fp64 values).
    """
    q = np.asarray(q, dtype=np.uint8)
    B, next_n, H, D = q.shape
    kv_cache = np.asarray(kv_cache, dtype=np.uint8)
    assert kv_cache.shape[1] >= fp8_page_bytes(page_size, D)
    qd = formats.decode_e4m3fn(q)

    def kfun(b, npg, L):
        return gather_fp8_tokens(kv_cache, block_table[b, :npg], L, page_size, D)

    return _score_rows(kfun, qd, np.asarray(weights, np.float32), context_lens,
                       block_table, max_context_len, page_size, next_n, rows,
                       want_tol, want_fp64)


def paged_mqa_logits_fp4(q, q_scale, kv_cache, weights, context_lens,
                         block_table, max_context_len, page_size=64, rows=None,
                         want_tol=False, want_fp64=False):
    """MXFP4 variant: E2M1 q and K with E8M0 scales per 32 elements of D.

    q: uint8 [B, next_n, H, D/2] packed; q_scale: uint8 [B, next_n, H, D/32];
    kv_cache: uint8 [num_pages, page bytes]; the rest as for fp8.  The K
    token scale is 1 (the block scales carry the magnitude).
    """
    q = np.asarray(q, dtype=np.uint8)
    B, next_n, H, Dh = q.shape
    D = 2 * Dh
    kv_cache = np.asarray(kv_cache, dtype=np.uint8)
    assert kv_cache.shape[1] >= fp4_page_bytes(page_size, D)
    qd = formats.decode_e2m1_packed(q) * np.repeat(
        formats.decode_e8m0(np.asarray(q_scale, np.uint8)), 32, axis=-1)

    def kfun(b, npg, L):
        k = gather_fp4_tokens(kv_cache, block_table[b, :npg], L, page_size, D)
        return k, np.ones(L, dtype=np.float64)

    return _score_rows(kfun, qd, np.asarray(weights, np.float32), context_lens,
                       block_table, max_context_len, page_size, next_n, rows,
                       want_tol, want_fp64)
