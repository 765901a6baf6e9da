"""Loaders for the hand-derived fixtures in tests/golden/.

Each fixture stores raw input bytes and the exact expected logits, worked
out by hand from the scoring rule (see the ``source`` and ``derivation``
fields of each JSON file).  ``embed`` re-packs a fixture into the dimensions
the GPU kernels are built for (64 heads, head_dim 128, 64-token pages) by
zero padding, which leaves every expected value unchanged.
"""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _expected(vals):
    return np.array([-np.inf if v == "-inf" else float(v) for v in vals], dtype=np.float64)


def _bound(vals):
    """Hand-derived sum_h |w_h| |X_h| per entry; 0 where the entry is masked."""
    return np.array([0.0 if v is None else float(v) for v in vals], dtype=np.float64)


def load_fp8(case_index=0):
    with open(os.path.join(GOLDEN, "hand_fp8.json")) as f:
        fx = json.load(f)
    H, D, P = fx["num_heads"], fx["head_dim"], fx["page_size"]
    q = np.array([[[bytes.fromhex(h) for h in row] for row in b] for b in fx["q_hex"]], dtype=object)
    qa = np.zeros((len(fx["q_hex"]), fx["next_n"], H, D), dtype=np.uint8)
    for b in range(qa.shape[0]):
        for j in range(qa.shape[1]):
            for h in range(H):
                qa[b, j, h] = np.frombuffer(q[b, j, h], dtype=np.uint8)
    pages = []
    case = fx["cases"][case_index]
    for pi, pg in enumerate(fx["pages"]):
        vals = np.concatenate([np.frombuffer(bytes.fromhex(t), np.uint8) for t in pg["values_hex"]])
        sc = np.array(pg["scales"], dtype="<f4")
        pages.append(np.concatenate([vals, sc.view(np.uint8)]))
    kv = np.stack(pages)
    bt = np.array(fx["block_table"], dtype=np.int32)
    if case["scale_override"]:
        t = case["scale_override"]["token"]
        phys = bt[0, t // P]
        off = P * D + 4 * (t % P)
        kv[phys, off:off + 4] = np.array([case["scale_override"]["scale"]], "<f4").view(np.uint8)
    return {"q": qa, "kv_cache": kv, "weights": np.array(fx["weights"], np.float32),
            "context_lens": np.array(fx["context_lens"], np.int32), "block_table": bt,
            "max_context_len": fx["max_context_len"], "page_size": P, "next_n": fx["next_n"],
            "expected": _expected(case["expected"])[None, :], "num_cases": len(fx["cases"]),
            "bound": _bound(case["bound"])[None, :]}


def load_fp4():
    with open(os.path.join(GOLDEN, "hand_fp4.json")) as f:
        fx = json.load(f)
    H, D, P = fx["num_heads"], fx["head_dim"], fx["page_size"]
    B = len(fx["context_lens"])
    q = np.zeros((B, fx["next_n"], H, D // 2), dtype=np.uint8)
    for b, rowb in enumerate(fx["q_bytes"]):
        for j, rowj in enumerate(rowb):
            for h, spec in enumerate(rowj):
                for k, v in spec.items():
                    q[b, j, h, int(k)] = int(v, 16)
    qs = np.array(fx["q_scale"], dtype=np.uint8).reshape(B, fx["next_n"], H, D // 32)
    pages = []
    for pg in fx["pages"]:
        vals = np.full((P, D // 2), int(pg.get("fill", "00"), 16), dtype=np.uint8)
        for t, spec in enumerate(pg["tokens"]):
            for k, v in spec.items():
                vals[t, int(k)] = int(v, 16)
        sc = np.array(pg["scales"], dtype=np.uint8).reshape(P, D // 32)
        pages.append(np.concatenate([vals.reshape(-1), sc.reshape(-1)]))
    return {"q": q, "q_scale": qs, "kv_cache": np.stack(pages),
            "weights": np.array(fx["weights"], np.float32),
            "context_lens": np.array(fx["context_lens"], np.int32),
            "block_table": np.array(fx["block_table"], np.int32),
            "max_context_len": fx["max_context_len"], "page_size": P, "next_n": fx["next_n"],
            "expected": _expected(fx["cases"][0]["expected"])[None, :],
            "bound": _bound(fx["cases"][0]["bound"])[None, :]}


def _tokens_fp8(fx):
    """Per logical token: (value bytes [D], scale float32) of row 0."""
    P = fx["page_size"]
    D = fx["q"].shape[-1]
    out = []
    for t in range(int(fx["context_lens"][0])):
        pg = fx["kv_cache"][fx["block_table"][0, t // P]]
        s = pg[P * D + 4 * (t % P):P * D + 4 * (t % P) + 4].view("<f4")[0]
        out.append((pg[(t % P) * D:(t % P + 1) * D], s))
    return out


def embed_fp8(fx, H=64, D=128, P=64, num_pages=3, phys=1):
    """Zero-pad a one-row fp8 fixture to (H, D, P); its tokens go to page ``phys``."""
    h0, d0 = fx["q"].shape[2], fx["q"].shape[3]
    q = np.zeros((1, 1, H, D), np.uint8)
    q[0, 0, :h0, :d0] = fx["q"][0, 0]
    w = np.zeros((1, H), np.float32)
    w[0, :h0] = fx["weights"][0]
    kv = np.full((num_pages, P * D + 4 * P), 0x7E, np.uint8)
    kv[:, P * D:] = np.full(P, 2.0 ** 60, "<f4").view(np.uint8)
    for t, (vals, s) in enumerate(_tokens_fp8(fx)):
        kv[phys, t * D:t * D + D] = 0
        kv[phys, t * D:t * D + d0] = vals
        kv[phys, P * D + 4 * t:P * D + 4 * t + 4] = np.array([s], "<f4").view(np.uint8)
    M = fx["max_context_len"]
    bt = np.full((1, max(1, -(-M // P))), (phys + 1) % num_pages, np.int32)
    bt[0, 0] = phys
    return {"q": q, "kv_cache": kv, "weights": w, "context_lens": fx["context_lens"].copy(),
            "block_table": bt, "max_context_len": M, "page_size": P, "next_n": 1,
            "expected": fx["expected"], "bound": fx["bound"]}


def embed_fp4(fx, H=64, D=128, P=64, num_pages=3, phys=2):
    """Zero-pad a one-row MXFP4 fixture to (H, D, P); its tokens go to page ``phys``."""
    h0, dh0 = fx["q"].shape[2], fx["q"].shape[3]
    q = np.zeros((1, 1, H, D // 2), np.uint8)
    q[0, 0, :h0, :dh0] = fx["q"][0, 0]
    qs = np.full((1, 1, H, D // 32), 127, np.uint8)
    qs[0, 0, :h0, :dh0 // 16] = fx["q_scale"][0, 0]
    w = np.zeros((1, H), np.float32)
    w[0, :h0] = fx["weights"][0]
    p0 = fx["page_size"]
    d0 = 2 * dh0
    vb = P * D // 2
    kv = np.full((num_pages, vb + P * D // 32), 0x77, np.uint8)
    kv[:, vb:] = 167
    for t in range(int(fx["context_lens"][0])):
        src = fx["kv_cache"][fx["block_table"][0, t // p0]]
        slot = t % p0
        kv[phys, t * D // 2:(t + 1) * D // 2] = 0
        kv[phys, t * D // 2:t * D // 2 + dh0] = src[slot * dh0:(slot + 1) * dh0]
        kv[phys, vb + t * D // 32:vb + (t + 1) * D // 32] = 127
        nb = d0 // 32
        kv[phys, vb + t * D // 32:vb + t * D // 32 + nb] = src[p0 * dh0 + slot * nb:p0 * dh0 + (slot + 1) * nb]
    M = fx["max_context_len"]
    bt = np.full((1, max(1, -(-M // P))), (phys + 1) % num_pages, np.int32)
    bt[0, 0] = phys
    return {"q": q, "q_scale": qs, "kv_cache": kv, "weights": w,
            "context_lens": fx["context_lens"].copy(), "block_table": bt,
            "max_context_len": M, "page_size": P, "next_n": 1, "expected": fx["expected"],
            "bound": fx["bound"]}
