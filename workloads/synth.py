"""Seeded synthetic workloads for paged MQA logits.

Input recipe (one ``numpy.random.Generator(PCG64(seed))`` per workload, values
drawn in this fixed order):

1. context lengths (uniform integers, or a clipped lognormal);
2. zero-length rows (a random subset of the stated fraction, plus row 0 when
   the workload forces it);
3. physical pages: ``perm = rng.permutation(pool)``; logical pages of all rows
   in row-major order take ``perm[0], perm[1], ...``; the remaining pool pages
   are poison pages;
4. a 63-bit seed for a ``torch.Generator`` that draws the bulk normals
   (torch's CPU sampler is several times faster than numpy's and gives the
   same stream for any thread count or chunking);
5. q ~ N(0, 1) (float32, torch stream), quantized to the variant's format;
6. K rows ~ N(0, 1) (float32, torch stream), drawn row by row in token order
   and quantized per token (fp8: scale = amax/448, values = e4m3(k/scale)) or
   per 32-element block (MXFP4, shared exponent floor(log2 amax) - 2);
7. with ``negative_scales`` (fp8 tests only), the signs of the token scales;
8. head weights ~ N(0, 1) / sqrt(H) (float32, numpy stream).

Bytes that no correct implementation reads hold large finite poison: unused
pool pages, the slots of a row's last page at or beyond its context length,
and block-table entries past a row's last page (they name poison pages).  A
stray read therefore produces a huge wrong value, never a fault.

Quantization uses torch's float8_e4m3fn cast (round to nearest even; inputs
are clamped to +-448 first) and, for E2M1, round-half-to-even on the E2M1 grid
with saturation at 6.  Quantization only shapes the input
data: the oracle and the GPU read the same bytes.
"""
from dataclasses import dataclass, replace

import numpy as np
import torch

H_DEFAULT = 64
D_DEFAULT = 128
PAGE_DEFAULT = 64

FP8_POISON_VALUE = 0x7E            # e4m3 448
FP8_POISON_SCALE = np.float32(2.0 ** 60)
FP4_POISON_VALUE = 0x77            # two e2m1 6.0 nibbles
FP4_POISON_SCALE = 127 + 40        # e8m0 2^40


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    variant: str                  # "fp8" or "fp4"
    batch: int
    next_n: int
    ctx_kind: str                 # "uniform" or "lognormal"
    ctx_lo: int
    ctx_hi: int
    ctx_median: float = 0.0
    ctx_sigma: float = 0.0
    zero_frac: float = 0.0
    row0_zero: bool = False
    max_context_len: int = 0
    pool_factor: float = 1.2
    seed: int = 0
    num_heads: int = 64


CONFIGS = {
    "tiny_fp8": WorkloadConfig("tiny_fp8", "fp8", 4, 1, "uniform", 0, 1024,
                               row0_zero=True, max_context_len=1024,
                               pool_factor=1.0, seed=0),
    "mid_fp8": WorkloadConfig("mid_fp8", "fp8", 64, 1, "uniform", 1024, 32768,
                              max_context_len=32768, seed=1),
    "large_fp8": WorkloadConfig("large_fp8", "fp8", 2048, 1, "lognormal", 1, 65536,
                                ctx_median=4096.0, ctx_sigma=1.0, zero_frac=0.10,
                                max_context_len=65536, seed=2),
    "spec_fp8": WorkloadConfig("spec_fp8", "fp8", 256, 2, "uniform", 8192, 131072,
                               max_context_len=131072, seed=3),
    "mxfp4": WorkloadConfig("mxfp4", "fp4", 512, 1, "uniform", 1024, 131072,
                            zero_frac=0.05, max_context_len=131072, seed=4),
    # the large_fp8 lengths with query blocks of 32 and 16 heads
    "large_fp8_h32": WorkloadConfig("large_fp8_h32", "fp8", 2048, 1, "lognormal", 1, 65536,
                                    ctx_median=4096.0, ctx_sigma=1.0, zero_frac=0.10,
                                    max_context_len=65536, seed=2, num_heads=32),
    "large_fp8_h16": WorkloadConfig("large_fp8_h16", "fp8", 2048, 1, "lognormal", 1, 65536,
                                    ctx_median=4096.0, ctx_sigma=1.0, zero_frac=0.10,
                                    max_context_len=65536, seed=2, num_heads=16),
}


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def draw_context_lens(cfg: WorkloadConfig, rng=None) -> np.ndarray:
    """Steps 1-2 of the recipe: int32 [B] context lengths."""
    rng = _rng(cfg.seed) if rng is None else rng
    B = cfg.batch
    if cfg.ctx_kind == "uniform":
        ctx = rng.integers(cfg.ctx_lo, cfg.ctx_hi + 1, size=B)
    elif cfg.ctx_kind == "lognormal":
        x = np.exp(rng.normal(np.log(cfg.ctx_median), cfg.ctx_sigma, size=B))
        ctx = np.clip(np.rint(x), cfg.ctx_lo, cfg.ctx_hi)
    else:
        raise ValueError(cfg.ctx_kind)
    ctx = ctx.astype(np.int64)
    nz = int(round(cfg.zero_frac * B))
    if nz:
        ctx[rng.choice(B, size=nz, replace=False)] = 0
    if cfg.row0_zero:
        ctx[0] = 0
    return ctx.astype(np.int32)


def quantize_e4m3(x: np.ndarray) -> np.ndarray:
    """float32 -> E4M3fn bytes, round to nearest even, clamped to +-448."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).clamp_(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def quantize_fp8_tokens(k: np.ndarray):
    """Per-token fp8 quantization: (bytes uint8 [n, D], scale float32 [n])."""
    t = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float32))
    amax = t.abs().amax(dim=1)
    scale = amax / 448.0
    safe = torch.where(scale > 0, scale, torch.ones_like(scale))
    codes = (t / safe[:, None]).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    codes[scale == 0] = 0
    return codes.numpy(), scale.numpy().astype(np.float32)


# Rounding boundaries between consecutive E2M1 magnitudes (0, 0.5, 1, 1.5, 2,
# 3, 4, 6).  A value equal to a midpoint rounds to the even code: the
# midpoints above an odd code are moved down by one ulp so that, with
# bucketize's "boundary[i-1] < v <= boundary[i]" rule, ties go up there and
# down everywhere else.  The bucket index is the E2M1 magnitude code.
_E2M1_BOUNDS = torch.tensor([0.25, np.nextafter(np.float32(0.75), np.float32(0)), 1.25,
                             np.nextafter(np.float32(1.75), np.float32(0)), 2.5,
                             np.nextafter(np.float32(3.5), np.float32(0)), 5.0],
                            dtype=torch.float32)


def quantize_mxfp4(x: np.ndarray):
    """MXFP4 quantization of [..., D]: (packed uint8 [..., D/2], e8m0 [..., D/32]).

    Shared exponent per 32 consecutive elements: floor(log2 amax) - 2 (the
    largest E2M1 exponent is 2), clamped to [-127, 127]; an all-zero block
    gets code 0.  Each scaled element (an exact power-of-two rescale) is
    rounded to the nearest E2M1 magnitude, ties to the even code, and
    saturates at 6.
    """
    x = np.asarray(x, dtype=np.float32)
    shp = x.shape
    D = shp[-1]
    blk = torch.from_numpy(np.ascontiguousarray(x)).reshape(-1, D // 32, 32)
    amax = blk.abs().amax(dim=2)
    ex = (torch.frexp(amax).exponent - 3).clamp_(-127, 127)     # floor(log2 amax) - 2
    code_s = torch.where(amax > 0, ex + 127, torch.zeros_like(ex)).to(torch.uint8)
    v = blk * torch.ldexp(torch.ones_like(amax), -ex)[..., None]
    code = torch.bucketize(v.abs(), _E2M1_BOUNDS, out_int32=True).to(torch.uint8)
    code |= ((v < 0) & (code > 0)).to(torch.uint8) << 3
    code = code.reshape(-1, D)
    packed = code[:, 0::2] | (code[:, 1::2] << 4)
    return (packed.numpy().reshape(shp[:-1] + (D // 2,)),
            code_s.numpy().reshape(shp[:-1] + (D // 32,)))


def _torch_normals(rng):
    g = torch.Generator()
    g.manual_seed(int(rng.integers(0, 2 ** 63 - 1)))

    def draw(*shape):
        return torch.randn(shape, generator=g, dtype=torch.float32).numpy()
    return draw


def _pages_needed(ctx, page_size):
    return (np.asarray(ctx, np.int64) + page_size - 1) // page_size


def _layout_pages(rng, ctx, page_size, pool_factor, bt_stride):
    npg = _pages_needed(ctx, page_size)
    needed = int(npg.sum())
    pool = max(needed + 1, int(np.ceil(needed * pool_factor)))
    perm = rng.permutation(pool).astype(np.int32)
    spare = perm[needed:]
    B = len(ctx)
    bt = np.empty((B, bt_stride), dtype=np.int32)
    # block-table entries past a row's last page name poison pages
    bt[:] = spare[np.arange(B * bt_stride) % len(spare)].reshape(B, bt_stride)
    pos = 0
    for b in range(B):
        n = int(npg[b])
        if n > bt_stride:
            raise ValueError(f"row {b} needs {n} pages > block_table stride {bt_stride}")
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    return bt, pool, npg


def make_fp8(context_lens, next_n=1, max_context_len=None, seed=0, pool_factor=1.2,
             num_heads=H_DEFAULT, head_dim=D_DEFAULT, page_size=PAGE_DEFAULT,
             bt_stride=None, negative_scales=False, rng=None):
    """fp8 inputs for the given context lengths (steps 3-6 of the recipe).

    With ``negative_scales`` a random half of the token scales is negated (an
    input the formula allows; it exercises ReLU(scale * s) with scale < 0).
    """
    rng = _rng(seed) if rng is None else rng
    ctx = np.asarray(context_lens, dtype=np.int32)
    B = len(ctx)
    M = int(max_context_len if max_context_len is not None else max(1, int(ctx.max(initial=0))))
    if bt_stride is None:
        bt_stride = max(1, -(-max(M, int(ctx.max(initial=0))) // page_size))
    H, D, P = num_heads, head_dim, page_size
    bt, pool, npg = _layout_pages(rng, ctx, P, pool_factor, bt_stride)
    normal = _torch_normals(rng)
    q = quantize_e4m3(normal(B, next_n, H, D))
    vbytes = P * D
    kv = np.empty((pool, vbytes + 4 * P), dtype=np.uint8)
    kv[:, :vbytes] = FP8_POISON_VALUE
    kv[:, vbytes:] = np.frombuffer(np.full(P, FP8_POISON_SCALE, "<f4").tobytes(), np.uint8)
    for b in range(B):
        L = int(ctx[b])
        if L == 0:
            continue
        n = int(npg[b])
        codes, scale = quantize_fp8_tokens(normal(L, D))
        vals = np.full((n * P, D), FP8_POISON_VALUE, dtype=np.uint8)
        vals[:L] = codes
        sc = np.full(n * P, FP8_POISON_SCALE, dtype="<f4")
        sc[:L] = scale
        pages = bt[b, :n]
        kv[pages, :vbytes] = vals.reshape(n, vbytes)
        kv[pages, vbytes:] = sc.view(np.uint8).reshape(n, 4 * P)
    if negative_scales:
        s = kv[:, vbytes:].copy().view("<f4")
        flip = rng.random(s.shape) < 0.5
        s[flip] = -s[flip]
        kv[:, vbytes:] = s.view(np.uint8)
    w = (rng.standard_normal((B * next_n, H), dtype=np.float32) /
         np.float32(np.sqrt(H))).astype(np.float32)
    return {"variant": "fp8", "q": q, "kv_cache": kv, "weights": w,
            "context_lens": ctx, "block_table": bt, "max_context_len": M,
            "next_n": next_n, "page_size": P}


def make_fp4(context_lens, next_n=1, max_context_len=None, seed=0, pool_factor=1.2,
             num_heads=H_DEFAULT, head_dim=D_DEFAULT, page_size=PAGE_DEFAULT,
             bt_stride=None, rng=None):
    """MXFP4 inputs for the given context lengths (steps 3-6 of the recipe)."""
    rng = _rng(seed) if rng is None else rng
    ctx = np.asarray(context_lens, dtype=np.int32)
    B = len(ctx)
    M = int(max_context_len if max_context_len is not None else max(1, int(ctx.max(initial=0))))
    if bt_stride is None:
        bt_stride = max(1, -(-max(M, int(ctx.max(initial=0))) // page_size))
    H, D, P = num_heads, head_dim, page_size
    bt, pool, npg = _layout_pages(rng, ctx, P, pool_factor, bt_stride)
    normal = _torch_normals(rng)
    q, q_scale = quantize_mxfp4(normal(B, next_n, H, D))
    vbytes = P * D // 2
    sbytes = P * D // 32
    kv = np.empty((pool, vbytes + sbytes), dtype=np.uint8)
    kv[:, :vbytes] = FP4_POISON_VALUE
    kv[:, vbytes:] = FP4_POISON_SCALE
    for b in range(B):
        L = int(ctx[b])
        if L == 0:
            continue
        n = int(npg[b])
        packed, scl = quantize_mxfp4(normal(L, D))
        vals = np.full((n * P, D // 2), FP4_POISON_VALUE, dtype=np.uint8)
        vals[:L] = packed
        ss = np.full((n * P, D // 32), FP4_POISON_SCALE, dtype=np.uint8)
        ss[:L] = scl
        pages = bt[b, :n]
        kv[pages, :vbytes] = vals.reshape(n, vbytes)
        kv[pages, vbytes:] = ss.reshape(n, sbytes)
    w = (rng.standard_normal((B * next_n, H), dtype=np.float32) /
         np.float32(np.sqrt(H))).astype(np.float32)
    return {"variant": "fp4", "q": q, "q_scale": q_scale, "kv_cache": kv, "weights": w,
            "context_lens": ctx, "block_table": bt, "max_context_len": M,
            "next_n": next_n, "page_size": P}


def make_workload(cfg, **overrides):
    """Full inputs of a named configuration (or a WorkloadConfig)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if overrides:
        cfg = replace(cfg, **overrides)
    rng = _rng(cfg.seed)
    ctx = draw_context_lens(cfg, rng)
    maker = make_fp8 if cfg.variant == "fp8" else make_fp4
    data = maker(ctx, next_n=cfg.next_n, max_context_len=cfg.max_context_len,
                 pool_factor=cfg.pool_factor, num_heads=cfg.num_heads, rng=rng)
    data["config"] = cfg
    return data
