"""Seeded synthetic inputs for the attention forward and the DFlash2 ring steps.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both the HIP path (through the binding) and the fp64
oracle read the arrays it returns, on the host, byte for byte.

Draws are numpy ``Generator(PCG64)`` float32 samples.  Large arrays are filled
in fixed-size chunks, chunk ``i`` drawn from ``SeedSequence(seed).spawn`` child
``i``, so the values do not depend on the thread count.  Conversions to the
storage types are library casts: numpy ``astype(float16)`` and torch's
``to(bfloat16)`` (both round to nearest even).  bf16 arrays are returned as
uint16 bit patterns.

Workloads (sizes as given for the five benchmark configurations):
  prefill_case("tiny" | "causal2k" | "chunked8k" | "chunked8k_pad", ...)
  paged_case(...)   -- paged decode, 16-token pages, permuted page pool
  dflash_case(...)  -- ring window + drafted rows, with forced-wrap variants
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_CHUNK = 1 << 22  # elements per independently seeded chunk


def _threads() -> int:
    import os
    return max(1, min(16, os.cpu_count() or 1))


def normal_f32(n: int, seed, std: float = 1.0) -> np.ndarray:
    """n float32 draws of N(0, std^2), chunk-seeded (deterministic for any thread count)."""
    out = np.empty(n, dtype=np.float32)
    nchunks = max(1, (n + _CHUNK - 1) // _CHUNK)
    seeds = np.random.SeedSequence(seed).spawn(nchunks)

    def fill(i):
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(seeds[i]))
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        if std != 1.0:
            out[lo:hi] *= np.float32(std)

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def to_f16(x: np.ndarray) -> np.ndarray:
    return x.astype(np.float16)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16) via torch's round-to-nearest-even cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _kv_store(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    return to_f16(x) if kv_dtype == "f16" else to_bf16_bits(x)


# --------------------------------------------------------------------------- prefill
@dataclass
class PrefillCase:
    name: str
    q: np.ndarray            # f32 [B, R, H, D] (or bf16 bits when q_dtype == "bf16")
    k: np.ndarray            # f16 [B, KV, HK, D] (or bf16 bits)
    v: np.ndarray
    mask: Optional[np.ndarray]  # [B, H|1, R, KV] f16 (or bf16 bits) or None
    scale: float
    kv_len: int
    q_dtype: str = "f32"
    kv_dtype: str = "f16"
    mask_dtype: str = "f16"
    visible_pairs: int = 0   # (query, key) pairs at or below each row's frontier, summed over rows
    meta: dict = field(default_factory=dict)


def _frontier_mask(rows: int, kv_len: int, cached: int, holes: float, rng) -> tuple:
    """0/-inf f16 mask [rows, kv_len]: row i sees keys j <= cached + i; with
    holes > 0, each earlier key j < cached + i is also hidden with probability
    `holes` (i.i.d. per (row, key)); the diagonal key is always kept."""
    j = np.arange(kv_len)[None, :]
    i = np.arange(rows)[:, None]
    visible = j <= cached + i
    if holes > 0:
        u = rng.random((rows, kv_len), dtype=np.float32)
        hole = (u < holes) & (j < cached + i)
        visible &= ~hole
    mask = np.where(visible, np.float16(0.0), np.float16(-np.inf)).astype(np.float16)
    frontier = int(np.minimum(cached + np.arange(rows) + 1, kv_len).sum())
    return mask, frontier


def prefill_synthetic(name: str, *, rows: int, kv_len: int, cached: int, n_heads: int,
                      n_kv_heads: int, head_dim: int, seed: int, q_std: float, kv_std: float,
                      holes: float = 0.0, batch: int = 1, kv_dtype: str = "f16",
                      kv_rows_alloc: Optional[int] = None, mask_cols: Optional[int] = None,
                      scale: float = 1.0, mask_dtype: str = "f16") -> PrefillCase:
    """Prefill over one contiguous KV range with a frontier (causal) mask.

    K/V are laid out [B, KV, HK, D] (row stride HK*D, head stride D).  With
    kv_rows_alloc > kv_len the extra K/V rows are zero and the mask columns
    past kv_len are -inf (a padded call); mask_cols sets the mask width.
    mask_dtype "bf16" stores the same 0/-inf mask as bf16 bit patterns."""
    rng = np.random.Generator(np.random.PCG64(seed))
    kv_alloc = kv_rows_alloc or kv_len
    mcols = mask_cols or kv_alloc
    q = normal_f32(batch * rows * n_heads * head_dim, [seed, 1], q_std).reshape(batch, rows, n_heads, head_dim)
    kf = np.zeros((batch, kv_alloc, n_kv_heads, head_dim), np.float32)
    vf = np.zeros_like(kf)
    kf[:, :kv_len] = normal_f32(batch * kv_len * n_kv_heads * head_dim, [seed, 2], kv_std).reshape(
        batch, kv_len, n_kv_heads, head_dim)
    vf[:, :kv_len] = normal_f32(batch * kv_len * n_kv_heads * head_dim, [seed, 3], kv_std).reshape(
        batch, kv_len, n_kv_heads, head_dim)
    m, frontier = _frontier_mask(rows, kv_len, cached, holes, rng)
    mask = np.full((batch, 1, rows, mcols), np.float16(-np.inf), np.float16)
    mask[:, 0, :, :kv_len] = m
    if mask_dtype == "bf16":
        mask = to_bf16_bits(mask.astype(np.float32))
    return PrefillCase(name, q, _kv_store(kf, kv_dtype), _kv_store(vf, kv_dtype), mask, scale, kv_len,
                       kv_dtype=kv_dtype, mask_dtype=mask_dtype, visible_pairs=frontier * batch,
                       meta=dict(rows=rows, kv_len=kv_len, n_heads=n_heads, n_kv_heads=n_kv_heads,
                                 head_dim=head_dim, batch=batch, cached=cached, holes=holes))


def prefill_case(name: str) -> PrefillCase:
    """The four prefill configurations at full size."""
    if name == "tiny":          # 64 queries, 192 cached + 64 new, GQA 4:1, d 256, seed 0
        return prefill_synthetic(name, rows=64, kv_len=256, cached=192, n_heads=4, n_kv_heads=1,
                                 head_dim=256, seed=0, q_std=1 / 16, kv_std=1.0)
    if name == "causal2k":      # 2048 x 2048 causal, 16/8 heads, d 256, seed 1
        return prefill_synthetic(name, rows=2048, kv_len=2048, cached=0, n_heads=16, n_kv_heads=8,
                                 head_dim=256, seed=1, q_std=1 / 16, kv_std=1.0)
    if name == "chunked8k":     # 4096 new rows over 4096 cached + 4096 new, 16/2 heads, d 512, 10% holes
        return prefill_synthetic(name, rows=4096, kv_len=8192, cached=4096, n_heads=16, n_kv_heads=2,
                                 head_dim=512, seed=2, q_std=1 / math.sqrt(512), kv_std=0.5, holes=0.1)
    if name == "chunked8k_pad":  # 8190 KV rows (4094 cached) padded to 8192: zero rows, -inf columns
        return prefill_synthetic(name, rows=4096, kv_len=8190, cached=4094, n_heads=16, n_kv_heads=2,
                                 head_dim=512, seed=2, q_std=1 / math.sqrt(512), kv_std=0.5, holes=0.1,
                                 kv_rows_alloc=8192)
    raise KeyError(name)


# --------------------------------------------------------------------------- paged decode
@dataclass
class PagedCase:
    q: np.ndarray            # f32 [B, H, D]
    k_pool: np.ndarray       # f16 [num_pages, page_size, HK, D]
    v_pool: np.ndarray
    page_table: np.ndarray   # int32 [B, max_pages], -1 past the end
    context_lens: np.ndarray  # int32 [B]
    scale: float
    max_context: int
    meta: dict = field(default_factory=dict)


def paged_case(*, batch: int = 64, ctx_lo: int = 512, ctx_hi: int = 16384, page_size: int = 16,
               num_pages: int = 65536, n_heads: int = 32, n_kv_heads: int = 8, head_dim: int = 128,
               seed: int = 3, max_pages: Optional[int] = None, poison_unused: bool = False,
               context_lens: Optional[np.ndarray] = None, kv_dtype: str = "f16") -> PagedCase:
    """Paged decode: context lengths ~ U{ctx_lo..ctx_hi}; logical page j of
    sequence b is pool page perm[off_b + j] with perm a seeded permutation of
    the pool and off_b the pages used by earlier sequences.  Used slots hold
    N(0,1) K/V; unused slots hold 0 (or NaN with poison_unused)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if context_lens is None:
        ctx = rng.integers(ctx_lo, ctx_hi, size=batch, endpoint=True).astype(np.int32)
    else:
        ctx = np.asarray(context_lens, dtype=np.int32)
    max_pages = max_pages or -(-ctx_hi // page_size)
    perm = rng.permutation(num_pages).astype(np.int32)
    pages_per_seq = -(-ctx.astype(np.int64) // page_size)
    assert pages_per_seq.sum() <= num_pages and pages_per_seq.max() <= max_pages
    page_table = np.full((batch, max_pages), -1, np.int32)
    off = 0
    for b in range(batch):
        n = int(pages_per_seq[b])
        page_table[b, :n] = perm[off:off + n]
        off += n
    q = normal_f32(batch * n_heads * head_dim, [seed, 1]).reshape(batch, n_heads, head_dim)
    fill = np.float16(np.nan) if poison_unused else np.float16(0)
    shape = (num_pages, page_size, n_kv_heads, head_dim)
    pools = []
    for which in (2, 3):
        pool = np.full(shape, fill, np.float16) if kv_dtype == "f16" else np.full(
            shape, 0x7FC0 if poison_unused else 0, np.uint16)
        used = page_table[page_table >= 0]
        vals = normal_f32(used.size * page_size * n_kv_heads * head_dim, [seed, which]).reshape(
            used.size, page_size, n_kv_heads, head_dim)
        # slots at or past the context end inside each sequence's last page are unused
        row = 0
        for b in range(batch):
            n = int(pages_per_seq[b])
            tail = int(ctx[b]) - (n - 1) * page_size
            if n > 0 and tail < page_size:
                vals[row + n - 1, tail:] = np.nan if poison_unused else 0.0
            row += n
        pool[used] = _kv_store(vals, kv_dtype)
        pools.append(pool)
    return PagedCase(q, pools[0], pools[1], page_table, ctx, 1.0 / math.sqrt(head_dim),
                     int(min(ctx_hi, max_pages * page_size)),
                     meta=dict(batch=batch, page_size=page_size, num_pages=num_pages, n_heads=n_heads,
                               n_kv_heads=n_kv_heads, head_dim=head_dim, kv_dtype=kv_dtype))


# --------------------------------------------------------------------------- dflash ring
@dataclass
class DFlashCase:
    geom: tuple              # (lanes, q_heads, kv_heads, head_dim, rows, window)
    max_commit: int
    ring_k: np.ndarray       # bf16 bits [b, hk, w, d]
    ring_v: np.ndarray
    cur_q: np.ndarray        # f32 [b, r, h, d]
    cur_k: np.ndarray        # f32 [b, r, hk, d]
    cur_v: np.ndarray
    cache_lengths: np.ndarray   # u32 [b]
    write_positions: np.ndarray  # u32 [b]
    commit_counts: np.ndarray    # u32 [b]
    scale: float


def dflash_case(*, lanes: int = 4, q_heads: int = 32, kv_heads: int = 8, head_dim: int = 128,
                rows: int = 16, window: int = 4096, seed: int = 4, forced_wrap: bool = False,
                cache_lengths=None, write_positions=None, commit_counts=None) -> DFlashCase:
    """Block-verify inputs: ring K/V ~ N(0,1) in every slot (bf16), current
    Q/K/V ~ N(0,1) (f32), L ~ U{rows+1..window}, wp = L mod window, counts ~
    U{1..rows}.  forced_wrap overrides lanes 0..2: lane 0 L = window, wp = 0
    (packing wraps), lane 1 wp = window - 6 with count = rows (commit wraps),
    lane 2 wp != L mod window."""
    b, h, hk, d, r, w = lanes, q_heads, kv_heads, head_dim, rows, window
    rng = np.random.Generator(np.random.PCG64(seed))
    ring_k = to_bf16_bits(normal_f32(b * hk * w * d, [seed, 1])).reshape(b, hk, w, d)
    ring_v = to_bf16_bits(normal_f32(b * hk * w * d, [seed, 2])).reshape(b, hk, w, d)
    cur_q = normal_f32(b * r * h * d, [seed, 3]).reshape(b, r, h, d)
    cur_k = normal_f32(b * r * hk * d, [seed, 4]).reshape(b, r, hk, d)
    cur_v = normal_f32(b * r * hk * d, [seed, 5]).reshape(b, r, hk, d)
    L = rng.integers(min(r + 1, w), w, size=b, endpoint=True).astype(np.uint32)
    wp = (L % w).astype(np.uint32)
    cnt = rng.integers(1, r, size=b, endpoint=True).astype(np.uint32)
    if forced_wrap:
        if b > 0:
            L[0], wp[0] = w, 0
        if b > 1:
            wp[1], cnt[1] = (w - 6) % w, r
        if b > 2:
            wp[2] = (int(L[2]) + 3) % w
    if cache_lengths is not None:
        L = np.asarray(cache_lengths, np.uint32)
    if write_positions is not None:
        wp = np.asarray(write_positions, np.uint32)
    if commit_counts is not None:
        cnt = np.asarray(commit_counts, np.uint32)
    return DFlashCase((b, h, hk, d, r, w), r, ring_k, ring_v, cur_q, cur_k, cur_v, L, wp, cnt,
                      1.0 / math.sqrt(d))


# --------------------------------------------------------------------------- multi-token paged
@dataclass
class PagedMultiCase:
    paged: PagedCase
    q: np.ndarray                # f32 [B, T, H, D]
    query_lens: np.ndarray       # int32 [B], in [0, T]
    position_starts: np.ndarray  # int32 [B]: the new tokens are the last query_lens of the context


def paged_multi_case(*, max_tokens: int, seed: int = 5, query_lens=None, **paged_kwargs) -> PagedMultiCase:
    """Multi-token paged attention inputs: a paged decode case whose last
    query_lens[b] context tokens are the new ones (their K/V already in the
    pages), query_lens ~ U{1..max_tokens} capped by the context, Q ~ N(0,1)."""
    pc = paged_case(seed=seed, **paged_kwargs)
    rng = np.random.Generator(np.random.PCG64([seed, 7]))
    b = pc.context_lens.shape[0]
    if query_lens is None:
        ql = rng.integers(1, max_tokens, size=b, endpoint=True).astype(np.int32)
    else:
        ql = np.asarray(query_lens, np.int32)
    ql = np.minimum(ql, pc.context_lens).astype(np.int32)
    starts = (pc.context_lens - ql).astype(np.int32)
    h, d = pc.q.shape[1], pc.q.shape[2]
    q = normal_f32(b * max_tokens * h * d, [seed, 8]).reshape(b, max_tokens, h, d)
    return PagedMultiCase(pc, q, ql, starts)

