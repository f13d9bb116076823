"""fp64 CPU oracle for the attention forward and the DFlash2 ring steps.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``.  The product package never imports
it.  The arithmetic lives in ``oracle.c`` (plain C, fp64); this module builds
it with gcc, loads it with ctypes and converts numpy arguments.

Functions follow the pages as cited in ``oracle.c``:
  attention        -- O1, batched strided masked GQA (two-pass softmax)
  paged_decode     -- O2, single query over a page table
  paged_prefill    -- O1 over keys gathered through a page table, causal by position
  paged_prepare    -- per-head RMS norm, rotary embedding, K/V write into the pages
  dflash_pack/mask/commit/mask_rows -- O3..O5 and the mask-rows step
  dflash_verify_attention -- O1 over the outputs of O3 and O4 (the verify step)
  bf16_from_f32    -- round-to-nearest-even f32 -> bf16 bits
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F64, F32, F16, BF16 = 0, 1, 2, 3


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (OpenMP over independent output rows)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-Wall",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        i64, dbl, vp, ip = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
        lib.oracle_attention.argtypes = (
            [i64] * 6 + [dbl]
            + [vp, ip, i64, i64, i64] * 4
            + [vp, i64, i64, i64])
        lib.oracle_attention.restype = None
        lib.oracle_paged_decode.argtypes = (
            [i64] * 6 + [dbl] + [vp, ip, i64, i64] + [vp, vp, ip, i64, i64, i64]
            + [vp, vp] + [vp, i64, i64])
        lib.oracle_paged_decode.restype = None
        lib.oracle_dflash_pack.argtypes = [i64] * 6 + [vp] * 10
        lib.oracle_dflash_mask.argtypes = [i64] * 4 + [vp, vp]
        lib.oracle_dflash_commit.argtypes = [i64] * 5 + [vp] * 6
        lib.oracle_dflash_mask_rows.argtypes = [i64] * 3 + [vp, vp]
        lib.oracle_bf16_from_f32_array.argtypes = [vp, vp, i64]
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = dbl
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f64.restype = dbl
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _dtype_code(a: np.ndarray, bf16: bool = False) -> int:
    if a.dtype == np.float64:
        return F64
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float16:
        return F16
    if a.dtype == np.uint16 and bf16:
        return BF16
    raise TypeError("unsupported oracle element type %s (bf16 arrays pass as uint16 with bf16=True)" % a.dtype)


def _strides(a: np.ndarray):
    return [s // a.itemsize for s in a.strides]


def attention(q, k, v, mask=None, *, scale: float, q_bf16=False, kv_bf16=False, mask_bf16=False):
    """O1.  q [B, R, H, D], k/v [B, KV, HK, D], mask [B, H|1, R, KV] (any strides,
    any of f64/f32/f16 or bf16-as-uint16).  Returns float64 O [B, R, H, D]."""
    lib = _load()
    B, R, H, D = q.shape
    _, KV, HK, D2 = k.shape
    assert D2 == D and v.shape == k.shape and H % HK == 0
    q, k, v = (a if a.strides[-1] == a.itemsize else np.ascontiguousarray(a) for a in (q, k, v))
    if mask is not None and mask.strides[-1] != mask.itemsize:
        mask = np.ascontiguousarray(mask)
    o = np.zeros((B, R, H, D), dtype=np.float64)
    if KV == 0:
        return o  # no keys: every row sees nothing and is 0, as for a fully masked row
    qs, ks, vs = _strides(q), _strides(k), _strides(v)
    if mask is not None:
        assert mask.shape[0] == B and mask.shape[2] == R and mask.shape[3] == KV
        ms = _strides(mask)
        m_hs = 0 if mask.shape[1] == 1 else ms[1]
        mptr, mcode = _ptr(mask), _dtype_code(mask, mask_bf16)
        m_bs, m_rs = ms[0], ms[2]
        assert ms[3] == 1, "mask keys must be contiguous"
    else:
        mptr, mcode, m_bs, m_hs, m_rs = None, F64, 0, 0, 0
    for a, s in ((q, qs), (k, ks), (v, vs)):
        assert s[3] == 1, "head_dim must be contiguous"
    lib.oracle_attention(
        B, R, KV, H, HK, D, float(scale),
        _ptr(q), _dtype_code(q, q_bf16), qs[0], qs[1], qs[2],
        _ptr(k), _dtype_code(k, kv_bf16), ks[0], ks[1], ks[2],
        _ptr(v), _dtype_code(v, kv_bf16), vs[0], vs[1], vs[2],
        mptr, mcode, m_bs, m_hs, m_rs,
        _ptr(o), R * H * D, H * D, D)
    return o


def paged_decode(q, k_pool, v_pool, page_table, context_lens, *, scale: float, kv_bf16=False):
    """O2.  q [B, H, D]; pools [num_pages, page_size, HK, D] (any element strides
    shared by K and V); page_table int32 [B, max_pages]; context_lens int32 [B].
    Returns float64 O [B, H, D]."""
    lib = _load()
    B, H, D = q.shape
    _, P, HK, D2 = k_pool.shape
    assert D2 == D and v_pool.shape == k_pool.shape and _strides(k_pool) == _strides(v_pool)
    page_table = np.ascontiguousarray(page_table, dtype=np.int32)
    context_lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    qs, ps = _strides(q), _strides(k_pool)
    o = np.zeros((B, H, D), dtype=np.float64)
    lib.oracle_paged_decode(
        B, H, HK, D, P, page_table.shape[1], float(scale),
        _ptr(q), _dtype_code(q), qs[0], qs[1],
        _ptr(k_pool), _ptr(v_pool), _dtype_code(k_pool, kv_bf16), ps[0], ps[1], ps[2],
        _ptr(page_table), _ptr(context_lens), _ptr(o), H * D, D)
    return o


def paged_prefill(q, k_pool, v_pool, page_table, query_lens, position_starts, *, scale: float, cap: int,
                  kv_bf16=False):
    """Multi-token paged attention: query token i of sequence b sits at position
    s_b + i (s_b = position_starts[b]) and attends to the keys t <= s_b + i of
    its sequence, key t read from pool page page_table[b, t // P], slot t % P.
    The keys of the sequence (its context, s_b + query_lens[b], clamped to cap)
    are gathered, then O1 runs with the causal mask.  Rows i >= query_lens[b]
    are NaN.  Returns float64 O [B, T, H, D]."""
    B, T, H, D = q.shape
    P = k_pool.shape[1]
    o = np.full((B, T, H, D), np.nan)
    for b in range(B):
        n = min(max(int(query_lens[b]), 0), T)
        if n == 0:
            continue
        st = min(max(int(position_starts[b]), 0), cap)
        ctx = min(st + n, cap)
        t = np.arange(ctx)
        pages = np.asarray(page_table)[b, t // P]
        kb = np.asarray(k_pool)[pages, t % P][None]
        vb = np.asarray(v_pool)[pages, t % P][None]
        mask = np.where(t[None, :] <= st + np.arange(n)[:, None], 0.0, -np.inf)[None, None]
        o[b, :n] = attention(q[b:b + 1, :n], kb, vb, mask, scale=scale, kv_bf16=kv_bf16)[0]
    return o


def rms_norm(x, w, eps):
    """x / sqrt(mean(x^2) + eps) * w over the last axis, in float64."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, np.float64)


def rope(x, position, rope_dim, theta, interleaved):
    """Rotate pair i of the first rope_dim features by position * theta^(-2i/rope_dim):
    pairs (2i, 2i+1) if interleaved, else (i, i + rope_dim/2).  float64."""
    x = np.array(x, np.float64, copy=True)
    half = rope_dim // 2
    i = np.arange(half, dtype=np.float64)
    ang = float(position) * np.power(float(theta), -2.0 * i / rope_dim)
    c, s = np.cos(ang), np.sin(ang)
    if interleaved:
        a, b = x[..., 0:rope_dim:2].copy(), x[..., 1:rope_dim:2].copy()
        x[..., 0:rope_dim:2] = a * c - b * s
        x[..., 1:rope_dim:2] = a * s + b * c
    else:
        a, b = x[..., :half].copy(), x[..., half:rope_dim].copy()
        x[..., :half] = a * c - b * s
        x[..., half:rope_dim] = a * s + b * c
    return x


def paged_prepare(q_raw, k_raw, v_raw, q_norm, k_norm, page_table, query_lens, position_starts, k_pool, v_pool, *,
                  rope_dim, theta, eps, interleaved, cap, kv_bf16=False):
    """The prepare step: token t < query_lens[b] at position s = position_starts[b] + t;
    Q and K heads RMS-normed (weights [heads or 1, D]; None: no norm) then rotated;
    prepared Q returned (float64 [B, T, H, D], NaN for rows past query_lens); K
    (rotated) and V (as is) rounded to the pool type and written at page
    page_table[b, s // P], slot s % P while s < cap.  Returns (q_out, k_pool, v_pool)."""
    B, T, H, _ = q_raw.shape
    D = k_pool.shape[-1]
    P = k_pool.shape[1]
    kp, vp = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    q_out = np.full((B, T, H, D), np.nan)

    def to_pool(x):
        x32 = np.asarray(x, np.float32)
        return bf16_from_f32(x32) if kv_bf16 else x32.astype(np.float16)

    for b in range(B):
        n = min(max(int(query_lens[b]), 0), T)
        st = max(int(position_starts[b]), 0)
        for t in range(n):
            s = st + t
            q = np.asarray(q_raw[b, t, :, :D], np.float64)
            k = np.asarray(k_raw[b, t, :, :D], np.float64)
            if q_norm is not None:
                q = rms_norm(q, q_norm, eps)
                k = rms_norm(k, k_norm, eps)
            q_out[b, t] = rope(q, s, rope_dim, theta, interleaved)
            if s < cap:
                page = int(page_table[b, s // P])
                kp[page, s % P] = to_pool(rope(k, s, rope_dim, theta, interleaved))
                vp[page, s % P] = to_pool(np.asarray(v_raw[b, t, :, :D], np.float32))
    return q_out, kp, vp


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


def dflash_pack(geom, ring_k, ring_v, cur_q, cur_k, cur_v, cache_lengths, write_positions):
    """O3.  geom = (lanes, q_heads, kv_heads, head_dim, rows, window).  bf16 as uint16."""
    lib = _load()
    b, h, hk, d, r, w = geom
    k = w - 1 + r
    ring_k, ring_v = _c(ring_k, np.uint16), _c(ring_v, np.uint16)
    cur_q, cur_k, cur_v = _c(cur_q, np.float32), _c(cur_k, np.float32), _c(cur_v, np.float32)
    L, wp = _c(cache_lengths, np.uint32), _c(write_positions, np.uint32)
    assert ring_k.shape == (b, hk, w, d) and cur_q.shape == (b, r, h, d) and cur_k.shape == (b, r, hk, d)
    pq = np.empty((b, h, r, d), np.uint16)
    pk = np.empty((b, hk, k, d), np.uint16)
    pv = np.empty((b, hk, k, d), np.uint16)
    lib.oracle_dflash_pack(b, h, hk, d, r, w, _ptr(ring_k), _ptr(ring_v), _ptr(cur_q), _ptr(cur_k),
                           _ptr(cur_v), _ptr(L), _ptr(wp), _ptr(pq), _ptr(pk), _ptr(pv))
    return pq, pk, pv


def dflash_mask(geom, cache_lengths):
    """O4.  Returns bf16 bits uint16 [lanes, q_heads, rows, packed_len]."""
    lib = _load()
    b, h, hk, d, r, w = geom
    L = _c(cache_lengths, np.uint32)
    m = np.empty((b, h, r, w - 1 + r), np.uint16)
    lib.oracle_dflash_mask(b, h, r, w, _ptr(L), _ptr(m))
    return m


def dflash_verify_attention(geom, ring_k, ring_v, cur_q, cur_k, cur_v, cache_lengths, write_positions, *,
                            scale: float):
    """The block-verify attention: pack (O3), mask (O4), then masked GQA
    attention (O1) over the packed buffers with bf16 Q/K/V and mask, exactly
    as the pack page's dispatch sequence feeds them.  Returns float64 O
    [lanes, q_heads, rows, head_dim]."""
    pq, pk, pv = dflash_pack(geom, ring_k, ring_v, cur_q, cur_k, cur_v, cache_lengths, write_positions)
    m = dflash_mask(geom, cache_lengths)
    o = attention(pq.transpose(0, 2, 1, 3), pk.transpose(0, 2, 1, 3), pv.transpose(0, 2, 1, 3), m, scale=scale,
                  q_bf16=True, kv_bf16=True, mask_bf16=True)
    return np.ascontiguousarray(o.transpose(0, 2, 1, 3))


def dflash_commit(geom, max_commit, new_k, new_v, commit_counts, write_positions, ring_k, ring_v):
    """O5.  Returns updated copies of ring_k, ring_v (bf16 bits)."""
    lib = _load()
    b, h, hk, d, r, w = geom
    new_k, new_v = _c(new_k, np.float32), _c(new_v, np.float32)
    assert new_k.shape == (b, max_commit, hk, d)
    rk, rv = np.array(ring_k, dtype=np.uint16, copy=True), np.array(ring_v, dtype=np.uint16, copy=True)
    cnt, wp = _c(commit_counts, np.uint32), _c(write_positions, np.uint32)
    lib.oracle_dflash_commit(b, hk, d, w, max_commit, _ptr(new_k), _ptr(new_v), _ptr(cnt), _ptr(wp),
                             _ptr(rk), _ptr(rv))
    return rk, rv


def dflash_mask_rows(lanes, rows, hidden, mask_embedding, draft_input):
    """Mask-rows step.  Returns an updated copy of the f32 draft input [lanes*rows, hidden]."""
    lib = _load()
    emb = _c(mask_embedding, np.uint16)
    out = np.array(draft_input, dtype=np.float32, copy=True)
    assert emb.shape == (hidden,) and out.shape == (lanes * rows, hidden)
    lib.oracle_dflash_mask_rows(lanes, rows, hidden, _ptr(emb), _ptr(out))
    return out


def bf16_from_f32(x) -> np.ndarray:
    """f32 -> bf16 bits (uint16), round to nearest even."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib.oracle_bf16_from_f32_array(_ptr(x), _ptr(out), x.size)
    return out


def f16_to_f64(bits: int) -> float:
    return _load().oracle_f16_to_f64(bits)


def bf16_to_f64(bits: int) -> float:
    return _load().oracle_bf16_to_f64(bits)
