"""Masked grouped-query attention forward for MI355X (gfx950): Python binding.

Every function here marshals torch tensors (device memory, streams) into a
call of the same name in libattn.so (include/attn.h) and does nothing else;
all arithmetic runs in the library's HIP kernels.

    attn_prefill       -- prefill / block-verify attention over a contiguous KV range
    attn_paged_decode  -- single-query attention over a paged KV cache
    attn_paged_prefill -- multi-token causal attention over a paged KV cache
    attn_paged_prepare -- Q/K RMS norm, rotary embedding, K/V write into the pages
    dflash_pack, dflash_mask, dflash_commit, dflash_mask_rows -- DFlash2 ring steps
    dflash_verify_attention -- block-verify attention read from the ring in place
    dflash_validate, kv_pad, prefill_workspace_bytes, decode_workspace_bytes,
    verify_workspace_bytes
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import _ffi
from ._ffi import AttnError, DFlashParams, DecodeParams, PagedPrefillParams, PrefillParams, PrepareParams, check

__all__ = [
    "AttnError", "DFlashParams", "attn_prefill", "attn_paged_decode", "attn_paged_prefill", "paged_prefill_params",
    "paged_prefill_workspace_bytes", "attn_paged_prepare", "dflash_pack", "dflash_mask",
    "dflash_commit", "dflash_mask_rows", "dflash_validate", "kv_pad", "prefill_params", "decode_params",
    "prefill_workspace_bytes", "decode_workspace_bytes", "dflash_verify_attention", "verify_workspace_bytes",
    "prefill_status", "attn_paged_decode_noalloc",
]

_DTYPES = {torch.float32: _ffi.ATTN_F32, torch.float16: _ffi.ATTN_F16, torch.bfloat16: _ffi.ATTN_BF16}


def _code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError("unsupported dtype %s" % t.dtype) from None


def _cap(t: torch.Tensor) -> int:
    """Elements addressable from t's first element to the end of its storage."""
    return t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _scratch(workspace: Optional[torch.Tensor], need: int, device, stream) -> torch.Tensor:
    """The caller's workspace when it holds `need` bytes, else a new one.  A new one is
    allocated while the stream the kernels run on is current, so the caching allocator
    hands its block to no work on another stream before those kernels are done with it."""
    if workspace is not None and workspace.numel() * workspace.element_size() >= need:
        return workspace
    if stream is None:
        s = torch.cuda.current_stream(device)
    elif isinstance(stream, torch.cuda.Stream):
        s = stream
    else:
        s = torch.cuda.ExternalStream(int(stream), device=device)
    with torch.cuda.stream(s):
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device)


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def kv_pad(kv_len: int) -> int:
    return _ffi.lib().attn_kv_pad(kv_len)


# --------------------------------------------------------------------------- prefill
def prefill_params(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: Optional[torch.Tensor],
                   out: torch.Tensor, *, scale: float, kv_len: Optional[int] = None) -> PrefillParams:
    """q [B, R, H, D]; k, v [B, KVrows, HK, D]; mask [B, H|1, R, cols] or None; out [B, R, H, D]."""
    B, R, H, D = q.shape
    p = PrefillParams()
    p.batch, p.rows, p.n_heads, p.head_dim = B, R, H, D
    p.kv_len = k.shape[1] if kv_len is None else kv_len
    p.n_kv_heads = k.shape[2]
    p.q_dtype, p.kv_dtype = _code(q), _code(k)
    p.mask_dtype = _ffi.ATTN_NONE if mask is None else _code(mask)
    p.scale = scale
    p.q_bs, p.q_rs, p.q_hs = q.stride(0), q.stride(1), q.stride(2)
    p.k_bs, p.k_rs, p.k_hs = k.stride(0), k.stride(1), k.stride(2)
    p.v_bs, p.v_rs, p.v_hs = v.stride(0), v.stride(1), v.stride(2)
    p.o_bs, p.o_rs, p.o_hs = out.stride(0), out.stride(1), out.stride(2)
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        if t.stride(3) != 1:
            raise ValueError("%s: head_dim must be contiguous" % name)
    if v.dtype != k.dtype:
        raise TypeError("k and v must share a dtype")
    if out.dtype != torch.float32:
        raise TypeError("out must be float32")
    if mask is not None:
        if mask.stride(3) != 1:
            raise ValueError("mask: keys must be contiguous")
        p.m_bs, p.m_rs = mask.stride(0), mask.stride(2)
        p.m_hs = 0 if mask.shape[1] == 1 else mask.stride(1)
        p.m_cap = _cap(mask)
    p.q_cap, p.k_cap, p.v_cap, p.o_cap = _cap(q), _cap(k), _cap(v), _cap(out)
    return p


def prefill_workspace_bytes(p: PrefillParams) -> int:
    n = ctypes.c_size_t(0)
    check(_ffi.lib().attn_prefill_workspace_bytes(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: Optional[torch.Tensor],
                 out: torch.Tensor, *, scale: float, kv_len: Optional[int] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """O = softmax(scale * Q K^T + mask) V into `out` (float32), on the device."""
    p = prefill_params(q, k, v, mask, out, scale=scale, kv_len=kv_len)
    workspace = _scratch(workspace, prefill_workspace_bytes(p), q.device, stream)
    check(_ffi.lib().attn_prefill(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  None if mask is None else mask.data_ptr(), out.data_ptr(), workspace.data_ptr(),
                                  _nbytes(workspace), _stream(stream)))
    return out


def prefill_status(workspace: torch.Tensor) -> tuple:
    """(error flags, merged row blocks): words 0 and 1 of the status block at the start of
    a prefill workspace, read once the call that used it has completed."""
    words = workspace[:8].view(torch.int32).cpu().numpy().view("uint32")
    return int(words[0]), int(words[1])


# --------------------------------------------------------------------------- paged decode
def decode_params(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, page_table: torch.Tensor,
                  out: torch.Tensor, *, scale: float, max_context: int) -> DecodeParams:
    """q, out [B, H, D] float32; pools [num_pages, page_size, HK, D] sharing strides; page_table int32 [B, P]."""
    B, H, D = q.shape
    num_pages, page_size, HK, D2 = k_pool.shape
    if D2 != D or tuple(v_pool.shape) != tuple(k_pool.shape) or v_pool.stride() != k_pool.stride():
        raise ValueError("k_pool and v_pool must have the same shape and strides, head_dim matching q")
    if k_pool.dtype != v_pool.dtype or q.dtype != torch.float32 or out.dtype != torch.float32:
        raise TypeError("q/out must be float32 and the pools share one dtype")
    if page_table.dtype != torch.int32 or not page_table.is_contiguous() or page_table.shape[0] != B:
        raise ValueError("page_table must be a contiguous int32 [batch, max_pages] tensor")
    if q.stride(2) != 1 or out.stride(2) != 1 or k_pool.stride(3) != 1:
        raise ValueError("head_dim must be contiguous")
    p = DecodeParams()
    p.batch, p.n_heads, p.n_kv_heads, p.head_dim = B, H, HK, D
    p.page_size, p.max_pages_per_seq, p.num_pages, p.max_context = page_size, page_table.shape[1], num_pages, max_context
    p.kv_dtype = _code(k_pool)
    p.scale = scale
    p.q_bs, p.q_hs, p.o_bs, p.o_hs = q.stride(0), q.stride(1), out.stride(0), out.stride(1)
    p.kv_page_stride, p.kv_token_stride, p.kv_head_stride = k_pool.stride(0), k_pool.stride(1), k_pool.stride(2)
    p.q_cap, p.o_cap = _cap(q), _cap(out)
    p.kv_cap = min(_cap(k_pool), _cap(v_pool))
    return p


def decode_workspace_bytes(p: DecodeParams) -> int:
    n = ctypes.c_size_t(0)
    check(_ffi.lib().attn_paged_decode_workspace_bytes(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def attn_paged_decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, page_table: torch.Tensor,
                      context_lens: torch.Tensor, out: torch.Tensor, *, scale: float, max_context: int,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    p = decode_params(q, k_pool, v_pool, page_table, out, scale=scale, max_context=max_context)
    if context_lens.dtype != torch.int32 or not context_lens.is_contiguous() or context_lens.numel() != q.shape[0]:
        raise ValueError("context_lens must be a contiguous int32 [batch] tensor")
    workspace = _scratch(workspace, decode_workspace_bytes(p), q.device, stream)
    check(_ffi.lib().attn_paged_decode(ctypes.byref(p), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                       page_table.data_ptr(), context_lens.data_ptr(), out.data_ptr(),
                                       workspace.data_ptr(), _nbytes(workspace), _stream(stream)))
    return out


def attn_paged_decode_noalloc(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                              page_table: torch.Tensor, context_lens: torch.Tensor, out: torch.Tensor, *,
                              scale: float, max_context: int, stream=None) -> torch.Tensor:
    """attn_paged_decode with the library's static per-GPU scratch array instead of a
    workspace: allocates nothing.  Calls that overlap in time on one GPU race."""
    p = decode_params(q, k_pool, v_pool, page_table, out, scale=scale, max_context=max_context)
    if context_lens.dtype != torch.int32 or not context_lens.is_contiguous() or context_lens.numel() != q.shape[0]:
        raise ValueError("context_lens must be a contiguous int32 [batch] tensor")
    check(_ffi.lib().attn_paged_decode_noalloc(ctypes.byref(p), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                               page_table.data_ptr(), context_lens.data_ptr(), out.data_ptr(),
                                               _stream(stream)))
    return out


# --------------------------------------------------------------------------- multi-token paged attention
def paged_prefill_params(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, page_table: torch.Tensor,
                         out: torch.Tensor, *, scale: float, max_context: int) -> PagedPrefillParams:
    """q, out [B, T, H, D] float32; pools [num_pages, page_size, HK, D] sharing strides; page_table int32 [B, P]."""
    B, T, H, D = q.shape
    num_pages, page_size, HK, D2 = k_pool.shape
    if D2 != D or tuple(v_pool.shape) != tuple(k_pool.shape) or v_pool.stride() != k_pool.stride():
        raise ValueError("k_pool and v_pool must have the same shape and strides, head_dim matching q")
    if tuple(out.shape) != (B, T, H, D):
        raise ValueError("out must have q's shape")
    if k_pool.dtype != v_pool.dtype or q.dtype != torch.float32 or out.dtype != torch.float32:
        raise TypeError("q/out must be float32 and the pools share one dtype")
    if page_table.dtype != torch.int32 or not page_table.is_contiguous() or page_table.shape[0] != B:
        raise ValueError("page_table must be a contiguous int32 [batch, max_pages] tensor")
    if q.stride(3) != 1 or out.stride(3) != 1 or k_pool.stride(3) != 1:
        raise ValueError("head_dim must be contiguous")
    p = PagedPrefillParams()
    p.batch, p.n_heads, p.n_kv_heads, p.head_dim = B, H, HK, D
    p.page_size, p.max_pages_per_seq, p.num_pages, p.max_context = page_size, page_table.shape[1], num_pages, max_context
    p.max_tokens = T
    p.kv_dtype = _code(k_pool)
    p.scale = scale
    p.q_bs, p.q_ts, p.q_hs = q.stride(0), q.stride(1), q.stride(2)
    p.o_bs, p.o_ts, p.o_hs = out.stride(0), out.stride(1), out.stride(2)
    p.kv_page_stride, p.kv_token_stride, p.kv_head_stride = k_pool.stride(0), k_pool.stride(1), k_pool.stride(2)
    p.q_cap, p.o_cap = _cap(q), _cap(out)
    p.kv_cap = min(_cap(k_pool), _cap(v_pool))
    return p


def paged_prefill_workspace_bytes(p: PagedPrefillParams) -> int:
    n = ctypes.c_size_t(0)
    check(_ffi.lib().attn_paged_prefill_workspace_bytes(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def attn_paged_prefill(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, page_table: torch.Tensor,
                       query_lens: torch.Tensor, position_starts: torch.Tensor, out: torch.Tensor, *, scale: float,
                       max_context: int, workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Query token i of sequence b (position position_starts[b] + i) attends to the keys at or
    before its position; rows i >= query_lens[b] of `out` are left as they are."""
    p = paged_prefill_params(q, k_pool, v_pool, page_table, out, scale=scale, max_context=max_context)
    for t, n in ((query_lens, "query_lens"), (position_starts, "position_starts")):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() != q.shape[0]:
            raise ValueError("%s must be a contiguous int32 [batch] tensor" % n)
    workspace = _scratch(workspace, paged_prefill_workspace_bytes(p), q.device, stream)
    check(_ffi.lib().attn_paged_prefill(ctypes.byref(p), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                        page_table.data_ptr(), query_lens.data_ptr(), position_starts.data_ptr(),
                                        out.data_ptr(), workspace.data_ptr(), _nbytes(workspace), _stream(stream)))
    return out


def attn_paged_prepare(q_raw: torch.Tensor, k_raw: torch.Tensor, v_raw: torch.Tensor,
                       q_norm: Optional[torch.Tensor], k_norm: Optional[torch.Tensor], page_table: torch.Tensor,
                       query_lens: torch.Tensor, position_starts: torch.Tensor, q_out: torch.Tensor,
                       k_pool: torch.Tensor, v_pool: torch.Tensor, *, rope_dim: int, rope_theta: float,
                       rope_interleaved: bool, epsilon: float, max_context: int, stream=None) -> torch.Tensor:
    """q_raw [B, T, H, >=D], k_raw/v_raw [B, T, HK, >=D] float32; q_norm/k_norm float32 [H|1, D] / [HK|1, D]
    or None (no norm); q_out [B, T, H, D] float32; pools [num_pages, page_size, HK, D] f16/bf16."""
    B, T, H, _ = q_raw.shape
    num_pages, page_size, HK, D = k_pool.shape
    if tuple(q_out.shape) != (B, T, H, D) or tuple(k_raw.shape[:3]) != (B, T, HK) or \
            tuple(v_raw.shape[:3]) != (B, T, HK) or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("inconsistent shapes")
    if v_pool.stride() != k_pool.stride() or k_pool.dtype != v_pool.dtype:
        raise ValueError("k_pool and v_pool must share strides and dtype")
    for t, n in ((q_raw, "q_raw"), (k_raw, "k_raw"), (v_raw, "v_raw"), (q_out, "q_out")):
        _want(t, (torch.float32,), n)
        if t.stride(3) != 1:
            raise ValueError("%s: features must be contiguous" % n)
    for t, n in ((query_lens, "query_lens"), (position_starts, "position_starts")):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() != B:
            raise ValueError("%s must be a contiguous int32 [batch] tensor" % n)
    if page_table.dtype != torch.int32 or not page_table.is_contiguous() or page_table.shape[0] != B:
        raise ValueError("page_table must be a contiguous int32 [batch, max_pages] tensor")
    p = PrepareParams()
    p.batch, p.n_heads, p.n_kv_heads, p.head_dim, p.max_tokens = B, H, HK, D, T
    p.rope_dim, p.rope_interleaved, p.qk_norm = rope_dim, int(bool(rope_interleaved)), int(q_norm is not None)
    p.page_size, p.max_pages_per_seq, p.num_pages, p.max_context = page_size, page_table.shape[1], num_pages, max_context
    p.kv_dtype = _code(k_pool)
    p.epsilon, p.rope_theta = epsilon, rope_theta
    p.qr_bs, p.qr_ts, p.qr_hs = q_raw.stride(0), q_raw.stride(1), q_raw.stride(2)
    p.kr_bs, p.kr_ts, p.kr_hs = k_raw.stride(0), k_raw.stride(1), k_raw.stride(2)
    p.vr_bs, p.vr_ts, p.vr_hs = v_raw.stride(0), v_raw.stride(1), v_raw.stride(2)
    p.qo_bs, p.qo_ts, p.qo_hs = q_out.stride(0), q_out.stride(1), q_out.stride(2)
    p.kv_page_stride, p.kv_token_stride, p.kv_head_stride = k_pool.stride(0), k_pool.stride(1), k_pool.stride(2)
    p.qr_cap, p.kr_cap, p.vr_cap, p.qo_cap = _cap(q_raw), _cap(k_raw), _cap(v_raw), _cap(q_out)
    p.kv_cap = min(_cap(k_pool), _cap(v_pool))
    qn = kn = None
    if q_norm is not None:
        if k_norm is None:
            raise ValueError("q_norm and k_norm go together")
        for t, n in ((q_norm, "q_norm"), (k_norm, "k_norm")):
            _want(t, (torch.float32,), n)
            if t.dim() != 2 or t.shape[1] != D or t.stride(1) != 1:
                raise ValueError("%s must be [heads or 1, head_dim] with contiguous features" % n)
        p.qn_hs = 0 if q_norm.shape[0] == 1 else q_norm.stride(0)
        p.kn_hs = 0 if k_norm.shape[0] == 1 else k_norm.stride(0)
        p.qn_cap, p.kn_cap = _cap(q_norm), _cap(k_norm)
        qn, kn = q_norm.data_ptr(), k_norm.data_ptr()
    check(_ffi.lib().attn_paged_prepare(ctypes.byref(p), q_raw.data_ptr(), k_raw.data_ptr(), v_raw.data_ptr(), qn, kn,
                                        page_table.data_ptr(), query_lens.data_ptr(), position_starts.data_ptr(),
                                        q_out.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), _stream(stream)))
    return q_out


# --------------------------------------------------------------------------- DFlash2 ring steps
def _dflash(params) -> DFlashParams:
    if isinstance(params, DFlashParams):
        return params
    return DFlashParams(*[int(x) for x in params])


def _bytes(tensors: Sequence[torch.Tensor]):
    for t in tensors:
        if not t.is_contiguous():
            raise ValueError("DFlash2 buffers must be contiguous")
    arr = (ctypes.c_uint64 * len(tensors))(*[t.numel() * t.element_size() for t in tensors])
    return arr


_U16 = (torch.bfloat16, torch.int16, torch.uint16)
_U32 = (torch.int32, torch.uint32)


def _want(t: torch.Tensor, dtypes, name: str):
    if t.dtype not in dtypes:
        raise TypeError("%s must be one of %s, got %s" % (name, dtypes, t.dtype))


def dflash_validate(params) -> None:
    """Raise AttnError unless the geometry passes the pack page's validate() rules."""
    check(_ffi.lib().dflash_validate(ctypes.byref(_dflash(params))))


def dflash_pack(params, ring_k, ring_v, cur_q, cur_k, cur_v, cache_lengths, write_positions,
                packed_q, packed_k, packed_v, *, stream=None) -> None:
    p = _dflash(params)
    bufs = [ring_k, ring_v, cur_q, cur_k, cur_v, cache_lengths, write_positions, packed_q, packed_k, packed_v]
    for t, n in zip((ring_k, ring_v, packed_q, packed_k, packed_v), ("ring_k", "ring_v", "packed_q", "packed_k",
                                                                     "packed_v")):
        _want(t, _U16, n)
    for t, n in zip((cur_q, cur_k, cur_v), ("cur_q", "cur_k", "cur_v")):
        _want(t, (torch.float32,), n)
    _want(cache_lengths, _U32, "cache_lengths")
    _want(write_positions, _U32, "write_positions")
    check(_ffi.lib().dflash_pack(ctypes.byref(p), *[t.data_ptr() for t in bufs], _bytes(bufs), _stream(stream)))


def dflash_mask(params, cache_lengths, mask, *, stream=None) -> None:
    p = _dflash(params)
    _want(cache_lengths, _U32, "cache_lengths")
    _want(mask, _U16, "mask")
    check(_ffi.lib().dflash_mask(ctypes.byref(p), cache_lengths.data_ptr(), mask.data_ptr(),
                                 _bytes([cache_lengths, mask]), _stream(stream)))


def dflash_commit(params, new_k, new_v, commit_counts, write_positions, ring_k, ring_v, *, stream=None) -> None:
    p = _dflash(params)
    bufs = [new_k, new_v, commit_counts, write_positions, ring_k, ring_v]
    _want(new_k, (torch.float32,), "new_k")
    _want(new_v, (torch.float32,), "new_v")
    _want(commit_counts, _U32, "commit_counts")
    _want(write_positions, _U32, "write_positions")
    _want(ring_k, _U16, "ring_k")
    _want(ring_v, _U16, "ring_v")
    check(_ffi.lib().dflash_commit(ctypes.byref(p), *[t.data_ptr() for t in bufs], _bytes(bufs), _stream(stream)))


def verify_workspace_bytes(params) -> int:
    n = ctypes.c_size_t(0)
    check(_ffi.lib().dflash_verify_workspace_bytes(ctypes.byref(_dflash(params)), ctypes.byref(n)))
    return n.value


def dflash_verify_attention(params, ring_k, ring_v, cur_q, cur_k, cur_v, cache_lengths, write_positions, out, *,
                            scale: float, workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out f32 [lanes, q_heads, rows, head_dim] = the block-verify attention over
    the drafted rows and the ring's visible rows, without packing."""
    p = _dflash(params)
    bufs = [ring_k, ring_v, cur_q, cur_k, cur_v, cache_lengths, write_positions, out]
    _want(ring_k, _U16, "ring_k")
    _want(ring_v, _U16, "ring_v")
    for t, n in zip((cur_q, cur_k, cur_v, out), ("cur_q", "cur_k", "cur_v", "out")):
        _want(t, (torch.float32,), n)
    _want(cache_lengths, _U32, "cache_lengths")
    _want(write_positions, _U32, "write_positions")
    workspace = _scratch(workspace, verify_workspace_bytes(p), out.device, stream)
    check(_ffi.lib().dflash_verify_attention(ctypes.byref(p), float(scale), *[t.data_ptr() for t in bufs],
                                             workspace.data_ptr(), _nbytes(workspace), _bytes(bufs),
                                             _stream(stream)))
    return out


def dflash_mask_rows(lanes: int, rows: int, hidden: int, mask_embedding, draft_input, *, stream=None) -> None:
    _want(mask_embedding, _U16, "mask_embedding")
    _want(draft_input, (torch.float32,), "draft_input")
    check(_ffi.lib().dflash_mask_rows(lanes, rows, hidden, mask_embedding.data_ptr(), draft_input.data_ptr(),
                                      _bytes([mask_embedding, draft_input]), _stream(stream)))
