"""Pins for the oracle's attention (O1) and paged decode (O2).

The oracle is checked against things other than itself: closed forms,
invariants, exhaustive checks of its float widening, and torch's float64
scaled_dot_product_attention (a library routine with its own code path) on
small shapes.  A dropped term, a wrong sign, a wrong head mapping, a scaled
mask or a transposed operand in oracle.c fails at least one test here.
"""
import math

import numpy as np
import pytest
import torch

import workloads

RTOL = 1e-12


def _sdpa_f64(q, k, v, mask, scale):
    """Library reference: q [B,R,H,D], k/v [B,KV,HK,D], mask [B,H|1,R,KV] (float64 arrays)."""
    B, R, H, D = q.shape
    HK = k.shape[2]
    g = H // HK
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(0, 2, 1, 3)))             # B,H,R,D
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(0, 2, 1, 3))).repeat_interleave(g, dim=1)
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(0, 2, 1, 3))).repeat_interleave(g, dim=1)
    am = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask))
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=am, scale=scale)
    return out.numpy().transpose(0, 2, 1, 3)


def _rand(shape, seed, dtype=np.float64):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape).astype(dtype)


# --------------------------------------------------------------------------- widening
def test_f16_widening_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_widening_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([orc.bf16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# --------------------------------------------------------------------------- closed forms
def test_single_visible_key_returns_its_value(orc):
    q, k, v = _rand((1, 3, 2, 16), 1), _rand((1, 7, 1, 16), 2), _rand((1, 7, 1, 16), 3)
    mask = np.full((1, 1, 3, 7), -np.inf)
    for i, j in enumerate((4, 0, 6)):
        mask[0, 0, i, j] = 0.25  # one visible key per row, non-zero additive value
    o = orc.attention(q, k, v, mask, scale=0.7)
    for i, j in enumerate((4, 0, 6)):
        for h in range(2):
            assert np.array_equal(o[0, i, h], v[0, j, 0])


def test_equal_scores_give_mean_of_visible_values(orc):
    q = np.zeros((1, 2, 1, 8))
    k, v = _rand((1, 5, 1, 8), 4), _rand((1, 5, 1, 8), 5)
    mask = np.zeros((1, 1, 2, 5))
    mask[0, 0, 1, 3:] = -np.inf
    o = orc.attention(q, k, v, mask, scale=1.0)
    np.testing.assert_allclose(o[0, 0, 0], v[0, :, 0].mean(axis=0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[0, 1, 0], v[0, :3, 0].mean(axis=0), rtol=0, atol=1e-15)


@pytest.mark.parametrize("gap", [-3.0, 0.5, 2.0, 30.0])
def test_two_keys_weights_are_logistic(orc, gap):
    # s_0 - s_1 = scale*(q.k0 - q.k1) + (m0 - m1) = gap: weight of key 0 is 1/(1+exp(-gap))
    d = 4
    q = np.zeros((1, 1, 1, d)); q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, 2, 1, d)); k[0, 0, 0, 0] = 2.0; k[0, 1, 0, 0] = 0.5
    v = np.zeros((1, 2, 1, d)); v[0, 0, 0, :] = [1, 0, 3, -1]; v[0, 1, 0, :] = [0, 1, -2, 5]
    scale = 0.5
    m1 = 0.25
    m0 = gap - scale * (2.0 - 0.5) + m1          # the mask is added after the scale
    mask = np.array([m0, m1]).reshape(1, 1, 1, 2)
    o = orc.attention(q, k, v, mask, scale=scale)
    w0 = 1.0 / (1.0 + math.exp(-gap))
    np.testing.assert_allclose(o[0, 0, 0], w0 * v[0, 0, 0] + (1 - w0) * v[0, 1, 0], rtol=1e-13, atol=1e-15)


def test_fully_masked_row_is_zero(orc):
    q, k, v = _rand((1, 2, 1, 8), 6), _rand((1, 4, 1, 8), 7), _rand((1, 4, 1, 8), 8)
    mask = np.zeros((1, 1, 2, 4)); mask[0, 0, 1, :] = -np.inf
    o = orc.attention(q, k, v, mask, scale=1.0)
    assert np.all(o[0, 1] == 0.0) and np.all(np.isfinite(o))
    assert np.any(o[0, 0] != 0.0)


def test_no_keys_equals_every_key_masked(orc):
    """With no keys at all a row sees nothing, as with every key masked: O = 0.  The
    paged form at cap 0 gives such rows for the new tokens and NaN past them."""
    q = _rand((1, 3, 2, 8), 9)
    empty = orc.attention(q, np.zeros((1, 0, 1, 8)), np.zeros((1, 0, 1, 8)), None, scale=1.0)
    k, v = _rand((1, 2, 1, 8), 10), _rand((1, 2, 1, 8), 11)
    masked = orc.attention(q, k, v, np.full((1, 1, 3, 2), -np.inf), scale=1.0)
    assert empty.shape == masked.shape and np.all(empty == 0.0) and np.all(masked == 0.0)
    mc = workloads.paged_multi_case(max_tokens=4, batch=2, ctx_lo=4, ctx_hi=30, num_pages=8, n_heads=2, n_kv_heads=1,
                                    head_dim=128, seed=64, query_lens=[3, 1])
    pc = mc.paged
    got = orc.paged_prefill(mc.q, pc.k_pool, pc.v_pool, pc.page_table, mc.query_lens, mc.position_starts,
                            scale=pc.scale, cap=0)
    assert np.all(got[0, :3] == 0.0) and np.all(np.isnan(got[0, 3:]))
    assert np.all(got[1, :1] == 0.0) and np.all(np.isnan(got[1, 1:]))


def test_no_mask_equals_zero_mask(orc):
    q, k, v = _rand((2, 3, 4, 8), 9), _rand((2, 6, 2, 8), 10), _rand((2, 6, 2, 8), 11)
    a = orc.attention(q, k, v, None, scale=0.3)
    b = orc.attention(q, k, v, np.zeros((2, 1, 3, 6)), scale=0.3)
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------- invariants
def test_per_row_mask_shift_is_invisible(orc):
    q, k, v = _rand((1, 4, 2, 8), 12), _rand((1, 9, 1, 8), 13), _rand((1, 9, 1, 8), 14)
    mask = _rand((1, 1, 4, 9), 15)
    shift = np.array([0.0, 5.0, -7.5, 100.0]).reshape(1, 1, 4, 1)
    a = orc.attention(q, k, v, mask, scale=0.4)
    b = orc.attention(q, k, v, mask + shift, scale=0.4)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_key_permutation_is_invisible(orc):
    q, k, v = _rand((1, 3, 2, 8), 16), _rand((1, 11, 2, 8), 17), _rand((1, 11, 2, 8), 18)
    mask = np.where(_rand((1, 2, 3, 11), 19) > 0.8, -np.inf, 0.0)
    perm = np.random.Generator(np.random.PCG64(20)).permutation(11)
    a = orc.attention(q, k, v, mask, scale=0.5)
    b = orc.attention(q, k[:, perm], v[:, perm], mask[..., perm], scale=0.5)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_masked_padding_keys_are_invisible(orc):
    q, k, v = _rand((1, 3, 2, 8), 21), _rand((1, 10, 1, 8), 22), _rand((1, 10, 1, 8), 23)
    mask = np.zeros((1, 1, 3, 10))
    kp = np.concatenate([k, np.zeros((1, 6, 1, 8))], axis=1)
    vp = np.concatenate([v, np.zeros((1, 6, 1, 8))], axis=1)
    mp = np.concatenate([mask, np.full((1, 1, 3, 6), -np.inf)], axis=3)
    a = orc.attention(q, k, v, mask, scale=0.5)
    b = orc.attention(q, kp, vp, mp, scale=0.5)
    assert np.array_equal(a, b)


def test_gqa_uses_floor_head_mapping(orc):
    # 6 query heads over 3 KV heads (g = 2): head h reads KV head h // 2; h % 3 would differ for h = 1..4
    q, k, v = _rand((1, 2, 6, 8), 24), _rand((1, 5, 3, 8), 25), _rand((1, 5, 3, 8), 26)
    o = orc.attention(q, k, v, None, scale=0.6)
    kr = np.repeat(k, 2, axis=2)
    vr = np.repeat(v, 2, axis=2)
    o_mha = orc.attention(q, kr, vr, None, scale=0.6)
    assert np.array_equal(o, o_mha)
    wrong = orc.attention(q, np.tile(k, (1, 1, 2, 1)), np.tile(v, (1, 1, 2, 1)), None, scale=0.6)
    assert not np.allclose(o, wrong)


def test_output_in_convex_hull_of_visible_values(orc):
    q, k, v = _rand((1, 5, 2, 8), 27), _rand((1, 12, 1, 8), 28), _rand((1, 12, 1, 8), 29)
    mask = np.where(np.arange(12)[None, None, None, :] <= np.arange(5)[None, None, :, None] + 4, 0.0, -np.inf)
    o = orc.attention(q, k, v, mask, scale=2.0)
    for i in range(5):
        vis = v[0, : i + 5, 0]
        assert np.all(o[0, i] >= vis.min(axis=0) - 1e-12) and np.all(o[0, i] <= vis.max(axis=0) + 1e-12)


# --------------------------------------------------------------------------- library cross-check
@pytest.mark.parametrize("B,R,KV,H,HK,D,per_head", [
    (1, 5, 9, 4, 1, 16, False),
    (2, 7, 13, 6, 3, 32, True),
    (1, 16, 40, 8, 2, 64, False),
])
def test_matches_torch_sdpa_float64(orc, B, R, KV, H, HK, D, per_head):
    q, k, v = _rand((B, R, H, D), 30), _rand((B, KV, HK, D), 31), _rand((B, KV, HK, D), 32)
    mh = H if per_head else 1
    rng = np.random.Generator(np.random.PCG64(33))
    mask = np.where(rng.random((B, mh, R, KV)) < 0.3, -np.inf, rng.standard_normal((B, mh, R, KV)))
    mask[..., 0] = 0.0  # keep one key per row so the library does not produce NaN rows
    scale = 1.0 / math.sqrt(D)
    o = orc.attention(q, k, v, mask, scale=scale)
    ref = _sdpa_f64(q, k, v, mask if per_head else np.broadcast_to(mask, (B, H, R, KV)), scale)
    np.testing.assert_allclose(o, ref, rtol=1e-11, atol=1e-12)


def test_strided_f16_inputs_match_library(orc):
    """The same buffers and strides the GPU sees: f32 Q, f16 K/V with row stride HK*D."""
    case = workloads.prefill_synthetic("t", rows=24, kv_len=40, cached=16, n_heads=4, n_kv_heads=2,
                                       head_dim=32, seed=34, q_std=0.25, kv_std=1.0, holes=0.2)
    o = orc.attention(case.q, case.k, case.v, case.mask, scale=case.scale)
    ref = _sdpa_f64(case.q.astype(np.float64), case.k.astype(np.float64), case.v.astype(np.float64),
                    np.broadcast_to(case.mask.astype(np.float64), (1, 4, 24, 40)), case.scale)
    np.testing.assert_allclose(o, ref, rtol=1e-11, atol=1e-12)


def test_bf16_inputs_widen_exactly(orc):
    bits = workloads.to_bf16_bits(_rand((1, 6, 1, 8), 35, np.float32))
    kbits = workloads.to_bf16_bits(_rand((1, 9, 1, 8), 36, np.float32))
    vbits = workloads.to_bf16_bits(_rand((1, 9, 1, 8), 37, np.float32))
    o = orc.attention(bits, kbits, vbits, None, scale=0.3, q_bf16=True, kv_bf16=True)
    widen = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().numpy()
    ref = _sdpa_f64(widen(bits), widen(kbits), widen(vbits), None, 0.3)
    np.testing.assert_allclose(o, ref, rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------- paged decode
def test_paged_matches_gathered_library(orc):
    case = workloads.paged_case(batch=5, ctx_lo=1, ctx_hi=70, page_size=16, num_pages=64, n_heads=4,
                                n_kv_heads=2, head_dim=16, seed=38)
    o = orc.paged_decode(case.q, case.k_pool, case.v_pool, case.page_table, case.context_lens, scale=case.scale)
    for b in range(5):
        n = int(case.context_lens[b])
        t = np.arange(n)
        pages = case.page_table[b, t // 16]
        kk = case.k_pool[pages, t % 16].astype(np.float64)[None]       # 1, n, HK, D
        vv = case.v_pool[pages, t % 16].astype(np.float64)[None]
        ref = _sdpa_f64(case.q[b][None, None].astype(np.float64), kk, vv, None, case.scale)
        np.testing.assert_allclose(o[b], ref[0, 0], rtol=1e-11, atol=1e-12)


def test_paged_ignores_unused_slots_and_pages(orc):
    clean = workloads.paged_case(batch=4, ctx_lo=1, ctx_hi=50, num_pages=32, n_heads=2, n_kv_heads=1,
                                 head_dim=8, seed=39)
    poisoned = workloads.paged_case(batch=4, ctx_lo=1, ctx_hi=50, num_pages=32, n_heads=2, n_kv_heads=1,
                                    head_dim=8, seed=39, poison_unused=True)
    a = orc.paged_decode(clean.q, clean.k_pool, clean.v_pool, clean.page_table, clean.context_lens, scale=0.5)
    b = orc.paged_decode(poisoned.q, poisoned.k_pool, poisoned.v_pool, poisoned.page_table,
                         poisoned.context_lens, scale=0.5)
    assert np.array_equal(a, b) and np.all(np.isfinite(b))


def test_paged_equals_contiguous_attention(orc):
    case = workloads.paged_case(batch=3, ctx_lo=20, ctx_hi=60, num_pages=16, n_heads=4, n_kv_heads=2,
                                head_dim=8, seed=40)
    o = orc.paged_decode(case.q, case.k_pool, case.v_pool, case.page_table, case.context_lens, scale=0.5)
    for b in range(3):
        n = int(case.context_lens[b])
        t = np.arange(n)
        kk = case.k_pool[case.page_table[b, t // 16], t % 16][None]
        vv = case.v_pool[case.page_table[b, t // 16], t % 16][None]
        c = orc.attention(case.q[b][None, None], kk, vv, None, scale=0.5)
        assert np.array_equal(o[b], c[0, 0])


# --------------------------------------------------------------------------- multi-token paged
@pytest.mark.parametrize("page_size,seed", [(16, 61), (5, 62)])
def test_paged_prefill_rows_are_decode_steps(orc, page_size, seed):
    """Token i of a multi-token call is a decode step of the context that ends at
    it: the paged decode path (keys read slot by slot through the page table in
    C) with context position_start + i + 1 gives the same row."""
    mc = workloads.paged_multi_case(max_tokens=6, seed=seed, batch=4, ctx_lo=1, ctx_hi=90, page_size=page_size,
                                    num_pages=96, n_heads=4, n_kv_heads=2, head_dim=128)
    pc = mc.paged
    got = orc.paged_prefill(mc.q, pc.k_pool, pc.v_pool, pc.page_table, mc.query_lens, mc.position_starts,
                            scale=0.7, cap=pc.max_context)
    for b in range(4):
        n = int(mc.query_lens[b])
        assert np.all(np.isnan(got[b, n:]))
        for i in range(n):
            ctx = np.zeros(4, np.int32)
            ctx[b] = mc.position_starts[b] + i + 1
            q1 = np.zeros(pc.q.shape, np.float32)
            q1[b] = mc.q[b, i]
            dec = orc.paged_decode(q1, pc.k_pool, pc.v_pool, pc.page_table, ctx, scale=0.7)
            np.testing.assert_allclose(got[b, i], dec[b], rtol=1e-12, atol=1e-12)


def test_paged_prefill_one_token_is_decode(orc):
    pc = workloads.paged_case(batch=3, ctx_lo=1, ctx_hi=70, num_pages=40, n_heads=4, n_kv_heads=1, head_dim=128,
                              seed=63)
    q = pc.q[:, None]
    got = orc.paged_prefill(q, pc.k_pool, pc.v_pool, pc.page_table, np.ones(3, np.int32), pc.context_lens - 1,
                            scale=pc.scale, cap=pc.max_context)
    dec = orc.paged_decode(pc.q, pc.k_pool, pc.v_pool, pc.page_table, pc.context_lens, scale=pc.scale)
    np.testing.assert_allclose(got[:, 0], dec, rtol=1e-12, atol=1e-12)

