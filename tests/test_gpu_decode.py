"""GPU parity of attn_paged_decode against the fp64 oracle, elementwise within
|err| <= 2e-3 * (1 + |ref|): oracle-sized page tables, bf16 and head_dim 256,
page sizes 1-3 with contexts of up to 16k tokens, one unit of about 69 pieces,
context lengths outside [0, max_context] (clamped), empty contexts, NaN-poisoned unused slots, the interleaved K/V token record,
paged == contiguous (through attn_prefill, within a bound derived from the f16
rounding of P), the same logical KV under two different physical page
placements (bit-identical), the full-size paged-decode configuration (64
sequences, contexts 512..16384, 65536-page pool), every sequence, in the
benchmark's launch configuration, and replays of a captured HIP graph."""
import math

import numpy as np
import pytest
import torch

import attention_flash_attn_03_amd as fa
import workloads
from gpu_util import announce, assert_close, dev

pytestmark = pytest.mark.gpu


def _run(case, k_pool=None, v_pool=None, max_context=None):
    bf = case.meta["kv_dtype"] == "bf16"
    q = dev(case.q)
    kp = dev(case.k_pool, bf) if k_pool is None else k_pool
    vp = dev(case.v_pool, bf) if v_pool is None else v_pool
    out = torch.full(case.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    fa.attn_paged_decode(q, kp, vp, dev(case.page_table), dev(case.context_lens), out, scale=case.scale,
                         max_context=case.max_context if max_context is None else max_context)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _oracle(orc, case, seqs=None):
    sel = slice(None) if seqs is None else seqs
    return orc.paged_decode(case.q[sel], case.k_pool, case.v_pool, case.page_table[sel], case.context_lens[sel],
                            scale=case.scale, kv_bf16=case.meta["kv_dtype"] == "bf16")


@pytest.mark.parametrize("kw", [
    dict(batch=6, ctx_lo=1, ctx_hi=700, num_pages=300, n_heads=8, n_kv_heads=2, head_dim=128, seed=31),
    dict(batch=4, ctx_lo=100, ctx_hi=3000, num_pages=800, n_heads=4, n_kv_heads=4, head_dim=128, seed=32),
    dict(batch=3, ctx_lo=1, ctx_hi=900, num_pages=200, n_heads=8, n_kv_heads=1, head_dim=256, seed=33,
         kv_dtype="bf16"),
    dict(batch=5, ctx_lo=5000, ctx_hi=9000, num_pages=3000, n_heads=16, n_kv_heads=2, head_dim=128, seed=34),
])
def test_decode_oracle_sized(orc, kw):
    announce("decode %s" % kw)
    case = workloads.paged_case(**kw)
    assert_close(_run(case), _oracle(orc, case), "decode")


@pytest.mark.parametrize("page_size", [1, 2, 3])
def test_small_pages_long_contexts(orc, page_size):
    """Page sizes below 4 bound the tiles per range by the page-id buffer (32 * page_size
    tiles); contexts long enough (about 160k tokens over 8 KV heads) that the device sets
    more than the minimum 32 tiles per range where that bound allows it.  Every row."""
    announce("decode page_size %d, long contexts" % page_size)
    case = workloads.paged_case(batch=12, ctx_lo=11000, ctx_hi=16000, page_size=page_size,
                                num_pages=-(-12 * 16000 // page_size), n_heads=32, n_kv_heads=8, head_dim=128,
                                seed=36 + page_size)
    assert_close(_run(case), _oracle(orc, case), "decode small pages")


def test_unit_of_more_than_64_pieces(orc):
    """One sequence, one head, a 70k-token context: the line is short, so ranges take the
    minimum 32 tiles and the unit is cut into about 69 pieces, past the 64 (m, l) one pass
    of the reduce reads."""
    announce("decode, one unit of about 69 pieces")
    case = workloads.paged_case(batch=1, num_pages=4400, n_heads=1, n_kv_heads=1, head_dim=128, seed=38,
                                context_lens=np.array([70000], np.int32), ctx_hi=70000)
    assert_close(_run(case), _oracle(orc, case), "decode many pieces")


def test_out_of_range_contexts_are_clamped(orc):
    """Context lengths below 0 and past max_context are clamped to [0, max_context] (the
    oracle is given the clamped lengths); a length clamped to 0 gives a zero row."""
    announce("decode with out-of-range context lengths")
    case = workloads.paged_case(batch=4, ctx_lo=20, ctx_hi=400, num_pages=120, n_heads=8, n_kv_heads=2,
                                head_dim=128, seed=39)
    cap = 300
    lens = np.array([-5, 50, cap + 100, 2 ** 31 - 1], np.int32)
    pt = case.page_table.copy()
    free = np.argwhere(pt < 0)
    pt[free[:, 0], free[:, 1]] = (5 * free[:, 0] + 11 * free[:, 1]) % case.k_pool.shape[0]
    moved = workloads.PagedCase(case.q, case.k_pool, case.v_pool, pt, lens, case.scale, cap, case.meta)
    got = _run(moved, max_context=cap)
    assert np.all(got[0] == 0.0)
    clipped = workloads.PagedCase(case.q, case.k_pool, case.v_pool, pt, np.clip(lens, 0, cap).astype(np.int32),
                                  case.scale, cap, case.meta)
    assert_close(got, _oracle(orc, clipped), "decode clamped")


def test_empty_and_one_token_contexts(orc):
    announce("decode empty contexts")
    case = workloads.paged_case(batch=4, num_pages=64, n_heads=4, n_kv_heads=2, head_dim=128, seed=35,
                                ctx_hi=100, context_lens=np.array([0, 1, 17, 0], np.int32))
    got = _run(case)
    assert np.all(got[[0, 3]] == 0.0)
    assert_close(got, _oracle(orc, case), "decode short")


def test_poisoned_unused_slots_are_never_read(orc):
    announce("decode NaN-poisoned unused slots")
    kw = dict(batch=5, ctx_lo=1, ctx_hi=400, num_pages=200, n_heads=8, n_kv_heads=2, head_dim=128, seed=36)
    clean = workloads.paged_case(**kw)
    poisoned = workloads.paged_case(poison_unused=True, **kw)
    a, b = _run(clean), _run(poisoned)
    assert np.all(np.isfinite(b))
    assert np.array_equal(a, b)


def test_interleaved_token_record(orc):
    """The token record [2 (K, V), kv_heads, head_dim] of one pool: k_pool = base,
    v_pool = base + kv_heads*head_dim, token stride 2*kv_heads*head_dim."""
    announce("decode interleaved K/V record")
    case = workloads.paged_case(batch=3, ctx_lo=10, ctx_hi=300, num_pages=80, n_heads=4, n_kv_heads=2, head_dim=128,
                                seed=37)
    rec = np.stack([case.k_pool, case.v_pool], axis=2)          # [pages, slot, 2, hk, d]
    base = dev(rec)
    kview = base[:, :, 0]
    vview = base[:, :, 1]
    assert kview.stride() == vview.stride()
    got = _run(case, k_pool=kview, v_pool=vview)
    assert_close(got, _oracle(orc, case), "interleaved")


def _p_rounding_bound(orc, q, kk, vv, o, scale):
    """Largest |O_a - O_b| between two kernels that both round Q and K/V to the same f16
    values, round every probability p to f16 and divide by the sum of the rounded p,
    but against different running maxima and in different f32 orders.  For one kernel,
    with weights w_j = p_j / l and n keys:
      f16 rounding of p above 2^-14 (relative 2^-11):  2^-11 sum_j w_j |v_j - O|
      below 2^-14 (absolute 2^-25, and l >= 1):         n 2^-25 max_j |v_j - O|
      f32 accumulation of sum p v and of l:             2 n 2^-24 sum_j w_j (|v_j| + |O|)
    with |v_j - O| <= |v_j| + |O| and sum_j w_j |v_j| the attention of |V|, taken from
    the oracle.  Two kernels: twice that."""
    n = kk.shape[1]
    a = orc.attention(q, kk, np.abs(vv), scale=scale)
    ao = np.abs(o)
    vmax = float(np.max(np.abs(vv)))
    one = 2.0 ** -11 * (a + ao) + n * 2.0 ** -25 * (vmax + ao) + 2 * n * 2.0 ** -24 * (a + ao)
    return 2 * one


def test_paged_equals_contiguous_prefill(orc):
    """The same logical KV through the page table (decode kernel) and as one
    contiguous range (prefill kernel): both match the oracle, and each other
    within the bound that their f16 rounding of the probabilities against
    different running maxima allows (about half the oracle bound here)."""
    announce("decode paged vs contiguous prefill")
    case = workloads.paged_case(batch=3, ctx_lo=200, ctx_hi=600, num_pages=200, n_heads=8, n_kv_heads=2,
                                head_dim=128, seed=38)
    paged = _run(case)
    ref = _oracle(orc, case)
    assert_close(paged, ref, "paged")
    for b in range(3):
        n = int(case.context_lens[b])
        t = np.arange(n)
        kk = case.k_pool[case.page_table[b, t // 16], t % 16][None]
        vv = case.v_pool[case.page_table[b, t // 16], t % 16][None]
        out = torch.zeros((1, 1, 8, 128), dtype=torch.float32, device="cuda")
        fa.attn_prefill(dev(case.q[b][None, None]), dev(kk), dev(vv), None, out, scale=case.scale)
        torch.cuda.synchronize()
        contiguous = out.cpu().numpy()[0, 0].astype(np.float64)
        assert_close(contiguous, ref[b], "contiguous")
        bound = _p_rounding_bound(orc, case.q[b][None, None], kk, vv, ref[b][None, None], case.scale)[0, 0]
        d = np.abs(paged[b] - contiguous)
        assert np.all(d <= bound), "paged vs contiguous: |d| %g above the rounding bound %g" % (
            float(d.max()), float(bound.flat[np.argmax(d - bound)]))


def relocate_pages(case, seed):
    """The same logical KV with every pool page moved to another physical page:
    pool page p goes to page sigma[p] and the page table follows it."""
    rng = np.random.Generator(np.random.PCG64(seed))
    sigma = rng.permutation(case.k_pool.shape[0]).astype(np.int32)
    k2, v2 = np.empty_like(case.k_pool), np.empty_like(case.v_pool)
    k2[sigma], v2[sigma] = case.k_pool, case.v_pool
    pt2 = np.where(case.page_table >= 0, sigma[np.maximum(case.page_table, 0)], -1).astype(np.int32)
    return k2, v2, pt2


def test_page_placement_is_invisible(orc):
    """Two page tables holding the same logical KV in different physical pages give
    bit-identical output."""
    announce("decode same logical KV, two physical page placements")
    case = workloads.paged_case(batch=7, ctx_lo=1, ctx_hi=2500, num_pages=1200, n_heads=16, n_kv_heads=4,
                                head_dim=128, seed=39)
    a = _run(case)
    k2, v2, pt2 = relocate_pages(case, 391)
    moved = workloads.PagedCase(case.q, k2, v2, pt2, case.context_lens, case.scale, case.max_context, case.meta)
    b = _run(moved)
    assert np.array_equal(a, b)
    assert_close(a, _oracle(orc, case), "decode")


def test_full_size_config_every_sequence(orc):
    announce("decode full size (64 seqs, 65536-page pool), every sequence")
    case = workloads.paged_case()
    got = _run(case)
    assert_close(got, _oracle(orc, case), "decode full size")


def test_graph_replays_match_eager(orc):
    """attn_paged_decode captured in a HIP graph (its grid sized from the device's
    occupancy, its tiles per range set on the device) and replayed four times, with an
    eager call on the same workspace between replays: every replay gives the eager bits."""
    announce("paged decode captured in a graph, four replays")
    case = workloads.paged_case(batch=12, ctx_lo=200, ctx_hi=9000, num_pages=8000, n_heads=32, n_kv_heads=8,
                                head_dim=128, seed=91)
    q, kp, vp = dev(case.q), dev(case.k_pool), dev(case.v_pool)
    pt, ctx = dev(case.page_table), dev(case.context_lens)
    out = torch.full(case.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    p = fa.decode_params(q, kp, vp, pt, out, scale=case.scale, max_context=case.max_context)
    ws = torch.empty(fa.decode_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    eager = torch.full_like(out, float("nan"))
    fa.attn_paged_decode(q, kp, vp, pt, ctx, eager, scale=case.scale, max_context=case.max_context, workspace=ws)
    torch.cuda.synchronize()
    want = eager.cpu().numpy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            fa.attn_paged_decode(q, kp, vp, pt, ctx, out, scale=case.scale, max_context=case.max_context,
                                 workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), want), "replay %d" % rep
        if rep == 1:
            fa.attn_paged_decode(q, kp, vp, pt, ctx, eager, scale=case.scale, max_context=case.max_context,
                                 workspace=ws)
            torch.cuda.synchronize()
            assert np.array_equal(eager.cpu().numpy(), want)
    ref = orc.paged_decode(case.q, case.k_pool, case.v_pool, case.page_table, case.context_lens, scale=case.scale)
    assert_close(want, ref, "graph decode")
