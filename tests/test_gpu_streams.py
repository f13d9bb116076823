"""The wrappers that allocate a workspace themselves, called on a side stream.

Each call is queued behind a GPU sleep on the side stream, and the default
stream then allocates blocks of the same size and fills them with 0xFF while
the call's kernels have not run yet.  A workspace allocated for the default
stream would be handed to those fills; the binding allocates it for the
stream the kernels run on, so every output still matches the fp64 oracle
within |err| <= 2e-3 * (1 + |ref|)."""
import math

import numpy as np
import pytest
import torch

import attention_flash_attn_03_amd as fa
import workloads
from gpu_util import announce, assert_close, dev

pytestmark = pytest.mark.gpu

SLEEP_CYCLES = 50_000_000  # about 20 ms of GPU time ahead of the call on the side stream


def _race(call, nbytes):
    """Run call() on a fresh side stream behind a sleep, then churn the default stream's pool."""
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        torch.cuda._sleep(SLEEP_CYCLES)
        call(side)
    junk = []
    for _ in range(4):
        t = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        t.fill_(0xFF)
        junk.append(t)
    torch.cuda.synchronize()
    del junk


def test_prefill_on_side_stream(orc):
    announce("prefill on a side stream")
    case = workloads.prefill_synthetic("t", rows=192, kv_len=192, cached=0, n_heads=2, n_kv_heads=1, head_dim=128,
                                       seed=61, q_std=1 / math.sqrt(128), kv_std=1.0, scale=1.0)
    q, k, v, m = dev(case.q), dev(case.k), dev(case.v), dev(case.mask)
    out = torch.full(case.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    need = fa.prefill_workspace_bytes(fa.prefill_params(q, k, v, m, out, scale=1.0))
    _race(lambda s: fa.attn_prefill(q, k, v, m, out, scale=1.0, stream=s), need)
    assert_close(out.cpu().numpy(), orc.attention(case.q, case.k, case.v, case.mask, scale=1.0), "side stream")


def test_paged_decode_on_side_stream(orc):
    announce("paged decode on a side stream")
    case = workloads.paged_case(batch=6, ctx_lo=100, ctx_hi=3000, num_pages=1200, n_heads=8, n_kv_heads=2,
                                head_dim=128, seed=62)
    q, kp, vp = dev(case.q), dev(case.k_pool), dev(case.v_pool)
    pt, ctx = dev(case.page_table), dev(case.context_lens)
    out = torch.full(case.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    need = fa.decode_workspace_bytes(fa.decode_params(q, kp, vp, pt, out, scale=case.scale,
                                                      max_context=case.max_context))
    _race(lambda s: fa.attn_paged_decode(q, kp, vp, pt, ctx, out, scale=case.scale, max_context=case.max_context,
                                         stream=s), need)
    ref = orc.paged_decode(case.q, case.k_pool, case.v_pool, case.page_table, case.context_lens, scale=case.scale)
    assert_close(out.cpu().numpy(), ref, "side stream")


def test_paged_prefill_on_side_stream(orc):
    announce("paged prefill on a side stream")
    mc = workloads.paged_multi_case(max_tokens=16, batch=4, ctx_lo=100, ctx_hi=2000, num_pages=600, n_heads=8,
                                    n_kv_heads=2, head_dim=128, seed=63)
    pc = mc.paged
    q, kp, vp = dev(mc.q), dev(pc.k_pool), dev(pc.v_pool)
    pt, ql, st = dev(pc.page_table), dev(mc.query_lens), dev(mc.position_starts)
    out = torch.zeros(mc.q.shape, dtype=torch.float32, device="cuda")
    need = fa.paged_prefill_workspace_bytes(fa.paged_prefill_params(q, kp, vp, pt, out, scale=pc.scale,
                                                                    max_context=pc.max_context))
    _race(lambda s: fa.attn_paged_prefill(q, kp, vp, pt, ql, st, out, scale=pc.scale, max_context=pc.max_context,
                                          stream=s), need)
    ref = orc.paged_prefill(mc.q, pc.k_pool, pc.v_pool, pc.page_table, mc.query_lens, mc.position_starts,
                            scale=pc.scale, cap=pc.max_context)
    got = out.cpu().numpy()
    for b, n in enumerate(mc.query_lens):
        assert_close(got[b, :int(n)], ref[b, :int(n)], "side stream (sequence %d)" % b)


def test_verify_attention_on_side_stream(orc):
    announce("pack-free verify attention on a side stream")
    c = workloads.dflash_case(lanes=2, q_heads=8, kv_heads=2, head_dim=128, rows=8, window=512, seed=64)
    b, h, hk, d, r, w = c.geom
    prm = fa.DFlashParams(b, h, hk, d, r, w, w - 1 + r, c.max_commit)

    def bf(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

    def u32(a):
        return torch.from_numpy(a.view(np.int32)).cuda()

    args = (bf(c.ring_k), bf(c.ring_v), dev(c.cur_q), dev(c.cur_k), dev(c.cur_v), u32(c.cache_lengths),
            u32(c.write_positions))
    out = torch.full((b, h, r, d), float("nan"), dtype=torch.float32, device="cuda")
    need = fa.verify_workspace_bytes(prm)
    _race(lambda s: fa.dflash_verify_attention(prm, *args, out, scale=c.scale, stream=s), need)
    ref = orc.dflash_verify_attention(c.geom, c.ring_k, c.ring_v, c.cur_q, c.cur_k, c.cur_v, c.cache_lengths,
                                      c.write_positions, scale=c.scale)
    assert_close(out.cpu().numpy(), ref, "side stream")
