"""attn_paged_decode_noalloc (the library's static per-GPU scratch array instead
of a workspace) against attn_paged_decode on the same inputs: bit-identical
outputs (same kernels, same launch), and within |err| <= 2e-3 * (1 + |ref|) of
the fp64 oracle.  Two calls in a row, the second smaller, so the second reuses
the scratch the first filled; then the paged workload at full size; then the
call captured in a HIP graph and replayed."""
import numpy as np
import pytest
import torch

import attention_flash_attn_03_amd as fa
import workloads
from gpu_util import announce, assert_close, dev

pytestmark = pytest.mark.gpu


def _both(case):
    q, kp, vp = dev(case.q), dev(case.k_pool), dev(case.v_pool)
    pt, ctx = dev(case.page_table), dev(case.context_lens)
    a = torch.full(case.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    b = torch.full(case.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    fa.attn_paged_decode(q, kp, vp, pt, ctx, a, scale=case.scale, max_context=case.max_context)
    fa.attn_paged_decode_noalloc(q, kp, vp, pt, ctx, b, scale=case.scale, max_context=case.max_context)
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy()


def test_noalloc_matches_workspace_call_twice(orc):
    for kw in (dict(batch=9, ctx_lo=300, ctx_hi=6000, num_pages=3600, n_heads=16, n_kv_heads=4, head_dim=128,
                    seed=81),
               dict(batch=3, ctx_lo=1, ctx_hi=900, num_pages=200, n_heads=8, n_kv_heads=2, head_dim=256, seed=82)):
        announce("noalloc decode %s" % kw)
        case = workloads.paged_case(**kw)
        with_ws, no_ws = _both(case)
        assert np.array_equal(with_ws, no_ws)
        ref = orc.paged_decode(case.q, case.k_pool, case.v_pool, case.page_table, case.context_lens,
                               scale=case.scale)
        assert_close(no_ws, ref, "noalloc decode")


def test_noalloc_full_size_paged_workload(orc):
    announce("noalloc decode, full paged workload")
    case = workloads.paged_case()
    with_ws, no_ws = _both(case)
    assert np.array_equal(with_ws, no_ws)
    seqs = np.arange(0, 64, 9)
    ref = orc.paged_decode(case.q[seqs], case.k_pool, case.v_pool, case.page_table[seqs], case.context_lens[seqs],
                           scale=case.scale)
    assert_close(no_ws[seqs], ref, "noalloc decode full size")


def test_noalloc_under_graph_capture(orc):
    """The entry point for callers that cannot allocate, captured in a HIP graph and
    replayed three times with a workspace call between replays: every replay gives the
    workspace call's bits."""
    announce("noalloc decode captured in a graph, three replays")
    case = workloads.paged_case(batch=6, ctx_lo=50, ctx_hi=5000, num_pages=2200, n_heads=16, n_kv_heads=4,
                                head_dim=128, seed=83)
    q, kp, vp = dev(case.q), dev(case.k_pool), dev(case.v_pool)
    pt, ctx = dev(case.page_table), dev(case.context_lens)
    want, _ = _both(case)
    out = torch.full(case.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            fa.attn_paged_decode_noalloc(q, kp, vp, pt, ctx, out, scale=case.scale, max_context=case.max_context)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), want), "replay %d" % rep
        _both(case)  # eager calls between replays, one of them on the shared scratch
    ref = orc.paged_decode(case.q, case.k_pool, case.v_pool, case.page_table, case.context_lens, scale=case.scale)
    assert_close(want, ref, "noalloc graph decode")
