"""GPU parity of the DFlash2 ring steps against the oracle: bit-exact.

Covers the worked example printed on the mlx-native 0.21.1
dflash2_attention_pack.rs page, the block-verify configuration at full size
(4 lanes, 16 drafted rows, window 4096, 32/8 heads, d 128), forced wrap of
pack and commit, a head_dim 256 geometry and the mask-rows step."""
import json
import os

import numpy as np
import pytest
import torch

import attention_flash_attn_03_amd as fa
import workloads
from gpu_util import announce, dev, host_u16

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _params(case):
    b, h, hk, d, r, w = case.geom
    return fa.DFlashParams(b, h, hk, d, r, w, w - 1 + r, case.max_commit)


def _run_pack_mask(case):
    b, h, hk, d, r, w = case.geom
    k = w - 1 + r
    p = _params(case)
    rk, rv = dev(case.ring_k, True), dev(case.ring_v, True)
    cq, ck, cv = dev(case.cur_q), dev(case.cur_k), dev(case.cur_v)
    L, wp = dev(case.cache_lengths), dev(case.write_positions)
    # poison the outputs so unwritten elements show
    pq = torch.full((b, h, r, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    pk = torch.full((b, hk, k, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    pv = torch.full((b, hk, k, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    mask = torch.full((b, h, r, k), 7.0, dtype=torch.bfloat16, device="cuda")
    fa.dflash_pack(p, rk, rv, cq, ck, cv, L, wp, pq, pk, pv)
    fa.dflash_mask(p, L, mask)
    torch.cuda.synchronize()
    return pq, pk, pv, mask


def _check_pack_mask(orc, case):
    pq, pk, pv, mask = _run_pack_mask(case)
    opq, opk, opv = orc.dflash_pack(case.geom, case.ring_k, case.ring_v, case.cur_q, case.cur_k, case.cur_v,
                                    case.cache_lengths, case.write_positions)
    omask = orc.dflash_mask(case.geom, case.cache_lengths)
    assert np.array_equal(host_u16(pq), opq)
    assert np.array_equal(host_u16(pk), opk)
    assert np.array_equal(host_u16(pv), opv)
    assert np.array_equal(host_u16(mask), omask)


def _check_commit(orc, case):
    p = _params(case)
    rk, rv = dev(case.ring_k, True), dev(case.ring_v, True)
    fa.dflash_commit(p, dev(case.cur_k), dev(case.cur_v), dev(case.commit_counts), dev(case.write_positions), rk, rv)
    torch.cuda.synchronize()
    ork, orv = orc.dflash_commit(case.geom, case.max_commit, case.cur_k, case.cur_v, case.commit_counts,
                                 case.write_positions, case.ring_k, case.ring_v)
    assert np.array_equal(host_u16(rk), ork)
    assert np.array_equal(host_u16(rv), orv)


def test_worked_example_on_gpu(orc):
    announce("dflash worked example")
    g = json.load(open(os.path.join(GOLDEN, "dflash_worked_example.json")))
    ring_k = np.zeros((1, 1, 4, 128), np.uint16)
    ring_v = np.zeros((1, 1, 4, 128), np.uint16)
    ring_k[0, 0, :, 0] = workloads.to_bf16_bits(np.array(g["ring_k_first_element_per_slot"], np.float32))
    ring_v[0, 0, :, 0] = workloads.to_bf16_bits(np.array(g["ring_v_first_element_per_slot"], np.float32))
    cq = np.zeros((1, 2, 1, 128), np.float32); cq.reshape(-1)[0] = 40.0
    ck = np.zeros((1, 2, 1, 128), np.float32); ck.reshape(-1)[[0, 128]] = [20.0, 21.0]
    cv = np.zeros((1, 2, 1, 128), np.float32); cv.reshape(-1)[[0, 128]] = [30.0, 31.0]
    case = workloads.DFlashCase((1, 1, 1, 128, 2, 4), 2, ring_k, ring_v, cq, ck, cv,
                                np.array([3], np.uint32), np.array([1], np.uint32), np.array([2], np.uint32), 1.0)
    pq, pk, pv, mask = _run_pack_mask(case)
    assert host_u16(pq).reshape(-1)[0] == g["expect_packed_q_0"]
    keys = host_u16(pk).reshape(-1)
    assert [int(keys[i * 128]) for i in range(5)] == g["expect_packed_k_row_firsts"]
    assert [int(m) for m in host_u16(mask).reshape(-1)[:10]] == g["expect_mask_first_10"]
    _check_pack_mask(orc, case)
    p = _params(case)
    rk = dev(ring_k, True)
    rv = dev(ring_v, True)
    fa.dflash_commit(p, dev(ck), dev(cv), dev(case.commit_counts), dev(case.write_positions), rk, rv)
    torch.cuda.synchronize()
    ring = host_u16(rk).reshape(-1)
    for idx, val in g["expect_ring_k_after_commit"].items():
        assert ring[int(idx)] == val


@pytest.mark.parametrize("forced_wrap", [False, True])
def test_block_verify_config_full_size(orc, forced_wrap):
    announce("dflash full size forced_wrap=%s" % forced_wrap)
    case = workloads.dflash_case(forced_wrap=forced_wrap)
    _check_pack_mask(orc, case)
    _check_commit(orc, case)


def test_head_dim_256_and_small_window(orc):
    announce("dflash d256 small window")
    for seed in range(3):
        case = workloads.dflash_case(lanes=3, q_heads=6, kv_heads=2, head_dim=256, rows=5, window=9, seed=10 + seed,
                                     forced_wrap=True)
        _check_pack_mask(orc, case)
        _check_commit(orc, case)


def test_edge_lengths_positions_and_counts(orc):
    """Cache length 0, lengths past the window, write positions past the window
    (taken mod window) and commit counts 0 and past max_commit."""
    announce("dflash edge values")
    case = workloads.dflash_case(lanes=4, q_heads=4, kv_heads=1, head_dim=128, rows=4, window=12, seed=20,
                                 cache_lengths=[0, 12, 50, 7], write_positions=[0, 11, 30, 5],
                                 commit_counts=[0, 4, 9, 2])
    _check_pack_mask(orc, case)
    _check_commit(orc, case)


def test_mask_rows(orc):
    announce("dflash mask rows")
    g = json.load(open(os.path.join(GOLDEN, "dflash_mask_rows_example.json")))
    emb = workloads.to_bf16_bits(np.array(g["mask_embedding"], np.float32))
    draft = np.array(g["draft_input"], np.float32).reshape(g["lanes"] * g["rows"], g["hidden"])
    t = dev(draft)
    fa.dflash_mask_rows(g["lanes"], g["rows"], g["hidden"], dev(emb, True), t)
    torch.cuda.synchronize()
    assert t.cpu().numpy().reshape(-1).tolist() == g["expect"]
    rng = np.random.Generator(np.random.PCG64(5))
    emb = workloads.to_bf16_bits(rng.standard_normal(1000).astype(np.float32))
    draft = rng.standard_normal((4 * 16, 1000)).astype(np.float32)
    t = dev(draft)
    fa.dflash_mask_rows(4, 16, 1000, dev(emb, True), t)
    torch.cuda.synchronize()
    assert np.array_equal(t.cpu().numpy(), orc.dflash_mask_rows(4, 16, 1000, emb, draft))
