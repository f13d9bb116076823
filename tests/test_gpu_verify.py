"""GPU parity of dflash_verify_attention (block-verify attention read from the
ring in place) against the oracle's pack -> mask -> attention, elementwise
within |err| <= 2e-3 * (1 + |ref|).

Covers the full-size block-verify configuration (4 lanes, 16 drafted rows,
window 4096, 32/8 heads, d 128) and its forced-wrap variant, agreement with
the packed path on the GPU, empty and full caches, cache lengths past the
window, write positions past the window, ring slots outside the visible
range poisoned with NaN, head_dim 256, MHA, several query-head groups per KV
head and row counts that leave a partial 16-column slice."""
import numpy as np
import pytest
import torch

import attention_flash_attn_03_amd as fa
import workloads
from gpu_util import announce, assert_close, dev

pytestmark = pytest.mark.gpu


def _params(case):
    b, h, hk, d, r, w = case.geom
    return fa.DFlashParams(b, h, hk, d, r, w, w - 1 + r, case.max_commit)


def _run(case, ring_k=None, ring_v=None):
    b, h, hk, d, r, w = case.geom
    out = torch.full((b, h, r, d), float("nan"), dtype=torch.float32, device="cuda")
    rk = dev(case.ring_k if ring_k is None else ring_k, True)
    rv = dev(case.ring_v if ring_v is None else ring_v, True)
    fa.dflash_verify_attention(_params(case), rk, rv, dev(case.cur_q), dev(case.cur_k), dev(case.cur_v),
                               dev(case.cache_lengths), dev(case.write_positions), out, scale=case.scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _oracle(orc, case):
    return orc.dflash_verify_attention(case.geom, case.ring_k, case.ring_v, case.cur_q, case.cur_k, case.cur_v,
                                       case.cache_lengths, case.write_positions, scale=case.scale)


def test_full_size_verify(orc):
    announce("verify attention full size (4 lanes, w 4096, h 32/8, d 128)")
    case = workloads.dflash_case()
    assert_close(_run(case), _oracle(orc, case), "verify full size")


def test_full_size_forced_wrap_matches_packed_path(orc):
    announce("verify attention forced wrap vs packed path")
    case = workloads.dflash_case(forced_wrap=True)
    b, h, hk, d, r, w = case.geom
    fused = _run(case)
    ref = _oracle(orc, case)
    assert_close(fused, ref, "verify forced wrap")
    # the packed path on the GPU: pack, mask, attn_prefill over the packed buffers
    k = w - 1 + r
    p = _params(case)
    pq = torch.empty((b, h, r, d), dtype=torch.bfloat16, device="cuda")
    pk = torch.empty((b, hk, k, d), dtype=torch.bfloat16, device="cuda")
    pv = torch.empty_like(pk)
    mask = torch.empty((b, h, r, k), dtype=torch.bfloat16, device="cuda")
    L, wp = dev(case.cache_lengths), dev(case.write_positions)
    fa.dflash_pack(p, dev(case.ring_k, True), dev(case.ring_v, True), dev(case.cur_q), dev(case.cur_k),
                   dev(case.cur_v), L, wp, pq, pk, pv)
    fa.dflash_mask(p, L, mask)
    out = torch.empty((b, h, r, d), dtype=torch.float32, device="cuda")
    fa.attn_prefill(pq.permute(0, 2, 1, 3), pk.permute(0, 2, 1, 3), pv.permute(0, 2, 1, 3), mask,
                    out.permute(0, 2, 1, 3), scale=case.scale)
    torch.cuda.synchronize()
    packed = out.cpu().numpy()
    assert_close(packed, ref, "packed path")
    assert_close(fused, packed.astype(np.float64), "fused vs packed")


@pytest.mark.parametrize("lengths,positions", [
    ([0, 1, 4096, 5000], [0, 4095, 17, 9000]),   # empty cache, one row, full, past the window; wp past w
    ([63, 64, 65, 4095], [64, 0, 4096 + 63, 1]),  # lengths around a tile edge
])
def test_lengths_and_positions(orc, lengths, positions):
    announce("verify attention lengths %s positions %s" % (lengths, positions))
    case = workloads.dflash_case(cache_lengths=lengths, write_positions=positions, seed=41)
    assert_close(_run(case), _oracle(orc, case), "verify lengths")


def test_unreached_ring_slots_are_never_read(orc):
    """Slots no row sees hold NaN; the output must not change."""
    announce("verify attention with NaN outside the visible ring range")
    case = workloads.dflash_case(lanes=3, window=512, cache_lengths=[100, 0, 300], write_positions=[250, 7, 511],
                                 seed=42)
    b, h, hk, d, r, w = case.geom
    rk, rv = case.ring_k.copy(), case.ring_v.copy()
    for lane in range(b):
        reach = min(int(case.cache_lengths[lane]), w - 1)
        seen = {(int(case.write_positions[lane]) % w - 1 - j) % w for j in range(reach)}
        for s in range(w):
            if s not in seen:
                rk[lane, :, s] = 0x7FC0
                rv[lane, :, s] = 0x7FC0
    assert_close(_run(case, rk, rv), _oracle(orc, case), "verify NaN outside")


@pytest.mark.parametrize("lanes,h,hk,d,r,w,seed", [
    (2, 8, 2, 256, 16, 700, 43),    # head_dim 256 (32-key tiles)
    (3, 4, 4, 128, 5, 300, 44),     # MHA, 5 rows: one partial 16-column slice
    (2, 16, 2, 128, 16, 1000, 45),  # 8 heads per KV head: two query-head groups of 4
    (1, 6, 2, 128, 7, 200, 46),     # 3 heads x 7 rows = 21 columns (two slices, one partial)
    (4, 2, 1, 256, 2, 129, 47),     # 2 rows, tiny window
])
def test_geometries(orc, lanes, h, hk, d, r, w, seed):
    announce("verify attention lanes=%d h=%d/%d d=%d r=%d w=%d" % (lanes, h, hk, d, r, w))
    case = workloads.dflash_case(lanes=lanes, q_heads=h, kv_heads=hk, head_dim=d, rows=r, window=w, seed=seed)
    assert_close(_run(case), _oracle(orc, case), "verify geometry")


def test_rejects_bad_arguments():
    case = workloads.dflash_case(lanes=1, window=64, rows=4, q_heads=4, kv_heads=2, seed=48)
    b, h, hk, d, r, w = case.geom
    out = torch.empty((b, h, r, d), dtype=torch.float32, device="cuda")
    with pytest.raises(fa.AttnError):
        fa.dflash_verify_attention(_params(case), dev(case.ring_k, True), dev(case.ring_v, True), dev(case.cur_q),
                                   dev(case.cur_k), dev(case.cur_v), dev(case.cache_lengths),
                                   dev(case.write_positions), out[:, :, :2].contiguous(), scale=case.scale)
    with pytest.raises(fa.AttnError):
        fa.dflash_verify_attention(_params(case), dev(case.ring_k, True), dev(case.ring_v, True), dev(case.cur_q),
                                   dev(case.cur_k), dev(case.cur_v), dev(case.cache_lengths),
                                   dev(case.write_positions), out, scale=float("inf"))
