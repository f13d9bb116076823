"""GPU parity of attn_prefill against the fp64 oracle, elementwise within
|err| <= 2e-3 * (1 + |ref|).

Oracle-sized cases span several 64-key tiles with ragged query and key tails,
including causal shapes whose launch shares the heaviest row blocks between
two workgroups (the merge of their partial results is counted in the status
block and must have run).  The full-size prefill configurations run in the
launch configuration the benchmark times: every query row of the causal 2k
case, and rows of every row block of the chunked d 512 cases.  Edge cases:
fully masked rows, padded vs unpadded KV, per-head bf16 masks with the KV
range split across workgroups, bf16 Q/K/V, f32 Q with bf16 K/V at head_dim
128/256/512 with f16, bf16 or no mask, strided views, GQA mapping.  Every
call's status block must show no expired wait."""
import math

import numpy as np
import pytest
import torch

import attention_flash_attn_03_amd as fa
import workloads
from gpu_util import announce, assert_close, dev

pytestmark = pytest.mark.gpu


def _call(case, kv_len=None, mask=True):
    """One attn_prefill call; returns (O, row blocks merged across workgroups)."""
    bf = case.kv_dtype == "bf16"
    q = dev(case.q, case.q_dtype == "bf16")
    k, v = dev(case.k, bf), dev(case.v, bf)
    m = dev(case.mask, case.mask_dtype == "bf16") if (mask and case.mask is not None) else None
    B, R, H, D = case.q.shape
    out = torch.full((B, R, H, D), float("nan"), dtype=torch.float32, device="cuda")
    kv = kv_len if kv_len is not None else case.kv_len
    p = fa.prefill_params(q, k, v, m, out, scale=case.scale, kv_len=kv)
    ws = torch.full((fa.prefill_workspace_bytes(p),), 0xA5, dtype=torch.uint8, device="cuda")
    fa.attn_prefill(q, k, v, m, out, scale=case.scale, kv_len=kv, workspace=ws)
    torch.cuda.synchronize()
    flags, merged = fa.prefill_status(ws)
    assert flags == 0, "status block flags 0x%x after the call" % flags
    return out.cpu().numpy(), merged


def _run(case, kv_len=None, mask=True):
    return _call(case, kv_len, mask)[0]


def _oracle(orc, case, rows=None, kv_len=None, mask=True):
    kv = kv_len if kv_len is not None else case.kv_len
    q = case.q if rows is None else case.q[:, rows]
    m = None
    if mask and case.mask is not None:
        m = case.mask[..., :kv] if rows is None else case.mask[:, :, rows, :kv]
    return orc.attention(q, case.k[:, :kv], case.v[:, :kv], m, scale=case.scale,
                         q_bf16=case.q_dtype == "bf16", kv_bf16=case.kv_dtype == "bf16",
                         mask_bf16=case.mask_dtype == "bf16")


def test_tiny_config_full(orc):
    announce("prefill tiny (64 x 256, 4/1 heads, d 256)")
    case = workloads.prefill_case("tiny")
    assert_close(_run(case), _oracle(orc, case), "tiny")


@pytest.mark.parametrize("rows,kv_len,cached,h,hk,d,holes,seed", [
    (200, 200, 0, 4, 2, 256, 0.0, 11),     # causal, ragged tails on both axes
    (96, 330, 234, 8, 2, 256, 0.1, 12),    # chunked with holes, ragged KV
    (70, 260, 190, 4, 1, 512, 0.1, 13),    # head_dim 512 (two head-dim slices)
    (130, 200, 70, 6, 3, 128, 0.0, 14),    # head_dim 128
    (33, 64, 31, 2, 2, 128, 0.3, 15),      # exactly one KV tile, MHA
])
def test_prefill_oracle_sized(orc, rows, kv_len, cached, h, hk, d, holes, seed):
    announce("prefill rows=%d kv=%d h=%d/%d d=%d holes=%g" % (rows, kv_len, h, hk, d, holes))
    case = workloads.prefill_synthetic("t", rows=rows, kv_len=kv_len, cached=cached, n_heads=h, n_kv_heads=hk,
                                       head_dim=d, seed=seed, q_std=1 / math.sqrt(d), kv_std=1.0, holes=holes,
                                       scale=1.0)
    assert_close(_run(case), _oracle(orc, case), "prefill")


@pytest.mark.parametrize("rows,h,hk,d,batch,kv_dtype", [
    (192, 2, 1, 128, 1, "f16"),    # three row blocks: the heavy one is shared, the middle one is alone
    (192, 2, 1, 256, 1, "f16"),
    (512, 32, 16, 128, 2, "f16"),  # 256 workgroups, every pair shared
    (512, 16, 8, 512, 2, "f16"),   # head_dim 512 (two head-dim slices), 256 workgroups
    (192, 2, 1, 128, 1, "bf16"),   # f32 Q + bf16 K/V; the first rows see one to a few keys
    (1024, 16, 8, 256, 2, "bf16"),  # eight-wave workgroups: 256 of them
    (512, 16, 8, 512, 2, "bf16"),
])
def test_prefill_shared_row_blocks(orc, rows, h, hk, d, batch, kv_dtype):
    """Causal shapes whose launch pairs heavy and light row blocks and cuts the
    heavy one between the two workgroups; every row against the oracle."""
    announce("prefill shared row blocks rows=%d h=%d/%d d=%d batch=%d %s" % (rows, h, hk, d, batch, kv_dtype))
    case = workloads.prefill_synthetic("t", rows=rows, kv_len=rows, cached=0, n_heads=h, n_kv_heads=hk,
                                       head_dim=d, seed=40 + d + rows, q_std=1 / math.sqrt(d), kv_std=1.0,
                                       batch=batch, scale=1.0, kv_dtype=kv_dtype)
    got, merged = _call(case)
    assert merged > 0, "no row block was shared and merged: the shape does not reach the merge"
    assert_close(got, _oracle(orc, case), "shared row blocks")


@pytest.mark.parametrize("d", [128, 256, 512])
@pytest.mark.parametrize("mask_dtype", [None, "f16", "bf16"])
def test_f32_q_bf16_kv(orc, d, mask_dtype):
    """f32 Q against bf16 K/V (Q carried as a hi + lo bf16 pair), ragged KV tail."""
    announce("prefill f32 Q + bf16 K/V d=%d mask=%s" % (d, mask_dtype))
    case = workloads.prefill_synthetic("t", rows=90, kv_len=301, cached=211, n_heads=4, n_kv_heads=2, head_dim=d,
                                       seed=50 + d, q_std=1 / math.sqrt(d), kv_std=1.0, holes=0.1,
                                       kv_dtype="bf16", mask_dtype=mask_dtype or "f16", scale=1.0)
    has_mask = mask_dtype is not None
    assert_close(_run(case, mask=has_mask), _oracle(orc, case, mask=has_mask), "f32 Q + bf16 K/V")


def test_f32_q_bf16_kv_verify_shaped(orc):
    """f32 Q + bf16 K/V at head_dim 256 with a per-head bf16 mask and few query rows:
    the two-wave launch with the KV range split across workgroups."""
    announce("prefill f32 Q + bf16 K/V d=256, per-head bf16 mask, split KV")
    rng = np.random.Generator(np.random.PCG64(59))
    b, h, hk, r, kv, d = 2, 4, 2, 16, 777, 256
    q = (rng.standard_normal((b, r, h, d)) / 16).astype(np.float32)
    k = workloads.to_bf16_bits(rng.standard_normal((b, kv, hk, d)).astype(np.float32))
    v = workloads.to_bf16_bits(rng.standard_normal((b, kv, hk, d)).astype(np.float32))
    mask = np.where(rng.random((b, h, r, kv)) < 0.6, np.float32(0.0), np.float32(-np.inf))
    mask[:, :, 2, :] = -np.inf
    case = workloads.PrefillCase("verify256", q, k, v, workloads.to_bf16_bits(mask), 1.0, kv, q_dtype="f32",
                                 kv_dtype="bf16", mask_dtype="bf16")
    got = _run(case)
    assert np.all(got[:, 2] == 0.0)
    assert_close(got, _oracle(orc, case), "verify-shaped d 256")


def test_bf16_kv_no_mask_batched(orc):
    announce("prefill bf16 K/V, no mask, batch 3")
    case = workloads.prefill_synthetic("t", rows=80, kv_len=150, cached=70, n_heads=4, n_kv_heads=2, head_dim=128,
                                       seed=16, q_std=1.0, kv_std=1.0, batch=3, kv_dtype="bf16",
                                       scale=1 / math.sqrt(128))
    assert_close(_run(case, mask=False), _oracle(orc, case, mask=False), "bf16 no mask")


def test_fully_masked_rows_are_zero(orc):
    announce("prefill fully masked rows")
    case = workloads.prefill_synthetic("t", rows=64, kv_len=128, cached=64, n_heads=2, n_kv_heads=1, head_dim=256,
                                       seed=17, q_std=0.1, kv_std=1.0)
    case.mask[:, :, ::5, :] = np.float16(-np.inf)
    got = _run(case)
    assert np.all(got[:, ::5] == 0.0)
    assert_close(got, _oracle(orc, case), "masked rows")


@pytest.mark.parametrize("d", [128, 256, 512])
@pytest.mark.parametrize("kv_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("rows,kv_len,masked", [(1, 1, False), (1, 65, True), (5, 1, False), (3, 33, True)])
def test_smallest_shapes(orc, d, kv_dtype, rows, kv_len, masked):
    """One query row, one key, and other shapes smaller than a single tile: the ragged
    stage is the only stage, and (with one key) every row's softmax is a single 1."""
    announce("prefill small shape rows=%d kv=%d d=%d %s masked=%s" % (rows, kv_len, d, kv_dtype, masked))
    case = workloads.prefill_synthetic("t", rows=rows, kv_len=kv_len, cached=kv_len - rows if kv_len >= rows else 0,
                                       n_heads=4, n_kv_heads=2, head_dim=d, seed=26, q_std=1 / math.sqrt(d),
                                       kv_std=1.0, kv_dtype=kv_dtype)
    got = _run(case, mask=masked)
    assert_close(got, _oracle(orc, case, mask=masked), "small shape")
    if kv_len == 1 and not masked:
        # softmax over one key is 1: O is that key's V (as the kernel's K/V type holds it)
        v0 = case.v[:, 0].astype(np.float64) if case.v.dtype != np.uint16 else None
        if v0 is not None:
            want = np.repeat(v0, 2, axis=1)[:, None]  # [B, 1, H, D] from [B, HK, D], 2 query heads per KV head
            assert np.array_equal(got, np.broadcast_to(want, got.shape).astype(np.float32))


def test_padded_and_unpadded_kv_agree(orc):
    announce("prefill padded vs unpadded KV")
    case = workloads.prefill_synthetic("t", rows=64, kv_len=190, cached=126, n_heads=4, n_kv_heads=1, head_dim=512,
                                       seed=18, q_std=1 / math.sqrt(512), kv_std=0.5, holes=0.1, kv_rows_alloc=192)
    ref = _oracle(orc, case)
    padded = _run(case, kv_len=192)    # zero rows, -inf columns 190..191
    unpadded = _run(case, kv_len=190)  # those rows never read
    assert_close(padded, ref, "padded")
    assert_close(unpadded, ref, "unpadded")
    assert_close(padded, unpadded.astype(np.float64), "padded vs unpadded", tol=1e-5)


def test_per_head_bf16_mask_with_kv_split(orc):
    """The block-verify shape: 16 rows per lane, per-head bf16 mask [b, h, r, k]
    with an odd row stride, bf16 Q/K/V, few query blocks so the KV range is split."""
    announce("prefill verify-shaped (per-head bf16 mask, split KV)")
    rng = np.random.Generator(np.random.PCG64(19))
    b, h, hk, r, kv, d = 2, 8, 2, 16, 1031, 128
    q = workloads.to_bf16_bits(rng.standard_normal((b, r, h, d)).astype(np.float32))
    k = workloads.to_bf16_bits(rng.standard_normal((b, kv, hk, d)).astype(np.float32))
    v = workloads.to_bf16_bits(rng.standard_normal((b, kv, hk, d)).astype(np.float32))
    vis = rng.random((b, h, r, kv)) < 0.7
    mask = np.where(vis, np.float32(0.0), np.float32(-np.inf))
    mask[:, :, 3, :] = -np.inf                     # one fully masked row
    mask[:, :, 5, :] = rng.standard_normal((b, h, kv)).astype(np.float32)  # general additive values
    mbits = workloads.to_bf16_bits(mask)
    case = workloads.PrefillCase("verify", q, k, v, mbits, 1 / math.sqrt(d), kv, q_dtype="bf16", kv_dtype="bf16",
                                 mask_dtype="bf16")
    got = _run(case)
    assert np.all(got[:, 3] == 0.0)
    assert_close(got, _oracle(orc, case), "verify-shaped")


def test_strided_views(orc):
    """Q, K, V and O as strided views into larger buffers."""
    announce("prefill strided views")
    case = workloads.prefill_synthetic("t", rows=100, kv_len=140, cached=40, n_heads=4, n_kv_heads=2, head_dim=128,
                                       seed=21, q_std=0.2, kv_std=1.0)
    qbig = torch.zeros((1, 100, 6, 136), dtype=torch.float32, device="cuda")
    qbig[:, :, 1:5, 8:] = dev(case.q)
    q = qbig[:, :, 1:5, 8:]
    kbig = torch.zeros((1, 140, 3, 144), dtype=torch.float16, device="cuda")
    kbig[:, :, :2, 16:] = dev(case.k)
    vbig = torch.zeros((1, 140, 2, 2, 128), dtype=torch.float16, device="cuda")
    vbig[:, :, :, 1, :] = dev(case.v)
    v = vbig[:, :, :, 1, :]
    out_big = torch.zeros((1, 100, 5, 132), dtype=torch.float32, device="cuda")
    out = out_big[:, :, :4, 4:]
    fa.attn_prefill(q, kbig[:, :, :2, 16:], v, dev(case.mask), out, scale=1.0)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), _oracle(orc, case), "strided")
    assert torch.all(out_big[:, :, 4] == 0) and torch.all(out_big[:, :, :, :4] == 0)


def test_gqa_matches_repeated_kv(orc):
    announce("prefill GQA vs repeated KV")
    case = workloads.prefill_synthetic("t", rows=64, kv_len=128, cached=64, n_heads=8, n_kv_heads=2, head_dim=256,
                                       seed=22, q_std=1 / 16, kv_std=1.0)
    gqa = _run(case)
    rep = workloads.PrefillCase("rep", case.q, np.repeat(case.k, 4, axis=2), np.repeat(case.v, 4, axis=2),
                                case.mask, case.scale, case.kv_len)
    mha = _run(rep)
    # The two calls get different launch shapes (query heads per workgroup, keys per
    # stage), so their probabilities are rounded to f16 against different running
    # maxima: they agree to the attention bound, not bit for bit.  A wrong KV-head
    # mapping would be off by O(1).
    assert_close(gqa, mha.astype(np.float64), "gqa vs mha")
    assert_close(gqa, _oracle(orc, case), "gqa")
    assert_close(mha, _oracle(orc, rep), "mha")


def test_gqa_matches_repeated_kv_bitwise(orc):
    """Unmasked, with neither KV splits nor row-block pairing in either launch: every query
    column then sees the same stages in the same order under either head mapping, and its
    scores, softmax and P V do not depend on the other columns of its tile, so GQA and the
    repeated-KV MHA call agree bit for bit."""
    announce("prefill GQA vs repeated KV, bitwise (unmasked, 1024 x 1024, 16/4 heads, d 128)")
    case = workloads.prefill_synthetic("t", rows=1024, kv_len=1024, cached=0, n_heads=16, n_kv_heads=4,
                                       head_dim=128, seed=23, q_std=1 / math.sqrt(128), kv_std=1.0)
    gqa = _run(case, mask=False)
    rep = workloads.PrefillCase("rep", case.q, np.repeat(case.k, 4, axis=2), np.repeat(case.v, 4, axis=2),
                                case.mask, case.scale, case.kv_len)
    mha = _run(rep, mask=False)
    assert np.array_equal(gqa, mha), "GQA and repeated-KV MHA differ: max |d| %g" % float(np.max(np.abs(gqa - mha)))
    rows = np.arange(0, 1024, 37)
    assert_close(gqa[:, rows], _oracle(orc, case, rows=rows, mask=False), "gqa unmasked")


def test_mask_heads_more_than_2gib_apart(orc):
    """A per-head f16 mask whose two heads lie 2 GiB apart (a strided view of one allocation)
    and whose rows have an odd key count: the tile classification reads it one key per lane
    with 64-bit offsets, and the attention kernel reads its masked tiles element by element.
    Every row is compared with the oracle."""
    announce("prefill per-head mask, heads 2 GiB apart (96 x 301, 2/1 heads, d 128)")
    kw = dict(rows=96, kv_len=301, cached=205, n_heads=2, n_kv_heads=1, head_dim=128,
              q_std=1 / math.sqrt(128), kv_std=1.0, holes=0.1)
    case = workloads.prefill_synthetic("t", seed=24, **kw)
    other = workloads.prefill_synthetic("t", seed=25, **kw)  # head 1: the same frontier, other holes
    mask = np.concatenate([case.mask, other.mask], axis=1)   # [1, 2, 96, 301] f16
    gap = 1 << 30                                             # elements between the heads: 2 GiB
    n = 96 * 301
    big = torch.empty((gap + n,), dtype=torch.float16, device="cuda")
    big[:n] = torch.from_numpy(np.ascontiguousarray(mask[0, 0]).reshape(-1)).cuda()
    big[gap:gap + n] = torch.from_numpy(np.ascontiguousarray(mask[0, 1]).reshape(-1)).cuda()
    m = big.as_strided((1, 2, 96, 301), (0, gap, 301, 1))
    q, k, v = dev(case.q), dev(case.k), dev(case.v)
    out = torch.full(case.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    p = fa.prefill_params(q, k, v, m, out, scale=case.scale)
    ws = torch.full((fa.prefill_workspace_bytes(p),), 0xA5, dtype=torch.uint8, device="cuda")
    fa.attn_prefill(q, k, v, m, out, scale=case.scale, workspace=ws)
    torch.cuda.synchronize()
    flags, _ = fa.prefill_status(ws)
    assert flags == 0, "status block flags 0x%x after the call" % flags
    got = out.cpu().numpy()
    del big, m
    ref = orc.attention(case.q, case.k, case.v, mask, scale=case.scale)
    assert_close(got, ref, "heads 2 GiB apart")


def _rows_per_block(rows, block, per, seed):
    """`per` distinct rows from every block of `block` consecutive rows (first and last included)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    pick = [0, rows - 1]
    for b0 in range(0, rows, block):
        n = min(block, rows - b0)
        pick += list(b0 + rng.choice(n, min(per, n), replace=False))
    return np.unique(pick)


def test_full_size_causal2k_every_row(orc):
    announce("prefill full size causal2k, every row")
    case = workloads.prefill_case("causal2k")
    got, merged = _call(case)
    assert merged > 0
    assert_close(got, _oracle(orc, case), "causal2k")


@pytest.mark.parametrize("name,block", [("chunked8k", 16), ("chunked8k_pad", 32)])
def test_full_size_chunked_every_row_block(orc, name, block):
    """A row of every `block`-row block (no coarser than the launch's row blocks, so
    both sides of every shared row block are covered)."""
    announce("prefill full size %s, a row of every %d-row block" % (name, block))
    case = workloads.prefill_case(name)
    got, _ = _call(case)
    rows = _rows_per_block(case.q.shape[1], block, 1, 23)
    assert_close(got[:, rows], _oracle(orc, case, rows=rows), name)
    if name == "chunked8k_pad":
        unpadded = _run(case, kv_len=8190)
        assert_close(got, unpadded.astype(np.float64), "padded vs unpadded", tol=1e-5)
