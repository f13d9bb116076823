"""GPU parity of attn_prefill against the fp64 oracle, elementwise within
|err| <= 2e-3 * (1 + |ref|).

Oracle-sized cases span several 64-key tiles with ragged query and key tails;
the full-size prefill configurations run in the launch configuration the
benchmark times and are checked on sampled query rows.  Edge cases: fully
masked rows, padded vs unpadded KV, per-head bf16 masks with the KV range
split across workgroups, bf16 Q/K/V, no mask, strided views, GQA mapping."""
import math

import numpy as np
import pytest
import torch

import attention_flash_attn_03_amd as fa
import workloads
from gpu_util import announce, assert_close, dev

pytestmark = pytest.mark.gpu


def _run(case, kv_len=None, mask=True):
    bf = case.kv_dtype == "bf16"
    q = dev(case.q, case.q_dtype == "bf16")
    k, v = dev(case.k, bf), dev(case.v, bf)
    m = dev(case.mask, case.mask_dtype == "bf16") if (mask and case.mask is not None) else None
    B, R, H, D = case.q.shape
    out = torch.full((B, R, H, D), float("nan"), dtype=torch.float32, device="cuda")
    fa.attn_prefill(q, k, v, m, out, scale=case.scale, kv_len=kv_len if kv_len is not None else case.kv_len)
    torch.cuda.synchronize()
    return out.cpu().numpy()


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


def _sampled_rows(rows, n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    pick = np.unique(np.concatenate([[0, rows - 1], rng.choice(rows, n, replace=False)]))
    return pick


@pytest.mark.parametrize("name,nrows", [("causal2k", 48), ("chunked8k", 12), ("chunked8k_pad", 8)])
def test_full_size_configs_sampled(orc, name, nrows):
    announce("prefill full size %s (sampled rows)" % name)
    case = workloads.prefill_case(name)
    got = _run(case)
    rows = _sampled_rows(case.q.shape[1], nrows, 23)
    assert_close(got[:, rows], _oracle(orc, case, rows=rows), name)
    if name == "chunked8k_pad":
        unpadded = _run(case, kv_len=8190)
        padded = _run(case, kv_len=8192)
        assert_close(padded, unpadded.astype(np.float64), "padded vs unpadded", tol=1e-5)
