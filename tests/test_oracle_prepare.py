"""Pins for the oracle's prepare step (per-head RMS norm, rotary embedding, K/V
write into the pages).

Pinned by properties the pages' operation fixes: a rotation at position 0 is
the identity; rotations keep each pair's length; rotated dot products depend
only on the relative position; the interleaved and half-split pairings are a
fixed permutation apart; pair i turns by position * theta^(-2i/rope_dim)
(checked at i = 0 and i = 1 against the textbook rotation); RMS norm gives
unit root-mean-square and is scale invariant; the page write touches exactly
the slots of the new positions and stores V as its rounding."""
import numpy as np
import pytest

import workloads


def test_rope_position_zero_is_identity(orc):
    x = np.random.Generator(np.random.PCG64(1)).standard_normal((3, 128))
    for inter in (True, False):
        assert np.array_equal(orc.rope(x, 0, 64, 10000.0, inter), x)


@pytest.mark.parametrize("inter", [True, False])
def test_rope_keeps_pair_lengths_and_tail(orc, inter):
    rng = np.random.Generator(np.random.PCG64(2))
    x = rng.standard_normal((4, 128))
    y = orc.rope(x, 12345, 96, 5e5, inter)
    if inter:
        pairs = lambda z: np.hypot(z[:, 0:96:2], z[:, 1:96:2])
    else:
        pairs = lambda z: np.hypot(z[:, :48], z[:, 48:96])
    np.testing.assert_allclose(pairs(y), pairs(x), rtol=1e-12)
    assert np.array_equal(y[:, 96:], x[:, 96:])


@pytest.mark.parametrize("inter", [True, False])
def test_rope_dot_products_depend_on_relative_position(orc, inter):
    rng = np.random.Generator(np.random.PCG64(3))
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    base = orc.rope(q, 40, 128, 10000.0, inter) @ orc.rope(k, 7, 128, 10000.0, inter)
    for shift in (1, 100, 9000):
        got = orc.rope(q, 40 + shift, 128, 10000.0, inter) @ orc.rope(k, 7 + shift, 128, 10000.0, inter)
        assert abs(got - base) < 1e-9 * (1 + abs(base))
    # and it does depend on it
    other = orc.rope(q, 41, 128, 10000.0, inter) @ orc.rope(k, 7, 128, 10000.0, inter)
    assert abs(other - base) > 1e-3


def test_rope_pairings_are_a_permutation_apart(orc):
    rng = np.random.Generator(np.random.PCG64(4))
    x = rng.standard_normal((2, 256))
    rd = 128
    perm = np.arange(256)
    perm[0:rd:2], perm[1:rd:2] = np.arange(rd // 2), np.arange(rd // 2, rd)  # interleaved slot <- half-split feature
    half = orc.rope(x, 777, rd, 1e4, False)
    inter = orc.rope(x[:, perm], 777, rd, 1e4, True)
    np.testing.assert_allclose(inter, half[:, perm], rtol=1e-12, atol=1e-12)


def test_rope_frequencies(orc):
    """rope_dim 4: pair 0 turns by the position, pair 1 by position / sqrt(theta)."""
    x = np.array([1.0, 0.0, 1.0, 0.0])
    pos, theta = 3.0, 10000.0
    y = orc.rope(x, pos, 4, theta, True)
    assert np.allclose(y, [np.cos(pos), np.sin(pos), np.cos(pos / 100.0), np.sin(pos / 100.0)], atol=1e-15)
    y = orc.rope(np.array([1.0, 1.0, 0.0, 0.0]), pos, 4, theta, False)
    assert np.allclose(y, [np.cos(pos), np.cos(pos / 100.0), np.sin(pos), np.sin(pos / 100.0)], atol=1e-15)


def test_rms_norm_unit_rms_and_scale_invariance(orc):
    rng = np.random.Generator(np.random.PCG64(5))
    x = rng.standard_normal((5, 128))
    y = orc.rms_norm(x, np.ones(128), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-13)
    np.testing.assert_allclose(orc.rms_norm(3.5 * x, np.ones(128), 0.0), y, rtol=1e-13)
    w = rng.standard_normal(128)
    np.testing.assert_allclose(orc.rms_norm(x, w, 0.0), y * w, rtol=1e-13)
    # epsilon enters under the root: a zero row stays zero, a tiny row is damped
    assert not orc.rms_norm(np.zeros(128), np.ones(128), 1e-6).any()


def test_prepare_writes_exactly_the_new_slots(orc):
    pc = workloads.paged_case(batch=3, ctx_lo=20, ctx_hi=60, page_size=8, num_pages=40, n_heads=4, n_kv_heads=2,
                              head_dim=128, seed=9)
    rng = np.random.Generator(np.random.PCG64(6))
    T = 5
    ql = np.array([5, 0, 3], np.int32)
    st = (pc.context_lens - ql).astype(np.int32)
    q_raw = rng.standard_normal((3, T, 4, 128)).astype(np.float32)
    k_raw = rng.standard_normal((3, T, 2, 128)).astype(np.float32)
    v_raw = rng.standard_normal((3, T, 2, 128)).astype(np.float32)
    q_out, kp, vp = orc.paged_prepare(q_raw, k_raw, v_raw, None, None, pc.page_table, ql, st, pc.k_pool, pc.v_pool,
                                      rope_dim=128, theta=1e4, eps=1e-6, interleaved=False, cap=pc.max_context)
    written = np.zeros(kp.shape[:2], bool)
    for b in range(3):
        assert np.all(np.isnan(q_out[b, ql[b]:])) and not np.any(np.isnan(q_out[b, :ql[b]]))
        for t in range(ql[b]):
            s = st[b] + t
            page, slot = pc.page_table[b, s // 8], s % 8
            written[page, slot] = True
            assert np.array_equal(vp[page, slot], v_raw[b, t].astype(np.float16))
            np.testing.assert_allclose(kp[page, slot].astype(np.float64),
                                       orc.rope(k_raw[b, t].astype(np.float64), s, 128, 1e4, False),
                                       rtol=2e-3, atol=2e-3)
    assert np.array_equal(kp[~written], pc.k_pool[~written])
    assert np.array_equal(vp[~written], pc.v_pool[~written])
    assert written.sum() == 8
