"""Pins for the oracle's DFlash2 steps (pack O3, mask O4, commit O5, mask rows)
and its f32 -> bf16 rounding.

Pinned by: the worked examples printed on the mlx-native 0.21.1
dflash2_attention_pack.rs page (tests/golden/), a ring buffer simulated from
scratch token by token, a window reading stated in absolute positions, brute
force over tiny geometries, and torch's bf16 cast.
"""
import json
import os

import numpy as np
import pytest
import torch

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _torch_bf16(x):
    return workloads.to_bf16_bits(np.asarray(x, np.float32))


# --------------------------------------------------------------------------- bf16 rounding
def test_bf16_hand_values(orc):
    cases = {
        0x3F800000: 0x3F80,  # 1.0
        0x3F808000: 0x3F80,  # exact tie, kept part even -> down
        0x3F818000: 0x3F82,  # exact tie, kept part odd -> up
        0x3F808001: 0x3F81,  # just above the tie -> up
        0x3F807FFF: 0x3F80,  # just below the tie -> down
        0x7F7FFFFF: 0x7F80,  # largest finite rounds to +inf
        0xFF7FFFFF: 0xFF80,
        0x7F800000: 0x7F80,  # +inf
        0xFF800000: 0xFF80,  # -inf
        0x00000001: 0x0000,  # smallest subnormal -> +0
        0x00018000: 0x0002,  # subnormal tie, odd -> up (subnormals are kept, not flushed)
        0x80008000: 0x8000,  # negative subnormal tie, even -> -0
        0x7F800001: 0x7FC0,  # signalling NaN gets the quiet bit
        0xFFC12345: 0xFFC1,  # quiet NaN keeps sign and upper payload
    }
    x = np.array(list(cases.keys()), np.uint32).view(np.float32)
    got = orc.bf16_from_f32(x)
    assert [int(g) for g in got] == list(cases.values())


def test_bf16_matches_torch_on_random_bits(orc):
    rng = np.random.Generator(np.random.PCG64(7))
    bits = rng.integers(0, 2**32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    finite = ~np.isnan(x)
    got = orc.bf16_from_f32(x)
    ref = _torch_bf16(x)
    assert np.array_equal(got[finite], ref[finite])
    nan_out = got[~finite]
    assert np.all((nan_out & 0x7F80) == 0x7F80) and np.all((nan_out & 0x7F) | 0x40)
    assert np.array_equal(nan_out >> 15, (bits[~finite] >> 31).astype(np.uint16))


# --------------------------------------------------------------------------- worked examples
def _worked_example_inputs(g):
    geo = g["geometry"]
    b, h, hk, d, r, w = (geo[k] for k in ("lanes", "q_heads", "kv_heads", "head_dim", "rows", "window"))
    ring_k = np.zeros((b, hk, w, d), np.uint16)
    ring_v = np.zeros((b, hk, w, d), np.uint16)
    ring_k[0, 0, :, 0] = _torch_bf16(g["ring_k_first_element_per_slot"])
    ring_v[0, 0, :, 0] = _torch_bf16(g["ring_v_first_element_per_slot"])
    cq = np.zeros((b, r, h, d), np.float32)
    ck = np.zeros((b, r, hk, d), np.float32)
    cv = np.zeros((b, r, hk, d), np.float32)
    for arr, key in ((cq, "current_q_nonzero"), (ck, "current_k_nonzero"), (cv, "current_v_nonzero")):
        flat = arr.reshape(-1)
        for idx, val in g[key].items():
            flat[int(idx)] = val
    L = np.array(g["cache_lengths"], np.uint32)
    wp = np.array(g["write_positions"], np.uint32)
    return (b, h, hk, d, r, w), ring_k, ring_v, cq, ck, cv, L, wp


def test_pack_mask_commit_worked_example(orc):
    g = _golden("dflash_worked_example.json")
    geom, ring_k, ring_v, cq, ck, cv, L, wp = _worked_example_inputs(g)
    pq, pk, pv = orc.dflash_pack(geom, ring_k, ring_v, cq, ck, cv, L, wp)
    assert pq.reshape(-1)[0] == g["expect_packed_q_0"]
    keys = pk.reshape(-1)
    assert [int(keys[i * 128]) for i in range(5)] == g["expect_packed_k_row_firsts"]
    assert list(_torch_bf16(g["expect_packed_k_row_firsts_values"])) == g["expect_packed_k_row_firsts"]
    mask = orc.dflash_mask(geom, L).reshape(-1)
    assert [int(m) for m in mask[:10]] == g["expect_mask_first_10"]
    counts = np.array(g["commit_counts"], np.uint32)
    rk, rv = orc.dflash_commit(geom, g["geometry"]["max_commit"], ck, cv, counts, wp, ring_k, ring_v)
    for idx, val in g["expect_ring_k_after_commit"].items():
        assert rk.reshape(-1)[int(idx)] == val


def test_mask_rows_worked_example(orc):
    g = _golden("dflash_mask_rows_example.json")
    emb = _torch_bf16(g["mask_embedding"])
    out = orc.dflash_mask_rows(g["lanes"], g["rows"], g["hidden"], emb,
                               np.array(g["draft_input"], np.float32).reshape(g["lanes"] * g["rows"], g["hidden"]))
    assert out.reshape(-1).tolist() == g["expect"]


# --------------------------------------------------------------------------- ring simulation
class Ring:
    """A ring buffer simulated token by token: slot = write pointer, pointer
    advances by one per token, length counts tokens ever written."""

    def __init__(self, w, d, start_wp):
        self.w, self.d = w, d
        self.slots = np.zeros((w, d), np.uint16)
        self.wp = start_wp
        self.length = 0
        self.history = []

    def append(self, row_bits):
        self.slots[self.wp] = row_bits
        self.wp = (self.wp + 1) % self.w
        self.length += 1
        self.history.append(row_bits.copy())


def _geometries():
    for w in (3, 4, 5, 8):
        for r in range(2, min(4, w - 1) + 1):
            yield w, r


@pytest.mark.parametrize("w,r", list(_geometries()))
def test_pack_reads_the_ring_newest_first(orc, w, r):
    d, h, hk = 8, 2, 1
    rng = np.random.Generator(np.random.PCG64(100 + w * 10 + r))
    for start in range(w):
        for n_tokens in range(0, w + 3):
            ring = Ring(w, d, start)
            for _ in range(n_tokens):
                ring.append(rng.integers(1, 60000, size=d, dtype=np.uint16))
            cq = rng.standard_normal((1, r, h, d)).astype(np.float32)
            ck = rng.standard_normal((1, r, hk, d)).astype(np.float32)
            cv = rng.standard_normal((1, r, hk, d)).astype(np.float32)
            L = np.array([min(ring.length, w)], np.uint32)
            wp = np.array([ring.wp], np.uint32)
            rk = ring.slots[None, None]
            pq, pk, pv = orc.dflash_pack((1, h, hk, d, r, w), rk, rk, cq, ck, cv, L, wp)
            # drafted rows first, in order, rounded by torch's cast; Q transposed to [b, h, r, d]
            assert np.array_equal(pk[0, 0, :r], _torch_bf16(ck[0, :, 0]))
            assert np.array_equal(pv[0, 0, :r], _torch_bf16(cv[0, :, 0]))
            assert np.array_equal(pq[0], _torch_bf16(cq[0].transpose(1, 0, 2)))
            # then the cache, newest token first, as far as it goes
            for j in range(w - 1):
                if j < int(L[0]):
                    assert np.array_equal(pk[0, 0, r + j], ring.history[-1 - j])
                else:
                    assert not pk[0, 0, r + j].any()


@pytest.mark.parametrize("w,r", list(_geometries()))
def test_mask_is_a_window_in_absolute_positions(orc, w, r):
    """Row i sits at absolute position L+i.  It sees every drafted row and the
    cached tokens a (0 <= a < L) with L+i-a < w: a window of w positions that
    ends at the row itself.  Cached token a is packed at r + (L-1-a)."""
    h = 3
    for L in range(0, w + 3):
        mask = orc.dflash_mask((1, h, 1, 8, r, w), np.array([L], np.uint32))
        k = w - 1 + r
        for i in range(r):
            want = np.full(k, 0xFF80, np.uint16)
            want[:r] = 0
            for a in range(L):
                p = r + (L - 1 - a)
                if p < k and (L + i) - a < w:
                    want[p] = 0
            for hh in range(h):
                assert np.array_equal(mask[0, hh, i], want), (L, i)
        vis = (mask[0, 0] == 0).sum(axis=1)
        assert np.all(np.diff(vis) <= 0)


@pytest.mark.parametrize("w,r", list(_geometries()))
def test_commit_then_pack_extends_the_cache(orc, w, r):
    """Commit n rows at wp, advance wp and L: packing again shows the committed
    rows newest first, followed by the old cache shifted by n."""
    d, hk = 8, 1
    rng = np.random.Generator(np.random.PCG64(200 + w * 10 + r))
    for L0 in range(0, w + 1):
        for wp0 in range(w):
            for n in range(0, r + 2):  # n > max_commit is clamped
                ring = rng.integers(1, 60000, size=(1, hk, w, d), dtype=np.uint16)
                new = rng.standard_normal((1, r, hk, d)).astype(np.float32)
                cnt = np.array([n], np.uint32)
                rk, rv = orc.dflash_commit((1, 1, hk, d, r, w), r, new, new, cnt, np.array([wp0], np.uint32),
                                           ring, ring)
                m = min(n, r)
                # only the committed slots changed
                changed = {(wp0 + c) % w for c in range(m)}
                for s in range(w):
                    if s in changed:
                        c = (s - wp0) % w
                        assert np.array_equal(rk[0, 0, s], _torch_bf16(new[0, c, 0]))
                    else:
                        assert np.array_equal(rk[0, 0, s], ring[0, 0, s])
                # committing again is a no-op
                rk2, _ = orc.dflash_commit((1, 1, hk, d, r, w), r, new, new, cnt, np.array([wp0], np.uint32),
                                           rk, rv)
                assert np.array_equal(rk2, rk)
                # pack before and after
                z = np.zeros((1, r, 1, d), np.float32)
                _, before, _ = orc.dflash_pack((1, 1, hk, d, r, w), ring, ring, z, z, z,
                                               np.array([L0], np.uint32), np.array([wp0], np.uint32))
                _, after, _ = orc.dflash_pack((1, 1, hk, d, r, w), rk, rk, z, z, z,
                                              np.array([L0 + m], np.uint32), np.array([(wp0 + m) % w], np.uint32))
                for j in range(w - 1):
                    if j < m:
                        assert np.array_equal(after[0, 0, r + j], _torch_bf16(new[0, m - 1 - j, 0]))
                    elif j < L0 + m:
                        assert np.array_equal(after[0, 0, r + j], before[0, 0, r + j - m])


def test_full_size_case_shapes(orc):
    case = workloads.dflash_case(lanes=2, window=64, rows=4, q_heads=4, kv_heads=2, head_dim=128,
                                 forced_wrap=True)
    pq, pk, pv = orc.dflash_pack(case.geom, case.ring_k, case.ring_v, case.cur_q, case.cur_k, case.cur_v,
                                 case.cache_lengths, case.write_positions)
    assert pq.shape == (2, 4, 4, 128) and pk.shape == (2, 2, 64 - 1 + 4, 128)
    m = orc.dflash_mask(case.geom, case.cache_lengths)
    assert m.shape == (2, 4, 4, 67) and set(np.unique(m)) <= {0, 0xFF80}


# --------------------------------------------------------------------------- verify attention
def _bits_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("w,r", [(5, 2), (8, 3), (8, 4)])
def test_verify_attention_matches_direct_softmax(orc, w, r):
    """The verify step's attention computed per query row straight from rings
    simulated token by token: row i attends over the drafted rows (bf16 by
    torch's cast) and the newest cached tokens its window reaches (the j-th
    newest while j < min(L, w - 1 - i)), softmax in float64 with numpy.  Two
    lanes in different states; GQA with two query heads per KV head."""
    d, h, hk = 8, 4, 2
    g = h // hk
    rng = np.random.Generator(np.random.PCG64(300 + 10 * w + r))
    scale = 0.7
    for start in range(w):
        for n_tokens in (0, 1, w - 2, w, w + 3):
            lanes = []
            for lane in range(2):
                ring = Ring(w, hk * d, (start + 3 * lane) % w)
                ring_v = Ring(w, hk * d, (start + 3 * lane) % w)
                for _ in range(n_tokens + lane):
                    ring.append(_torch_bf16(rng.standard_normal(hk * d)))
                    ring_v.append(_torch_bf16(rng.standard_normal(hk * d)))
                lanes.append((ring, ring_v))
            rk = np.stack([ln[0].slots.reshape(w, hk, d).transpose(1, 0, 2) for ln in lanes])
            rv = np.stack([ln[1].slots.reshape(w, hk, d).transpose(1, 0, 2) for ln in lanes])
            cq = rng.standard_normal((2, r, h, d)).astype(np.float32)
            ck = rng.standard_normal((2, r, hk, d)).astype(np.float32)
            cv = rng.standard_normal((2, r, hk, d)).astype(np.float32)
            L = np.array([min(ln[0].length, w) for ln in lanes], np.uint32)
            wp = np.array([ln[0].wp for ln in lanes], np.uint32)
            got = orc.dflash_verify_attention((2, h, hk, d, r, w), rk, rv, cq, ck, cv, L, wp, scale=scale)
            assert got.shape == (2, h, r, d)
            for b, (ring, ring_v) in enumerate(lanes):
                for hh in range(h):
                    kv = hh // g
                    for i in range(r):
                        keys = [_bits_to_f64(_torch_bf16(ck[b, p, kv])) for p in range(r)]
                        vals = [_bits_to_f64(_torch_bf16(cv[b, p, kv])) for p in range(r)]
                        for j in range(len(ring.history)):
                            if j < int(L[b]) and j < w - 1 - i:
                                keys.append(_bits_to_f64(ring.history[-1 - j].reshape(hk, d)[kv]))
                                vals.append(_bits_to_f64(ring_v.history[-1 - j].reshape(hk, d)[kv]))
                        q = _bits_to_f64(_torch_bf16(cq[b, i, hh]))
                        s = scale * (np.array(keys) @ q)
                        p = np.exp(s - s.max())
                        want = (p @ np.array(vals)) / p.sum()
                        assert np.allclose(got[b, hh, i], want, rtol=1e-12, atol=1e-12), (start, n_tokens, b, hh, i)
