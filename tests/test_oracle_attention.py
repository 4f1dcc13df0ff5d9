"""Pins for the block-sparse prefill attention oracle (oracle/attention.py): a scalar
brute force with the attended positions written out by hand, and the properties any
attention has.  CPU only."""

import math

import numpy as np

from oracle import attention


def test_attended_positions_hand_worked():
    # ratio 4: row 2 at position 10 + 2 = 12 has 13 // 4 = 3 complete blocks (positions 0..11);
    # its tail is position 12 alone.  Listed blocks 2 and 0 (in that order), 3 is not yet
    # complete and -1 is padding.
    got = attention.attended_positions([2, -1, 3, 0], first_pos=10, r=2, ratio=4)
    assert got.tolist() == [8, 9, 10, 11, 0, 1, 2, 3, 12]
    # row 1 at position 11: 12 // 4 = 3 complete blocks, block 2 now complete, empty tail
    assert attention.attended_positions([2], 10, 1, 4).tolist() == [8, 9, 10, 11]
    # nothing listed: the tail only (positions 8..10 for the row at position 10)
    assert attention.attended_positions([-1, -1], 10, 0, 4).tolist() == [8, 9, 10]


def _case(seed=3, rows=3, nq=4, nkv=2, hd=8, pages=6, block_size=4):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((rows, nq, hd))
    k = rng.standard_normal((pages, block_size, nkv, hd))
    v = rng.standard_normal((pages, block_size, nkv, hd))
    bt = rng.permutation(pages)
    return q, k, v, bt


def test_prefill_attn_brute_force():
    q, k, v, bt = _case()
    lists = np.array([[1, -1], [0, 2], [3, 1]])
    first_pos, ratio, block_size, nkv = 12, 4, 4, 2
    out = attention.prefill_attn(q, k, v, bt, lists, first_pos, ratio, block_size, nkv, 0.35)
    # hand-listed positions: rows at 12, 13, 14 have 3 complete blocks each; tails 12, 12..13, 12..14
    attended = {0: [4, 5, 6, 7, 12], 1: [0, 1, 2, 3, 8, 9, 10, 11, 12, 13], 2: [4, 5, 6, 7, 12, 13, 14]}
    for r in range(3):
        for h in range(4):
            kvh = h // 2
            s = [0.35 * math.fsum(q[r, h, d] * k[bt[p // 4], p % 4, kvh, d] for d in range(8)) for p in attended[r]]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = math.fsum(e)
            for d in range(8):
                exp = math.fsum(e[j] / z * v[bt[p // 4], p % 4, kvh, d] for j, p in enumerate(attended[r]))
                assert abs(out[r, h, d] - exp) <= 1e-12


def test_prefill_attn_properties():
    q, k, v, bt = _case(seed=4, rows=2, nq=6, nkv=3, hd=16, pages=8, block_size=8)
    lists = np.array([[2, 0, 5], [1, -1, -1]])
    base = attention.prefill_attn(q, k, v, bt, lists, 47, 8, 8, 3, 0.25)
    # the list order does not matter (a set of blocks)
    perm = attention.prefill_attn(q, k, v, bt, lists[:, ::-1], 47, 8, 8, 3, 0.25)
    np.testing.assert_allclose(perm, base, rtol=1e-13, atol=1e-14)
    # a zero query weighs every attended position equally: the mean of their values
    qz = q.copy()
    qz[1, 4] = 0.0
    outz = attention.prefill_attn(qz, k, v, bt, lists, 47, 8, 8, 3, 0.25)
    pos = attention.attended_positions(lists[1], 47, 1, 8)
    mean = v[bt[pos // 8], pos % 8, 2].mean(axis=0)                 # head 4 reads KV head 2
    np.testing.assert_allclose(outz[1, 4], mean, rtol=1e-13, atol=1e-14)
    # every output is a convex combination of the attended values
    for r in range(2):
        pos = attention.attended_positions(lists[r], 47, r, 8)
        for h in range(6):
            vals = v[bt[pos // 8], pos % 8, h // 2]
            assert np.all(base[r, h] <= vals.max(axis=0) + 1e-12) and np.all(base[r, h] >= vals.min(axis=0) - 1e-12)
    # one attended position returns its value exactly; none returns zeros
    one = attention.prefill_attn(q, k, v, bt, np.array([[-1], [-1]]), 47, 8, 8, 3, 0.25)   # row 0 at 47: tail empty
    np.testing.assert_array_equal(one[0], 0.0)
    np.testing.assert_allclose(one[1, 0], v[bt[48 // 8], 48 % 8, 0], rtol=0, atol=0)       # row 1 at 48: tail 48
