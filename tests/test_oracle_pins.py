"""Pins for the CPU oracle: checks against what the pages fix and against mathematics,
never against the oracle's own formulas retyped.  CPU only."""

import heapq
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import indexer, nvfp4, qsa
from tests.insertion_topk import insertion_topk
from workloads import make
from workloads.configs import csa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- E2M1

def test_e2m1_matches_commit_encoding_table():
    for bits, value in _read_table("e2m1_encoding.txt"):
        code = int(bits, 2)
        assert nvfp4.e2m1_decode(code) == float(value)
        # sign bit (bit 3) negates: the listing's dequant_fp4_scalar
        neg = nvfp4.e2m1_decode(code | 8)
        assert neg == -float(value) and math.copysign(1.0, neg) == -1.0


def test_e2m1_matches_commit_lut():
    (row,) = _read_table("e2m1_lut.txt")
    lut = [float(v) for v in row]
    assert list(nvfp4.e2m1_decode(np.arange(8))) == lut


def test_e2m1_closed_form_bias1():
    # E2M1 with exponent bias 1: e = bits[2:1], m = bit0; e == 0 is subnormal m * 2^-1.
    for n in range(16):
        e, m, s = (n >> 1) & 3, n & 1, n >> 3
        v = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        assert nvfp4.e2m1_decode(n) == (-v if s else v)


def test_e2m1_is_not_the_raw_integer_decode():
    # commit 79ef87f9a9: "Old (WRONG): val = (int)(nibble & 0x07) * scale"
    wrong = np.arange(8, dtype=np.float64)
    right = nvfp4.e2m1_decode(np.arange(8))
    differ = [i for i in range(8) if wrong[i] != right[i]]
    assert differ == [1, 2, 3, 4, 5, 6, 7]


def test_nibble_order_low_first():
    # listing dequant_fp4_scalar: lane 0 = low nibble (element 2b), lane 1 = high nibble
    b = np.array([[0x31, 0xF0]], dtype=np.uint8)
    nib = nvfp4.unpack_nibbles(b)
    assert nib.tolist() == [[0x1, 0x3, 0x0, 0xF]]
    assert nvfp4.e2m1_decode(nib).tolist() == [[0.5, 1.5, 0.0, -6.0]]


# ---------------------------------------------------------------- E4M3

def test_e4m3_matches_library_all_codes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = nvfp4.e4m3_decode(np.arange(256))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))
    assert np.isnan(got).sum() == 2


def test_e4m3_hand_spot_values():
    for byte, value in _read_table("e4m3_spot.txt"):
        got = float(nvfp4.e4m3_decode(int(byte, 16)))
        if value == "nan":
            assert math.isnan(got)
        else:
            assert got == float(value)
            assert math.copysign(1.0, got) == math.copysign(1.0, float(value))


def test_code_values_exact_in_fp16_and_f32():
    # every finite (E2M1, E4M3) product is representable in fp16: exact NVFP4 code values
    v = nvfp4.e2m1_decode(np.arange(16))[:, None] * nvfp4.e4m3_decode(np.arange(256))[None, :]
    fin = np.isfinite(v)
    assert np.array_equal(v[fin].astype(np.float16).astype(np.float64), v[fin])


# ---------------------------------------------------------------- layout / address

def test_group_scale_assignment():
    # 16 consecutive elements share a scale byte (listing NVFP4 notes)
    keys = np.full((1, 16), 0x22, dtype=np.uint8)          # 32 elements of code 2 -> 1.0
    sc = np.array([[0x38, 0x40]], dtype=np.uint8)           # 1.0, 2.0
    c = nvfp4.code_values(keys, sc)
    assert c.tolist() == [[1.0] * 16 + [2.0] * 16]


def test_address_resolution_reveals_table():
    P, epb, D = 7, 3, 32
    keys = np.full((P, epb, D // 2), 0x22, dtype=np.uint8)  # every code value 1.0
    sc = np.full((P, epb, D // 16), 0x38, dtype=np.uint8)
    g = np.arange(1, P + 1, dtype=np.float32)              # page p encodes p + 1
    rng = np.random.default_rng(5)
    bt = rng.permutation(P).astype(np.int32)
    c, gg = nvfp4.dequant_row(keys, sc, g, bt, P * epb, epb)
    for s in range(P * epb):
        assert gg[s] == bt[s // epb] + 1
    assert np.all(c == 1.0)


def test_physical_permutation_invariance():
    w = make(1)
    rng = np.random.default_rng(11)
    perm = rng.permutation(w.P)                 # new slot of old page p is perm[p]
    inv = np.argsort(perm)
    keys2 = w.keys_fp4[inv]
    sc2 = w.key_scale[inv]
    g2 = w.key_gscale[inv]
    bt2 = perm[w.block_table].astype(np.int32)
    a = indexer.scores(w.q, w.w, w.keys_fp4, w.key_scale, w.key_gscale, w.block_table, w.valid_lens, w.epb)
    b = indexer.scores(w.q, w.w, keys2, sc2, g2, bt2, w.valid_lens, w.epb)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_duplicate_page_gives_equal_scores():
    w = make(1)
    bt = w.block_table.copy()
    bt[:, 5] = bt[:, 2]
    rows = indexer.scores(w.q, w.w, w.keys_fp4, w.key_scale, w.key_gscale, bt, w.valid_lens, w.epb)
    r = rows[0]
    assert np.array_equal(r[5 * w.epb:6 * w.epb], r[2 * w.epb:3 * w.epb])
    idx, _ = indexer.topk(r, w.P * w.epb)
    pos = {int(s): i for i, s in enumerate(idx)}
    for j in range(w.epb):     # equal scores: the lower index ranks first
        assert pos[2 * w.epb + j] < pos[5 * w.epb + j]


def test_dequant_f32_is_one_rounding_of_the_exact_product():
    # Code 0b011 (1.5) with scale byte 0x3A (1.25) and global scale g = 1 + 2^-22 (an fp32
    # value).  Worked by hand: c = 1.875 and c*g = 1.875 + 3.75 * 2^-23; the fp32 spacing
    # on [1, 2) is 2^-23, so one rounding gives 1.875 + 4 * 2^-23.  The listing's code
    # rounds e4m3*g first: 1.25 + 2.5 * 2^-23 is a tie that goes to the even 1.25 + 2 * 2^-23,
    # and 1.5 times that is 1.875 + 3 * 2^-23 -- a different float.
    keys = np.array([[0x03, 0, 0, 0, 0, 0, 0, 0]], dtype=np.uint8)
    sc = np.array([[0x3A]], dtype=np.uint8)
    c = nvfp4.code_values(keys, sc)
    assert c[0, 0] == 1.875 and np.all(c[0, 1:] == 0.0)
    g = np.array([np.float32(1.0 + 2.0 ** -22)], dtype=np.float32)
    assert float(g[0]) == 1.0 + 2.0 ** -22
    k = nvfp4.dequant_f32(c, g)
    assert k.dtype == np.float32
    assert float(k[0, 0]) == 1.875 + 4 * 2.0 ** -23
    assert float(k[0, 0]) != 1.875 + 3 * 2.0 ** -23


# ---------------------------------------------------------------- scores

def _hand_case():
    with open(os.path.join(GOLDEN, "hand_worked_scores.json")) as f:
        h = json.load(f)
    D, H, epb, P = h["D"], h["H"], h["epb"], h["P"]
    keys = np.zeros((P, epb, D // 2), dtype=np.uint8)
    for p, e, b, v in h["keys_fp4_nonzero"]:
        keys[p, e, b] = int(v, 16)
    sc = np.array([[[int(x, 16) for x in g] for g in e] for e in h["key_scale"]], dtype=np.uint8)
    g = np.array(h["key_gscale"], dtype=np.float32)
    bt = np.array(h["block_table"], dtype=np.int32)
    vl = np.array(h["valid_lens"], dtype=np.int32)
    T = bt.shape[0]
    q = np.zeros((T, H, D), dtype=np.float32)
    for t, hh, d, v in h["q_nonzero"]:
        q[t, hh, d] = v
    w = np.array(h["w"], dtype=np.float32)
    return h, q, w, keys, sc, g, bt, vl


def test_hand_worked_scores_and_topk():
    h, q, w, keys, sc, g, bt, vl = _hand_case()
    idx, val, rows = indexer.score_topk(q, w, keys, sc, g, bt, vl, h["epb"], h["top_k"])
    for t in range(len(rows)):
        assert rows[t].tolist() == h["expected_scores"][t]
        assert idx[t].tolist() == h["expected_topk"][t]


def test_one_hot_query_reads_code_values():
    # q[h] = e_{d_h}: I[s] = sum_h w_h * max(0, k[s, d_h]) exactly
    w1 = make(1)
    T, H, D = 1, 3, w1.D
    dims = [0, 17, 63]
    q = np.zeros((T, H, D), dtype=np.float32)
    for hh, d in enumerate(dims):
        q[0, hh, d] = 1.0
    ww = np.array([[0.25, 1.0, 4.0]], dtype=np.float32)
    rows = indexer.scores(q, ww, w1.keys_fp4, w1.key_scale, w1.key_gscale, w1.block_table[:1], [500], w1.epb)
    c, gg = nvfp4.dequant_row(w1.keys_fp4, w1.key_scale, w1.key_gscale, w1.block_table[0], 500, w1.epb)
    exp = sum(ww[0, i] * np.maximum(c[:, d] * gg, 0.0) for i, d in enumerate(dims))
    assert np.array_equal(rows[0], exp)


def test_score_invariants():
    w = make(1)
    base = indexer.scores(w.q, w.w, w.keys_fp4, w.key_scale, w.key_gscale, w.block_table, w.valid_lens, w.epb)
    q2 = (w.q * 4.0).astype(np.float32)
    s2 = indexer.scores(q2, w.w, w.keys_fp4, w.key_scale, w.key_gscale, w.block_table, w.valid_lens, w.epb)
    g2 = (w.key_gscale * 0.5).astype(np.float32)
    s3 = indexer.scores(w.q, w.w, w.keys_fp4, w.key_scale, g2, w.block_table, w.valid_lens, w.epb)
    wz = w.w.copy()
    wz[:, 1:] = 0
    s4 = indexer.scores(w.q, wz, w.keys_fp4, w.key_scale, w.key_gscale, w.block_table, w.valid_lens, w.epb)
    for t in range(w.T):
        assert np.all(base[t] >= 0)                  # ReLU with w >= 0
        assert np.array_equal(s2[t], 4.0 * base[t])  # homogeneous in q (power of 2: exact)
        assert np.array_equal(s3[t], 0.5 * base[t])  # homogeneous in gscale
        assert np.all(s4[t] <= base[t] + 1e-12)
        assert len(base[t]) == w.valid_lens[t]


def test_negative_gscale_and_weight_follow_relu_of_scaled_key():
    w = make(1)
    g = w.key_gscale.copy()
    g[::3] = -g[::3]
    ww = w.w.copy()
    ww[:, 0] = -ww[:, 0]
    rows = indexer.scores(w.q, ww, w.keys_fp4, w.key_scale, g, w.block_table, w.valid_lens, w.epb)
    t = 1
    c, gg = nvfp4.dequant_row(w.keys_fp4, w.key_scale, g, w.block_table[t], w.valid_lens[t], w.epb)
    k = c * gg[:, None]
    for s in (0, 1, 100, 699):
        exp = sum(float(ww[t, h]) * max(0.0, float(np.dot(w.q[t, h].astype(np.float64), k[s]))) for h in range(w.H))
        assert rows[t][s] == pytest.approx(exp, rel=1e-14, abs=1e-14)


def _brute_force_scores(w, t):
    """Scalar loops with an independent decode: E2M1 from its bit fields, E4M3 via torch."""
    out = []
    e4 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).tolist()
    for s in range(int(w.valid_lens[t])):
        p = int(w.block_table[t][s // w.epb])
        slot = s % w.epb
        g = float(w.key_gscale[p])
        key = []
        for d in range(w.D):
            byte = int(w.keys_fp4[p, slot, d // 2])
            n = byte & 15 if d % 2 == 0 else byte >> 4
            e, m = (n >> 1) & 3, n & 1
            v = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
            if n & 8:
                v = -v
            key.append(v * e4[int(w.key_scale[p, slot, d // 16])] * g)
        total = 0.0
        for h in range(w.H):
            dot = math.fsum(float(w.q[t, h, d]) * key[d] for d in range(w.D))
            total += float(w.w[t, h]) * max(dot, 0.0)
        out.append(total)
    return out


def test_brute_force_matches_on_tiny_config():
    w = make(1)
    rows = indexer.scores(w.q, w.w, w.keys_fp4, w.key_scale, w.key_gscale, w.block_table, w.valid_lens, w.epb)
    for t in (1, 3):
        bf = _brute_force_scores(w, t)
        np.testing.assert_allclose(rows[t], bf, rtol=1e-13, atol=1e-13)


def test_bf16_q_upcast_exact():
    x = np.array([1.0, -2.5, 3.140625, 1e-3], dtype=np.float32)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(indexer.upcast(bits, "bf16"), ref)


# ---------------------------------------------------------------- top-k

@pytest.mark.parametrize("k", [1, 5, 32, 40])
def test_topk_three_ways(k):
    w = make(1)
    rows = indexer.scores(w.q, w.w, w.keys_fp4, w.key_scale, w.key_gscale, w.block_table, w.valid_lens, w.epb)
    for t in range(w.T):
        r = rows[t]
        idx, val = indexer.topk(r, k)
        hb, hs = insertion_topk(list(r), k)
        assert idx.tolist() == hb
        nl = heapq.nlargest(k, ((v, -s) for s, v in enumerate(r)))
        exp = [-s for _, s in nl] + [-1] * (k - len(nl))
        assert idx.tolist() == exp


def test_topk_ties_and_padding():
    # all-zero scores: the first K indices, then -1
    idx, val = indexer.topk(np.zeros(17), 32)
    assert idx.tolist() == list(range(17)) + [-1] * 15
    assert np.all(np.isneginf(val[17:]))
    # -0.0 and 0.0 tie; lower index first
    idx, _ = indexer.topk(np.array([0.0, -0.0, 1.0, -0.0]), 4)
    assert idx.tolist() == [2, 0, 1, 3]
    # empty row
    idx, _ = indexer.topk(np.zeros(0), 3)
    assert idx.tolist() == [-1, -1, -1]


def test_tiny_config_short_row_zero_ties():
    w = make(1)
    rows = indexer.scores(w.q, w.w, w.keys_fp4, w.key_scale, w.key_gscale, w.block_table, w.valid_lens, w.epb)
    r = rows[3]                               # valid_len 17 < k = 32
    idx, _ = indexer.topk(r, w.top_k)
    assert sorted(idx[:17].tolist()) == list(range(17)) and np.all(idx[17:] == -1)
    zeros = [s for s in idx[:17] if r[s] == 0.0]
    assert zeros == sorted(zeros)
    assert all(0 <= s < w.valid_lens[t] for t in range(w.T) for s in indexer.topk(rows[t], w.top_k)[0] if s >= 0)


# ---------------------------------------------------------------- QSA

def test_rms_norm_matches_library():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 128))
    wt = rng.normal(0, 0.1, 128)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), weight=torch.from_numpy(1 + wt), eps=1e-6).numpy()
    np.testing.assert_allclose(qsa.rms_norm(x, wt, 1e-6), ref, rtol=1e-14, atol=1e-15)


def test_rope_closed_form_and_properties():
    D, rot, theta = 128, 64, 1e4
    e0 = np.zeros(D)
    e0[0] = 1.0
    pos = 7
    r = qsa.rope(e0, pos, rot, theta)
    assert r[0] == pytest.approx(math.cos(7.0)) and r[32] == pytest.approx(math.sin(7.0))
    e5 = np.zeros(D)
    e5[5] = 1.0
    ang = pos * theta ** (-10 / 64)
    r5 = qsa.rope(e5, pos, rot, theta)
    assert r5[5] == pytest.approx(math.cos(ang)) and r5[37] == pytest.approx(math.sin(ang))
    rng = np.random.default_rng(1)
    x = rng.standard_normal(D)
    y = rng.standard_normal(D)
    assert np.array_equal(qsa.rope(x, 0, rot, theta), x)                 # pos 0 is identity
    assert np.array_equal(qsa.rope(x, 99, 0, theta), x)                  # rot 0 is a no-op
    rx = qsa.rope(x, 12345, rot, theta)
    assert np.array_equal(rx[rot:], x[rot:])                             # untouched tail
    for i in range(rot // 2):                                            # pairs keep their norm
        assert math.hypot(rx[i], rx[i + 32]) == pytest.approx(math.hypot(x[i], x[i + 32]))
    # q(p) . k(p') depends only on p - p'
    a = qsa.rope(x, 1000, rot, theta) @ qsa.rope(y, 990, rot, theta)
    b = qsa.rope(x, 20, rot, theta) @ qsa.rope(y, 10, rot, theta)
    assert a == pytest.approx(b, rel=1e-9)


def test_block_pool_reduces_to_norm_and_mean():
    rng = np.random.default_rng(2)
    raw = rng.standard_normal((64, 32))
    wz = np.zeros(32)
    # ratio 1, rot 0: each block key is the RMSNorm of its single raw key
    out = qsa.block_pool(raw, wz, 0, 64, 1, 0, 1e4, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(raw), (32,), eps=1e-6).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-13)
    # ratio 4: mean of the 4 raw keys, then norm (rot 0)
    out4 = qsa.block_pool(raw, wz, 2, 3, 4, 0, 1e4, 1e-6)
    m = np.stack([raw[4 * b:4 * b + 4].mean(0) for b in (2, 3, 4)])
    ref4 = torch.nn.functional.rms_norm(torch.from_numpy(m), (32,), eps=1e-6).numpy()
    np.testing.assert_allclose(out4, ref4, rtol=1e-13)
    assert qsa.block_pool(raw, wz, 0, 0, 4, 0, 1e4, 1e-6).shape == (0, 32)


def test_qsa_score_rows_brute_force_and_mask():
    rng = np.random.default_rng(4)
    rows, H, hd, nb, ratio, first = 3, 2, 16, 10, 4, 30
    q = rng.standard_normal((rows, H, hd))
    k = rng.standard_normal((nb, hd))
    s, valid = qsa.score_rows(q, k, first, ratio)
    # rows at positions 30, 31, 32 with 4 tokens per block: blocks 0..6 hold tokens 0..27
    # (complete at 30), block 7 completes with token 31; the table holds 10 blocks
    assert valid.tolist() == [7, 8, 8]
    for r in range(rows):
        for b in range(nb):
            if b >= valid[r]:
                assert s[r, b] == -np.inf
            else:
                exp = sum(max(0.0, math.fsum(q[r, h, d] * k[b, d] for d in range(hd))) for h in range(H)) / 4.0
                assert s[r, b] == pytest.approx(exp, rel=1e-13)


def _rot(a, b, ang):
    return a * math.cos(ang) - b * math.sin(ang), a * math.sin(ang) + b * math.cos(ang)


def test_qprep_rows_hand_worked():
    # Two rows at positions 5 and 6 (first_pos 5), two heads of 4 dims read from rows of
    # width qkw = 10 (the last two columns are not q), rot = 4 (pairs (0,2) and (1,3)),
    # theta = 100: pair 0 turns by pos, pair 1 by pos * 100^(-1/2) = pos / 10.  eps = 0.
    qk = np.array([[1, 1, 1, 1, 2, 0, 0, 0, 100, -100],
                   [0, 3, 0, 4, -1, -1, 1, 1, 7, 7]], dtype=np.float64)
    wq = np.array([0.0, 0.5, -0.5, 1.0])             # scale 1 + w = (1, 1.5, 0.5, 2)
    got = qsa.qprep_rows(qk, wq, 2, 5, 10, 2, 4, 4, 100.0, 0.0)
    assert got.shape == (2, 2, 4)
    # normalised and scaled by hand: rms of (1,1,1,1) and (2,0,0,0) and (-1,-1,1,1) is 1,
    # of (0,3,0,4) it is 2.5
    normed = {(0, 0): (1.0, 1.5, 0.5, 2.0), (0, 1): (2.0, 0.0, 0.0, 0.0),
              (1, 0): (0.0, 1.8, 0.0, 3.2), (1, 1): (-1.0, -1.5, 0.5, 2.0)}
    for (r, h), (n0, n1, n2, n3) in normed.items():
        pos = 5 + r
        o0, o2 = _rot(n0, n2, pos * 1.0)
        o1, o3 = _rot(n1, n3, pos / 10.0)
        np.testing.assert_allclose(got[r, h], [o0, o1, o2, o3], rtol=1e-13, atol=1e-14)


def test_block_pool_rotates_at_the_block_first_position():
    # ratio 2: block b pools raw rows 2b, 2b+1 and sits at position 2b.  Blocks 3 and 4:
    # means (1,1,1,1) and (2,0,0,0), both of rms 1; rot = 4, theta = 100 (pair 1 turns
    # by pos / 10), eps = 0.  The other raw rows must not be read.
    raw = np.full((10, 4), 50.0)
    raw[6], raw[7] = [0, 2, 1, 1], [2, 0, 1, 1]
    raw[8], raw[9] = [3, 0, 0, 0], [1, 0, 0, 0]
    wk = np.array([0.0, 0.5, -0.5, 1.0])
    got = qsa.block_pool(raw, wk, 3, 2, 2, 4, 100.0, 0.0)
    assert got.shape == (2, 4)
    for i, (pos, (n0, n1, n2, n3)) in enumerate([(6, (1.0, 1.5, 0.5, 2.0)), (8, (2.0, 0.0, 0.0, 0.0))]):
        o0, o2 = _rot(n0, n2, pos * 1.0)
        o1, o3 = _rot(n1, n3, pos / 10.0)
        np.testing.assert_allclose(got[i], [o0, o1, o2, o3], rtol=1e-13, atol=1e-14)


def test_qprep_decode_query_hand_worked():
    # the projection row (0,3,0,4 | -1,-1,1,1) of the hand-worked prefill case, now a single
    # decode query at position 6 with no extra columns; same normalisation and rotation
    got = qsa.qprep(np.array([0, 3, 0, 4, -1, -1, 1, 1], dtype=np.float64), np.array([0.0, 0.5, -0.5, 1.0]),
                    2, 4, 4, 6, 100.0, 0.0)
    for h, (n0, n1, n2, n3) in enumerate([(0.0, 1.8, 0.0, 3.2), (-1.0, -1.5, 0.5, 2.0)]):
        o0, o2 = _rot(n0, n2, 6.0)
        o1, o3 = _rot(n1, n3, 0.6)
        np.testing.assert_allclose(got[h], [o0, o1, o2, o3], rtol=1e-13, atol=1e-14)


def test_score_blocks_brute_force_and_no_causal_cut():
    rng = np.random.default_rng(6)
    H, hd, nb = 3, 16, 12
    q = rng.standard_normal((H, hd))
    k = rng.standard_normal((nb + 5, hd))        # the table is longer than the blocks scored
    got = qsa.score_blocks(q, k, nb)
    assert got.shape == (nb,)
    for b in range(nb):
        exp = sum(max(0.0, math.fsum(q[h, d] * k[b, d] for d in range(hd))) for h in range(H)) / 4.0
        assert got[b] == pytest.approx(exp, rel=1e-13)
    # a prefill row whose complete-block count is nb scores the same blocks
    rows, valid = qsa.score_rows(q[None], k[:nb], first_pos=nb * 4 - 1, ratio=4)
    assert valid.tolist() == [nb]
    np.testing.assert_allclose(rows[0], got, rtol=1e-14)


def test_complete_blocks_literal():
    # positions 14..18 with 4 tokens per block: tokens 0..15 fill blocks 0..3 at position 15
    assert qsa.complete_blocks(14, 5, 4, 100).tolist() == [3, 4, 4, 4, 4]
    assert qsa.complete_blocks(14, 5, 4, 4).tolist() == [3, 4, 4, 4, 4]
    assert qsa.complete_blocks(14, 5, 4, 3).tolist() == [3, 3, 3, 3, 3]      # capped by the table
    assert qsa.complete_blocks(0, 3, 1, 10).tolist() == [1, 2, 3]             # ratio 1: every token


def test_generator_is_deterministic():
    a = make(1)
    b = make(1)
    for f in ("q", "w", "keys_fp4", "key_scale", "key_gscale", "block_table", "valid_lens"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = csa("x", [9], T=2, H=4, D=64, epb=16, P=8, max_lb=8, top_k=4, valid_lens=[5, 6], dist="gauss", table="per_row")
    assert not np.array_equal(c.block_table[0], c.block_table[1])
