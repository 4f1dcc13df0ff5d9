"""Pins for the gather oracle (oracle/gather.py): checks against library conversions,
hand-worked values and layouts built so that every gathered element names its source.
CPU only."""

import numpy as np
import torch

from oracle import gather
from workloads.gather import make_gather, make_qsa_gather


def _bf16_of_f32(x):
    """torch's float32 -> bfloat16 conversion (one RNE rounding of a float32 value)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_matches_library_on_float32_values():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    special = np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.3895314e38, 3.4028235e38, 1e-40, -1e-45,
                        1.00390625, 1.01171875, 1.0078125 + 2 ** -23, 9.183549615799121e-41], dtype=np.float32)
    for v in (x, special):
        assert np.array_equal(gather.bf16_rne(v.astype(np.float64)), _bf16_of_f32(v))
    assert gather.bf16_rne(np.array([np.nan]))[0] & 0x7FFF == 0x7FC0


def test_bf16_rne_rounds_the_exact_value_once():
    # E4M3 byte 0x39 is 1.125; the fp32 scale with bits 0x3f69c71c is 15320860 * 2^-24.
    # Their product is 137887740 * 2^-27, which lies 2^-25 below the bfloat16 tie point
    # 1 + 7/256 = 137887744 * 2^-27.  One rounding goes down to 1 + 6/256 = 1.0234375
    # (bits 0x3F83).  Rounding to fp32 first lands exactly on the tie (the distance is
    # under half an fp32 spacing), and ties-to-even then gives 1 + 8/256 (0x3F84).
    s = np.array([0x3F69C71C], dtype=np.uint32).view(np.float32)
    assert float(s[0]) * 2 ** 24 == 15320860
    exact = 1.125 * float(s[0])
    assert exact * 2 ** 27 == 137887740
    assert gather.bf16_rne(np.array([exact]))[0] == 0x3F83
    assert _bf16_of_f32(np.array([exact], dtype=np.float32))[0] == 0x3F84   # the two-rounding result


def _one_hot_pool(P=6, epb=3, d_nope=256, d_rope=64, group=128):
    """Entry (p, e): every FP8 code is 0x38 (1.0) and its two group scales are 2p+1 and
    -(e+1)/4 (exact in bfloat16); its rope dim d holds 8p + e + (d mod 2)/2 (7 significant
    bits: exact in bfloat16)."""
    fp8 = np.full((P, epb, d_nope), 0x38, dtype=np.uint8)
    scale = np.zeros((P, epb, d_nope // group), dtype=np.float32)
    rope = np.zeros((P, epb, d_rope), dtype=np.float32)
    for p in range(P):
        for e in range(epb):
            scale[p, e] = [2 * p + 1, -(e + 1) / 4]
            rope[p, e] = 8 * p + e + (np.arange(d_rope) % 2) / 2
    return fp8, scale, _bf16_of_f32(rope), rope


def test_gather_kv_resolves_entries_through_the_table():
    P, epb = 6, 3
    fp8, scale, rope_bits, rope = _one_hot_pool(P, epb)
    bt = np.array([[4, 0, 5, 2, 1, 3], [1, 1, 2, 0, 3, 5]], dtype=np.int32)
    idx = np.array([[0, 5, 17, -1, 9], [3, 4, -1, -1, 16]], dtype=np.int32)
    out = gather.gather_kv(fp8, scale, rope_bits, bt, idx, epb, 128)
    assert out.shape == (2, 5, 320) and out.dtype == np.uint16
    vals = torch.from_numpy(out.view(np.int16)).view(torch.bfloat16).float().numpy()
    for t in range(2):
        for i in range(5):
            s = int(idx[t, i])
            if s < 0:
                assert np.all(out[t, i] == 0)
                continue
            p, e = int(bt[t, s // epb]), s % epb
            assert np.all(vals[t, i, :128] == 2 * p + 1)
            assert np.all(vals[t, i, 128:256] == -(e + 1) / 4)
            assert np.array_equal(out[t, i, 256:], rope_bits[p, e])          # the rope half is copied
            assert np.array_equal(vals[t, i, 256:], rope[p, e])


def test_gather_kv_dequant_of_each_code_is_the_library_value():
    # all 256 E4M3 bytes (NaN codes excluded) with scale 1: the value of each code, which
    # bfloat16 holds exactly (4 significant bits, exponents 2^-9 .. 2^8)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    fp8 = codes.reshape(1, 1, -1)[:, :, :254]
    fp8 = np.concatenate([fp8, np.zeros((1, 1, 2), np.uint8)], axis=-1)          # 256 dims
    scale = np.ones((1, 1, 2), np.float32)
    rope_bits = np.zeros((1, 1, 0), np.uint16)
    out = gather.gather_kv(fp8, scale, rope_bits, np.zeros((1, 1), np.int32), np.zeros((1, 1), np.int32), 1, 128)
    lib = torch.from_numpy(fp8.reshape(-1)).view(torch.float8_e4m3fn).to(torch.bfloat16)
    assert np.array_equal(out.reshape(-1), lib.view(torch.int16).numpy().view(np.uint16))


def test_gather_kv_fp8_round_trip_error_bound():
    # [commits] c2f705a21a states an FP8 round trip under 0.01 absolute.  For values in
    # [-0.12, 0.12] with the group scale amax/448, an E4M3 code carries 3 mantissa bits
    # (relative error <= 2^-4, so <= 0.0075 here), and the bfloat16 result adds <= 2^-9
    # relative: under 0.01.
    w = make_gather("round_trip", [31], T=2, P=8, epb=16, max_lb=8, top_k=64, d_nope=512, d_rope=64,
                    amp=0.12)
    out = gather.gather_kv(w.fp8, w.scale, w.rope_bits, w.block_table, w.topk_idx, w.epb, w.group)
    vals = torch.from_numpy(out.view(np.int16)).view(torch.bfloat16).double().numpy()
    for t in range(w.T):
        for i, s in enumerate(w.topk_idx[t]):
            if s < 0:
                continue
            p, e = int(w.block_table[t, s // w.epb]), int(s) % w.epb
            orig = w.source[p, e]
            assert np.max(np.abs(vals[t, i, : w.d_nope] - orig)) < 0.01


def test_qsa_gather_is_a_copy_of_the_selected_rows():
    block_size, nkv, hd, nb = 4, 2, 8, 5
    k = np.arange(nb * block_size * nkv * hd, dtype=np.uint16).reshape(nb, block_size, nkv, hd)
    v = (k + 30000).astype(np.uint16)
    bt = np.array([3, 0, 4, 1, 2], dtype=np.int32)
    sel = np.array([0, 7, 19, 8, 3], dtype=np.int64)
    ko, vo = gather.qsa_gather(k, v, bt, sel, block_size)
    assert ko.shape == (5, nkv, hd)
    for i, s in enumerate(sel):          # brute force, one element at a time
        for h in range(nkv):
            for d in range(hd):
                assert ko[i, h, d] == k[bt[s // block_size], s % block_size, h, d]
                assert vo[i, h, d] == v[bt[s // block_size], s % block_size, h, d]
    w = make_qsa_gather("qg", [32], n_blocks=64, block_size=16, nkv=2, hd=64, n_sel=100)
    ko, vo = gather.qsa_gather(w.k_cache, w.v_cache, w.block_table, w.sel, w.block_size)
    assert ko.shape == (100, 2, 64) and vo.shape == (100, 2, 64)


def test_gather_kv_rounds_the_product_once():
    # the hand-worked value of test_bf16_rne_rounds_the_exact_value_once, through the gather
    fp8 = np.full((1, 1, 128), 0x39, dtype=np.uint8)
    scale = np.array([0x3F69C71C], dtype=np.uint32).view(np.float32).reshape(1, 1, 1)
    out = gather.gather_kv(fp8, scale, np.zeros((1, 1, 0), np.uint16), np.zeros((1, 1), np.int32),
                           np.zeros((1, 1), np.int32), 1, 128)
    assert np.all(out == 0x3F83)
