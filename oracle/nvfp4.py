"""NVFP4 key decoding and paged-pool address resolution (float64 oracle).

Test infrastructure only; see the package docstring.

Sources (page titles as in the package docstring):
* Nibble position and sign bit: [listing], ``dequant_fp4_scalar`` -- lane 0 is the
  low nibble and lane 1 the high nibble of a packed byte; bit 3 of the nibble is
  the sign, bits 2..0 the magnitude code.
* Magnitude of the 3-bit code: [commits], e74c84458c (the LUT
  0, 0.5, 1, 1.5, 2, 3, 4, 6) and 79ef87f9a9 (the same values spelled out as the
  bias-1 E2M1 encoding, and the statement that the raw-integer reading was wrong).
* Group scale: [listing], NVFP4 notes and the main kernel -- one FP8 E4M3 byte
  per 16 consecutive elements (``__nv_fp8_e4m3``, i.e. the OCP E4M3 format).
* Global scale: [listing], main kernel -- one FP32 value per physical block
  (``key_gscale[num_phys_blocks]``).
* Pool layout and address: [listing], kernel signature and the "resolve physical
  location of entry s" step -- logical block ``s // epb``, slot ``s % epb``,
  physical block from ``block_table[t, logical_block]``, entry
  ``phys * epb + slot``.

Reading taken where the listing's code and comments disagree: the exact value of
an element is ``code * e4m3(scale)`` and the float32 dequantised key is one
round-to-nearest-even of ``code * e4m3(scale) * gscale`` (the product is exact in
float64).  The listing's own code rounds ``e4m3 * gscale`` first; its comment
gives the left-to-right order, which is the one followed here.
"""

from __future__ import annotations

import numpy as np

# [commits] e74c84458c: magnitudes of the 3-bit E2M1 code, indexed by the code.
E2M1_MAGNITUDE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)

GROUP = 16  # [listing] NVFP4 notes: one scale per 16 elements


def e2m1_decode(nibbles) -> np.ndarray:
    """Value of 4-bit E2M1 codes: bit 3 is the sign, bits 2..0 index the magnitude.

    A set sign bit negates the magnitude, so code 0x8 is -0.0 ([listing],
    ``dequant_fp4_scalar``: ``sign ? -val : val``).
    """
    n = np.asarray(nibbles, dtype=np.uint8)
    if np.any(n > 15):
        raise ValueError("E2M1 codes are 4-bit")
    mag = E2M1_MAGNITUDE[n & 7]
    return np.where((n >> 3) & 1, -mag, mag)


def e4m3_decode(codes) -> np.ndarray:
    """Value of OCP FP8 E4M3 bytes (bias 7, no infinities, 0x7F/0xFF are NaN).

    s.eeee.mmm: e == 0 is subnormal m/8 * 2^-6; otherwise (1 + m/8) * 2^(e-7);
    e == 15 with m == 7 is NaN.  Largest finite magnitude 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def unpack_nibbles(packed) -> np.ndarray:
    """[..., D/2] bytes -> [..., D] nibbles; element 2b is the low nibble of byte b."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def code_values(keys_fp4, key_scale) -> np.ndarray:
    """Exact element values c = E2M1(nibble) * E4M3(scale of its 16-group), float64.

    keys_fp4: [..., D/2] uint8, key_scale: [..., D/16] uint8.  Returns [..., D].
    """
    nib = unpack_nibbles(keys_fp4)
    d = nib.shape[-1]
    sc = np.asarray(key_scale, dtype=np.uint8)
    if sc.shape[-1] * GROUP != d:
        raise ValueError("key_scale must hold one byte per 16 elements")
    scale = np.repeat(e4m3_decode(sc), GROUP, axis=-1)
    return e2m1_decode(nib) * scale


def resolve(block_table_row, s, epb):
    """Logical entries s -> (physical block, physical entry) for one query's table row."""
    s = np.asarray(s, dtype=np.int64)
    lb = s // epb
    slot = s % epb
    phys = np.asarray(block_table_row, dtype=np.int64)[lb]
    return phys, phys * epb + slot


def dequant_row(keys_fp4, key_scale, key_gscale, block_table_row, valid_len, epb):
    """Keys of one query's logical entries [0, valid_len).

    Returns (c, g): c [valid_len, D] exact code values (float64) and g [valid_len]
    the FP32 global scale of each entry's physical block (as float64).  The key
    used for scoring is c * g, exact in float64.
    """
    P, e, half = keys_fp4.shape
    if e != epb:
        raise ValueError("keys_fp4 must be [P, epb, D/2]")
    s = np.arange(int(valid_len), dtype=np.int64)
    phys, entry = resolve(block_table_row, s, epb)
    if s.size and (phys.min() < 0 or phys.max() >= P):
        raise ValueError("block_table entry outside the pool")
    codes = keys_fp4.reshape(P * epb, half)[entry]
    scales = key_scale.reshape(P * epb, -1)[entry]
    c = code_values(codes, scales)
    g = np.asarray(key_gscale, dtype=np.float32).astype(np.float64)[phys]
    return c, g


def dequant_f32(c, g) -> np.ndarray:
    """Bit-exact float32 dequantised key: one RNE rounding of the exact c * g."""
    return (np.asarray(c, dtype=np.float64) * np.asarray(g, dtype=np.float64)[..., None]).astype(np.float32)
