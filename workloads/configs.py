"""The five synthetic indexer workloads, plus reduced-size variants for tests.

Stream seeds: workload ``i`` draws array stream ``j`` from
``np.random.SeedSequence([i, j])`` with j = 0 block_table, 1 valid_lens, 2 q,
3 w, 4 key values / nibbles, 5 scales, 6 global scales, 7 norm weights,
8 raw keys.  Reduced variants add a third entry to the seed so they never
alias a full-size draw.

Key encodings (storage only; nothing here decodes):
* ``dist="tiny"``: uniform random 4-bit codes, E4M3 group scales drawn as
  2^U(-4, 2) and rounded to E4M3, global scale 1.0.
* ``dist="gauss"``: N(0,1) vectors quantised per 16 elements with an
  absmax/6 scale: scale byte = E4M3_RNE(absmax / 6 / g), code = nearest E2M1
  point of x / (scale * g) (ties to the even code, magnitudes saturate at 6,
  sign bit = x < 0), global scale g ~ U(0.5, 2) per physical page.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

# E2M1 magnitude grid used only to *encode* synthetic keys (nearest point).
_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
_E4M3_MAX = 448.0


def _rng(seed, stream):
    return np.random.default_rng(np.random.SeedSequence(list(seed) + [stream]))


def e4m3_encode_rne(x) -> np.ndarray:
    """float -> OCP E4M3 byte, round to nearest even, saturating at +-448."""
    v = np.clip(np.asarray(x, dtype=np.float32), -_E4M3_MAX, _E4M3_MAX)
    return torch.from_numpy(np.ascontiguousarray(v)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e2m1_encode_rne(x) -> np.ndarray:
    """float -> 4-bit E2M1 code (nearest grid point, ties to the even code, saturating)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 6.0)
    mid = (_E2M1_GRID[:-1] + _E2M1_GRID[1:]) / 2
    code = np.searchsorted(mid, a, side="left")          # a <= mid[i] -> below point i+1
    at_mid = (code < len(mid)) & (a == mid[np.minimum(code, len(mid) - 1)])
    code = np.where(at_mid & (code % 2 == 1), code + 1, code)  # tie: prefer the even code
    sign = (x < 0).astype(np.uint8)
    return (code.astype(np.uint8) | (sign << 3)).astype(np.uint8)


def pack_nibbles(codes) -> np.ndarray:
    """[..., D] 4-bit codes -> [..., D/2] bytes; element 2b in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def to_bf16_bits(x) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32)))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def quantize_gauss(rng_vals, rng_g, P, epb, D):
    """N(0,1) keys -> (keys_fp4 [P,epb,D/2], key_scale [P,epb,D/16], gscale [P])."""
    g = rng_g.uniform(0.5, 2.0, size=P).astype(np.float32)
    x = rng_vals.standard_normal((P, epb, D // 16, 16), dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    scale_b = e4m3_encode_rne(amax / 6.0 / g[:, None, None])
    scale_v = torch.from_numpy(scale_b).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    denom = scale_v.astype(np.float64) * g[:, None, None].astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(denom[..., None] > 0, x / denom[..., None], 0.0)
    codes = e2m1_encode_rne(y).reshape(P, epb, D)
    return pack_nibbles(codes), scale_b.reshape(P, epb, D // 16), g


def quantize_tiny(rng_vals, rng_s, P, epb, D):
    keys = rng_vals.integers(0, 256, size=(P, epb, D // 2), dtype=np.uint8)
    sc = e4m3_encode_rne(np.exp2(rng_s.uniform(-4.0, 2.0, size=(P, epb, D // 16))))
    return keys, sc, np.ones(P, dtype=np.float32)


@dataclass
class Workload:
    name: str
    kind: str                      # "csa" or "qsa"
    top_k: int
    # CSA fields
    T: int = 0
    H: int = 0
    D: int = 0
    epb: int = 0
    P: int = 0
    max_lb: int = 0
    q: Optional[np.ndarray] = None          # float32 [T,H,D] or uint16 bf16 bits
    q_dtype: str = "f32"
    w: Optional[np.ndarray] = None          # float32 [T,H]
    keys_fp4: Optional[np.ndarray] = None   # uint8 [P,epb,D/2]
    key_scale: Optional[np.ndarray] = None  # uint8 [P,epb,D/16]
    key_gscale: Optional[np.ndarray] = None  # float32 [P]
    block_table: Optional[np.ndarray] = None  # int32 [T,max_lb]
    valid_lens: Optional[np.ndarray] = None   # int32 [T]
    # QSA fields
    raw_keys: Optional[np.ndarray] = None   # uint16 bf16 bits [n_tok, hd]
    k_norm_w: Optional[np.ndarray] = None
    q_norm_w: Optional[np.ndarray] = None
    qk: Optional[np.ndarray] = None         # uint16 bf16 bits [rows, qkw]
    rows: int = 0
    first_pos: int = 0
    n_heads: int = 0
    hd: int = 0
    rot: int = 0
    theta: float = 0.0
    eps: float = 0.0
    ratio: int = 0
    n_blocks: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def pairs(self) -> int:
        """Number of valid (query, key) pairs scored."""
        if self.kind == "csa":
            return int(np.asarray(self.valid_lens, dtype=np.int64).sum())
        pos = self.first_pos + np.arange(self.rows, dtype=np.int64)
        return int(np.minimum((pos + 1) // self.ratio, self.n_blocks).sum()) * 1


def csa(name, seed, T, H, D, epb, P, max_lb, top_k, valid_lens, dist, q_dtype="f32",
        w_scale=1.0, table="shared") -> Workload:
    """Generic paged NVFP4 workload.  ``valid_lens`` is an int array or a callable(rng, T)."""
    r_bt, r_v, r_q, r_w, r_k, r_s, r_g = (_rng(seed, j) for j in range(7))
    if table == "shared":
        row = r_bt.permutation(P)[:max_lb].astype(np.int32)
        bt = np.tile(row, (T, 1))
    elif table == "per_row":
        bt = np.stack([r_bt.permutation(P)[:max_lb] for _ in range(T)]).astype(np.int32)
    elif table == "disjoint":   # every row its own pages: no page is shared between rows
        assert P >= T * max_lb
        bt = r_bt.permutation(P)[: T * max_lb].reshape(T, max_lb).astype(np.int32)
    else:
        raise ValueError(table)
    vl = valid_lens(r_v, T) if callable(valid_lens) else valid_lens
    vl = np.asarray(vl, dtype=np.int32)
    qf = r_q.standard_normal((T, H, D), dtype=np.float32)
    q = to_bf16_bits(qf) if q_dtype == "bf16" else qf
    w = (r_w.uniform(0.0, 1.0, size=(T, H)) * w_scale).astype(np.float32)
    if dist == "tiny":
        keys, sc, g = quantize_tiny(r_k, r_s, P, epb, D)
    elif dist == "gauss":
        keys, sc, g = quantize_gauss(r_k, r_g, P, epb, D)
    else:
        raise ValueError(dist)
    return Workload(name=name, kind="csa", top_k=top_k, T=T, H=H, D=D, epb=epb, P=P, max_lb=max_lb,
                    q=q, q_dtype=q_dtype, w=w, keys_fp4=keys, key_scale=sc, key_gscale=g,
                    block_table=bt, valid_lens=vl)


def qsa(name, seed, n_tok, hd, ratio, rows, n_heads, top_k, rot=64, theta=1e4, eps=1e-6,
        first_pos=None) -> Workload:
    r_w = _rng(seed, 7)
    r_raw = _rng(seed, 8)
    r_q = _rng(seed, 2)
    raw = to_bf16_bits(r_raw.standard_normal((n_tok, hd), dtype=np.float32))
    k_w = r_w.normal(0.0, 0.1, size=hd).astype(np.float32)
    q_w = r_w.normal(0.0, 0.1, size=hd).astype(np.float32)
    qk = to_bf16_bits(r_q.standard_normal((rows, n_heads * hd), dtype=np.float32))
    if first_pos is None:
        first_pos = n_tok - rows
    return Workload(name=name, kind="qsa", top_k=top_k, raw_keys=raw, k_norm_w=k_w, q_norm_w=q_w, qk=qk,
                    rows=rows, first_pos=first_pos, n_heads=n_heads, hd=hd, rot=rot, theta=theta, eps=eps,
                    ratio=ratio, n_blocks=n_tok // ratio)


def _uniform_valid(lo, hi):
    return lambda rng, T: rng.integers(lo, hi + 1, size=T)


def make(i: int, reduced: int = 0) -> Workload:
    """Workload ``i`` (1..5).  ``reduced > 0`` shrinks it for full-oracle tests."""
    seed = [i] if not reduced else [i, 1000 + reduced]
    if i == 1:
        return csa("tiny_decode", seed, T=4, H=4, D=64, epb=16, P=64, max_lb=64, top_k=32,
                   valid_lens=np.array([1024, 700, 333, 17]), dist="tiny")
    if i == 2:
        if reduced:
            return csa("decode_reduced", seed, T=3, H=64, D=128, epb=64, P=64, max_lb=48, top_k=256,
                       valid_lens=np.array([3072, 2000, 1537]), dist="gauss", w_scale=1 / 64)
        return csa("decode_T8_S65536", seed, T=8, H=64, D=128, epb=64, P=2048, max_lb=1024, top_k=2048,
                   valid_lens=_uniform_valid(32768, 65536), dist="gauss", w_scale=1 / 64)
    if i == 3:
        if reduced:
            return csa("long_decode_reduced", seed, T=4, H=64, D=128, epb=64, P=512, max_lb=256, top_k=2048,
                       valid_lens=np.array([16384, 9001, 12345, 2049]), dist="gauss", w_scale=1 / 64)
        return csa("long_decode_T32_S262144", seed, T=32, H=64, D=128, epb=64, P=8192, max_lb=4096,
                   top_k=2048, valid_lens=_uniform_valid(131072, 262144), dist="gauss", w_scale=1 / 64)
    if i == 4:
        T = 4096 if not reduced else 300
        stride = 4 if not reduced else 4
        pos = np.arange(T) * stride
        vl = (pos + 1) // 4
        P = 64 if not reduced else 5
        return csa("prefill_T4096" if not reduced else "prefill_reduced", seed, T=T, H=64, D=128, epb=64,
                   P=P, max_lb=P, top_k=512 if not reduced else 64, valid_lens=vl, dist="gauss",
                   q_dtype="bf16", w_scale=1 / 64)
    if i == 5:
        if reduced:
            return qsa("qsa_reduced", seed, n_tok=16 * 700, hd=128, ratio=16, rows=40, n_heads=32, top_k=64)
        return qsa("qsa_prefill", seed, n_tok=524288, hd=128, ratio=16, rows=2048, n_heads=32, top_k=256)
    raise ValueError(i)


def make_diag(name: str) -> Workload:
    """Diagnostic workloads that are not configurations of their own.

    ``hbm_true_T32_S262144``: the long-decode shape (32 rows, S=262144, H=64, D=128,
    64 keys per page, top_k=2048, valid lengths U{131072..262144}) where every row
    reads its own 4096 pages of a 131072-page pool (604 MB of NVFP4 keys, more than
    the 256 MB last-level cache), so that every key byte a row reads comes from DRAM.
    Keys use the uniform-code encoding (``dist="tiny"``) to keep generation fast.
    """
    if name == "hbm_true_T32_S262144":
        return csa(name, [3, 100], T=32, H=64, D=128, epb=64, P=131072, max_lb=4096, top_k=2048,
                   valid_lens=_uniform_valid(131072, 262144), dist="tiny", w_scale=1 / 64, table="disjoint")
    raise ValueError(name)


CONFIGS = {
    1: "tiny_decode",
    2: "decode_T8_S65536",
    3: "long_decode_T32_S262144",
    4: "prefill_T4096",
    5: "qsa_prefill",
}
