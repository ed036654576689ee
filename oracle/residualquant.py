"""ResidualQuant CPU oracle: cross-loop residual KV quantization and decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing under ``oracle/`` is part of the product:
only ``tests/``, the package's ``smoke()`` check and the benchmark's CPU
baseline leg may import it.  It shares no code with the HIP path and never
takes an input or an expected value from it.

Plain and slow on purpose: float64 numpy, one formula per step, in the order
the pages give it.  Sources (four web pages about "ResidualQuant: KV Cache
Quantization for Looped Transformers with 2-Bit Residuals"):

* explainer page (learnaivisually.com), paragraph "So ResidualQuant keeps the
  final loop's KV ...": the last loop is the anchor, stored INT4; every earlier
  loop stores ``residual = KV(loop) - c * anchor`` at 2 bits, with ``c`` a
  least-squares coefficient per key or value vector; a fixed rotation is
  applied to the residual before quantization; attention rebuilds
  ``c * anchor + residual``.
* same page, paragraph "Which print is the master ...": shared anchor = two
  reads per loop, chained overlays need more; the current token stays BF16
  until its final loop and is quantized afterwards.
* same page, "Worked example": 4-bit anchor + three 2-bit residuals, FP8
  scale and offset per channel group, one BF16 coefficient per residual vector.
* arXiv digest (ai4snews), Figure 1 caption and ablation paragraph: group size
  g = 32, last-loop residual, least-squares scaling, rotation of the residual
  (not of the KV), INT4/INT2 mixed precision; Huginn-3.5B runs its 32 loops as
  8 groups of 4.

Readings adopted where the pages are silent:
asymmetric min/max quantizer ``x_hat = z + q * s`` with FP8-E4M3 offset ``z``
rounded down and scale ``s`` the smallest E4M3 value >= 2^-9 that covers the
group maximum; codes rounded half-to-even; ``c`` rounded to BF16 once from the
exact quotient and used rounded; groups are contiguous channels (of the rotated
vector for residuals); chained variant references the *reconstructed* next
loop; softmax scale 1/sqrt(d); the current token attends to itself with its
BF16 K/V.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

from .formats import (E4M3_POSITIVE, bf16_bits, bf16_from_bits, bf16_round, e4m3_decode,
                      e4m3_encode, e4m3_floor)

TILE = 64   # tokens per cache tile


@dataclasses.dataclass(frozen=True)
class Config:
    head_dim: int
    group: int
    anchor_bits: int
    resid_bits: int
    loops_per_group: int
    n_groups: int
    chained: bool
    n_kv_heads: int
    n_q_heads: int
    max_batch: int
    max_ctx: int
    scale_rule: int = 0     # 0: least-squares c; 1: norm-ratio c (the digest's appendix alternative)
    # residual width of each local loop 0..L-2 (empty: resid_bits for all).  The commentary page
    # ("它压的根本不是 KV" section) remarks that the loops near the anchor keep thinner residuals
    # and the farther ones more bits; these widths express that allocation.
    resid_bits_loop: Tuple[int, ...] = ()

    @property
    def n_loops(self) -> int:
        return self.loops_per_group * self.n_groups

    def rbits(self, l: int) -> int:
        """Residual width of local loop l (< L-1)."""
        return self.resid_bits_loop[l] if self.resid_bits_loop else self.resid_bits


# ---------------------------------------------------------------------------
# quantizer (explainer worked example: FP8 scale + offset per group; digest: g = 32)
# ---------------------------------------------------------------------------

def quantize(x: np.ndarray, bits: int, group: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Asymmetric group quantizer over the last axis.

    For each group of ``group`` contiguous channels with minimum m and maximum M:
    offset z = largest E4M3 value <= m; scale s = smallest E4M3 value >= 2^-9
    with z + (2^bits - 1) * s >= M (found by testing every positive E4M3 value);
    code = clamp(round_half_even((x - z) / s), 0, 2^bits - 1).
    Returns integer codes (..., d), offsets (..., d/group), scales (..., d/group).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % group == 0
    n = 2 ** bits - 1
    xg = x.reshape(x.shape[:-1] + (d // group, group))
    lo = xg.min(axis=-1)
    hi = xg.max(axis=-1)
    z = e4m3_floor(lo)
    covers = (z[..., None] + n * E4M3_POSITIVE) >= hi[..., None]
    if not np.all(covers.any(axis=-1)):
        raise ValueError("group range exceeds what an E4M3 scale can cover")
    s = E4M3_POSITIVE[np.argmax(covers, axis=-1)]
    t = (xg - z[..., None]) / s[..., None]
    codes = np.clip(np.rint(t), 0, n).astype(np.int64)
    return codes.reshape(x.shape), z, s


def dequantize(codes: np.ndarray, z: np.ndarray, s: np.ndarray, group: int) -> np.ndarray:
    """x_hat = z + code * s, per group of contiguous channels."""
    codes = np.asarray(codes)
    d = codes.shape[-1]
    cg = codes.reshape(codes.shape[:-1] + (d // group, group)).astype(np.float64)
    return (z[..., None] + cg * s[..., None]).reshape(codes.shape)


# ---------------------------------------------------------------------------
# least-squares coefficient (explainer: "c is a least-squares coefficient computed
# for each key or value vector"; digest: stored in BF16)
# ---------------------------------------------------------------------------

def ls_coefficient(x: np.ndarray, ref: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """c* = <x, ref> / <ref, ref> (0 when ref is all zero) and c = BF16(c*)."""
    num = np.sum(x * ref, axis=-1)
    den = np.sum(ref * ref, axis=-1)
    exact = np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0)
    return bf16_round(exact), exact


def norm_ratio_coefficient(x: np.ndarray, ref: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """c* = ||x|| / ||ref|| (0 when ref is all zero) and c = BF16(c*).

    The digest names norm-ratio scaling (ablation section, appendix table) as the
    alternative to least squares without printing it; the plain reading is the ratio of
    the Euclidean norms, which matches the magnitude of c * ref to that of x and ignores
    the direction."""
    xx = np.sum(x * x, axis=-1)
    rr = np.sum(ref * ref, axis=-1)
    exact = np.where(rr > 0, np.sqrt(xx / np.where(rr > 0, rr, 1.0)), 0.0)
    return bf16_round(exact), exact


def coefficient(x: np.ndarray, ref: np.ndarray, cfg: "Config") -> Tuple[np.ndarray, np.ndarray]:
    """The scaling rule the configuration selects."""
    return norm_ratio_coefficient(x, ref) if cfg.scale_rule == 1 else ls_coefficient(x, ref)


# ---------------------------------------------------------------------------
# encoding one anchor group of loops for one (KV head, K|V)
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Encoded:
    """Codes and metadata of one anchor group for a set of tokens.

    anchor = (codes, z, s); resid[l] = (codes, z, s, c) for loops l = 0..L-2
    (loop L-1 of the group is the anchor).  Leading axes are the tokens'.
    """
    anchor: Tuple[np.ndarray, np.ndarray, np.ndarray]
    resid: List[Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]]


def encode(xs: np.ndarray, rot: np.ndarray, cfg: Config) -> Encoded:
    """Quantize the K (or V) vectors of all loops of one anchor group.

    xs: (L, ..., d) values of loops 0..L-1 (loop L-1 is the anchor, the last loop).
    rot: (d, d) rotation R for this (KV head, K|V).

    Shared anchor (explainer, "With one shared master, each other loop needs two
    reads"): every loop l < L-1 is referenced to the dequantized anchor a_hat.
    Chained (same paragraph, the alternative design): loop l is referenced to the
    reconstruction of loop l+1, and the anchor closes the chain.
    For each non-anchor loop: c = BF16(<x, ref>/<ref, ref>) (or the norm ratio, see
    ``coefficient``); y = x - c * ref; r = R y; r is group-quantized at the residual width.
    """
    L = xs.shape[0]
    g = cfg.group
    R = np.asarray(rot, dtype=np.float64)
    qa, za, sa = quantize(xs[L - 1], cfg.anchor_bits, g)
    a_hat = dequantize(qa, za, sa, g)
    resid: List = [None] * (L - 1)
    ref = a_hat
    for l in range(L - 2, -1, -1):
        c, _ = coefficient(xs[l], ref, cfg)
        y = xs[l] - c[..., None] * ref
        r = y @ R.T                                  # r = R y, tokens as rows
        qr, zr, sr = quantize(r, cfg.rbits(l), g)
        resid[l] = (qr, zr, sr, c)
        if cfg.chained:
            ref = c[..., None] * ref + dequantize(qr, zr, sr, g) @ R   # c * ref + R^T r_hat
    return Encoded((qa, za, sa), resid)


def reconstruct(enc: Encoded, loop: int, rot: np.ndarray, cfg: Config) -> np.ndarray:
    """Rebuilt K (or V) of local loop ``loop``: a_hat for the anchor loop, otherwise
    c * ref + R^T r_hat with ref = a_hat (shared) or the rebuilt loop+1 (chained)."""
    L = cfg.loops_per_group
    g = cfg.group
    R = np.asarray(rot, dtype=np.float64)
    a_hat = dequantize(*enc.anchor, g)
    if loop == L - 1:
        return a_hat
    if not cfg.chained:
        qr, zr, sr, c = enc.resid[loop]
        return c[..., None] * a_hat + dequantize(qr, zr, sr, g) @ R
    ref = a_hat
    for l in range(L - 2, loop - 1, -1):
        qr, zr, sr, c = enc.resid[l]
        ref = c[..., None] * ref + dequantize(qr, zr, sr, g) @ R
    return ref


# ---------------------------------------------------------------------------
# byte layout of the packed cache
# ---------------------------------------------------------------------------

class Layout:
    """Byte layout of the packed cache (one flat buffer).

    Blocks are ordered [batch][KV head][K|V]; each block holds n_groups * L planes
    in global loop order (the anchor plane is the last of its group); each plane is
    ceil(max_ctx/64) tiles of 64 tokens.  A tile is
      codes block : 64 rows of d*bits/8 bytes; channel i sits at bit i*bits of its row
                    (little-endian within the row); bits is the plane's own width
      meta block  : 64 rows of 2*(d/group) bytes; byte 2j = E4M3 offset, 2j+1 = E4M3 scale
                    of channel group j
      c block     : residual planes only, 64 little-endian BF16 values.
    """

    def __init__(self, cfg: Config):
        self.cfg = cfg
        d, g = cfg.head_dim, cfg.group
        L = cfg.loops_per_group
        self.n_tiles = -(-cfg.max_ctx // TILE)
        self.a_row = d * cfg.anchor_bits // 8
        self.m_row = 2 * (d // g)
        self.a_tile = TILE * (self.a_row + self.m_row)
        self.r_rows = [d * cfg.rbits(l) // 8 for l in range(L - 1)]
        self.r_tiles = [TILE * (r + self.m_row + 2) for r in self.r_rows]
        self.group_bytes = self.n_tiles * (self.a_tile + sum(self.r_tiles))
        self.block_bytes = cfg.n_groups * self.group_bytes
        self.total_bytes = cfg.max_batch * cfg.n_kv_heads * 2 * self.block_bytes

    @property
    def r_row(self) -> int:
        """Residual code bytes per token row (uniform widths only)."""
        assert len(set(self.r_rows)) <= 1
        return self.r_rows[0]

    @property
    def r_tile(self) -> int:
        assert len(set(self.r_tiles)) <= 1
        return self.r_tiles[0]

    def plane_offset(self, b: int, h: int, x: int, loop: int) -> int:
        cfg = self.cfg
        L = cfg.loops_per_group
        k, l = divmod(loop, L)
        off = ((b * cfg.n_kv_heads + h) * 2 + x) * self.block_bytes + k * self.group_bytes
        off += self.n_tiles * sum(self.r_tiles[:l])      # residual planes of loops < l
        return off

    def bytes_per_token_head(self) -> Tuple[int, int]:
        """(anchor, residual) bytes per token per KV head per K|V (uniform widths)."""
        return self.a_row + self.m_row, self.r_row + self.m_row + 2

    def bytes_per_token_loop(self) -> List[int]:
        """Bytes per token per KV head per K|V of each local loop's plane (anchor last)."""
        return [r + self.m_row + 2 for r in self.r_rows] + [self.a_row + self.m_row]


def _pack_bits(codes: np.ndarray, bits: int) -> np.ndarray:
    """(..., d) integer codes -> (..., d*bits/8) bytes, channel i at bit i*bits."""
    per = 8 // bits
    c = codes.reshape(codes.shape[:-1] + (codes.shape[-1] // per, per)).astype(np.uint32)
    out = np.zeros(c.shape[:-1], dtype=np.uint32)
    for k in range(per):
        out |= c[..., k] << (k * bits)
    return out.astype(np.uint8)


def _unpack_bits(rows: np.ndarray, bits: int) -> np.ndarray:
    per = 8 // bits
    mask = (1 << bits) - 1
    r = rows.astype(np.int64)
    parts = [(r >> (k * bits)) & mask for k in range(per)]
    return np.stack(parts, axis=-1).reshape(rows.shape[:-1] + (rows.shape[-1] * per,))


def _meta_bytes(z: np.ndarray, s: np.ndarray) -> np.ndarray:
    m = np.stack([e4m3_encode(z), e4m3_encode(s)], axis=-1)
    return m.reshape(m.shape[:-2] + (m.shape[-2] * 2,))


def _plane_views(cache: np.ndarray, lay: Layout, off: int, l: int):
    """Views (codes, meta, c) of local loop l's plane as [n_tiles][64][row] arrays."""
    n = lay.n_tiles
    resid = l < lay.cfg.loops_per_group - 1
    row = lay.r_rows[l] if resid else lay.a_row
    tile = lay.r_tiles[l] if resid else lay.a_tile
    plane = cache[off: off + n * tile].reshape(n, tile)
    codes = plane[:, : TILE * row].reshape(n, TILE, row)
    meta = plane[:, TILE * row: TILE * (row + lay.m_row)].reshape(n, TILE, lay.m_row)
    c = plane[:, TILE * (row + lay.m_row):].reshape(n, TILE, 2) if resid else None
    return codes, meta, c


def write_tokens(cache: np.ndarray, lay: Layout, b: int, h: int, x: int, group_idx: int,
                 positions: np.ndarray, enc: Encoded) -> None:
    """Store the encoding of tokens (leading axis of ``enc`` arrays) at token slots ``positions``."""
    cfg = lay.cfg
    L = cfg.loops_per_group
    positions = np.asarray(positions)
    ti, tj = positions // TILE, positions % TILE
    for l in range(L):
        off = lay.plane_offset(b, h, x, group_idx * L + l)
        if l == L - 1:
            qa, za, sa = enc.anchor
            codes, meta, _ = _plane_views(cache, lay, off, l)
            codes[ti, tj] = _pack_bits(qa, cfg.anchor_bits)
            meta[ti, tj] = _meta_bytes(za, sa)
        else:
            qr, zr, sr, c = enc.resid[l]
            codes, meta, cb = _plane_views(cache, lay, off, l)
            codes[ti, tj] = _pack_bits(qr, cfg.rbits(l))
            meta[ti, tj] = _meta_bytes(zr, sr)
            cb[ti, tj] = bf16_bits(c).view(np.uint8).reshape(c.shape + (2,))


def read_tokens(cache: np.ndarray, lay: Layout, b: int, h: int, x: int, group_idx: int,
                n_tokens: int) -> Encoded:
    """Decode the stored codes and metadata of token slots 0..n_tokens-1."""
    cfg = lay.cfg
    L = cfg.loops_per_group
    nd = cfg.head_dim // cfg.group
    pos = np.arange(n_tokens)
    ti, tj = pos // TILE, pos % TILE
    anchor = None
    resid: List = [None] * (L - 1)
    for l in range(L):
        off = lay.plane_offset(b, h, x, group_idx * L + l)
        is_res = l < L - 1
        codes, meta, cb = _plane_views(cache, lay, off, l)
        m = meta[ti, tj].reshape(n_tokens, nd, 2)
        z, s = e4m3_decode(m[..., 0]), e4m3_decode(m[..., 1])
        if is_res:
            q = _unpack_bits(codes[ti, tj], cfg.rbits(l))
            cbits = cb[ti, tj].copy().view(np.uint16).reshape(n_tokens)
            resid[l] = (q, z, s, bf16_from_bits(cbits))
        else:
            q = _unpack_bits(codes[ti, tj], cfg.anchor_bits)
            anchor = (q, z, s)
    return Encoded(anchor, resid)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray, sm_scale: float) -> np.ndarray:
    """Softmax attention of one query vector over rows of keys/values."""
    s = (keys @ q) * sm_scale
    p = np.exp(s - s.max())
    return (p @ values) / p.sum()


def decode_attention(cache: np.ndarray, lay: Layout, loop: int, q: np.ndarray,
                     k_cur: np.ndarray, v_cur: np.ndarray, ctx_len: Sequence[int],
                     rot: np.ndarray, sm_scale: float,
                     heads: Optional[Sequence[Tuple[int, int]]] = None) -> np.ndarray:
    """Decode attention at global loop ``loop`` over the packed cache, brute force.

    q: (B, Hq, d); k_cur, v_cur: (B, Hkv, d) current-token K/V of this loop (BF16 values);
    ctx_len: tokens already in the cache per batch row; rot: (Hkv, 2, d, d).
    Every cached token's K and V are rebuilt in full (reconstruct), the current token
    is appended as the last entry, and plain softmax attention is taken per query head
    (query head hq reads KV head hq // (Hq/Hkv)).  ``heads`` restricts the work to a
    list of (b, hq); the other outputs are NaN.
    """
    cfg = lay.cfg
    B, Hq, d = q.shape
    G = Hq // cfg.n_kv_heads
    k_grp, l_loc = divmod(loop, cfg.loops_per_group)
    out = np.full((B, Hq, d), np.nan)
    todo = heads if heads is not None else [(b, hq) for b in range(B) for hq in range(Hq)]
    cache_kv = {}
    for b, hq in todo:
        h = hq // G
        if (b, h) not in cache_kv:
            n = int(ctx_len[b])
            kv = []
            for x in range(2):
                enc = read_tokens(cache, lay, b, h, x, k_grp, n)
                kv.append(reconstruct(enc, l_loc, rot[h, x], cfg))
            keys = np.concatenate([kv[0], k_cur[b, h][None, :]], axis=0)
            values = np.concatenate([kv[1], v_cur[b, h][None, :]], axis=0)
            cache_kv[(b, h)] = (keys, values)
        keys, values = cache_kv[(b, h)]
        out[b, hq] = attention(np.asarray(q[b, hq], dtype=np.float64), keys, values, sm_scale)
    return out


def decode_attention_factored(enc_k: Encoded, enc_v: Encoded, loop: int, q: np.ndarray,
                              k_cur: np.ndarray, v_cur: np.ndarray, rot_k: np.ndarray,
                              rot_v: np.ndarray, sm_scale: float, cfg: Config) -> np.ndarray:
    """The same attention for one query and one (b, KV head), rearranged the way a
    decode kernel evaluates it without rebuilding K/V: score = C*(q.a_hat) +
    sum_k gamma_k (R q).r_hat_k, output = (sum_j p_j C_j a_hat_j + R^T sum_j p_j
    sum_k gamma_k r_hat_k + p_cur v_cur) / sum p.  Shared anchor: C = c, one residual
    with gamma = 1.  Chained at loop l: C = prod_{m=l}^{L-2} c_m and gamma_k =
    prod_{m=l}^{k-1} c_m for k = l..L-2.  Used only as a self-check of ``attention``."""
    L = cfg.loops_per_group
    g = cfg.group
    q = np.asarray(q, dtype=np.float64)

    def terms(enc: Encoded):
        a_hat = dequantize(*enc.anchor, g)
        n = a_hat.shape[0]
        if loop == L - 1:
            return a_hat, np.ones(n), []
        ks = list(range(loop, L - 1)) if cfg.chained else [loop]
        coef = np.ones(n)
        parts = []
        for k in ks:
            qr, zr, sr, c = enc.resid[k]
            parts.append((coef.copy(), dequantize(qr, zr, sr, g)))
            coef = coef * c
        return a_hat, coef, parts

    a_k, C_k, parts_k = terms(enc_k)
    a_v, C_v, parts_v = terms(enc_v)
    u = np.asarray(rot_k, dtype=np.float64) @ q
    s = C_k * (a_k @ q)
    for gam, r_hat in parts_k:
        s = s + gam * (r_hat @ u)
    s_cur = float(np.asarray(k_cur, dtype=np.float64) @ q)
    s = np.concatenate([s, [s_cur]]) * sm_scale
    p = np.exp(s - s.max())
    pc, p_cur = p[:-1], p[-1]
    acc_a = (pc * C_v) @ a_v
    acc_r = np.zeros(q.shape[-1])
    for gam, r_hat in parts_v:
        acc_r = acc_r + (pc * gam) @ r_hat
    o = acc_a + np.asarray(rot_v, dtype=np.float64).T @ acc_r + p_cur * np.asarray(v_cur, np.float64)
    return o / p.sum()


# ---------------------------------------------------------------------------
# whole-cache helpers
# ---------------------------------------------------------------------------

def pack_context(kv: np.ndarray, rot: np.ndarray, cfg: Config, n_tokens: int,
                 cache: Optional[np.ndarray] = None, batches=None, heads=None) -> np.ndarray:
    """Encode tokens 0..n_tokens-1 of every loop into a fresh (or given) cache buffer.

    kv: (n_groups, L, 2, B, Hkv, >=n_tokens, d) values; rot: (Hkv, 2, d, d).
    ``batches``/``heads`` restrict the work to some (b, h) (other bytes stay untouched).
    """
    lay = Layout(cfg)
    if cache is None:
        cache = np.zeros(lay.total_bytes, dtype=np.uint8)
    L = cfg.loops_per_group
    bs = range(kv.shape[3]) if batches is None else batches
    hs = range(cfg.n_kv_heads) if heads is None else heads
    pos = np.arange(n_tokens)
    for b in bs:
        for h in hs:
            for x in range(2):
                for k in range(cfg.n_groups):
                    xs = np.asarray(kv[k, :, x, b, h, :n_tokens, :], dtype=np.float64)
                    enc = encode(xs, rot[h, x], cfg)
                    write_tokens(cache, lay, b, h, x, k, pos, enc)
    return cache

