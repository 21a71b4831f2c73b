"""Brute-force checks that pin the C oracle to definitions outside itself.

Test infrastructure only.  Every routine here takes a different route to the
quantity the oracle computes:

* ``select_exhaustive``: the saliency of a RoPE pair as the mean, over every
  (selection query, prefill key) combination of the head group, of the
  product of the two pair norms (PN-Mix, abstract and transcript), in fp64,
  ranked with a stable argsort — no factorization and no fixed point.
* ``nearest_level``: for an affine grid z + s*q, q = 0..L (SemKV, abstract),
  the code whose level is nearest in fp64, by exhaustive search.
* ``unpack_keys`` / ``unpack_values``: read the byte records bit by bit from
  the layout documented in include/kvq.h, written without the oracle's
  packing loops.
* ``attention_textbook``: softmax(scale * K q) . V with numpy in fp64.
"""
from __future__ import annotations

import numpy as np

GS = 32
D = 128


def select_exhaustive(q_sel: np.ndarray, k: np.ndarray, G: int):
    """q_sel [Hq][n_qry][128], k [Hkv][T][128] (fp64 values, one sequence).
    Returns (mean scores [Hkv][64], ranking [Hkv][64])."""
    Hkv = k.shape[0]
    scores = np.zeros((Hkv, 64))
    ranks = np.zeros((Hkv, 64), np.int64)
    for kh in range(Hkv):
        qn = np.hypot(q_sel[kh * G:(kh + 1) * G, :, :64],
                      q_sel[kh * G:(kh + 1) * G, :, 64:]).reshape(-1, 64)
        kn = np.hypot(k[kh, :, :64], k[kh, :, 64:])
        for j in range(64):
            scores[kh, j] = np.outer(qn[:, j], kn[:, j]).mean()
        ranks[kh] = np.argsort(-scores[kh], kind="stable")
    return scores, ranks


def nearest_level(x: np.ndarray, s: float, z: float, L: int):
    """Codes minimizing |x - (z + s*q)| over q = 0..L (fp64), and the distance
    from each x to the midpoint between its two nearest levels (to skip
    inputs that sit on a rounding boundary)."""
    levels = z + s * np.arange(L + 1, dtype=np.float64)
    d = np.abs(x[:, None] - levels[None, :])
    q = d.argmin(axis=1)
    ds = np.sort(d, axis=1)
    margin = ds[:, 1] - ds[:, 0] if L > 0 else np.full(len(x), np.inf)
    return q, margin


def _code(word: int, pos: int) -> int:
    return (int(word) >> (2 * pos)) & 3


def _pos(c: int) -> int:
    # bits 0 and 1 of c exchanged, as the layout specifies
    b0, b1 = c & 1, (c >> 1) & 1
    return (c & ~3) | (b0 << 1) | b1


def _tile_index(t: int) -> int:
    # inverse of "record e = 16T + r holds token 8(r//4) + 4T + r%4"
    T = (t // 4) % 2
    r = 4 * (t // 8) + t % 4
    return 16 * T + r


def _bit1_pos(c: int) -> int:
    # the bit of run channel c in a 1-bit word of the dense layout, tile half
    # T = 0 (T = 1: the same + 16; include/kvq.h, k_lo)
    return 4 * (c & 1) + ((c >> 1) & 1) + 8 * ((c >> 2) & 1) + 2 * (c >> 3)


def unpack_keys_dense1(k_lo, k_meta, one_bit_pairs):
    """One group record of the dense 1-bit layout -> (codes [128][32],
    s_bits [128], z_bits [128]).  Plane order: the 2-bit channels ascending
    (wl) and the 1-bit ones (ol), each a pair's first channel before the
    second ones; chunk kq = 2-bit run wl[16kq ..] then 1-bit run ol[16kq ..]."""
    one = set(int(p) for p in one_bit_pairs)
    wl = [c for c in range(D) if c % 64 not in one]
    ol = [c for c in range(D) if c % 64 in one]
    assert len(wl) == len(ol) == 64
    words = np.asarray(k_lo, np.uint32)
    codes = np.zeros((D, GS), np.int64)
    for t in range(GS):
        T, r = divmod(_tile_index(t), 16)
        for kq in range(4):
            w = int(words[(kq * 2 + T) * 16 + r])
            h = int(words[128 + kq * 16 + r]) >> (16 * T)
            for c in range(16):
                codes[wl[16 * kq + c], t] = _code(w, _pos(c))
                codes[ol[16 * kq + c], t] = (h >> _bit1_pos(c)) & 1
    meta = np.asarray(k_meta, np.uint16).reshape(8, 2, 16)
    s = np.zeros(D, np.uint16)
    z = np.zeros(D, np.uint16)
    for kq in range(4):
        for c in range(16):
            s[wl[16 * kq + c]], z[wl[16 * kq + c]] = meta[2 * kq, 0, c], meta[2 * kq, 1, c]
            s[ol[16 * kq + c]], z[ol[16 * kq + c]] = meta[2 * kq + 1, 0, c], meta[2 * kq + 1, 1, c]
    return codes, s, z


def unpack_keys(k_lo, k_hi, k_meta, salient: list[int], bits_hi: int):
    """One group record -> (codes [128][32], raw16 [len(salient)][32] or None,
    s_bits [128], z_bits [128]).  `salient` = ascending salient channels."""
    codes = np.zeros((D, GS), np.int64)
    for t in range(GS):
        e = _tile_index(t)
        T, r = divmod(e, 16)
        for c in range(D):
            w = c // 16
            kq, u = divmod(w, 2)
            word = k_lo[((kq * 2 + u) * 2 + T) * 16 + r]
            codes[c, t] = _code(word, _pos(c % 16))
    raw = None
    if salient and bits_hi == 4:
        words = np.frombuffer(np.asarray(k_hi, np.uint8).tobytes(), np.uint32)
        for t in range(GS):
            e = _tile_index(t)
            for d, c in enumerate(salient):
                codes[c, t] += 4 * _code(words[e], _pos(d))
    elif salient and bits_hi == 16:
        vals = np.frombuffer(np.asarray(k_hi, np.uint8).tobytes(), np.uint16)
        n = len(salient)
        raw = np.zeros((n, GS), np.uint16)
        for t in range(GS):
            e = _tile_index(t)
            raw[:, t] = vals[e * n:(e + 1) * n]
    meta = np.asarray(k_meta, np.uint16).reshape(8, 2, 16)  # run, (scale, zero), channel
    return codes, raw, meta[:, 0].reshape(D).copy(), meta[:, 1].reshape(D).copy()


def _v_digits(words, base: int, nslot: int, slot: int):
    """Digits [8 tokens][128] of one 8-token block stored in the v_codes word
    format: word base + (j * nslot + slot) * 16 + c."""
    d = np.zeros((8, D), np.int64)
    for j in range(4):
        for c in range(16):
            word = int(words[base + (j * nslot + slot) * 16 + c])
            for i in range(8):
                d[i, 32 * j + c] = _code(word & 0xFFFF, _pos(i))
                d[i, 32 * j + 16 + c] = _code(word >> 16, _pos(i))
    return d


def unpack_values(v_codes, v_meta, v_hi=None):
    """One group record -> (codes [32 slots][128], s_bits [32][4],
    z_bits [32][4], order [32]).  Without a v_hi record slot = position and
    every code is its two-bit digit.  With one (8 header words holding the
    32 order bytes slot -> position, then the high digits of the first
    n 8-slot blocks), the codes of those blocks are low digit + 4 * high
    digit."""
    codes = np.zeros((GS, D), np.int64)
    for kq in range(4):
        codes[8 * kq:8 * kq + 8] = _v_digits(v_codes, 0, 4, kq)
    order = np.arange(GS)
    if v_hi is not None and len(v_hi) > 0:
        nslot = (len(v_hi) - 8) // 64
        order = np.frombuffer(np.asarray(v_hi[:8], np.uint32).tobytes(), np.uint8).astype(np.int64)
        for kq in range(nslot):
            codes[8 * kq:8 * kq + 8] += 4 * _v_digits(v_hi, 8, nslot, kq)
    meta = np.asarray(v_meta, np.uint16).reshape(2, 4, GS)
    return codes, meta[0].T.copy(), meta[1].T.copy(), order


def attention_textbook(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                       sm_scale: float) -> np.ndarray:
    """q [128], K/V [T][128] fp64 -> softmax(sm_scale * K q) . V."""
    logits = sm_scale * (K @ q)
    w = np.exp(logits - logits.max())
    return (w / w.sum()) @ V
