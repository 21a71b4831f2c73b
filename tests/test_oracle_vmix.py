"""Pins of the oracle's two value precisions (SemKV, abstract: tokens ranked by
a model-internal score get one of two adjacent precisions; the page names no
indicator).  The reading: per 32-token group the n_vblk_hi of the four 8-token
blocks with the largest fixed-point value magnitude are quantized at bits_vhi
bits, the rest at 2 bits; the extra high digits are stored for kept blocks
only.

* Selection: the kept blocks are the top ones by a plain float64 sum of |v|
  wherever that sum separates them; a planted block is kept first; the kept
  sets are nested in n_vblk_hi; n_vblk_hi = 0 reproduces the 2-bit cache.
* Codes: every value's code is the nearest level of its token group's grid
  (brute force), with 2^bits_vhi levels in kept blocks and 4 elsewhere.
* Bytes: the brute-force unpacker rebuilds every code from v_codes + v_hi.
* Attention over those bytes equals textbook attention; more kept blocks
  give a smaller value error.
"""
import numpy as np
import pytest

import kvq_synth
import oracle
from oracle import brute

W = kvq_synth.Workload("vmix", 2, 4, 2, 300, n_qry=8, io_dtype="bf16", outliers="pct2x10",
                       n_pairs_hi=6, residual=64, seed=71)


@pytest.fixture(scope="module")
def data():
    d = kvq_synth.generate(W)
    _, pairs = oracle.select(d["q_sel"], d["k"], W.tokens, W.n_kv_heads, W.io_dtype)
    d["pairs"] = pairs
    return d


def _quant(data, n, bits=4, v=None):
    return oracle.quantize(data["k"], data["v"] if v is None else v, W.tokens, data["pairs"],
                           residual=W.residual, n_pairs_hi=W.n_pairs_hi, bits_hi=W.bits_hi,
                           io_dtype=W.io_dtype, n_vblk_hi=n, bits_vhi=bits)


def _vals(data, v=None):
    return kvq_synth.bits_to_f64((data["v"] if v is None else v)[:, :, :W.tokens], W.io_dtype)


def test_zero_kept_blocks_is_the_two_bit_cache(data):
    a = _quant(data, 0)
    b = oracle.quantize(data["k"], data["v"], W.tokens, data["pairs"], residual=W.residual,
                        n_pairs_hi=W.n_pairs_hi, bits_hi=W.bits_hi, io_dtype=W.io_dtype)
    for f in ("vcodes", "vs", "vz"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    assert np.all(a.vblk == 0) and a.vcodes.max() <= 3


def test_selection_matches_float_sums_and_is_nested(data):
    vf = np.abs(_vals(data))
    checked = 0
    prev = None
    for n in (1, 2, 3):
        qz = _quant(data, n)
        for b in range(W.batch):
            for kh in range(W.n_kv_heads):
                for g in range(qz.nq // 32):
                    e = vf[b, kh, 32 * g:32 * g + 32].reshape(4, 8 * 128).sum(axis=1)
                    order = np.argsort(-e, kind="stable")
                    srt = e[order]
                    mask = int(qz.vblk[b, kh, g])
                    assert bin(mask).count("1") == n
                    if prev is not None:
                        assert mask & prev[b, kh, g] == prev[b, kh, g]
                    # the fixed point drops under 1/4096 per value, 0.25 per block
                    if srt[n - 1] - srt[n] < 0.5:
                        continue
                    assert mask == sum(1 << int(k) for k in order[:n])
                    checked += 1
        prev = qz.vblk.copy()
    assert checked >= 20


def test_planted_block_is_kept(data):
    vf = _vals(data)
    for blk in range(4):
        vp = vf.copy()
        for g in range(W.tokens // 32):
            vp[:, :, 32 * g + 8 * blk:32 * g + 8 * blk + 8] *= 16
        v = data["v"].copy()
        v[:, :, :W.tokens] = kvq_synth.to_bits(vp, W.io_dtype)
        qz = _quant(data, 1, v=v)
        assert np.all(qz.vblk[:, :, :qz.nq // 32] == (1 << blk))


@pytest.mark.parametrize("n,bits", [(1, 4), (2, 3), (4, 4)])
def test_codes_are_nearest_levels(data, n, bits):
    qz = _quant(data, n, bits)
    vf = _vals(data)
    f16 = lambda x: np.asarray(x, np.uint16).view(np.float16).astype(np.float64)
    for b in range(W.batch):
        for kh in range(W.n_kv_heads):
            for g in range(qz.nq // 32):
                mask = int(qz.vblk[b, kh, g])
                for t in range(32):
                    L = (1 << bits) - 1 if (mask >> (t // 8)) & 1 else 3
                    for j in range(4):
                        s = f16(qz.vs[b, kh, g, t, j])
                        z = f16(qz.vz[b, kh, g, t, j])
                        x = vf[b, kh, 32 * g + t, 32 * j:32 * j + 32]
                        code = qz.vcodes[b, kh, g, t, 32 * j:32 * j + 32].astype(np.int64)
                        assert code.max() <= L
                        if s == 0:
                            continue
                        want, margin = brute.nearest_level(x, s, z, L)
                        ok = margin > 1e-6 * s
                        assert np.array_equal(code[ok], want[ok])


@pytest.mark.parametrize("n,bits", [(1, 4), (2, 3), (3, 4)])
def test_packed_bytes_and_attention(data, n, bits):
    qz = _quant(data, n, bits)
    pk = oracle.pack(qz)
    assert pk["v_hi"].shape[-1] == 4 + 64 * n
    q = data["q_dec"][:, :, 0]
    sm = float(np.float32(1.0 / np.sqrt(128.0)))
    out = oracle.attention(qz, q, sm)
    f16 = lambda x: float(np.uint16(x).view(np.float16))
    G, T = W.group_size, W.tokens
    for b in range(W.batch):
        for kh in range(W.n_kv_heads):
            K = np.zeros((T, 128))
            V = _vals(data)[b, kh].copy()
            sal = sorted([int(p) for p in qz.pairs[b, kh, :W.n_pairs_hi]] +
                         [int(p) + 64 for p in qz.pairs[b, kh, :W.n_pairs_hi]])
            K[:] = kvq_synth.bits_to_f64(data["k"][b, kh, :T], W.io_dtype)
            for g in range(qz.nq // 32):
                assert int(pk["v_hi"][b, kh, g, 0]) == int(qz.vblk[b, kh, g])
                vc, vs, vz = brute.unpack_values(pk["v_codes"][b, kh, g], pk["v_meta"][b, kh, g],
                                                 pk["v_hi"][b, kh, g])
                assert np.array_equal(vc, qz.vcodes[b, kh, g])
                for t in range(32):
                    for j in range(4):
                        V[32 * g + t, 32 * j:32 * j + 32] = (f16(vz[t, j]) + f16(vs[t, j]) *
                                                             vc[t, 32 * j:32 * j + 32])
                codes, _, s, z = brute.unpack_keys(pk["k_lo"][b, kh, g], pk["k_hi"][b, kh, g],
                                                   pk["k_meta"][b, kh, g], sal, W.bits_hi)
                for c in range(128):
                    K[32 * g:32 * g + 32, c] = f16(z[c]) + f16(s[c]) * codes[c]
            for h in range(kh * G, kh * G + G):
                qf = kvq_synth.bits_to_f64(q[b, h], W.io_dtype)
                ref = brute.attention_textbook(qf, K, V, sm)
                assert np.max(np.abs(out[b, h] - ref)) < 1e-12


def test_more_kept_blocks_smaller_value_error(data):
    vf = _vals(data)
    f16 = lambda x: np.asarray(x, np.uint16).view(np.float16).astype(np.float64)
    errs = []
    for n in (0, 1, 2, 4):
        qz = _quant(data, n)
        nq = qz.nq
        vh = (f16(qz.vz)[..., None] + f16(qz.vs)[..., None] *
              qz.vcodes.reshape(*qz.vcodes.shape[:4], 4, 32)).reshape(vf.shape[0], vf.shape[1], -1, 128)
        errs.append(np.abs(vh[:, :, :nq] - vf[:, :, :nq]).mean())
    assert errs[0] > errs[1] > errs[2] > errs[3]
