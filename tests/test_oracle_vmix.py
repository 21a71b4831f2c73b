"""Pins of the oracle's two value precisions by token (SemKV, abstract: tokens
ranked by a model-internal score get one of two adjacent precisions; the page
names no indicator).  The reading: each 32-token group's tokens are stored in
descending order of their key magnitude E_t = sum_c min(floor(4096 |k_t,c|),
2^20) (ties to the lower position); the values of the first 8 n_vblk_hi
tokens in that order are quantized at bits_vhi bits, the rest at 2 bits, and
the extra high digits are stored for those tokens only.

* Order: a permutation per group, the same for every n_vblk_hi > 0 and the
  identity at n_vblk_hi = 0; it sorts a plain float64 sum of |k| wherever that
  sum separates neighbours; planted large-key tokens come first; it does not
  depend on the values.
* Codes: every value's code is the nearest level of its token group's grid
  (brute force), with 2^bits_vhi levels for the leading tokens and 4 else.
* Bytes: the brute-force unpackers rebuild every key and value code from the
  records, whose slots hold the tokens in the stored order.
* Attention over those bytes (in slot order) equals textbook attention; more
  high-precision tokens give a smaller value error.
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


def _quant(data, n, bits=4, k=None, v=None):
    return oracle.quantize(data["k"] if k is None else k, data["v"] if v is None else v,
                           W.tokens, data["pairs"], residual=W.residual, n_pairs_hi=W.n_pairs_hi,
                           bits_hi=W.bits_hi, io_dtype=W.io_dtype, n_vblk_hi=n, bits_vhi=bits)


def _vals(x):
    return kvq_synth.bits_to_f64(x[:, :, :W.tokens], W.io_dtype)


def _groups(qz):
    for b in range(W.batch):
        for kh in range(W.n_kv_heads):
            for g in range(qz.nq // 32):
                yield b, kh, g


def test_zero_high_tokens_is_the_two_bit_cache(data):
    a = _quant(data, 0)
    b = oracle.quantize(data["k"], data["v"], W.tokens, data["pairs"], residual=W.residual,
                        n_pairs_hi=W.n_pairs_hi, bits_hi=W.bits_hi, io_dtype=W.io_dtype)
    for f in ("vcodes", "vs", "vz", "kcodes", "ks", "kz"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    assert np.all(a.order == np.arange(32)) and a.vcodes.max() <= 3
    pa, pb = oracle.pack(a), oracle.pack(b)
    for f in ("k_lo", "k_hi", "k_meta", "v_codes", "v_meta"):
        assert np.array_equal(pa[f], pb[f])


def test_order_sorts_float_key_sums(data):
    kf = np.abs(_vals(data["k"]))
    qz = _quant(data, 1)
    for n in (2, 4):
        assert np.array_equal(_quant(data, n).order, qz.order)
    # the values do not enter the order
    assert np.array_equal(_quant(data, 2, v=data["v"][:, ::-1].copy()).order, qz.order)
    checked = 0
    for b, kh, g in _groups(qz):
        o = qz.order[b, kh, g].astype(np.int64)
        assert sorted(o) == list(range(32))
        e = kf[b, kh, 32 * g:32 * g + 32].sum(axis=1)[o]
        # the fixed point drops under 1/4096 per value, 1/32 per token
        for i in range(31):
            if abs(e[i] - e[i + 1]) > 1 / 16:
                assert e[i] > e[i + 1]
                checked += 1
    assert checked >= 300


def test_planted_tokens_lead(data):
    kf = _vals(data["k"])
    rng = np.random.default_rng(3)
    for _ in range(3):
        kp = kf.copy()
        picks = []
        for g in range(W.tokens // 32):
            p = rng.choice(32, 8, replace=False)
            picks.append(set(int(x) for x in p))
            kp[:, :, 32 * g + p] *= 16
        k = data["k"].copy()
        k[:, :, :W.tokens] = kvq_synth.to_bits(kp, W.io_dtype)
        qz = _quant(data, 1, k=k)
        for b, kh, g in _groups(qz):
            assert set(int(x) for x in qz.order[b, kh, g, :8]) == picks[g]


@pytest.mark.parametrize("n,bits", [(1, 4), (2, 3), (4, 4)])
def test_codes_are_nearest_levels(data, n, bits):
    qz = _quant(data, n, bits)
    vf = _vals(data["v"])
    f16 = lambda x: np.asarray(x, np.uint16).view(np.float16).astype(np.float64)
    for b, kh, g in _groups(qz):
        slot = np.argsort(qz.order[b, kh, g])
        for t in range(32):
            L = (1 << bits) - 1 if slot[t] < 8 * n else 3
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
    assert pk["v_hi"].shape[-1] == 8 + 64 * n
    q = data["q_dec"][:, :, 0]
    sm = float(np.float32(1.0 / np.sqrt(128.0)))
    out = oracle.attention(qz, q, sm)
    f16 = lambda x: float(np.uint16(x).view(np.float16))
    G, T = W.group_size, W.tokens
    vf = _vals(data["v"])
    for b in range(W.batch):
        for kh in range(W.n_kv_heads):
            # rows in the records' slot order; the ring in position order
            K = kvq_synth.bits_to_f64(data["k"][b, kh, :T], W.io_dtype).copy()
            V = vf[b, kh].copy()
            sal = sorted([int(p) for p in qz.pairs[b, kh, :W.n_pairs_hi]] +
                         [int(p) + 64 for p in qz.pairs[b, kh, :W.n_pairs_hi]])
            for g in range(qz.nq // 32):
                vc, vs, vz, order = brute.unpack_values(pk["v_codes"][b, kh, g],
                                                        pk["v_meta"][b, kh, g],
                                                        pk["v_hi"][b, kh, g])
                assert np.array_equal(order, qz.order[b, kh, g])
                assert np.array_equal(vc, qz.vcodes[b, kh, g][order])
                kc, _, s, z = brute.unpack_keys(pk["k_lo"][b, kh, g], pk["k_hi"][b, kh, g],
                                                pk["k_meta"][b, kh, g], sal, W.bits_hi)
                assert np.array_equal(kc, qz.kcodes[b, kh, g][:, order])
                for t in range(32):
                    for j in range(4):
                        V[32 * g + t, 32 * j:32 * j + 32] = (f16(vz[t, j]) + f16(vs[t, j]) *
                                                             vc[t, 32 * j:32 * j + 32])
                for c in range(128):
                    K[32 * g:32 * g + 32, c] = f16(z[c]) + f16(s[c]) * kc[c]
            for h in range(kh * G, kh * G + G):
                qf = kvq_synth.bits_to_f64(q[b, h], W.io_dtype)
                ref = brute.attention_textbook(qf, K, V, sm)
                assert np.max(np.abs(out[b, h] - ref)) < 1e-12


def test_more_high_tokens_smaller_value_error(data):
    vf = _vals(data["v"])
    f16 = lambda x: np.asarray(x, np.uint16).view(np.float16).astype(np.float64)
    errs = []
    for n in (0, 1, 2, 4):
        qz = _quant(data, n)
        nq = qz.nq
        vh = (f16(qz.vz)[..., None] + f16(qz.vs)[..., None] *
              qz.vcodes.reshape(*qz.vcodes.shape[:4], 4, 32)).reshape(vf.shape[0], vf.shape[1], -1, 128)
        errs.append(np.abs(vh[:, :, :nq] - vf[:, :, :nq]).mean())
    assert errs[0] > errs[1] > errs[2] > errs[3]
