"""Pins of the oracle's in-place precision shrink (PM-KVQ review,
key_machinery: 2b-bit codes become b-bit codes with the zero point kept and
the step multiplied by 2^b + 1).

* The shift form the review prints and the definition round(X / (2^b + 1))
  agree on every input of every transition it names (2b = 16, 8, 4) and on
  2 -> 1, against exact rational rounding.
* On a quantized cache, every shrunk channel dequantizes to the nearest
  level of the new grid z + 5 s q, q = 0..3, to the value its old code
  dequantized to (brute force over levels), held as the 4-bit code 5 q under
  the unchanged scale; everything outside the shrunk channels and groups is
  untouched.
* Attention over the shrunk cache equals textbook attention over its bytes.
"""
from fractions import Fraction

import numpy as np
import pytest

import kvq_synth
import oracle
from oracle import brute


def _round_exact(x, d):
    f = Fraction(x, d)
    fl = f.numerator // f.denominator
    return fl + (1 if f - fl > Fraction(1, 2) else 0)  # d odd: no tie


@pytest.mark.parametrize("b", [1, 2, 4, 8])
def test_shift_form_equals_rounding_exhaustively(b):
    d = (1 << b) + 1
    for x in range(1 << (2 * b)):
        want = _round_exact(x, d)
        assert oracle.shrink_code(x, b) == want, x
        assert oracle.ers(x, b) == want, x
        assert 0 <= want <= (1 << b) - 1


W = kvq_synth.Workload("shrink", 1, 4, 2, 300, n_qry=8, io_dtype="bf16", outliers="pct2x10",
                       n_pairs_hi=6, residual=64, seed=41)


def _setup():
    d = kvq_synth.generate(W)
    _, pairs = oracle.select(d["q_sel"], d["k"], W.tokens, W.n_kv_heads, W.io_dtype)
    qz = oracle.quantize(d["k"], d["v"], W.tokens, pairs, residual=W.residual,
                         n_pairs_hi=W.n_pairs_hi, bits_hi=W.bits_hi, io_dtype=W.io_dtype)
    return d, pairs, qz


def _f16(b):
    return float(np.uint16(b).view(np.float16))


def test_shrunk_codes_are_nearest_new_levels():
    d, pairs, qz = _setup()
    ng = qz.nq // 32
    assert ng >= 5
    g0, g1 = 1, 4
    sh = oracle.shrink(qz, g0, g1)
    for b in range(W.batch):
        for kh in range(W.n_kv_heads):
            sal = {int(p) for p in pairs[b, kh, :W.n_pairs_hi]}
            for g in range(ng):
                for c in range(128):
                    old, new = qz.kcodes[b, kh, g, c], sh.kcodes[b, kh, g, c]
                    assert sh.kz[b, kh, g, c] == qz.kz[b, kh, g, c]
                    if not (g0 <= g < g1 and c % 64 in sal):
                        assert np.array_equal(old, new)
                        assert sh.ks[b, kh, g, c] == qz.ks[b, kh, g, c]
                        continue
                    s_old, z = _f16(qz.ks[b, kh, g, c]), _f16(qz.kz[b, kh, g, c])
                    assert sh.ks[b, kh, g, c] == qz.ks[b, kh, g, c]
                    x_hat = z + s_old * old.astype(np.float64)
                    q, _ = brute.nearest_level(x_hat, 5 * s_old, z, 3)
                    assert np.array_equal(new, 5 * q)
                    # the dequantized value is the new grid's level, exactly
                    assert np.array_equal(z + s_old * new.astype(np.float64),
                                          z + (5 * s_old) * q.astype(np.float64))
    # before the shrink the codes used the whole 4-bit range
    assert set(np.unique(qz.kcodes[:, :, g0:g1])) - {0, 5, 10, 15}
    assert set(np.unique(sh.kcodes[:, :, g0:g1])) <= {0, 1, 2, 3, 5, 10, 15}


def test_shrink_range_is_clamped_to_quantized_groups():
    _, _, qz = _setup()
    ng = qz.nq // 32
    a, b = oracle.shrink(qz, 0, ng), oracle.shrink(qz, -5, ng + 100)
    assert np.array_equal(a.kcodes, b.kcodes) and np.array_equal(a.ks, b.ks)
    c = oracle.shrink(qz, ng, ng + 3)
    assert np.array_equal(c.kcodes, qz.kcodes) and np.array_equal(c.ks, qz.ks)


def test_attention_over_shrunk_bytes_matches_textbook():
    d, pairs, qz = _setup()
    sh = oracle.shrink(qz, 0, qz.nq // 32)
    pk = oracle.pack(sh)
    q = d["q_dec"][:, :, 0]
    sm = float(np.float32(1.0 / np.sqrt(128.0)))
    out = oracle.attention(sh, q, sm)
    G = W.group_size
    T = W.tokens
    for b in range(W.batch):
        for kh in range(W.n_kv_heads):
            sal = sorted([int(p) for p in pairs[b, kh, :W.n_pairs_hi]] +
                         [int(p) + 64 for p in pairs[b, kh, :W.n_pairs_hi]])
            K = kvq_synth.bits_to_f64(d["k"][b, kh, :T], W.io_dtype).copy()
            V = kvq_synth.bits_to_f64(d["v"][b, kh, :T], W.io_dtype).copy()
            for g in range(sh.nq // 32):
                codes, _, s, z = brute.unpack_keys(pk["k_lo"][b, kh, g], pk["k_hi"][b, kh, g],
                                                   pk["k_meta"][b, kh, g], sal, 4)
                assert set(np.unique(codes[sal])) <= {0, 5, 10, 15}
                for c in range(128):
                    K[32 * g:32 * g + 32, c] = _f16(z[c]) + _f16(s[c]) * codes[c]
                vc, vs, vz, _ = brute.unpack_values(pk["v_codes"][b, kh, g], pk["v_meta"][b, kh, g])
                for t in range(32):
                    for j in range(4):
                        V[32 * g + t, 32 * j:32 * j + 32] = (_f16(vz[t, j]) + _f16(vs[t, j]) *
                                                             vc[t, 32 * j:32 * j + 32])
            for h in range(kh * G, kh * G + G):
                qf = kvq_synth.bits_to_f64(q[b, h], W.io_dtype)
                ref = brute.attention_textbook(qf, K, V, sm)
                assert np.max(np.abs(out[b, h] - ref)) < 1e-12
