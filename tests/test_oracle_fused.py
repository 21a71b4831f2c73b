"""Pins of the oracle's attention for a call that appends a token and decodes
in one step (PM-KVQ, key_machinery: new tokens are held at 16 bits first and
quantized later).  The reading: all T tokens after the append are attended,
with the quantized prefix of before the append, n_q(T-1), so a group that the
append packs is attended at 16 bits in that call.

* The identity the oracle uses, n_q(T, R+1) = n_q(T-1, R), holds for every T
  and R tried (closed form of n_q).
* Where the append packs no group the result is plain attention, bit for bit.
* Where it packs one, the result is textbook softmax attention over the
  first n_q(T-1) tokens rebuilt from the packed bytes by the brute-force
  unpackers and the remaining tokens at 16 bits, and it differs from the
  attention that reads the new group quantized.
* The attention of a one-launch call computed from the cache it finds
  (before the append) equals the one above on plain layouts, bit for bit,
  at steps with and without a pack.  On progressive layouts, at a step whose
  pack shrinks the groups crossing the window edges, it is textbook
  attention over the groups at their former widths plus 16-bit tokens, and
  differs from attention over the cache after the append.
"""
import numpy as np
import pytest

import kvq_synth
import oracle
from oracle import brute

SM = float(np.float32(1.0 / np.sqrt(128.0)))


def test_quantized_prefix_identity():
    for R in (32, 64, 96, 128):
        for T in range(1, 700):
            want = 32 * (max(0, T - 1 - R) // 32)
            assert oracle.n_quant(T - 1, R) == want
            assert oracle.n_quant(T, R + 1) == want


def _case(T, seed):
    w = kvq_synth.Workload("fused", 1, 4, 1, T, n_qry=8, io_dtype="bf16", outliers="pct2x10",
                           n_pairs_hi=6, residual=64, seed=seed)
    d = kvq_synth.generate(w)
    _, pairs = oracle.select(d["q_sel"], d["k"], T, 1, "bf16")
    qz = oracle.quantize(d["k"], d["v"], T, pairs, residual=64, n_pairs_hi=6, bits_hi=4,
                         io_dtype="bf16")
    return w, d, qz


@pytest.mark.parametrize("T", [40, 64 + 33, 64 + 32 * 4 + 17])
def test_no_group_packed_is_plain_attention(T):
    assert oracle.n_quant(T, 64) == oracle.n_quant(T - 1, 64)
    w, d, qz = _case(T, 5)
    q = d["q_dec"][:, :, 0]
    assert np.array_equal(oracle.attention_after_append(qz, q, SM), oracle.attention(qz, q, SM))


@pytest.mark.parametrize("T", [64 + 32, 64 + 32 * 5])
def test_packed_group_attended_at_sixteen_bits(T):
    R = 64
    assert oracle.n_quant(T, R) == oracle.n_quant(T - 1, R) + 32
    w, d, qz = _case(T, 6)
    pk = oracle.pack(qz)
    q = d["q_dec"][:, :, 0]
    got = oracle.attention_after_append(qz, q, SM)
    nq = oracle.n_quant(T - 1, R)
    f16 = lambda x: float(np.uint16(x).view(np.float16))
    sal = sorted([int(p) for p in qz.pairs[0, 0, :6]] + [int(p) + 64 for p in qz.pairs[0, 0, :6]])
    K = kvq_synth.bits_to_f64(d["k"][0, 0, :T], "bf16").copy()
    V = kvq_synth.bits_to_f64(d["v"][0, 0, :T], "bf16").copy()
    for g in range(nq // 32):
        codes, _, s, z = brute.unpack_keys(pk["k_lo"][0, 0, g], pk["k_hi"][0, 0, g],
                                           pk["k_meta"][0, 0, g], sal, 4)
        for c in range(128):
            K[32 * g:32 * g + 32, c] = f16(z[c]) + f16(s[c]) * codes[c]
        vc, vs, vz, _ = brute.unpack_values(pk["v_codes"][0, 0, g], pk["v_meta"][0, 0, g])
        for t in range(32):
            for j in range(4):
                V[32 * g + t, 32 * j:32 * j + 32] = f16(vz[t, j]) + f16(vs[t, j]) * vc[t, 32 * j:32 * j + 32]
    for h in range(4):
        ref = brute.attention_textbook(kvq_synth.bits_to_f64(q[0, h], "bf16"), K, V, SM)
        assert np.max(np.abs(got[0, h] - ref)) < 1e-12
    assert not np.array_equal(got, oracle.attention(qz, q, SM))


@pytest.mark.parametrize("T", [64 + 33, 64 + 32, 64 + 32 * 5, 64 + 32 * 4 + 17])
def test_one_launch_from_the_cache_before_equals_after_append(T):
    w = kvq_synth.Workload("fused", 1, 4, 1, T, n_qry=8, io_dtype="bf16", outliers="pct2x10",
                           n_pairs_hi=6, residual=64, seed=7)
    d = kvq_synth.generate(w)
    _, pairs = oracle.select(d["q_sel"], d["k"], T, 1, "bf16")
    kw = dict(residual=64, n_pairs_hi=6, bits_hi=4, io_dtype="bf16")
    before = oracle.quantize(d["k"], d["v"], T - 1, pairs, **kw)
    after = oracle.quantize(d["k"], d["v"], T, pairs, **kw)
    q = d["q_dec"][:, :, 0]
    assert np.array_equal(oracle.attention_one_launch(before, q, SM),
                          oracle.attention_after_append(after, q, SM))


def test_one_launch_progressive_reads_the_former_widths():
    # windows 2 (8-bit) / 5 (>= 4-bit), R = 64: the step T - 1 -> T packs
    # group 9, and the pack shrinks group 7 (reaching age 2: 8 -> 4 bits) and
    # group 4 (reaching age 5: 4 -> 2 bits), which this call still reads at 8
    # and 4 bits
    R, w8, w4 = 64, 2, 5
    T = R + 32 * 10
    assert oracle.n_quant(T, R) == oracle.n_quant(T - 1, R) + 32
    w = kvq_synth.Workload("fprog", 1, 4, 2, T, n_qry=8, io_dtype="bf16", outliers="pct2x10",
                           n_pairs_hi=6, residual=R, seed=8)
    d = kvq_synth.generate(w)
    _, pairs = oracle.select(d["q_sel"], d["k"], T, w.n_kv_heads, "bf16")
    kw = dict(residual=R, n_pairs_hi=6, bits_hi=4, io_dtype="bf16", prog_w8=w8, prog_w4=w4)
    before = oracle.quantize(d["k"], d["v"], T - 1, pairs, **kw)
    after = oracle.quantize(d["k"], d["v"], T, pairs, **kw)
    ngb = before.nq // 32
    assert ngb == 9
    widths = [oracle.prog_width(ngb - 1 - g, w8, w4) for g in range(ngb)]
    assert widths[7] == 8 and widths[4] == 4
    assert oracle.prog_width(ngb - 7, w8, w4) == 4 and oracle.prog_width(ngb - 4, w8, w4) == 2
    q = d["q_dec"][:, :, 0]
    got = oracle.attention_one_launch(before, q, SM)
    f16 = lambda b: np.asarray(b, np.uint16).view(np.float16).astype(np.float64)
    for kh in range(w.n_kv_heads):
        K = kvq_synth.bits_to_f64(d["k"][0, kh, :T], "bf16").copy()
        V = kvq_synth.bits_to_f64(d["v"][0, kh, :T], "bf16").copy()
        for g in range(ngb):
            s, z = f16(before.ks[0, kh, g]), f16(before.kz[0, kh, g])
            K[32 * g:32 * g + 32] = (z[:, None] + s[:, None] * before.kcodes[0, kh, g]).T
            vs, vz = f16(before.vs[0, kh, g]), f16(before.vz[0, kh, g])
            V[32 * g:32 * g + 32] = (vz.repeat(32, axis=1)
                                     + vs.repeat(32, axis=1) * before.vcodes[0, kh, g])
        for h in range(kh * 2, kh * 2 + 2):
            ref = brute.attention_textbook(kvq_synth.bits_to_f64(q[0, h], "bf16"), K, V, SM)
            assert np.max(np.abs(got[0, h] - ref)) < 1e-12
    assert not np.array_equal(got, oracle.attention_after_append(after, q, SM))
