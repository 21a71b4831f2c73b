"""Pins of the oracle's byte packing (against an independent bit-level
unpacker of the documented layout) and of its attention (against textbook
softmax attention with numpy, closed-form special cases and the
log-sum-exp identity)."""
import numpy as np
import pytest

import kvq_synth
import oracle
from oracle import brute


def _setup(w, T=None):
    d = kvq_synth.generate(w)
    T = w.tokens if T is None else T
    _, pairs = oracle.select(d["q_sel"], d["k"], w.tokens, w.n_kv_heads, w.io_dtype)
    qz = oracle.quantize(d["k"], d["v"], T, pairs, residual=w.residual,
                         n_pairs_hi=w.n_pairs_hi, bits_hi=w.bits_hi, io_dtype=w.io_dtype,
                         n_pairs_lo1=w.n_pairs_lo1)
    return d, pairs, qz


def _salient(pairs_row, n_hi):
    return sorted([int(p) for p in pairs_row[:n_hi]] + [int(p) + 64 for p in pairs_row[:n_hi]])


VARIANTS = [
    kvq_synth.WORKLOADS[0],
    kvq_synth.Workload("b", 2, 4, 2, 200, n_qry=8, io_dtype="bf16", outliers="pct2x10",
                       n_pairs_hi=6, residual=64, seed=5),
    kvq_synth.Workload("c", 1, 2, 1, 160, n_qry=8, io_dtype="bf16", n_pairs_hi=6,
                       bits_hi=16, residual=32, seed=6),
    kvq_synth.Workload("d", 1, 2, 1, 130, n_qry=8, io_dtype="fp16", n_pairs_hi=0,
                       residual=32, seed=7),
    # the 1.5-bit point: 32 pairs at 2 bits, the 32 lowest-ranked at 1 bit
    kvq_synth.Workload("e", 1, 4, 2, 170, n_qry=8, io_dtype="bf16", outliers="pct2x10",
                       n_pairs_hi=0, n_pairs_lo1=32, residual=32, seed=8),
    # 4-bit salient pairs, 2-bit middle, 1-bit tail
    kvq_synth.Workload("f", 1, 4, 1, 140, n_qry=8, io_dtype="fp16", n_pairs_hi=6,
                       n_pairs_lo1=16, residual=64, seed=9),
]


def _unpack(w, pk, pairs, b, kh, g, sal):
    """A key record read back bit by bit: the dense 1-bit layout (the
    1.5-bit point) or the 2-bit slot layout."""
    if oracle.dense1(w.n_pairs_hi, w.n_pairs_lo1):
        codes, s, z = brute.unpack_keys_dense1(pk["k_lo"][b, kh, g], pk["k_meta"][b, kh, g],
                                               pairs[b, kh, 64 - w.n_pairs_lo1:])
        return codes, None, s, z
    return brute.unpack_keys(pk["k_lo"][b, kh, g], pk["k_hi"][b, kh, g], pk["k_meta"][b, kh, g],
                             sal, w.bits_hi)


def test_dense_one_bit_layout_is_smaller():
    # the 1.5-bit point stores one bit per 1-bit code: 768 bytes of key codes
    # per group against 1024 for the 2.0-bit point; every bit position of a
    # 1-bit half-word is used once
    assert sorted(brute._bit1_pos(c) for c in range(16)) == list(range(16))
    w2 = VARIANTS[-2].replace(n_pairs_lo1=0)
    for w, words in ((VARIANTS[-2], 192), (w2, 256)):
        d, pairs, qz = _setup(w)
        assert oracle.pack(qz)["k_lo"].shape[-1] == words
    assert oracle.dense1(0, 32) and not oracle.dense1(6, 32) and not oracle.dense1(0, 16)


@pytest.mark.parametrize("w", VARIANTS, ids=lambda w: w.name)
def test_pack_roundtrip(w):
    d, pairs, qz = _setup(w)
    pk = oracle.pack(qz)
    ng = qz.nq // 32
    assert ng >= 1
    for b in range(w.batch):
        for kh in range(w.n_kv_heads):
            sal = _salient(pairs[b, kh], w.n_pairs_hi)
            for g in range(ng):
                codes, raw, s, z = _unpack(w, pk, pairs, b, kh, g, sal)
                assert np.array_equal(codes, qz.kcodes[b, kh, g])
                assert np.array_equal(s, qz.ks[b, kh, g]) and np.array_equal(z, qz.kz[b, kh, g])
                if raw is not None:
                    ref = d["k"][b, kh, 32 * g:32 * g + 32][:, sal].T
                    assert np.array_equal(raw, ref)
                vc, vs, vz, _ = brute.unpack_values(pk["v_codes"][b, kh, g], pk["v_meta"][b, kh, g])
                assert np.array_equal(vc, qz.vcodes[b, kh, g])
                assert np.array_equal(vs, qz.vs[b, kh, g]) and np.array_equal(vz, qz.vz[b, kh, g])
            # 4-bit channels hold codes up to 15, 2-bit ones up to 3
            lo = [c for c in range(128) if c not in sal]
            assert qz.kcodes[b, kh, :ng][:, lo].max() <= 3
            if sal and w.bits_hi == 4:
                assert qz.kcodes[b, kh, :ng][:, sal].max() > 3


def _dequant_from_bytes(w, d, pairs, pk, b, kh, T):
    """fp64 K^, V^ [T][128] of one (b, kv head), rebuilt from the packed
    bytes with the brute-force unpacker and the raw ring positions."""
    nq = oracle.n_quant(T, w.residual)
    f16 = lambda bits: np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)
    K = kvq_synth.bits_to_f64(d["k"][b, kh, :T], w.io_dtype).copy()
    V = kvq_synth.bits_to_f64(d["v"][b, kh, :T], w.io_dtype).copy()
    sal = _salient(pairs[b, kh], w.n_pairs_hi)
    for g in range(nq // 32):
        codes, raw, s, z = _unpack(w, pk, pairs, b, kh, g, sal)
        for c in range(128):
            if w.bits_hi == 16 and c in sal:
                continue
            K[32 * g:32 * g + 32, c] = f16(z[c]) + f16(s[c]) * codes[c]
        vc, vs, vz, _ = brute.unpack_values(pk["v_codes"][b, kh, g], pk["v_meta"][b, kh, g])
        for t in range(32):
            for j in range(4):
                V[32 * g + t, 32 * j:32 * j + 32] = f16(vz[t, j]) + f16(vs[t, j]) * vc[t, 32 * j:32 * j + 32]
    return K, V


@pytest.mark.parametrize("w", VARIANTS, ids=lambda w: w.name)
def test_attention_matches_textbook_over_unpacked_bytes(w):
    d, pairs, qz = _setup(w)
    pk = oracle.pack(qz)
    q = d["q_dec"][:, :, 0]
    sm = 1.0 / np.sqrt(128.0)
    out = oracle.attention(qz, q, sm)
    G = w.group_size
    for b in range(w.batch):
        for kh in range(w.n_kv_heads):
            K, V = _dequant_from_bytes(w, d, pairs, pk, b, kh, w.tokens)
            for h in range(kh * G, kh * G + G):
                qf = kvq_synth.bits_to_f64(q[b, h], w.io_dtype)
                ref = brute.attention_textbook(qf, K, V, float(np.float32(sm)))
                assert np.max(np.abs(out[b, h] - ref)) <= 1e-12


def test_all_sixteen_bit_mode_is_plain_attention():
    # residual window covering every token: nothing is quantized
    w = kvq_synth.Workload("hp", 1, 4, 2, 96, n_qry=8, io_dtype="bf16", residual=128, seed=8)
    d, pairs, qz = _setup(w)
    assert qz.nq == 0
    q = d["q_dec"][:, :, 0]
    out, lse = oracle.attention(qz, q, 0.125, with_lse=True)
    for h in range(4):
        qf = kvq_synth.bits_to_f64(q[0, h], "bf16")
        K = kvq_synth.bits_to_f64(d["k"][0, h // 2], "bf16")
        V = kvq_synth.bits_to_f64(d["v"][0, h // 2], "bf16")
        assert np.max(np.abs(out[0, h] - brute.attention_textbook(qf, K, V, 0.125))) <= 1e-12
        lg = 0.125 * (K @ qf)
        assert abs(lse[0, h] - np.log(np.exp(lg).sum())) <= 1e-10


def test_single_token_returns_its_value():
    w = kvq_synth.Workload("t1", 1, 2, 1, 1, n_qry=1, io_dtype="fp16", residual=32, seed=9)
    d, pairs, qz = _setup(w)
    out = oracle.attention(qz, d["q_dec"][:, :, 0], 0.088)
    v0 = kvq_synth.bits_to_f64(d["v"][0, 0, 0], "fp16")
    assert np.array_equal(out[0, 0], v0) and np.array_equal(out[0, 1], v0)


def test_zero_query_is_mean_of_dequantized_values():
    w = kvq_synth.WORKLOADS[0]
    d, pairs, qz = _setup(w)
    pk = oracle.pack(qz)
    out = oracle.attention(qz, np.zeros((1, 1, 128), np.uint16), 0.088)
    _, V = _dequant_from_bytes(w, d, pairs, pk, 0, 0, w.tokens)
    assert np.max(np.abs(out[0, 0] - V.mean(axis=0))) <= 1e-12


def test_lse_combine_identity():
    # merging two token ranges with the log-sum-exp rule equals the whole
    w = kvq_synth.Workload("lse", 1, 2, 1, 64, n_qry=8, io_dtype="bf16", residual=128, seed=10)
    d, pairs, _ = _setup(w)
    q = d["q_dec"][:, :, 0]
    parts = []
    for lo, hi in ((0, 40), (40, 64)):
        sub = {k: d[k][:, :, lo:hi] for k in ("k", "v")}
        qz = oracle.quantize(sub["k"], sub["v"], hi - lo, pairs, residual=128,
                             n_pairs_hi=6, bits_hi=4, io_dtype="bf16")
        parts.append(oracle.attention(qz, q, 0.1, with_lse=True))
    qz = oracle.quantize(d["k"], d["v"], 64, pairs, residual=128, n_pairs_hi=6,
                         bits_hi=4, io_dtype="bf16")
    whole, lse = oracle.attention(qz, q, 0.1, with_lse=True)
    m = np.maximum(parts[0][1], parts[1][1])
    w0, w1 = np.exp(parts[0][1] - m), np.exp(parts[1][1] - m)
    merged = (parts[0][0] * w0[..., None] + parts[1][0] * w1[..., None]) / (w0 + w1)[..., None]
    assert np.max(np.abs(merged - whole)) <= 1e-12
    assert np.max(np.abs(m + np.log(w0 + w1) - lse)) <= 1e-12


def test_record_sizes():
    # per group of 32 tokens: k_lo 1 KiB, k_meta 512 B, v 1 KiB + 512 B;
    # salient section 128 B (4-bit) or 32 tokens x 2 n_hi x 2 B (16-bit)
    assert oracle.k_hi_words(6, 4) == 128
    assert oracle.k_hi_words(6, 16) == 768
    assert oracle.k_hi_words(0, 4) == 0
    # residual rule: "last 32" at T=512/R=32 and 128 at T=32768/R=128
    assert 512 - oracle.n_quant(512, 32) == 32
    assert 32768 - oracle.n_quant(32768, 128) == 128
    assert oracle.n_quant(100, 128) == 0
    assert 200 - oracle.n_quant(200, 64) == 72


@pytest.mark.parametrize("w", [v for v in VARIANTS if v.n_pairs_lo1], ids=lambda w: w.name)
def test_one_bit_pairs(w):
    """Pairs of the n_pairs_lo1 lowest ranks get a two-level grid: s is the
    fp16 of the group's range, every code is the nearer of z and z + s; the
    other non-salient pairs keep four levels.  At 32 of 64 pairs the code
    bits average 1.5 per key channel."""
    d, pairs, qz = _setup(w)
    ng = qz.nq // 32
    f16 = lambda b: float(np.uint16(b).view(np.float16))
    for b in range(w.batch):
        for kh in range(w.n_kv_heads):
            ranked = [int(p) for p in pairs[b, kh]]
            one = set(ranked[64 - w.n_pairs_lo1:])
            two = set(ranked[w.n_pairs_hi:64 - w.n_pairs_lo1])
            bits = [1 if c % 64 in one else 2 if c % 64 in two else w.bits_hi for c in range(128)]
            if w.n_pairs_hi == 0 and w.n_pairs_lo1 == 32:
                assert sum(bits) == 1.5 * 128
            for g in range(ng):
                x = kvq_synth.bits_to_f64(d["k"][b, kh, 32 * g:32 * g + 32], w.io_dtype)
                for c in range(128):
                    codes = qz.kcodes[b, kh, g, c]
                    s, z = f16(qz.ks[b, kh, g, c]), f16(qz.kz[b, kh, g, c])
                    if bits[c] == 1:
                        assert codes.max() <= 1
                        assert z == f16(oracle.f32_to_half(x[:, c].min())[0])
                        assert s == f16(oracle.f32_to_half(np.float32(x[:, c].max() - z))[0])
                        if s > 0:
                            q, margin = brute.nearest_level(x[:, c], s, z, 1)
                            ok = margin > 1e-4 * s
                            assert np.array_equal(codes[ok], q[ok])
            lo2 = [c for c in range(128) if bits[c] == 2]
            assert qz.kcodes[b, kh, :ng][:, lo2].max() == 3
