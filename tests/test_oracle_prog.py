"""Pins of the oracle's progressive precision (PM-KVQ review, lead and
key_machinery: the cache starts at 16 bits and is shrunk through 8, 4 and 2
bits as it ages, each step in place by the equivalent right shift).

The oracle's reading: a group's width follows its age among the quantized
groups (8 bits for the newest prog_w8, 4 bits up to prog_w4, then the final
width); every group is quantized at 8 bits first and shrunk step by step,
the zero point kept and the step stored as fp16(s (2^b + 1)).

* The width schedule by age, every edge (w8 = 0, w8 = w4).
* Closed forms of the chain: in every quantized channel (keys) and channel
  group (values) the group minimum keeps code 0 and the maximum the top
  code 2^w - 1 at every width; data that lies on a 2-bit grid keeps the
  grid's codes exactly (85 k -> 5 k -> k).
* The quantization error after the chain: every dequantized value lies
  within 0.52 of its final step of the input (the bound that the three
  roundings and the fp16 steps allow), within 0.5 at 8 bits.
* The byte records, read bit by bit from the layout (digit 0 in k_lo /
  v_codes, digit 1 of salient keys in k_hi, digits 1..3 of the wide groups
  in their plane slots), give back the logical codes and metadata.
* Attention over those bytes equals textbook attention, and the 8-bit cache
  is far closer to unquantized attention than the 2-bit one.
"""
import numpy as np
import pytest

import kvq_synth
import oracle
from oracle import brute

W = kvq_synth.Workload("prog", 1, 4, 2, 32 * 10 + 64 + 20, n_qry=8, io_dtype="bf16",
                       outliers="pct2x10", n_pairs_hi=6, residual=64, seed=77)


def _f16(b):
    return np.asarray(b, np.uint16).view(np.float16).astype(np.float64)


def _setup(w8=2, w4=5, bits_hi=4, n_hi=6, io="bf16"):
    w = W.replace(bits_hi=bits_hi, n_pairs_hi=n_hi, io_dtype=io)
    d = kvq_synth.generate(w)
    _, pairs = oracle.select(d["q_sel"], d["k"], w.tokens, w.n_kv_heads, w.io_dtype)
    qz = oracle.quantize(d["k"], d["v"], w.tokens, pairs, residual=w.residual,
                         n_pairs_hi=w.n_pairs_hi, bits_hi=w.bits_hi, io_dtype=w.io_dtype,
                         prog_w8=w8, prog_w4=w4)
    return w, d, pairs, qz


def _salient(pairs, b, kh, n_hi):
    return sorted([int(p) for p in pairs[b, kh, :n_hi]] + [int(p) + 64 for p in pairs[b, kh, :n_hi]])


@pytest.mark.parametrize("w8,w4", [(0, 1), (0, 4), (2, 5), (3, 3), (6, 6)])
def test_width_schedule_by_age(w8, w4):
    for age in range(12):
        want = 8 if age < w8 else (4 if age < w4 else 2)
        assert oracle.prog_width(age, w8, w4) == want


@pytest.mark.parametrize("bits_hi", [4, 16])
def test_min_and_max_keep_the_end_codes_at_every_width(bits_hi):
    w, d, pairs, qz = _setup(bits_hi=bits_hi)
    ng = qz.nq // 32
    assert ng == 10
    for b in range(w.batch):
        for kh in range(w.n_kv_heads):
            sal = set(_salient(pairs, b, kh, w.n_pairs_hi))
            K = kvq_synth.bits_to_f64(d["k"][b, kh], w.io_dtype)
            V = kvq_synth.bits_to_f64(d["v"][b, kh], w.io_dtype)
            for g in range(ng):
                width = oracle.prog_width(ng - 1 - g, 2, 5)
                for c in range(128):
                    codes = qz.kcodes[b, kh, g, c].astype(np.int64)
                    if c in sal and bits_hi == 16:
                        assert not codes.any() and qz.ks[b, kh, g, c] == 0
                        continue
                    cw = 4 if (c in sal and width == 2) else width
                    x = K[32 * g:32 * g + 32, c]
                    if x.max() == x.min():
                        continue
                    assert codes.max() == (1 << cw) - 1 and codes.min() == 0
                    assert codes[np.argmax(x)] == (1 << cw) - 1
                    assert codes[np.argmin(x)] == 0
                for t in range(32):
                    for j in range(4):
                        x = V[32 * g + t, 32 * j:32 * j + 32]
                        vc = qz.vcodes[b, kh, g, t, 32 * j:32 * j + 32].astype(np.int64)
                        if x.max() == x.min():
                            continue
                        assert vc.max() == (1 << width) - 1 and vc.min() == 0
                        assert vc[np.argmax(x)] == (1 << width) - 1


def test_grid_data_keeps_its_codes_through_the_chain():
    # keys and values on a grid z + k * 2^-3 with every level k = 0..3
    # present in each channel group: 8-bit codes 85 k, 4-bit 5 k, 2-bit k
    rng = np.random.default_rng(5)
    B, Hkv, T, R = 1, 1, 32 * 6 + 32, 32
    lev = np.tile(np.arange(4), 8)
    k = np.zeros((B, Hkv, T, 128))
    v = np.zeros((B, Hkv, T, 128))
    kk = np.zeros((6, 128, 32), np.int64)
    vk = np.zeros((6, 32, 128), np.int64)
    for g in range(6):
        for c in range(128):
            kk[g, c] = rng.permutation(lev)
            k[0, 0, 32 * g:32 * g + 32, c] = -1.0 + 0.125 * kk[g, c]
        for t in range(32):
            for j in range(4):
                vk[g, t, 32 * j:32 * j + 32] = rng.permutation(lev)
            v[0, 0, 32 * g + t] = 0.5 + 0.125 * vk[g, t]
    # grid values have few significant bits: exact in bf16 (upper half of fp32)
    kb = (k.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    vb = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(kvq_synth.bits_to_f64(kb, "bf16"), k)
    pairs = np.tile(np.arange(64, dtype=np.int32), (B, Hkv, 1))
    qz = oracle.quantize(kb, vb, T, pairs, residual=R, n_pairs_hi=0, bits_hi=4,
                         io_dtype="bf16", prog_w8=2, prog_w4=4)
    ng = qz.nq // 32
    assert ng == 6
    for g in range(ng):
        mul = {8: 85, 4: 5, 2: 1}[oracle.prog_width(ng - 1 - g, 2, 4)]
        assert np.array_equal(qz.kcodes[0, 0, g].astype(np.int64), mul * kk[g])
        assert np.array_equal(qz.vcodes[0, 0, g].astype(np.int64), mul * vk[g])
        # the steps stay within fp16 rounding of the grid's own step
        step = 0.375 / ((1 << {85: 8, 5: 4, 1: 2}[mul]) - 1)
        assert np.allclose(_f16(qz.ks[0, 0, g]), step, rtol=3 * 2.0 ** -11)
        assert np.allclose(_f16(qz.vs[0, 0, g]), step, rtol=3 * 2.0 ** -11)


@pytest.mark.parametrize("io", ["bf16", "fp16"])
def test_dequantized_values_within_half_a_final_step(io):
    w, d, pairs, qz = _setup(io=io)
    ng = qz.nq // 32
    for b in range(w.batch):
        for kh in range(w.n_kv_heads):
            sal = set(_salient(pairs, b, kh, w.n_pairs_hi))
            K = kvq_synth.bits_to_f64(d["k"][b, kh], w.io_dtype)
            V = kvq_synth.bits_to_f64(d["v"][b, kh], w.io_dtype)
            for g in range(ng):
                width = oracle.prog_width(ng - 1 - g, 2, 5)
                lim = 0.5 + 1e-6 if width == 8 else 0.52
                s, z = _f16(qz.ks[b, kh, g]), _f16(qz.kz[b, kh, g])
                xh = z[:, None] + s[:, None] * qz.kcodes[b, kh, g]
                err = np.abs(xh - K[32 * g:32 * g + 32].T)
                assert np.all(err <= lim * s[:, None] + 1e-9), (g, err.max())
                vs, vz = _f16(qz.vs[b, kh, g]), _f16(qz.vz[b, kh, g])  # [32][4]
                vh = vz.repeat(32, axis=1) + vs.repeat(32, axis=1) * qz.vcodes[b, kh, g]
                err = np.abs(vh - V[32 * g:32 * g + 32])
                assert np.all(err <= lim * vs.repeat(32, axis=1) + 1e-9), (g, err.max())
                # the shrink is not a no-op: 2-bit groups are coarser than 8-bit ones
                if width == 2:
                    assert np.max(qz.vcodes[b, kh, g]) == 3


def _k_digits(words):
    """Digits [128][32] of a 256-word plane in the k_lo word format, read
    from the layout (word (w*2 + T)*16 + r, token at tile index 16T + r,
    channel 16w + c at position pi(c))."""
    out = np.zeros((128, 32), np.int64)
    for t in range(32):
        e = brute._tile_index(t)
        T, r = divmod(e, 16)
        for c in range(128):
            out[c, t] = brute._code(words[((c // 16) * 2 + T) * 16 + r], brute._pos(c % 16))
    return out


@pytest.mark.parametrize("w8,w4,bits_hi", [(2, 5, 4), (0, 3, 4), (3, 3, 16), (10, 10, 4)])
def test_byte_records_give_back_the_codes(w8, w4, bits_hi):
    w, d, pairs, qz = _setup(w8=w8, w4=w4, bits_hi=bits_hi)
    pk = oracle.pack(qz)
    ng = qz.nq // 32
    assert pk["k_pl"].shape[2] == w4 + 2 * w8
    slots = oracle.live_plane_slots(w.tokens, w.residual, w8, w4)
    assert len({s for _, s in slots}) == len(slots)  # live planes never share a slot
    for b in range(w.batch):
        for kh in range(w.n_kv_heads):
            sal = _salient(pairs, b, kh, w.n_pairs_hi)
            for g in range(ng):
                age = ng - 1 - g
                codes, raw, s, z = brute.unpack_keys(pk["k_lo"][b, kh, g], pk["k_hi"][b, kh, g],
                                                     pk["k_meta"][b, kh, g], sal, bits_hi)
                vc, vs, vz, _ = brute.unpack_values(pk["v_codes"][b, kh, g], pk["v_meta"][b, kh, g])
                assert np.array_equal(s, qz.ks[b, kh, g]) and np.array_equal(z, qz.kz[b, kh, g])
                assert np.array_equal(vs, qz.vs[b, kh, g]) and np.array_equal(vz, qz.vz[b, kh, g])
                if age < w4:
                    # digit 0 from k_lo, digits 1.. from the planes for every channel
                    kd = [brute.unpack_keys(pk["k_lo"][b, kh, g], pk["k_hi"][b, kh, g][:0],
                                            pk["k_meta"][b, kh, g], [], 4)[0]]
                    vd = [vc]
                    ps = [g % w4] + ([w4 + 2 * (g % w8), w4 + 2 * (g % w8) + 1] if age < w8 else [])
                    for p in ps:
                        kd.append(_k_digits(pk["k_pl"][b, kh, p]))
                        vd.append(np.concatenate([brute._v_digits(pk["v_pl"][b, kh, p], 0, 4, kq)
                                                  for kq in range(4)]))
                    codes = sum(dg * 4 ** i for i, dg in enumerate(kd))
                    vc = sum(dg * 4 ** i for i, dg in enumerate(vd))
                    if bits_hi == 4:
                        # k_hi still carries digit 1 of the salient channels
                        hi = brute.unpack_keys(pk["k_lo"][b, kh, g] * 0, pk["k_hi"][b, kh, g],
                                               pk["k_meta"][b, kh, g], sal, 4)[0]
                        assert np.array_equal(hi[sal] // 4, kd[1][sal])
                assert np.array_equal(codes, qz.kcodes[b, kh, g].astype(np.int64)), (g, age)
                assert np.array_equal(vc, qz.vcodes[b, kh, g].astype(np.int64)), (g, age)


def test_attention_over_progressive_bytes_matches_textbook():
    w, d, pairs, qz = _setup()
    q = d["q_dec"][:, :, 0]
    sm = float(np.float32(1.0 / np.sqrt(128.0)))
    out = oracle.attention(qz, q, sm)
    G, T = w.group_size, w.tokens
    ng = qz.nq // 32
    for b in range(w.batch):
        for kh in range(w.n_kv_heads):
            K = kvq_synth.bits_to_f64(d["k"][b, kh, :T], w.io_dtype).copy()
            V = kvq_synth.bits_to_f64(d["v"][b, kh, :T], w.io_dtype).copy()
            for g in range(ng):
                s, z = _f16(qz.ks[b, kh, g]), _f16(qz.kz[b, kh, g])
                K[32 * g:32 * g + 32] = (z[:, None] + s[:, None] * qz.kcodes[b, kh, g]).T
                vs, vz = _f16(qz.vs[b, kh, g]), _f16(qz.vz[b, kh, g])
                V[32 * g:32 * g + 32] = vz.repeat(32, axis=1) + vs.repeat(32, axis=1) * qz.vcodes[b, kh, g]
            for h in range(kh * G, kh * G + G):
                qf = kvq_synth.bits_to_f64(q[b, h], w.io_dtype)
                ref = brute.attention_textbook(qf, K, V, sm)
                assert np.max(np.abs(out[b, h] - ref)) < 1e-12


def test_eight_bit_cache_is_closest_to_unquantized_attention():
    errs = {}
    for key, (w8, w4) in {"8": (10, 10), "window": (2, 5), "2": (0, 1)}.items():
        w, d, pairs, qz = _setup(w8=w8, w4=w4)
        q = d["q_dec"][:, :, 0]
        sm = float(np.float32(1.0 / np.sqrt(128.0)))
        out = oracle.attention(qz, q, sm)
        e = 0.0
        for b in range(w.batch):
            for h in range(w.n_q_heads):
                kh = h // w.group_size
                K = kvq_synth.bits_to_f64(d["k"][b, kh, :w.tokens], w.io_dtype)
                V = kvq_synth.bits_to_f64(d["v"][b, kh, :w.tokens], w.io_dtype)
                ref = brute.attention_textbook(kvq_synth.bits_to_f64(q[b, h], w.io_dtype), K, V, sm)
                e = max(e, np.max(np.abs(out[b, h] - ref)))
        errs[key] = e
    assert errs["8"] < 0.1 * errs["2"], errs
    assert errs["window"] <= errs["2"] * 1.0001, errs
