"""Pins of the oracle's query-channel pruning at decode (Dual-QK, abstract:
keep a decode query's few large channels, drop the many small ones, and read
the key cache only for the kept ones).  The page gives no rule; the reading
keeps, per (b, kv head), the n_keep of the eight 16-channel key runs with
the largest summed |q| over the group's heads (fixed point: min(floor(4096
|q|), 2^20) per value; ties to the lower run), and every logit sums
q_c k^_c over the kept channels only.

* Selection: the kept set is the top n_keep by a plain float64 sum of |q|
  wherever that sum separates the runs; it does not change when heads are
  permuted inside a group or channels inside a run, nor when q is doubled
  for values whose fixed-point form is exact (multiples of 1/4096); a planted
  run is kept first; an all-zero query keeps runs 0 .. n_keep-1; a
  query far beyond the cap still ranks; the kept sets are nested in n_keep.
* Attention: n_keep = 8 is unpruned attention, bit for bit; otherwise it
  equals textbook softmax attention whose logits use only the kept channels'
  columns of the key matrix, rebuilt from the packed bytes by the brute-force
  unpacker (quantized groups) and from the 16-bit inputs (ring).
"""
import numpy as np
import pytest

import kvq_synth
import oracle
from oracle import brute

W = kvq_synth.Workload("prune", 2, 8, 2, 300, n_qry=8, io_dtype="bf16", outliers="pct2x10",
                       n_pairs_hi=6, residual=64, seed=61)


@pytest.fixture(scope="module")
def data():
    return kvq_synth.generate(W)


def _q(data):
    return data["q_dec"][:, :, 0]


def test_selection_matches_float_sums_where_separated(data):
    q = _q(data)
    G = W.group_size
    qf = np.abs(kvq_synth.bits_to_f64(q, W.io_dtype))
    checked = 0
    for n_keep in range(1, 8):
        keep = oracle.prune_chunks(q, W.n_kv_heads, W.io_dtype, n_keep)
        for b in range(W.batch):
            for kh in range(W.n_kv_heads):
                e = qf[b, kh * G:(kh + 1) * G].reshape(G, 8, 16).sum(axis=(0, 2))
                order = np.argsort(-e, kind="stable")
                srt = e[order]
                # the fixed point drops under 1/4096 per value: 1/256 per run and head
                if srt[n_keep - 1] - srt[n_keep] < G / 128:
                    continue  # too close for a float sum to decide
                want = np.zeros(8, bool)
                want[order[:n_keep]] = True
                assert np.array_equal(keep[b, kh], want)
                checked += 1
    assert checked >= 6


def test_selection_invariances(data):
    q = _q(data)
    G = W.group_size
    rng = np.random.default_rng(5)
    qf = kvq_synth.bits_to_f64(q, W.io_dtype)
    # heads permuted inside each group, channels permuted inside each run
    hp = np.concatenate([kh * G + rng.permutation(G) for kh in range(W.n_kv_heads)])
    cp = np.concatenate([16 * m + rng.permutation(16) for m in range(8)])
    q2 = q[:, hp][:, :, cp]
    # doubling: values rounded to multiples of 1/4096 (and below the cap)
    qr = np.clip(np.round(qf * 4096) / 4096, -100, 100)
    q = kvq_synth.to_bits(qr, W.io_dtype)
    assert np.array_equal(kvq_synth.bits_to_f64(q, W.io_dtype) * 4096,
                          np.round(kvq_synth.bits_to_f64(q, W.io_dtype) * 4096))
    q2 = q[:, hp][:, :, cp]
    q3 = kvq_synth.to_bits(2 * kvq_synth.bits_to_f64(q, W.io_dtype), W.io_dtype)
    for n_keep in range(1, 9):
        k0 = oracle.prune_chunks(q, W.n_kv_heads, W.io_dtype, n_keep)
        assert np.array_equal(k0, oracle.prune_chunks(q2, W.n_kv_heads, W.io_dtype, n_keep))
        assert np.array_equal(k0, oracle.prune_chunks(q3, W.n_kv_heads, W.io_dtype, n_keep))
        assert np.all(k0.sum(axis=2) == n_keep)
        if n_keep < 8:  # nested
            k1 = oracle.prune_chunks(q, W.n_kv_heads, W.io_dtype, n_keep + 1)
            assert np.all(k1[k0])


def test_planted_run_and_zero_query(data):
    q = _q(data)
    qf = kvq_synth.bits_to_f64(q, W.io_dtype)
    for m in range(8):
        qp = qf.copy()
        qp[:, :, 16 * m:16 * m + 16] *= 64
        keep = oracle.prune_chunks(kvq_synth.to_bits(qp, W.io_dtype), W.n_kv_heads, W.io_dtype, 1)
        want = np.zeros(8, bool)
        want[m] = True
        assert np.all(keep == want)
    zero = np.zeros_like(q)
    for n_keep in range(1, 8):
        keep = oracle.prune_chunks(zero, W.n_kv_heads, W.io_dtype, n_keep)
        assert np.all(keep == (np.arange(8) < n_keep))
    # huge values: every one capped at 2^20 / 4096 = 256; the run with the
    # most of them wins, whatever their size beyond the cap
    big = np.zeros((1, W.group_size, 128))
    big[0, :, 16 * 5:16 * 5 + 3] = 1e30
    big[0, :, 16 * 2:16 * 2 + 2] = 3e38
    big[0, :, 16 * 7] = 1000.0
    keep = oracle.prune_chunks(kvq_synth.to_bits(big, "bf16"), 1, "bf16", 1)
    assert np.array_equal(keep[0, 0], np.arange(8) == 5)


def _quantized(data):
    _, pairs = oracle.select(data["q_sel"], data["k"], W.tokens, W.n_kv_heads, W.io_dtype)
    return oracle.quantize(data["k"], data["v"], W.tokens, pairs, residual=W.residual,
                           n_pairs_hi=W.n_pairs_hi, bits_hi=W.bits_hi, io_dtype=W.io_dtype)


def test_keep_all_is_unpruned_attention(data):
    qz = _quantized(data)
    sm = float(np.float32(1.0 / np.sqrt(128.0)))
    a = oracle.attention(qz, _q(data), sm)
    b = oracle.attention_pruned(qz, _q(data), sm, 8)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("n_keep", [1, 3, 5, 7])
def test_pruned_attention_matches_textbook_on_kept_columns(data, n_keep):
    qz = _quantized(data)
    pk = oracle.pack(qz)
    q = _q(data)
    sm = float(np.float32(1.0 / np.sqrt(128.0)))
    out = oracle.attention_pruned(qz, q, sm, n_keep)
    keep = oracle.prune_chunks(q, W.n_kv_heads, W.io_dtype, n_keep)
    G, T = W.group_size, W.tokens
    f16 = lambda x: float(np.uint16(x).view(np.float16))
    for b in range(W.batch):
        for kh in range(W.n_kv_heads):
            sal = sorted([int(p) for p in qz.pairs[b, kh, :W.n_pairs_hi]] +
                         [int(p) + 64 for p in qz.pairs[b, kh, :W.n_pairs_hi]])
            K = kvq_synth.bits_to_f64(data["k"][b, kh, :T], W.io_dtype).copy()
            V = kvq_synth.bits_to_f64(data["v"][b, kh, :T], W.io_dtype).copy()
            for g in range(qz.nq // 32):
                codes, _, s, z = brute.unpack_keys(pk["k_lo"][b, kh, g], pk["k_hi"][b, kh, g],
                                                   pk["k_meta"][b, kh, g], sal, W.bits_hi)
                for c in range(128):
                    K[32 * g:32 * g + 32, c] = f16(z[c]) + f16(s[c]) * codes[c]
                vc, vs, vz, _ = brute.unpack_values(pk["v_codes"][b, kh, g], pk["v_meta"][b, kh, g])
                for t in range(32):
                    for j in range(4):
                        V[32 * g + t, 32 * j:32 * j + 32] = (f16(vz[t, j]) + f16(vs[t, j]) *
                                                             vc[t, 32 * j:32 * j + 32])
            cols = np.concatenate([np.arange(16 * m, 16 * m + 16) for m in range(8)
                                   if keep[b, kh, m]])
            for h in range(kh * G, kh * G + G):
                qf = kvq_synth.bits_to_f64(q[b, h], W.io_dtype)
                ref = brute.attention_textbook(qf[cols], K[:, cols], V, sm)
                assert np.max(np.abs(out[b, h] - ref)) < 1e-12
