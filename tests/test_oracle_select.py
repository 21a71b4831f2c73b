"""Pins of the oracle's pair selection (PN-Mix, abstract and transcript:
saliency of a RoPE pair = query pair norm x key pair norm, chosen once at
prefill) against an exhaustive mean over all query/key combinations, planted
outliers, RoPE invariance and token-order invariance."""
import numpy as np

import kvq_synth
import oracle
from oracle import brute


def _small(seed, io_dtype="bf16", T=96, Hq=4, Hkv=2, n_qry=8):
    return kvq_synth.Workload("t", 1, Hq, Hkv, T, n_qry=n_qry, io_dtype=io_dtype,
                              outliers="pairs4x8", seed=seed)


def _check_against_exhaustive(w, data):
    sums, pairs = oracle.select(data["q_sel"], data["k"], w.tokens, w.n_kv_heads, w.io_dtype)
    qf = kvq_synth.bits_to_f64(data["q_sel"][0], w.io_dtype)
    kf = kvq_synth.bits_to_f64(data["k"][0, :, :w.tokens], w.io_dtype)
    mean, rank = brute.select_exhaustive(qf, kf, w.group_size)
    n_q = w.group_size * w.n_qry
    for kh in range(w.n_kv_heads):
        # factorized fixed-point score == exhaustive mean, to fixed-point error
        fact = sums[0, kh, 0].astype(np.float64) * sums[0, kh, 1].astype(np.float64)
        fact /= n_q * w.tokens * 2.0 ** 48
        assert np.allclose(fact, mean[kh], rtol=1e-6, atol=0)
        # same ranking wherever neighbours are separated by more than that
        sc = mean[kh][rank[kh]]
        gap = (sc[:-1] - sc[1:]) / sc[:-1]
        if np.all(gap > 1e-5):
            assert np.array_equal(pairs[0, kh], rank[kh])
        else:
            assert set(pairs[0, kh]) == set(range(64))
            assert np.all(np.diff(mean[kh][pairs[0, kh]]) <= 1e-5 * sc[0])


def test_matches_exhaustive_mean():
    for seed in range(6):
        for dt in ("fp16", "bf16"):
            w = _small(seed, dt)
            _check_against_exhaustive(w, kvq_synth.generate(w))


def test_planted_outliers_rank_first():
    w = kvq_synth.WORKLOADS[0]
    data = kvq_synth.generate(w)
    _, pairs = oracle.select(data["q_sel"], data["k"], w.tokens, 1, w.io_dtype)
    planted = set(np.nonzero(data["outlier_scale"][0, 0] > 1)[0])
    assert len(planted) == 4
    assert set(pairs[0, 0, :4]) == planted


def test_rope_invariance():
    for seed in range(4):
        w = _small(seed, "fp16", T=64)
        d = kvq_synth.generate(w, keep_pre_rope=True)
        pre_q = kvq_synth.to_bits(d["q_sel_pre"], w.io_dtype)
        pre_k = kvq_synth.to_bits(d["k_pre"], w.io_dtype)
        s_pre, p_pre = oracle.select(pre_q, pre_k, w.tokens, w.n_kv_heads, w.io_dtype)
        s_post, p_post = oracle.select(d["q_sel"], d["k"], w.tokens, w.n_kv_heads, w.io_dtype)
        # the rotation preserves norms up to 16-bit rounding of the inputs
        a = s_pre.astype(np.float64)
        b = s_post.astype(np.float64)
        assert np.allclose(a, b, rtol=2e-3)
        for kh in range(w.n_kv_heads):
            sc = a[0, kh, 0] * a[0, kh, 1]
            srt = np.sort(sc)[::-1]
            if np.all((srt[:-1] - srt[1:]) / srt[:-1] > 1e-2):
                assert np.array_equal(p_pre[0, kh], p_post[0, kh])


def test_token_order_invariance_bit_exact():
    w = _small(3, "bf16", T=80)
    d = kvq_synth.generate(w)
    perm = np.random.default_rng(0).permutation(w.tokens)
    k2 = d["k"][:, :, perm]
    s1, p1 = oracle.select(d["q_sel"], d["k"], w.tokens, w.n_kv_heads, w.io_dtype)
    s2, p2 = oracle.select(d["q_sel"], k2, w.tokens, w.n_kv_heads, w.io_dtype)
    assert np.array_equal(s1, s2) and np.array_equal(p1, p2)


def test_rope_preserves_pair_norms():
    w = kvq_synth.WORKLOADS[0]
    d = kvq_synth.generate(w, keep_pre_rope=True)
    for pre, post in (("k_pre", "k_post"), ("q_sel_pre", "q_sel_post"),
                      ("q_dec_pre", "q_dec_post")):
        a, b = d[pre], d[post]
        na = np.hypot(a[..., :64], a[..., 64:])
        nb = np.hypot(b[..., :64], b[..., 64:])
        assert np.max(np.abs(na - nb)) <= 1e-12 * max(1.0, na.max())
        # and the rotation is not the identity
        assert np.max(np.abs(a - b)) > 0.1
