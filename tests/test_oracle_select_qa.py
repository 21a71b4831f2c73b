"""Pins of the oracle's query-aware channel score (MixKVQ, abstract: a key
channel's importance joins its intrinsic quantization difficulty with its
relevance to the query).  The page prints no formula; the reading scores a
channel by (sum of per-group key ranges) x (sum of |q|) in fixed point, a
pair by the sum over its two channels.  Parity with the page is therefore
unpinned; these tests pin the oracle to properties that reading must have."""
import numpy as np
import pytest

import kvq_synth
import oracle

W = kvq_synth.Workload("qa", 2, 8, 2, 256, n_qry=16, io_dtype="bf16", outliers="pct2x10",
                       n_pairs_hi=6, residual=32, seed=51)


@pytest.fixture(scope="module")
def data():
    return kvq_synth.generate(W)


def _score(q, k, T=W.tokens, dtype=W.io_dtype):
    return oracle.select_qa(q, k, T, W.n_kv_heads, dtype)


def test_order_invariances_bit_exact(data):
    q, k = data["q_sel"], data["k"][:, :, :W.tokens]
    S0, p0 = _score(q, k)
    rng = np.random.default_rng(3)
    # tokens shuffled inside every 32-token group: ranges unchanged
    kk = k.copy()
    for g in range(W.tokens // 32):
        perm = rng.permutation(32)
        kk[:, :, 32 * g:32 * g + 32] = kk[:, :, 32 * g + perm]
    # whole groups shuffled: integer sums unchanged
    gp = rng.permutation(W.tokens // 32)
    kg = np.concatenate([kk[:, :, 32 * g:32 * g + 32] for g in gp], axis=2)
    # queries shuffled within each head and heads within each KV group
    G = W.group_size
    qq = q[:, :, rng.permutation(W.n_qry)]
    hp = np.concatenate([kh * G + rng.permutation(G) for kh in range(W.n_kv_heads)])
    qq = qq[:, hp]
    S1, p1 = _score(qq, kg)
    assert np.array_equal(S0.view(np.uint64), S1.view(np.uint64))
    assert np.array_equal(p0, p1)


def test_sign_flips_bit_exact(data):
    q, k = data["q_sel"], data["k"][:, :, :W.tokens]
    S0, _ = _score(q, k)
    S1, _ = _score(q ^ np.uint16(0x8000), k ^ np.uint16(0x8000))
    assert np.array_equal(S0.view(np.uint64), S1.view(np.uint64))


def test_doubling_queries_doubles_scores(data):
    # |q| * 2^24 is an integer for every bf16 query of this data, so the
    # fixed-point relevance doubles exactly, and with it every score
    q, k = data["q_sel"], data["k"][:, :, :W.tokens]
    qf = kvq_synth.bits_to_f64(q, "bf16")
    assert np.all((np.abs(qf) * 2 ** 24) % 1 == 0)
    S0, p0 = _score(q, k)
    S1, p1 = _score(kvq_synth.to_bits(2 * qf, "bf16"), k)
    assert np.array_equal(S1, 2 * S0) and np.array_equal(p0, p1)


def test_degenerate_inputs_rank_by_pair_id(data):
    q, k = data["q_sel"], data["k"][:, :, :W.tokens]
    ident = np.broadcast_to(np.arange(64, dtype=np.int32), (W.batch, W.n_kv_heads, 64))
    S, p = _score(np.zeros_like(q), k)  # no relevance anywhere
    assert np.all(S == 0) and np.array_equal(p, ident)
    kc = np.broadcast_to(k[:, :, :1], k.shape).copy()  # constant keys: no difficulty
    S, p = _score(q, kc)
    assert np.all(S == 0) and np.array_equal(p, ident)
    S, p = _score(q, k[:, :, :31], T=31)  # no full group
    assert np.all(S == 0) and np.array_equal(p, ident)


def test_planted_pair_ranks_first(data):
    # a pair whose keys and queries are both scaled x8 has the largest range
    # and the largest |q| on both channels
    q = kvq_synth.bits_to_f64(data["q_sel"], "bf16")
    k = kvq_synth.bits_to_f64(data["k"][:, :, :W.tokens], "bf16")
    j = 37
    for arr in (q, k):
        arr[..., j] *= 8
        arr[..., j + 64] *= 8
    _, p = _score(kvq_synth.to_bits(q, "bf16"), kvq_synth.to_bits(k, "bf16"))
    assert np.all(p[:, :, 0] == j)
