"""Pins of two oracle rules that no value on the pages fixes:

* the ring of recent 16-bit tokens (PM-KVQ review, supporting_citations and
  key_machinery: recent tokens are held at 16 bits): the bytes orc_ring
  writes, read back through the slot formulas of include/kvq.h
  (slot = position mod (R + 32); ring_k [slot][128], ring_v
  [slot / 32][128][slot % 32]), hold exactly the positions [n_q(T), T), each
  once, and nothing else changes;
* the order of equal saliency scores (PN-Mix, abstract: pairs are ranked by
  their score; the order of equal scores is this library's rule: the lower
  pair id first), for both scorers, on planted exact ties.
"""
import ctypes

import numpy as np
import pytest

import kvq_synth
import oracle

D = 128


def _ring(k, v, T, R, fill=0xABCD):
    """orc_ring on sentinel-filled buffers: (ring_k [B][Hkv][RS][128],
    ring_v [B][Hkv][RS/32][128][32])."""
    B, Hkv, Tstride, _ = k.shape
    RS = R + 32
    rk = np.full((B, Hkv, RS, D), fill, np.uint16)
    rv = np.full((B, Hkv, RS // 32, D, 32), fill, np.uint16)
    lib = oracle._load()
    rc = lib.orc_ring(B, Hkv, oracle._p(k), oracle._p(v), Tstride, int(T), int(R),
                      oracle._p(rk), oracle._p(rv))
    assert rc == 0
    return rk, rv


def _tagged(B, Hkv, Tstride):
    """16-bit patterns unique per (sequence, head, position, channel) within a
    head: a misplaced copy names the position it came from."""
    p = np.arange(Tstride)[:, None] * D + np.arange(D)[None, :]
    base = (p % 65521).astype(np.uint16)
    k = np.broadcast_to(base, (B, Hkv, Tstride, D)).copy()
    v = np.broadcast_to(((base.astype(np.uint32) * 7 + 3) % 65521).astype(np.uint16),
                        (B, Hkv, Tstride, D)).copy()
    for b in range(B):
        for h in range(Hkv):
            k[b, h] ^= np.uint16((b * 131 + h * 17) & 0x7)
    return k, v


@pytest.mark.parametrize("R,T", [(32, 1), (32, 31), (32, 32), (32, 63), (32, 64), (32, 65),
                                 (32, 97), (64, 300), (128, 127), (128, 160), (128, 161),
                                 (128, 450)])
def test_ring_holds_exactly_the_recent_positions(R, T):
    B, Hkv, RS = 2, 3, R + 32
    k, v = _tagged(B, Hkv, T + 40)
    rk, rv = _ring(k, v, T, R)
    nq = oracle.n_quant(T, R)
    assert nq == 32 * (max(0, T - R) // 32)
    if T >= R:
        assert R <= T - nq <= R + 31  # at most RS tokens are raw
    live = set()
    for p in range(nq, T):
        s = p % RS
        assert s not in live  # no two raw positions share a slot
        live.add(s)
        assert np.array_equal(rk[:, :, s], k[:, :, p])
        assert np.array_equal(rv[:, :, s // 32, :, s % 32], v[:, :, p])
    # every other slot is untouched
    for s in range(RS):
        if s not in live:
            assert np.all(rk[:, :, s] == 0xABCD)
            assert np.all(rv[:, :, s // 32, :, s % 32] == 0xABCD)


@pytest.mark.parametrize("R", [32, 96])
def test_ring_of_one_more_token_differs_in_one_slot(R):
    # the ring of T + 1 tokens is the ring of T tokens with slot T mod RS
    # overwritten by token T (the append of the header); when n_q grows, the
    # slots of the group that left stay as they were (no longer read)
    B, Hkv, RS = 1, 2, R + 32
    k, v = _tagged(B, Hkv, 5 * R)
    for T in range(1, 4 * R):
        rk0, rv0 = _ring(k, v, T, R)
        rk1, rv1 = _ring(k, v, T + 1, R)
        s = T % RS
        assert np.array_equal(rk1[:, :, s], k[:, :, T])
        assert np.array_equal(rv1[:, :, s // 32, :, s % 32], v[:, :, T])
        for p in range(oracle.n_quant(T + 1, R), T):
            t = p % RS
            assert np.array_equal(rk1[:, :, t], rk0[:, :, t])
            assert np.array_equal(rv1[:, :, t // 32, :, t % 32], rv0[:, :, t // 32, :, t % 32])


def test_pack_carries_the_ring():
    # oracle.pack's ring equals orc_ring on the same positions (live slots)
    w = kvq_synth.Workload("r", 2, 4, 2, 230, n_qry=8, io_dtype="bf16", n_pairs_hi=6,
                           residual=64, seed=77)
    d = kvq_synth.generate(w)
    _, pairs = oracle.select(d["q_sel"], d["k"], w.tokens, w.n_kv_heads, w.io_dtype)
    qz = oracle.quantize(d["k"], d["v"], w.tokens, pairs, residual=w.residual,
                         n_pairs_hi=w.n_pairs_hi, bits_hi=w.bits_hi, io_dtype=w.io_dtype)
    pk = oracle.pack(qz)
    k = np.ascontiguousarray(d["k"], dtype=np.uint16)
    v = np.ascontiguousarray(d["v"], dtype=np.uint16)
    RS = w.residual + 32
    for p in range(qz.nq, w.tokens):
        s = p % RS
        assert np.array_equal(pk["ring_k"][:, :, s], k[:, :, p])
        assert np.array_equal(pk["ring_v"][:, :, s // 32, :, s % 32], v[:, :, p])


# ------------------------------------------------------------ ranking ties

def _tie_data(seed, io_dtype="bf16", T=96, Hq=4, Hkv=2, n_qry=8):
    w = kvq_synth.Workload("ties", 1, Hq, Hkv, T, n_qry=n_qry, io_dtype=io_dtype,
                           outliers="pairs4x8", seed=seed)
    return w, kvq_synth.generate(w)


def _plant_copies(x, src, dsts, swap=()):
    """Copies pair src's two channels into pairs dsts (both channels, every
    row); pairs in `swap` get them exchanged (j <-> j + 64), which keeps
    every pair norm."""
    x = x.copy()
    for j in dsts:
        a, b = x[..., src].copy(), x[..., src + 64].copy()
        if j in swap:
            a, b = b, a
        x[..., j], x[..., j + 64] = a, b
    return x


@pytest.mark.parametrize("scorer", ["pair_norm", "query_aware"])
def test_equal_scores_rank_the_lower_pair_first(scorer):
    for seed in range(4):
        w, d = _tie_data(seed)
        src = int(np.random.default_rng(seed).integers(64))
        dsts = sorted({(src + 9 * i + 3) % 64 for i in range(1, 5)} - {src})
        swap = set(dsts[::2])
        q = _plant_copies(d["q_sel"], src, dsts, swap)
        k = _plant_copies(d["k"], src, dsts, swap)
        if scorer == "pair_norm":
            sums, pairs = oracle.select(q, k, w.tokens, w.n_kv_heads, w.io_dtype)
            score = sums[..., 0, :].astype(np.float64) * sums[..., 1, :].astype(np.float64)
        else:
            score, pairs = oracle.select_qa(q, k, w.tokens, w.n_kv_heads, w.io_dtype)
        tied = sorted(set(dsts) | {src})
        for kh in range(w.n_kv_heads):
            sc = score[0, kh]
            # exchanged channels keep every pair norm, and the query-aware
            # score's two products only swap places in an IEEE sum, which
            # commutes: the tie is exact for both scorers
            assert len({sc[j] for j in tied}) == 1
            rank = list(pairs[0, kh])
            pos = [rank.index(j) for j in tied]
            # the tied pairs sit next to each other, lower id first
            assert pos == list(range(pos[0], pos[0] + len(tied))), (tied, pos)
            # and the whole ranking is sorted by (score descending, id ascending)
            assert rank == sorted(range(64), key=lambda j: (-sc[j], j))


def test_all_pairs_equal_give_the_identity_ranking():
    for scorer in ("pair_norm", "query_aware"):
        w, d = _tie_data(11)
        q = _plant_copies(d["q_sel"], 5, [j for j in range(64) if j != 5])
        k = _plant_copies(d["k"], 5, [j for j in range(64) if j != 5])
        if scorer == "pair_norm":
            _, pairs = oracle.select(q, k, w.tokens, w.n_kv_heads, w.io_dtype)
        else:
            _, pairs = oracle.select_qa(q, k, w.tokens, w.n_kv_heads, w.io_dtype)
        for kh in range(w.n_kv_heads):
            assert list(pairs[0, kh]) == list(range(64))
