"""GPU parity: the HIP library (through the C ABI) against the CPU oracle on
the same seeded inputs.  Indices, sums, codes, scales, zero points and ring
bytes must match bit for bit; attention outputs within max-abs 2e-3 (the
accuracy target for fp16/bf16 I/O with fp32 accumulation).  The bound is
checked on the kernel's fp32 result, read from the single split record (o / l
stored once as fp16, so half an fp16 ulp is added); the 16-bit output may
differ from that result by its own rounding, half an ulp of the output dtype,
which alone exceeds 2e-3 in bf16 once |o| >= 0.5."""
import numpy as np
import pytest
import torch

import kvq_synth
import oracle
from tests._gpu_case import (SM_SCALE, Case, check_output, check_single_split, compare_cache,
                              half_ulp, lse_merge, single_split)

pytestmark = pytest.mark.gpu

ATOL = 2e-3

SMALL = [
    kvq_synth.WORKLOADS[0],  # tiny: fp16, 8 pairs @4-bit, R = 32, T = 512
    kvq_synth.Workload("gqa4-ragged", 2, 8, 2, 1000, n_qry=16, io_dtype="bf16",
                       outliers="pct2x10", n_pairs_hi=6, residual=128, seed=21),
    kvq_synth.Workload("raw16-salient", 1, 8, 2, 700, n_qry=8, io_dtype="bf16",
                       n_pairs_hi=6, bits_hi=16, residual=64, seed=22),
    kvq_synth.Workload("no-salient-g1", 1, 3, 3, 333, n_qry=8, io_dtype="fp16",
                       n_pairs_hi=0, residual=32, seed=23),
    kvq_synth.Workload("g16", 1, 16, 1, 300, n_qry=4, io_dtype="bf16",
                       n_pairs_hi=8, residual=32, seed=24),
    # the 1.5-bit point (32 pairs at 2 bits, 32 at 1 bit) and a 4/2/1-bit mix
    kvq_synth.Workload("one-bit-1p5", 1, 8, 2, 420, n_qry=8, io_dtype="bf16",
                       outliers="pct2x10", n_pairs_hi=0, n_pairs_lo1=32, residual=64, seed=25),
    kvq_synth.Workload("mixed-4-2-1", 2, 4, 1, 260, n_qry=8, io_dtype="fp16",
                       n_pairs_hi=6, n_pairs_lo1=16, residual=32, seed=26),
]


def _ids(w):
    return w.name


@pytest.mark.parametrize("w", SMALL, ids=_ids)
def test_select_bit_exact(w):
    case = Case(w)
    sums, pairs = case.oracle_select()
    g = case.gpu_bytes()
    bad = np.argwhere(g["sums"] != sums)
    if len(bad):
        i = tuple(bad[0])
        print("sums mismatch at %d places, first %s gpu %d oracle %d" % (
            len(bad), i, g["sums"][i], sums[i]))
    assert np.array_equal(g["sums"], sums)
    assert np.array_equal(g["pairs"], pairs)


@pytest.mark.parametrize("w", SMALL, ids=_ids)
def test_quant_bit_exact(w):
    case = Case(w)
    qz = case.oracle_quant()
    assert qz.nq > 0
    compare_cache(case, qz, qz.nq // 32)


@pytest.mark.parametrize("w", SMALL, ids=_ids)
@pytest.mark.parametrize("n_splits", [1, 3, 64])
def test_decode_matches_oracle(w, n_splits):
    case = Case(w)
    qz = case.oracle_quant()
    q = case.d["q_dec"][:, :, 0]
    ref = oracle.attention(qz, q, SM_SCALE)
    got, part = case.decode(q, n_splits, partials=True)
    err = check_output(got, ref, w.io_dtype, ATOL)
    msg = "%s S=%d max|err| %.3g max|o| %.3g" % (w.name, n_splits, err, np.abs(ref).max())
    if n_splits == 1:
        e32 = check_single_split(part, ref, ATOL)
        msg += " split-record max|err| %.3g" % e32
    print(msg)


@pytest.mark.parametrize("T", [1, 31, 32, 33, 127, 160, 161, 193])
def test_decode_edge_lengths(T):
    # T < R (ring only), T = 1, and lengths either side of group boundaries
    w = kvq_synth.Workload("edge", 1, 4, 1, 200, n_qry=8, io_dtype="bf16", n_pairs_hi=6,
                           residual=128, seed=30)
    case = Case(w, T=T)
    qz = case.oracle_quant()
    if qz.nq:
        compare_cache(case, qz, qz.nq // 32)
    q = case.d["q_dec"][:, :, 0]
    ref = oracle.attention(qz, q, SM_SCALE)
    for S in (1, 5):
        got, part = case.decode(q, S, partials=True)
        check_output(got, ref, w.io_dtype, ATOL)
        if S == 1:
            check_single_split(part, ref, ATOL)


def test_all_sixteen_bit_mode_matches_textbook():
    # residual window over every token: the kernel reproduces plain attention
    w = kvq_synth.Workload("hp", 1, 8, 2, 250, n_qry=8, io_dtype="bf16", residual=256, seed=31)
    case = Case(w)
    q = case.d["q_dec"][:, :, 0]
    out, part = case.decode(q, 1, partials=True)
    out32 = single_split(part)
    qf = kvq_synth.bits_to_f64(q, "bf16")
    K = kvq_synth.bits_to_f64(case.d["k"][:, :, :250], "bf16")
    V = kvq_synth.bits_to_f64(case.d["v"][:, :, :250], "bf16")
    for h in range(8):
        lg = SM_SCALE * (K[0, h // 4] @ qf[0, h])
        p = np.exp(lg - lg.max())
        ref = (p / p.sum()) @ V[0, h // 4]
        assert np.all(np.abs(out32[0, h] - ref) <= 1e-4)
        assert np.all(np.abs(out[0, h] - ref) <= 1e-4 + half_ulp(ref, "bf16"))


def _dequantized_values(qz) -> np.ndarray:
    """v^ of every held token as fp64 [B][Hkv][T][128]: z + s * code for
    quantized tokens, the raw 16-bit value for ring tokens."""
    v = kvq_synth.bits_to_f64(qz.v[:, :, :qz.T], qz.io_dtype).copy()
    nq = qz.nq
    if nq:
        B, Hkv = v.shape[:2]
        ng = nq // 32
        s = qz.vs[:, :, :ng].astype(np.uint16).view(np.float16).astype(np.float64)
        z = qz.vz[:, :, :ng].astype(np.uint16).view(np.float16).astype(np.float64)
        c = qz.vcodes[:, :, :ng].astype(np.float64)  # [B][Hkv][ng][32][128]
        deq = np.repeat(z, 32, axis=-1) + np.repeat(s, 32, axis=-1) * c
        v[:, :, :nq] = deq.reshape(B, Hkv, nq, 128)
    return v


def test_split_counts_agree():
    # Every split count meets the oracle's 2e-3.  Between split counts the
    # fp32 records, merged on the host in fp64, differ only through the fp16
    # rounding of the softmax weights p = 2^(x - m), whose reference m is the
    # running max of the split: each weight moves by at most a relative
    # u = 2^-11, which moves a weighted mean by at most u * max |v - o| (the
    # same rounded weights form the numerator and the denominator), so two
    # split counts differ by at most 2u * max |v - o|.
    w = SMALL[1]
    case = Case(w)
    qz = case.oracle_quant()
    q = case.d["q_dec"][:, :, 0]
    ref = oracle.attention(qz, q, SM_SCALE)
    _, part1 = case.decode(q, 1, partials=True)
    base = single_split(part1)
    vhat = _dequantized_values(qz)  # [B][Hkv][T][128]
    G = w.group_size
    spread = np.array([[np.abs(vhat[b, h // G] - ref[b, h]).max() for h in range(w.n_q_heads)]
                       for b in range(w.batch)])[..., None]
    worst = 0.0
    for S in (7, 32, 256, 1024):  # 1024: the largest accepted
        got, part = case.decode(q, S, partials=True)
        check_output(got, ref, w.io_dtype, ATOL)
        merged = lse_merge(part)
        d = np.abs(merged - base)
        assert np.all(d <= 2 * 2.0 ** -11 * spread + 1e-6), "S=%d: %.3g" % (S, d.max())
        # the kernel's own merge is that combine rounded once to the io dtype
        assert np.all(np.abs(got - merged) <= half_ulp(merged, w.io_dtype) + 1e-6)
        worst = max(worst, float(d.max()))
    print("split counts: largest difference of merged records %.3g" % worst)


def test_deterministic():
    case = Case(SMALL[1])
    q = case.d["q_dec"][:, :, 0]
    a, b = case.decode(q, 16), case.decode(q, 16)
    assert np.array_equal(a, b)


def test_append_equals_prefill():
    # prefill T0, then n appends == prefill of T0 + n (same rank table)
    w = kvq_synth.Workload("app", 2, 8, 2, 200, n_qry=8, n_app=75, io_dtype="bf16",
                           n_pairs_hi=6, residual=64, seed=32)
    case = Case(w, T=w.tokens, max_tokens=w.max_tokens)
    from decode_attention_select_amd import kvq
    from tests._gpu_case import dev
    kn = dev(np.ascontiguousarray(case.d["k"][:, :, w.tokens:]))
    vn = dev(np.ascontiguousarray(case.d["v"][:, :, w.tokens:]))
    q = case.d["q_dec"][:, :, 0]
    for i in range(w.n_app):
        kvq.kvq_append(case.layout, kn[:, :, i].contiguous(), vn[:, :, i].contiguous(),
                       case.cache.struct)
        if i in (0, 40, w.n_app - 1):
            T = w.tokens + i + 1
            qz = case.oracle_quant(T=T)
            ref = oracle.attention(qz, q, SM_SCALE)
            check_output(case.decode(q, 8), ref, w.io_dtype, ATOL)
            _, part = case.decode(q, 1, partials=True)
            check_single_split(part, ref, ATOL)
    torch.cuda.synchronize()
    T = w.tokens + w.n_app
    qz = case.oracle_quant(T=T)
    compare_cache(case, qz, qz.nq // 32)
    assert kvq.kvq_check(case.cache.struct) == 0


def test_append_at_capacity_sets_error():
    w = kvq_synth.Workload("cap", 1, 4, 1, 96, n_qry=4, io_dtype="bf16", residual=32, seed=33)
    case = Case(w, T=96, max_tokens=96)
    from decode_attention_select_amd import kvq
    from tests._gpu_case import dev
    before = case.gpu_bytes()
    z = dev(np.zeros((1, 1, 128), np.uint16))
    kvq.kvq_append(case.layout, z, z, case.cache.struct)
    assert kvq.kvq_check(case.cache.struct) == 1
    after = case.gpu_bytes()
    for k in before:
        assert np.array_equal(before[k], after[k])


@pytest.mark.parametrize("n_splits", [2, 7, 64])
def test_workspace_reuse_sees_fresh_records(n_splits):
    # split records cross workgroups through the workspace; a reused workspace
    # must never feed one call's merge with another call's records
    from decode_attention_select_amd import kvq
    from tests._gpu_case import dev
    case = Case(SMALL[1])
    qs = [case.d["q_dec"][:, :, 0], np.ascontiguousarray(case.d["q_sel"][:, :, 0])]
    fresh = [case.decode(q, n_splits) for q in qs]
    ws = torch.zeros(kvq.kvq_workspace_bytes(case.layout, n_splits), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((case.w.batch, case.w.n_q_heads, 128), dtype=torch.int16, device="cuda")
    qd = [dev(q) for q in qs]
    for i in range(40):
        kvq.kvq_decode_attn(case.layout, qd[i % 2], case.cache.struct, SM_SCALE, n_splits, ws, out)
        got = kvq_synth.bits_to_f64(out.cpu().numpy().view(np.uint16), case.w.io_dtype)
        assert np.array_equal(got, fresh[i % 2]), "call %d" % i


def test_workspace_reuse_across_split_counts():
    # one workspace, sized for the largest call, serves calls with split
    # counts 64, 7, 64, 1024, 1, 64 in turn: the split counters sit at the
    # start of every layout, so each call finds them at zero; every output
    # equals that of a fresh workspace
    from decode_attention_select_amd import kvq
    from tests._gpu_case import dev
    case = Case(SMALL[1])
    q = case.d["q_dec"][:, :, 0]
    seq = [64, 7, 64, 1024, 1, 64]
    fresh = {S: case.decode(q, S) for S in set(seq)}
    ws = torch.zeros(max(kvq.kvq_workspace_bytes(case.layout, S) for S in seq), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((case.w.batch, case.w.n_q_heads, 128), dtype=torch.int16, device="cuda")
    qd = dev(q)
    for i, S in enumerate(seq):
        out.fill_(0x7fc0)
        kvq.kvq_decode_attn(case.layout, qd, case.cache.struct, SM_SCALE, S, ws, out)
        got = kvq_synth.bits_to_f64(out.cpu().numpy().view(np.uint16), case.w.io_dtype)
        assert np.array_equal(got, fresh[S]), "call %d (S=%d)" % (i, S)
    # the counters are back at zero after the last call
    t = ws[:case.w.batch * case.w.n_kv_heads * 256].cpu().numpy().view(np.uint32)
    assert not t.any()


@pytest.mark.parametrize("g0,g1", [(0, 3), (2, 100), (0, 1 << 20)])
def test_shrink_matches_oracle(g0, g1):
    # salient 4-bit codes shrunk in place to 2 bits: bytes equal the oracle's
    # shrunk cache; decoding over it matches the oracle's attention
    from decode_attention_select_amd import kvq
    w = kvq_synth.Workload("shrink", 2, 8, 2, 420, n_qry=8, io_dtype="bf16",
                           outliers="pct2x10", n_pairs_hi=6, residual=64, seed=42)
    case = Case(w)
    kvq.kvq_shrink(case.layout, case.cache.struct, g0, g1)
    torch.cuda.synchronize()
    qz = oracle.shrink(case.oracle_quant(), g0, g1)
    compare_cache(case, qz, qz.nq // 32)
    q = case.d["q_dec"][:, :, 0]
    ref = oracle.attention(qz, q, SM_SCALE)
    check_output(case.decode(q, 8), ref, w.io_dtype, ATOL)
    _, part = case.decode(q, 1, partials=True)
    check_single_split(part, ref, ATOL)


@pytest.mark.parametrize("w", SMALL, ids=_ids)
def test_select_qa_bit_exact(w):
    # the query-aware channel score: scores (as double bits) and ranks
    from decode_attention_select_amd import kvq
    from tests._gpu_case import dev
    case = Case(w)
    kvq.kvq_select_pairs_qa(case.layout, case.q_sel, w.n_qry, case.k_sel, w.tokens,
                            case.cache.struct)
    torch.cuda.synchronize()
    S, pairs = oracle.select_qa(case.d["q_sel"], case.d["k"], w.tokens, w.n_kv_heads, w.io_dtype)
    g = case.gpu_bytes()
    assert np.array_equal(g["sums"][:, :, 0], S.view(np.uint64))
    assert np.all(g["sums"][:, :, 1] == 0)
    assert np.array_equal(g["pairs"], pairs)


@pytest.mark.parametrize("w", SMALL, ids=_ids)
@pytest.mark.parametrize("n_keep", [1, 2, 3, 5, 7])
def test_pruned_decode_matches_oracle(w, n_keep):
    # query-channel pruning: logits over the kept 16-channel key runs only
    # (odd counts leave half of the last contraction empty)
    case = Case(w)
    if case.pruned_unsupported(3, n_keep):
        return  # the dense 1-bit layout: ENOTSUP, checked
    qz = case.oracle_quant()
    q = case.d["q_dec"][:, :, 0]
    ref = oracle.attention_pruned(qz, q, SM_SCALE, n_keep)
    for S in (1, 7):
        err = check_output(case.decode_pruned(q, S, n_keep), ref, w.io_dtype, ATOL)
        print("%s keep=%d S=%d max|err| %.3g" % (w.name, n_keep, S, err))


@pytest.mark.parametrize("w", [SMALL[1], SMALL[4], SMALL[6]], ids=_ids)
def test_pruned_choice_ties_to_the_lower_run(w):
    # runs 2 and 5 carry the same magnitudes (run 5 a permutation of run 2,
    # both x8 above the other runs), so their energies tie exactly and a
    # keep-1 decode must keep run 2, the lower one
    case = Case(w)
    if case.pruned_unsupported(3, 1):
        return
    qz = case.oracle_quant()
    qf = kvq_synth.bits_to_f64(case.d["q_dec"][:, :, 0], w.io_dtype)
    perm = np.random.default_rng(7).permutation(16)
    qp = qf.copy()
    qp[:, :, 32:48] *= 8
    qp[:, :, 80:96] = qp[:, :, 32:48][:, :, perm]
    q = kvq_synth.to_bits(qp, w.io_dtype)
    keep = oracle.prune_chunks(q, w.n_kv_heads, w.io_dtype, 1)
    assert keep[..., 2].all() and not keep[..., 5].any()
    ref = oracle.attention_pruned(qz, q, SM_SCALE, 1)
    # the output a choice of run 5 would give (the same query values, run 2
    # not kept): far from ref, so a wrong tie order fails the check below
    q5 = qp.copy()
    q5[:, :, 32:48] = 0
    wrong = oracle.attention_pruned(qz, kvq_synth.to_bits(q5, w.io_dtype), SM_SCALE, 1)
    assert np.abs(wrong - ref).max() > 10 * ATOL
    for S in (1, 3):
        err = check_output(case.decode_pruned(q, S, 1), ref, w.io_dtype, ATOL)
        print("%s tied runs S=%d max|err| %.3g" % (w.name, S, err))


def test_pruned_keep_all_equals_unpruned():
    w = SMALL[1]
    case = Case(w)
    q = case.d["q_dec"][:, :, 0]
    a = case.decode(q, 5)
    b = case.decode_pruned(q, 5, 8)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("T", [1, 33, 161])
def test_pruned_decode_edge_lengths(T):
    # ring-only and ragged lengths: ring keys are pruned as well
    w = kvq_synth.Workload("edge", 1, 4, 1, 200, n_qry=8, io_dtype="bf16", n_pairs_hi=6,
                           residual=128, seed=30)
    case = Case(w, T=T)
    qz = case.oracle_quant()
    q = case.d["q_dec"][:, :, 0]
    for n_keep in (1, 4, 5):
        ref = oracle.attention_pruned(qz, q, SM_SCALE, n_keep)
        check_output(case.decode_pruned(q, 3, n_keep), ref, w.io_dtype, ATOL)


VMIX = [
    kvq_synth.Workload("vmix-1x4", 2, 8, 2, 700, n_qry=8, io_dtype="bf16", outliers="pct2x10",
                       n_pairs_hi=6, residual=64, seed=81, n_vblk_hi=1, bits_vhi=4),
    kvq_synth.Workload("vmix-2x3-fp16", 1, 4, 1, 420, n_qry=8, io_dtype="fp16",
                       n_pairs_hi=8, residual=32, seed=82, n_vblk_hi=2, bits_vhi=3),
    kvq_synth.Workload("vmix-3x4-raw16", 1, 8, 2, 333, n_qry=8, io_dtype="bf16",
                       n_pairs_hi=6, bits_hi=16, residual=32, seed=83, n_vblk_hi=3, bits_vhi=4),
    kvq_synth.Workload("vmix-4x4-lo1", 1, 8, 2, 300, n_qry=8, io_dtype="bf16",
                       n_pairs_hi=0, n_pairs_lo1=32, residual=64, seed=84, n_vblk_hi=4,
                       bits_vhi=4),
]


@pytest.mark.parametrize("w", VMIX, ids=_ids)
def test_two_value_precisions_bit_exact_and_decode(w):
    # SemKV reading: each group's 8 n tokens of largest key magnitude, stored
    # first, at 3 or 4 bits; bytes (order headers and high digits included)
    # equal the oracle's, decoding matches its attention
    case = Case(w)
    qz = case.oracle_quant()
    compare_cache(case, qz, qz.nq // 32)
    q = case.d["q_dec"][:, :, 0]
    ref = oracle.attention(qz, q, SM_SCALE)
    for S in (1, 9):
        got, part = case.decode(q, S, partials=True)
        err = check_output(got, ref, w.io_dtype, ATOL)
        if S == 1:
            check_single_split(part, ref, ATOL)
        print("%s S=%d max|err| %.3g" % (w.name, S, err))


def test_two_value_precisions_append_equals_prefill():
    from decode_attention_select_amd import kvq
    from tests._gpu_case import dev
    w = VMIX[0]
    T0 = 100
    case = Case(w, T=T0, max_tokens=w.tokens)
    for t in range(T0, w.tokens):
        kvq.kvq_append(case.layout, dev(np.ascontiguousarray(case.d["k"][:, :, t])),
                       dev(np.ascontiguousarray(case.d["v"][:, :, t])), case.cache.struct)
    torch.cuda.synchronize()
    case.T = w.tokens
    qz = case.oracle_quant()
    compare_cache(case, qz, qz.nq // 32)


@pytest.mark.parametrize("w", VMIX, ids=_ids)
def test_two_value_precisions_with_pruned_decode(w):
    # pruning touches only the key side, the high value digits only the value
    # side: the pruned oracle over the two-precision cache
    case = Case(w)
    if case.pruned_unsupported():
        return  # the dense 1-bit layout: ENOTSUP, checked
    qz = case.oracle_quant()
    q = case.d["q_dec"][:, :, 0]
    for n_keep in (1, 4, 5, 6):
        ref = oracle.attention_pruned(qz, q, SM_SCALE, n_keep)
        for S in (1, 6):
            check_output(case.decode_pruned(q, S, n_keep), ref, w.io_dtype, ATOL)


@pytest.mark.parametrize("T", [1, 33, 95, 161])
def test_two_value_precisions_edge_lengths(T):
    # ring-only, one group and ragged lengths with kept value blocks
    w = kvq_synth.Workload("edge-vmix", 1, 4, 1, 200, n_qry=8, io_dtype="bf16", n_pairs_hi=6,
                           residual=32, seed=33, n_vblk_hi=1, bits_vhi=3)
    case = Case(w, T=T)
    qz = case.oracle_quant()
    if qz.nq:
        compare_cache(case, qz, qz.nq // 32)
    q = case.d["q_dec"][:, :, 0]
    ref = oracle.attention(qz, q, SM_SCALE)
    for S in (1, 5):
        got, part = case.decode(q, S, partials=True)
        check_output(got, ref, w.io_dtype, ATOL)
        if S == 1:
            check_single_split(part, ref, ATOL)


def _plant_zeros_and_ties(d, T, seed):
    """Keys and values with zero minima of both signs and with equal key
    magnitudes: in every group, some key channels and value channel groups
    are made non-negative with a -0 and a +0 planted in either order (the
    quantizer's zero point takes the sign of the first zero by position),
    and some tokens repeat another token's key row (equal ranking scores,
    decided by position) or have an all-zero key row."""
    rng = np.random.default_rng(seed)
    k, v = d["k"].copy(), d["v"].copy()
    B, H = k.shape[:2]
    for b in range(B):
        for h in range(H):
            for g in range(T // 32):
                base = 32 * g
                for c in rng.choice(128, 12, replace=False):
                    k[b, h, base:base + 32, c] &= 0x7FFF
                    p1, p2 = sorted(rng.choice(32, 2, replace=False))
                    s = rng.integers(2)
                    k[b, h, base + p1, c] = 0x8000 if s else 0x0000
                    k[b, h, base + p2, c] = 0x0000 if s else 0x8000
                for t in rng.choice(32, 6, replace=False):
                    j = rng.integers(4)
                    v[b, h, base + t, 32 * j:32 * j + 32] &= 0x7FFF
                    p1, p2 = sorted(rng.choice(32, 2, replace=False))
                    s = rng.integers(2)
                    v[b, h, base + t, 32 * j + p1] = 0x8000 if s else 0x0000
                    v[b, h, base + t, 32 * j + p2] = 0x0000 if s else 0x8000
                a, c2, z1, z2 = rng.choice(32, 4, replace=False)
                k[b, h, base + max(a, c2)] = k[b, h, base + min(a, c2)]
                k[b, h, base + z1] = 0
                k[b, h, base + z2] = 0x8000
    out = dict(d)
    out["k"], out["v"] = k, v
    return out


ZT = [
    kvq_synth.Workload("zeros-ties-vmix", 1, 8, 2, 420, n_qry=8, io_dtype="bf16",
                       n_pairs_hi=6, residual=32, seed=91, n_vblk_hi=2, bits_vhi=4),
    kvq_synth.Workload("zeros-ties-fp16", 1, 8, 2, 420, n_qry=8, io_dtype="fp16",
                       n_pairs_hi=6, residual=32, seed=92),
]


@pytest.mark.parametrize("w", ZT, ids=_ids)
@pytest.mark.parametrize("path", ["prefill", "append"])
def test_signed_zero_minima_and_tied_scores(w, path):
    from decode_attention_select_amd import kvq
    from tests._gpu_case import dev
    data = _plant_zeros_and_ties(kvq_synth.generate(w), w.tokens, w.seed)
    if path == "prefill":
        case = Case(w, data=data)
    else:
        T0 = 40
        case = Case(w, T=T0, max_tokens=w.tokens, data=data)
        for t in range(T0, w.tokens):
            kvq.kvq_append(case.layout, dev(np.ascontiguousarray(data["k"][:, :, t])),
                           dev(np.ascontiguousarray(data["v"][:, :, t])), case.cache.struct)
        torch.cuda.synchronize()
        case.T = w.tokens
    qz = case.oracle_quant()
    # the planted zero minima reach the oracle's zero points with both signs
    nq = qz.nq // 32
    assert np.any(qz.kz[:, :, :nq] == 0x8000) and np.any(qz.kz[:, :, :nq] == 0)
    assert np.any(qz.vz[:, :, :nq] == 0x8000) and np.any(qz.vz[:, :, :nq] == 0)
    compare_cache(case, qz, nq)
    q = case.d["q_dec"][:, :, 0]
    got = case.decode(q, 4)
    check_output(got, oracle.attention(qz, q, SM_SCALE), w.io_dtype, ATOL)


def test_state_no_call_wrote_stays_in_bounds():
    # a length beyond the capacity decodes as the capacity; a negative one is
    # reported by append and decodes as an empty cache
    from decode_attention_select_amd import kvq
    from tests._gpu_case import dev
    w = kvq_synth.Workload("cap", 1, 4, 1, 96, n_qry=4, io_dtype="bf16", residual=32, seed=33)
    case = Case(w, T=96, max_tokens=96)
    q = case.d["q_dec"][:, :, 0]
    want = case.decode(q, 3)
    lens = case.cache["len"].view(torch.int32)
    lens.fill_(96 + 1000)
    assert np.array_equal(case.decode(q, 3), want)
    lens.fill_(-5)
    z = dev(np.zeros((1, 1, 128), np.uint16))
    kvq.kvq_append(case.layout, z, z, case.cache.struct)
    assert kvq.kvq_check(case.cache.struct) == 2
    assert np.all(case.gpu_bytes()["len"] == -5)
    assert np.all(case.decode(q, 3) == 0)
    # two value precisions: values quantized over order bytes no key pass
    # wrote (0xFF) read inside their group; the usual order then gives the
    # oracle's bytes
    wv = VMIX[0]
    cv = Case(wv)
    cv.cache["v_hi"].fill_(0xFF)
    kvq.kvq_quant_values(cv.layout, dev(cv.d["v"][:, :, :cv.T]), cv.T, cv.cache.struct)
    torch.cuda.synchronize()
    kvq.kvq_quant_keys(cv.layout, dev(cv.d["k"][:, :, :cv.T]), cv.T, cv.cache.struct)
    kvq.kvq_quant_values(cv.layout, dev(cv.d["v"][:, :, :cv.T]), cv.T, cv.cache.struct)
    torch.cuda.synchronize()
    qz = cv.oracle_quant()
    compare_cache(cv, qz, qz.nq // 32)


FUSED = [
    kvq_synth.Workload("fused-gqa4", 2, 8, 2, 330, n_qry=8, io_dtype="bf16", outliers="pct2x10",
                       n_pairs_hi=6, residual=64, seed=101),
    kvq_synth.Workload("fused-fp16-g1", 1, 3, 3, 200, n_qry=8, io_dtype="fp16", n_pairs_hi=8,
                       residual=32, seed=102),
    kvq_synth.Workload("fused-raw16", 1, 8, 2, 230, n_qry=8, io_dtype="bf16", n_pairs_hi=6,
                       bits_hi=16, residual=32, seed=103),
    kvq_synth.Workload("fused-lo1-vmix", 1, 8, 2, 230, n_qry=8, io_dtype="bf16", n_pairs_hi=0,
                       n_pairs_lo1=32, residual=32, seed=104, n_vblk_hi=2, bits_vhi=4),
]


@pytest.mark.parametrize("w", FUSED, ids=_ids)
def test_append_and_decode_in_one_launch(w):
    # every step's output against the oracle of the fused call (the group
    # packed by a step is attended at 16 bits in that step), then every byte
    # against the prefill of the same tokens
    from decode_attention_select_amd import kvq
    from tests._gpu_case import dev
    T0 = w.tokens - 100
    case = Case(w, T=T0, max_tokens=w.tokens)
    pairs = case.oracle_select()[1]
    S = 3
    ws = torch.zeros(kvq.kvq_workspace_bytes(case.layout, S), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.int16, device="cuda")
    q_bits = case.d["q_dec"][:, :, 0]
    q = dev(q_bits)
    packed = 0
    for t in range(T0, w.tokens):
        kvq.kvq_append_decode_attn(case.layout, dev(np.ascontiguousarray(case.d["k"][:, :, t])),
                                   dev(np.ascontiguousarray(case.d["v"][:, :, t])), q,
                                   case.cache.struct, SM_SCALE, S, ws, out)
        qz = case.oracle_quant(T=t + 1, pairs=pairs)
        packed += oracle.n_quant(t + 1, w.residual) > oracle.n_quant(t, w.residual)
        got = kvq_synth.bits_to_f64(out.cpu().numpy().view(np.uint16), w.io_dtype)
        check_output(got, oracle.attention_after_append(qz, q_bits, SM_SCALE), w.io_dtype, ATOL)
    assert packed >= 2
    assert kvq.kvq_check(case.cache.struct) == 0
    case.T = w.tokens
    qz = case.oracle_quant(pairs=pairs)
    compare_cache(case, qz, qz.nq // 32)


def test_append_and_decode_at_capacity():
    # a full cache: error bit 0, nothing changes, the output is the plain decode
    from decode_attention_select_amd import kvq
    from tests._gpu_case import dev
    w = kvq_synth.Workload("cap", 1, 4, 1, 96, n_qry=4, io_dtype="bf16", residual=32, seed=33)
    case = Case(w, T=96, max_tokens=96)
    q_bits = case.d["q_dec"][:, :, 0]
    want = case.decode(q_bits, 3)
    before = case.gpu_bytes()
    ws = torch.zeros(kvq.kvq_workspace_bytes(case.layout, 3), dtype=torch.uint8, device="cuda")
    out = torch.empty((1, 4, 128), dtype=torch.int16, device="cuda")
    z = dev(np.zeros((1, 1, 128), np.uint16))
    kvq.kvq_append_decode_attn(case.layout, z, z, dev(q_bits), case.cache.struct, SM_SCALE, 3,
                               ws, out)
    assert kvq.kvq_check(case.cache.struct) == 1
    assert np.array_equal(kvq_synth.bits_to_f64(out.cpu().numpy().view(np.uint16), "bf16"), want)
    after = case.gpu_bytes()
    for k in before:
        assert np.array_equal(before[k], after[k])


@pytest.mark.parametrize("w", [
    kvq_synth.Workload("fused-from-one", 1, 8, 2, 100, n_qry=8, io_dtype="bf16", n_pairs_hi=6,
                       residual=32, seed=105),
    kvq_synth.Workload("fused-from-one-vmix", 1, 4, 1, 100, n_qry=8, io_dtype="fp16",
                       n_pairs_hi=6, residual=32, seed=106, n_vblk_hi=1, bits_vhi=3),
], ids=_ids)
def test_append_and_decode_from_one_token(w):
    # ring-only steps, then the first two packed groups (R = 32: at T = 64, 96)
    from decode_attention_select_amd import kvq
    from tests._gpu_case import dev
    case = Case(w, T=1, max_tokens=w.tokens)
    pairs = case.oracle_select()[1]
    ws = torch.zeros(kvq.kvq_workspace_bytes(case.layout, 2), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.int16, device="cuda")
    q_bits = case.d["q_dec"][:, :, 0]
    q = dev(q_bits)
    for t in range(1, w.tokens):
        kvq.kvq_append_decode_attn(case.layout, dev(np.ascontiguousarray(case.d["k"][:, :, t])),
                                   dev(np.ascontiguousarray(case.d["v"][:, :, t])), q,
                                   case.cache.struct, SM_SCALE, 2, ws, out)
        qz = case.oracle_quant(T=t + 1, pairs=pairs)
        got = kvq_synth.bits_to_f64(out.cpu().numpy().view(np.uint16), w.io_dtype)
        check_output(got, oracle.attention_after_append(qz, q_bits, SM_SCALE), w.io_dtype, ATOL)
    assert kvq.kvq_check(case.cache.struct) == 0
    case.T = w.tokens
    qz = case.oracle_quant(pairs=pairs)
    assert qz.nq == 64
    compare_cache(case, qz, qz.nq // 32)


DEGEN = [
    kvq_synth.Workload("degenerate-bf16", 2, 8, 2, 300, n_qry=8, io_dtype="bf16",
                       n_pairs_hi=6, residual=64, seed=111),
    kvq_synth.Workload("degenerate-fp16", 2, 8, 2, 300, n_qry=8, io_dtype="fp16",
                       n_pairs_hi=6, bits_hi=16, residual=64, seed=112),
]


@pytest.mark.parametrize("w", DEGEN, ids=_ids)
def test_degenerate_groups(w):
    # zero steps (s = 0): constant key channels, a group of identical key
    # rows, constant value groups; an all-zero query for one sequence
    # (uniform weights)
    rng = np.random.default_rng(w.seed)
    d = kvq_synth.generate(w)
    kf = kvq_synth.bits_to_f64(d["k"], w.io_dtype)
    vf = kvq_synth.bits_to_f64(d["v"], w.io_dtype)
    for c in rng.choice(128, 10, replace=False):
        kf[:, :, 0:32, c] = 0.75
    kf[:, :, 32:64, :] = kf[:, :, 32:33, :]
    for t in rng.choice(np.arange(64, 192), 12, replace=False):
        vf[:, :, t, 32:64] = -1.5
    d["k"] = kvq_synth.to_bits(kf, w.io_dtype)
    d["v"] = kvq_synth.to_bits(vf, w.io_dtype)
    q = d["q_dec"][:, :, 0].copy()
    q[1] = 0
    case = Case(w, data=d)
    qz = case.oracle_quant()
    assert np.any(qz.ks[:, :, :qz.nq // 32] == 0) and np.any(qz.vs[:, :, :qz.nq // 32] == 0)
    compare_cache(case, qz, qz.nq // 32)
    ref = oracle.attention(qz, q, SM_SCALE)
    for S in (1, 4):
        check_output(case.decode(q, S), ref, w.io_dtype, ATOL)


@pytest.mark.parametrize("w", DEGEN, ids=_ids)
def test_values_at_the_input_limit(w):
    # values up to the documented limit |x| <= 32752: every byte bit-exact
    # (scales near the top of fp16), outputs finite and within 2^-8 of each
    # output row's largest magnitude (the fp16 weights p*s carry 2^-11)
    from tests._gpu_case import half_ulp
    rng = np.random.default_rng(w.seed + 1)
    d = kvq_synth.generate(w)
    vf = kvq_synth.bits_to_f64(d["v"], w.io_dtype)
    big = 32752.0 if w.io_dtype == "fp16" else 32512.0  # largest value <= 32752 in the format
    for t in rng.choice(w.tokens, 20, replace=False):
        vf[:, :, t, rng.integers(128)] = big * (1 if rng.integers(2) else -1)
    d["v"] = kvq_synth.to_bits(vf, w.io_dtype)
    case = Case(w, data=d)
    qz = case.oracle_quant()
    compare_cache(case, qz, qz.nq // 32)
    q = d["q_dec"][:, :, 0]
    ref = oracle.attention(qz, q, SM_SCALE)
    for S in (1, 4):
        got = case.decode(q, S)
        assert np.all(np.isfinite(got))
        bound = (ATOL + half_ulp(ref, w.io_dtype) +
                 2.0 ** -8 * np.abs(ref).max(axis=-1, keepdims=True))
        assert np.all(np.abs(got - ref) <= bound), np.abs(got - ref).max()


@pytest.mark.parametrize("w", DEGEN, ids=_ids)
def test_keys_and_queries_at_the_input_limit(w):
    # keys up to the input limit and queries in the hundreds: every byte
    # bit-exact and every output finite (the products q*s, formed in fp16, are
    # kept in range by a power-of-two scaling of each head's query).  With
    # logits this large the softmax is nearly one-hot and its conditioning,
    # not the kernel, sets the error, so only finiteness and the bytes are
    # checked here.
    rng = np.random.default_rng(w.seed + 2)
    d = kvq_synth.generate(w)
    kf = kvq_synth.bits_to_f64(d["k"], w.io_dtype)
    big = 32752.0 if w.io_dtype == "fp16" else 32512.0
    for t in rng.choice(w.tokens, 20, replace=False):
        kf[:, :, t, rng.integers(128)] = big * (1 if rng.integers(2) else -1)
    d["k"] = kvq_synth.to_bits(kf, w.io_dtype)
    qf = kvq_synth.bits_to_f64(d["q_dec"][:, :, 0], w.io_dtype) * 256
    q = kvq_synth.to_bits(qf, w.io_dtype)
    case = Case(w, data=d)
    qz = case.oracle_quant()
    compare_cache(case, qz, qz.nq // 32)
    for S in (1, 4):
        assert np.all(np.isfinite(case.decode(q, S)))


def test_capacity_within_the_residual_window():
    # max_tokens <= R + 31: the cache has no quantized-group storage at all
    # (its own kernel variant) and every token lives in the ring: prefill,
    # decode, one-launch steps up to the capacity, then the capacity error
    from decode_attention_select_amd import kvq
    from tests._gpu_case import dev
    w = kvq_synth.Workload("ring-only-cap", 1, 8, 2, 60, n_qry=8, io_dtype="bf16", n_pairs_hi=6,
                           residual=32, seed=121)
    case = Case(w, T=40, max_tokens=60)
    assert case.NG == 0
    pairs = case.oracle_select()[1]
    q_bits = case.d["q_dec"][:, :, 0]
    qz = case.oracle_quant(pairs=pairs)
    for S in (1, 3):
        check_output(case.decode(q_bits, S), oracle.attention(qz, q_bits, SM_SCALE), w.io_dtype,
                     ATOL)
    ws = torch.zeros(kvq.kvq_workspace_bytes(case.layout, 3), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.int16, device="cuda")
    q = dev(q_bits)
    for t in range(40, 60):
        kvq.kvq_append_decode_attn(case.layout, dev(np.ascontiguousarray(case.d["k"][:, :, t])),
                                   dev(np.ascontiguousarray(case.d["v"][:, :, t])), q,
                                   case.cache.struct, SM_SCALE, 3, ws, out)
        qz = case.oracle_quant(T=t + 1, pairs=pairs)
        got = kvq_synth.bits_to_f64(out.cpu().numpy().view(np.uint16), w.io_dtype)
        check_output(got, oracle.attention_after_append(qz, q_bits, SM_SCALE), w.io_dtype, ATOL)
    assert kvq.kvq_check(case.cache.struct) == 0
    case.T = 60
    compare_cache(case, case.oracle_quant(pairs=pairs), 0)
    z = dev(np.zeros((1, 2, 128), np.uint16))
    kvq.kvq_append(case.layout, z, z, case.cache.struct)
    assert kvq.kvq_check(case.cache.struct) == 1


def _random_layouts(n, seed):
    """Seeded draws over the layout space the ABI accepts (small sizes)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.choice([1, 2, 4, 8, 16]))
        Hkv = int(rng.choice([1, 2, 3]))
        R = int(rng.choice([32, 64, 96, 128]))
        n_hi = int(rng.integers(0, 9))
        bits_hi = int(rng.choice([4, 16]))
        n_lo1 = int(rng.choice([0, 0, 8, 32]))
        nvb = int(rng.choice([0, 0, 1, 2, 3, 4]))
        T = int(rng.integers(1, 720))
        out.append(kvq_synth.Workload(
            "rand%d" % i, int(rng.integers(1, 3)), G * Hkv, Hkv, T + 1, n_qry=8,
            io_dtype=str(rng.choice(["fp16", "bf16"])),
            outliers=str(rng.choice(["none", "pairs4x8", "pct2x10"])), n_pairs_hi=n_hi,
            bits_hi=bits_hi, n_pairs_lo1=n_lo1, residual=R, seed=200 + i, n_vblk_hi=nvb,
            bits_vhi=int(rng.choice([3, 4]))))
    return out


@pytest.mark.parametrize("w", _random_layouts(12, 7), ids=_ids)
def test_random_layouts(w):
    # prefill w.tokens - 1 tokens: every byte; plain and pruned decode at a
    # drawn split count; one one-launch step (the last token)
    from decode_attention_select_amd import kvq
    from tests._gpu_case import dev
    rng = np.random.default_rng(w.seed)
    T0 = w.tokens - 1
    case = Case(w, T=T0, max_tokens=w.tokens)
    pairs = case.oracle_select()[1]
    if T0 >= 1:
        qz = case.oracle_quant(pairs=pairs)
        compare_cache(case, qz, qz.nq // 32)
        q = case.d["q_dec"][:, :, 0]
        S = int(rng.integers(1, 10))
        check_output(case.decode(q, S), oracle.attention(qz, q, SM_SCALE), w.io_dtype, ATOL)
        keep = int(rng.integers(1, 8))
        if not case.pruned_unsupported(S, keep):
            check_output(case.decode_pruned(q, S, keep),
                         oracle.attention_pruned(qz, q, SM_SCALE, keep), w.io_dtype, ATOL)
    S = int(rng.integers(1, 10))
    ws = torch.zeros(kvq.kvq_workspace_bytes(case.layout, S), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.int16, device="cuda")
    q_bits = case.d["q_dec"][:, :, 0]
    kvq.kvq_append_decode_attn(case.layout, dev(np.ascontiguousarray(case.d["k"][:, :, T0])),
                               dev(np.ascontiguousarray(case.d["v"][:, :, T0])), dev(q_bits),
                               case.cache.struct, SM_SCALE, S, ws, out)
    assert kvq.kvq_check(case.cache.struct) == 0
    case.T = w.tokens
    qz = case.oracle_quant(pairs=pairs)
    got = kvq_synth.bits_to_f64(out.cpu().numpy().view(np.uint16), w.io_dtype)
    check_output(got, oracle.attention_after_append(qz, q_bits, SM_SCALE), w.io_dtype, ATOL)
    compare_cache(case, qz, qz.nq // 32)


@pytest.mark.parametrize("w", _random_layouts(12, 7), ids=_ids)
def test_random_layouts_query_aware_and_shrink(w):
    # the query-aware scorer (scores and ranks), then, on the prefilled cache,
    # the shrink of a drawn group range (4-bit salient layouts): bytes and decode
    from decode_attention_select_amd import kvq
    from tests._gpu_case import dev
    rng = np.random.default_rng(w.seed + 7)
    case = Case(w, T=w.tokens)
    kvq.kvq_select_pairs_qa(case.layout, case.q_sel, w.n_qry, case.k_sel, w.tokens,
                            case.cache.struct)
    torch.cuda.synchronize()
    S, pairs_qa = oracle.select_qa(case.d["q_sel"], case.d["k"], w.tokens, w.n_kv_heads,
                                   w.io_dtype)
    g = case.gpu_bytes()
    assert np.array_equal(g["sums"][:, :, 0], S.view(np.uint64))
    assert np.array_equal(g["pairs"], pairs_qa)
    if w.bits_hi != 4 or w.n_pairs_hi == 0:
        return
    # re-prefill with the query-aware ranking in place, then shrink
    case2 = Case(w, T=w.tokens)
    kvq.kvq_select_pairs_qa(case2.layout, case2.q_sel, w.n_qry, case2.k_sel, w.tokens,
                            case2.cache.struct)
    kvq.kvq_quant_keys(case2.layout, dev(case2.d["k"][:, :, :w.tokens]), w.tokens,
                       case2.cache.struct)
    kvq.kvq_quant_values(case2.layout, dev(case2.d["v"][:, :, :w.tokens]), w.tokens,
                         case2.cache.struct)
    ng = oracle.n_quant(w.tokens, w.residual) // 32
    g0 = int(rng.integers(0, ng + 1))
    g1 = int(rng.integers(g0, ng + 2))
    kvq.kvq_shrink(case2.layout, case2.cache.struct, g0, g1)
    torch.cuda.synchronize()
    qz = oracle.shrink(case2.oracle_quant(pairs=pairs_qa), g0, min(g1, case2.NG))
    compare_cache(case2, qz, qz.nq // 32)
    q = case2.d["q_dec"][:, :, 0]
    check_output(case2.decode(q, 3), oracle.attention(qz, q, SM_SCALE), w.io_dtype, ATOL)
