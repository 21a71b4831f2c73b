"""GPU parity of progressive precision (PM-KVQ review, lead and
key_machinery: a cache held at 16 bits, then 8, 4 and 2 bits as it ages,
each step an in-place shrink by the equivalent right shift), through the C
ABI against the oracle on the same seeded inputs.

* Prefill: every byte of k_lo, k_hi, k_meta, v_codes, v_meta and of the live
  digit-plane slots equals the oracle's packing, for windows that cover part
  of the groups, all of them, none at 8 bits, and 8 bits straight to 2.
* Append: a run of appends across several group boundaries (each packing a
  group at 8 bits and shrinking the groups that reach the window edges)
  leaves exactly the bytes of a prefill of the same tokens.
* Decode: within 2e-3 of the oracle's fp64 attention over the current
  widths, at split counts where window groups fall to different waves and
  where one wave takes several; the one-split fp32 record as well.
* Append and decode in one launch: every step within 2e-3 of the oracle's
  attention from the cache the call found (window groups at their former
  widths, the packed group and the new token at 16 bits), and after every
  pack every byte equal to a prefill of the same tokens.
"""
import numpy as np
import pytest
import torch

import kvq_synth
import oracle
from decode_attention_select_amd import kvq
from tests._gpu_case import SM_SCALE, Case, check_output, check_single_split, compare_cache, dev

pytestmark = pytest.mark.gpu

ATOL = 2e-3

PROG = [
    # 13 quantized groups: 2 at 8 bits, 3 at 4 bits, 8 at 2 bits
    kvq_synth.Workload("prog-2-5", 1, 8, 2, 32 * 13 + 128 + 17, n_qry=8, io_dtype="bf16",
                       outliers="pct2x10", n_pairs_hi=6, residual=128, seed=61,
                       prog_w8=2, prog_w4=5),
    # no 8-bit window (groups leave the ring at 4 bits), fp16, G = 1
    kvq_synth.Workload("prog-0-3-g1", 2, 2, 2, 32 * 7 + 64 + 5, n_qry=8, io_dtype="fp16",
                       n_pairs_hi=8, residual=64, seed=62, prog_w8=0, prog_w4=3),
    # 8 bits straight to 2 (w8 == w4), raw 16-bit salient channels
    kvq_synth.Workload("prog-3-3-raw16", 1, 8, 2, 32 * 9 + 64 + 31, n_qry=8, io_dtype="bf16",
                       n_pairs_hi=6, bits_hi=16, residual=64, seed=63, prog_w8=3, prog_w4=3),
    # windows wider than the sequence (every group wide), no salient pairs, G = 16
    kvq_synth.Workload("prog-all-wide", 1, 16, 1, 32 * 4 + 32 + 9, n_qry=4, io_dtype="bf16",
                       n_pairs_hi=0, residual=32, seed=64, prog_w8=3, prog_w4=9),
    # GQA 4 at a longer context: 40 groups, windows of 4 and 16
    kvq_synth.Workload("prog-4-16-long", 1, 32, 8, 32 * 40 + 128 + 3, n_qry=8, io_dtype="bf16",
                       outliers="pct2x10", n_pairs_hi=6, residual=128, seed=65,
                       prog_w8=4, prog_w4=16),
]


def _ids(w):
    return w.name


@pytest.mark.parametrize("w", PROG, ids=_ids)
def test_prog_prefill_bytes(w):
    print("case", w.name, flush=True)
    case = Case(w)
    qz = case.oracle_quant()
    compare_cache(case, qz, qz.nq // 32)


@pytest.mark.parametrize("w", PROG, ids=_ids)
@pytest.mark.parametrize("n_splits", [1, 3, 16])
def test_prog_decode(w, n_splits):
    print("case", w.name, "S", n_splits, flush=True)
    case = Case(w)
    qz = case.oracle_quant()
    q = case.d["q_dec"][:, :, 0]
    ref = oracle.attention(qz, q, SM_SCALE)
    if n_splits == 1:
        got, part = case.decode(q, 1, partials=True)
        check_single_split(part, ref, ATOL)
    else:
        got = case.decode(q, n_splits)
    err = check_output(got, ref, w.io_dtype, ATOL)
    print("max err %.3g" % err)


@pytest.mark.parametrize("w8,w4", [(2, 5), (0, 2), (2, 2)])
def test_prog_appends_equal_prefill(w8, w4):
    # prefill, then appends that pack 4 groups: each pack enters at the width
    # of age 0 and shrinks the groups reaching ages w8 and w4
    w = kvq_synth.Workload("prog-app", 2, 8, 2, 32 * 6 + 64 + 20, n_qry=8, n_app=130,
                           io_dtype="bf16", outliers="pct2x10", n_pairs_hi=6, residual=64,
                           seed=66, prog_w8=w8, prog_w4=w4)
    print("case", w8, w4, flush=True)
    case = Case(w, T=w.tokens, max_tokens=w.max_tokens)
    kn = dev(np.ascontiguousarray(case.d["k"][:, :, w.tokens:]))
    vn = dev(np.ascontiguousarray(case.d["v"][:, :, w.tokens:]))
    q = case.d["q_dec"][:, :, 0]
    ng0 = oracle.n_quant(w.tokens, w.residual) // 32
    for i in range(w.n_app):
        kvq.kvq_append(case.layout, kn[:, :, i].contiguous(), vn[:, :, i].contiguous(),
                       case.cache.struct)
        T = w.tokens + i + 1
        ng = oracle.n_quant(T, w.residual) // 32
        if ng != oracle.n_quant(T - 1, w.residual) // 32 or i == w.n_app - 1:
            torch.cuda.synchronize()
            qz = case.oracle_quant(T=T)
            compare_cache(case, qz, ng)
            check_output(case.decode(q, 5), oracle.attention(qz, q, SM_SCALE), w.io_dtype, ATOL)
    assert oracle.n_quant(w.tokens + w.n_app, w.residual) // 32 - ng0 == 4
    assert kvq.kvq_check(case.cache.struct) == 0


FUSED_PROG = [
    kvq_synth.Workload("fprog-2-5", 2, 8, 2, 32 * 6 + 64 + 20, n_qry=8, n_app=100,
                       io_dtype="bf16", outliers="pct2x10", n_pairs_hi=6, residual=64, seed=68,
                       prog_w8=2, prog_w4=5),
    kvq_synth.Workload("fprog-0-2-g1", 1, 3, 3, 32 * 5 + 32 + 7, n_qry=8, n_app=100,
                       io_dtype="fp16", n_pairs_hi=8, residual=32, seed=69, prog_w8=0,
                       prog_w4=2),
    kvq_synth.Workload("fprog-2-2-raw16", 1, 8, 2, 32 * 4 + 32 + 30, n_qry=8, n_app=100,
                       io_dtype="bf16", n_pairs_hi=6, bits_hi=16, residual=32, seed=70,
                       prog_w8=2, prog_w4=2),
]


@pytest.mark.parametrize("w", FUSED_PROG, ids=_ids)
def test_prog_append_and_decode_in_one_launch(w):
    # each step's output against the oracle's attention from the cache the
    # call found; after each pack (its shrinks run once every split has read
    # the window groups) every byte against the prefill of the same tokens
    print("case", w.name, flush=True)
    case = Case(w, T=w.tokens, max_tokens=w.max_tokens)
    pairs = case.oracle_select()[1]
    S = 5
    ws = torch.zeros(kvq.kvq_workspace_bytes(case.layout, S), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.int16, device="cuda")
    q_bits = case.d["q_dec"][:, :, 0]
    q = dev(q_bits)
    packs = 0
    for i in range(w.n_app):
        t = w.tokens + i
        kvq.kvq_append_decode_attn(case.layout, dev(np.ascontiguousarray(case.d["k"][:, :, t])),
                                   dev(np.ascontiguousarray(case.d["v"][:, :, t])), q,
                                   case.cache.struct, SM_SCALE, S, ws, out)
        before = case.oracle_quant(T=t, pairs=pairs)
        got = kvq_synth.bits_to_f64(out.cpu().numpy().view(np.uint16), w.io_dtype)
        check_output(got, oracle.attention_one_launch(before, q_bits, SM_SCALE), w.io_dtype,
                     ATOL)
        if oracle.n_quant(t + 1, w.residual) > oracle.n_quant(t, w.residual):
            packs += 1
            qz = case.oracle_quant(T=t + 1, pairs=pairs)
            compare_cache(case, qz, qz.nq // 32)
    assert packs >= 3
    assert kvq.kvq_check(case.cache.struct) == 0
    qz = case.oracle_quant(T=w.tokens + w.n_app, pairs=pairs)
    compare_cache(case, qz, qz.nq // 32)


def test_prog_holds_less_than_an_eight_bit_cache():
    # the planes are the only storage above the 2-bit records: a progressive
    # cache with windows of 4 and 16 groups against one holding every group
    # of a 32K sequence at 8 bits
    base = kvq.make_layout(1, 32, 8, max_tokens=32768, prog_w8=4, prog_w4=16)
    wide = kvq.make_layout(1, 32, 8, max_tokens=32768, prog_w8=256, prog_w4=256)
    two = kvq.make_layout(1, 32, 8, max_tokens=32768)
    nb, nw, n2 = (sum(kvq.kvq_cache_sizes(x)) for x in (base, wide, two))
    assert nb - n2 == 8 * (16 + 2 * 4) * 1024 * 2
    assert nw - n2 == 8 * (256 + 2 * 256) * 1024 * 2
    assert nb < nw


def _random_prog_layouts(n, seed):
    """Seeded draws over the progressive layouts the ABI accepts (small sizes)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.choice([1, 2, 4, 8, 16]))
        Hkv = int(rng.choice([1, 2, 3]))
        R = int(rng.choice([32, 64, 128]))
        w4 = int(rng.integers(1, 14))
        w8 = int(rng.integers(0, w4 + 1))
        T = int(rng.integers(1, 900))
        out.append(kvq_synth.Workload(
            "prand%d" % i, int(rng.integers(1, 3)), G * Hkv, Hkv, T, n_qry=8, n_app=64,
            io_dtype=str(rng.choice(["fp16", "bf16"])),
            outliers=str(rng.choice(["none", "pairs4x8", "pct2x10"])),
            n_pairs_hi=int(rng.integers(0, 9)), bits_hi=int(rng.choice([4, 16])), residual=R,
            seed=400 + i, prog_w8=w8, prog_w4=w4))
    return out


@pytest.mark.parametrize("w", _random_prog_layouts(10, 11), ids=_ids)
def test_prog_random_layouts(w):
    # prefill: every byte and the decode at a drawn split count; then 32
    # appends (at least one pack): every byte and the decode again, and the
    # no-allocation entry point equal to the plain one; then 32 one-launch
    # steps at a drawn split count, each against the oracle's attention from
    # the cache the call found, and every byte at the end
    print("case", w, flush=True)
    rng = np.random.default_rng(w.seed)
    case = Case(w, T=w.tokens, max_tokens=w.max_tokens)
    pairs = case.oracle_select()[1]
    q = case.d["q_dec"][:, :, 0]
    qz = case.oracle_quant(pairs=pairs)
    compare_cache(case, qz, qz.nq // 32)
    S = int(rng.integers(1, 12))
    check_output(case.decode(q, S), oracle.attention(qz, q, SM_SCALE), w.io_dtype, ATOL)
    kn = dev(np.ascontiguousarray(case.d["k"][:, :, w.tokens:]))
    vn = dev(np.ascontiguousarray(case.d["v"][:, :, w.tokens:]))
    n1 = w.n_app // 2
    for i in range(n1):
        kvq.kvq_append(case.layout, kn[:, :, i].contiguous(), vn[:, :, i].contiguous(),
                       case.cache.struct)
    torch.cuda.synchronize()
    assert kvq.kvq_check(case.cache.struct) == 0
    case.T = w.tokens + n1
    qz = case.oracle_quant(pairs=pairs)
    compare_cache(case, qz, qz.nq // 32)
    S = int(rng.integers(1, 12))
    got = case.decode(q, S)
    check_output(got, oracle.attention(qz, q, SM_SCALE), w.io_dtype, ATOL)
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.int16, device="cuda")
    kvq.kvq_decode_attn_noalloc(case.layout, dev(q), case.cache.struct, SM_SCALE, S, out)
    torch.cuda.synchronize()
    assert np.array_equal(kvq_synth.bits_to_f64(out.cpu().numpy().view(np.uint16), w.io_dtype),
                          got)
    S = int(rng.integers(1, 12))
    ws = torch.zeros(kvq.kvq_workspace_bytes(case.layout, S), dtype=torch.uint8, device="cuda")
    qd = dev(q)
    for i in range(n1, w.n_app):
        t = w.tokens + i
        kvq.kvq_append_decode_attn(case.layout, kn[:, :, i].contiguous(), vn[:, :, i].contiguous(),
                                   qd, case.cache.struct, SM_SCALE, S, ws, out)
        before = case.oracle_quant(T=t, pairs=pairs)
        got = kvq_synth.bits_to_f64(out.cpu().numpy().view(np.uint16), w.io_dtype)
        check_output(got, oracle.attention_one_launch(before, q, SM_SCALE), w.io_dtype, ATOL)
    assert kvq.kvq_check(case.cache.struct) == 0
    case.T = w.tokens + w.n_app
    qz = case.oracle_quant(pairs=pairs)
    compare_cache(case, qz, qz.nq // 32)


def test_prog_guard_bands_survive():
    # every cache section (the plane windows included), the workspace and the
    # output between canary bands through prefill, appends that pack and
    # shrink, and decode at several split counts
    from tests.test_gpu_canary import Guarded
    w = kvq_synth.Workload("prog-canary", 2, 8, 2, 32 * 9 + 64 + 7, n_qry=8, n_app=70,
                           io_dtype="bf16", outliers="pct2x10", n_pairs_hi=6, residual=64,
                           seed=67, prog_w8=2, prog_w4=4)
    d = kvq_synth.generate(w)
    T0 = w.tokens
    layout = kvq.make_layout(w.batch, w.n_q_heads, w.n_kv_heads, n_pairs_hi=w.n_pairs_hi,
                             residual=w.residual, max_tokens=T0 + w.n_app + 8,
                             io_dtype=w.io_dtype, prog_w8=w.prog_w8, prog_w4=w.prog_w4)
    sizes = kvq.kvq_cache_sizes(layout)
    assert sizes[12] > 0 and sizes[13] > 0
    bufs = [Guarded(n) for n in sizes]
    cache = kvq.kvq_cache(*[b.ptr() for b in bufs])
    q_sel = Guarded(d["q_sel"].nbytes, d["q_sel"])
    k0 = Guarded(d["k"][:, :, :T0].nbytes, d["k"][:, :, :T0])
    v0 = Guarded(d["v"][:, :, :T0].nbytes, d["v"][:, :, :T0])
    q = Guarded(d["q_dec"][:, :, 0].nbytes, d["q_dec"][:, :, 0])
    out = Guarded(w.batch * w.n_q_heads * 128 * 2)
    S_list = [1, 3, 32]
    ws = Guarded(max(kvq.kvq_workspace_bytes(layout, S) for S in S_list))
    kvq.kvq_select_pairs(layout, q_sel.ptr(), w.n_qry, k0.ptr(), T0, cache)
    kvq.kvq_quant_keys(layout, k0.ptr(), T0, cache)
    kvq.kvq_quant_values(layout, v0.ptr(), T0, cache)
    inputs = [q_sel, k0, v0, q]
    for i in range(w.n_app):
        kn = Guarded(d["k"][:, :, T0 + i].nbytes, d["k"][:, :, T0 + i])
        vn = Guarded(d["v"][:, :, T0 + i].nbytes, d["v"][:, :, T0 + i])
        kvq.kvq_append(layout, kn.ptr(), vn.ptr(), cache)
        inputs += [kn, vn]
        if i % 23 == 0:
            for S in S_list:
                kvq.kvq_decode_attn(layout, q.ptr(), cache, SM_SCALE, S, ws.ptr(), out.ptr(),
                                    ws_bytes=ws.n)
    kvq.kvq_decode_attn_noalloc(layout, q.ptr(), cache, SM_SCALE, 3, out.ptr())
    torch.cuda.synchronize()
    assert kvq.kvq_check(cache) == 0
    bad = [kvq.BUF_NAMES[i] for i, b in enumerate(bufs) if not b.bands_intact()]
    bad += [nm for nm, b in (("workspace", ws), ("out", out)) if not b.bands_intact()]
    bad += ["input %d" % i for i, b in enumerate(inputs) if not b.bands_intact()]
    assert not bad, "guard bands overwritten: %s" % bad
