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
