"""kvq_decode_attn_noalloc: the decode entry point whose workspace is the
library's static per-GPU scratch array.  Through the C ABI, on calls in a
row (the second with a smaller layout, fewer splits and tokens, the third
with the first layout again), its
outputs equal kvq_decode_attn's on a fresh workspace bit for bit (the same
kernels) and meet the oracle's 2e-3; a layout whose workspace exceeds the
array is rejected before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import kvq_synth
import oracle
from decode_attention_select_amd import kvq
from tests._gpu_case import SM_SCALE, Case, check_output, dev

pytestmark = pytest.mark.gpu

ATOL = 2e-3


def _noalloc(case, q_bits, S):
    out = torch.full((case.w.batch, case.w.n_q_heads, 128), 0x7fc0, dtype=torch.int16,
                     device="cuda")
    kvq.kvq_decode_attn_noalloc(case.layout, dev(q_bits), case.cache.struct, SM_SCALE, S, out)
    torch.cuda.synchronize()
    return kvq_synth.bits_to_f64(out.cpu().numpy().view(np.uint16), case.w.io_dtype)


def test_noalloc_matches_decode_attn_on_two_calls():
    big = kvq_synth.Workload("noalloc-big", 2, 8, 2, 900, n_qry=8, io_dtype="bf16",
                             outliers="pct2x10", n_pairs_hi=6, residual=128, seed=301)
    small = kvq_synth.Workload("noalloc-small", 1, 4, 1, 230, n_qry=8, io_dtype="fp16",
                               n_pairs_hi=8, residual=32, seed=302)
    # big, then smaller, then big again: the third call's extra split
    # counters sit where the second call left its records
    for w, S in ((big, 48), (small, 3), (big, 48)):
        print("case", w.name, "S", S, flush=True)
        case = Case(w)
        q = case.d["q_dec"][:, :, 0]
        got = _noalloc(case, q, S)
        want = case.decode(q, S)
        assert np.array_equal(got, want), np.nanmax(np.abs(got - want))
        check_output(got, oracle.attention(case.oracle_quant(), q, SM_SCALE), w.io_dtype, ATOL)


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    # 64 sequences x 128 query heads at 1024 splits need far more
    # than the static array: rejected on the host, nothing enqueued
    L = kvq.make_layout(64, 128, 8, max_tokens=4096)
    assert kvq.kvq_workspace_bytes(L, 1024) > kvq.NOALLOC_WORKSPACE_BYTES
    st = kvq.lib().kvq_decode_attn_noalloc(ctypes.byref(L), ctypes.c_void_p(1 << 20),
                                           ctypes.byref(kvq.kvq_cache(*[1 << 20] * kvq.NBUF)),
                                           ctypes.c_float(0.088), 1024, ctypes.c_void_p(1 << 20),
                                           ctypes.c_void_p(0))
    assert st == -4  # KVQ_ECAPACITY
