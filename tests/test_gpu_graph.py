"""Decode steps captured in a HIP graph (torch.cuda.CUDAGraph around the C-ABI
calls, on the capturing stream) and replayed, the way a serving loop runs a
fixed step without per-call launch work.  The calls allocate nothing and
record no memset, so a step is capturable once its buffers exist.

Two caches are built from the same data: one is stepped eagerly, the other by
replays of a graph captured once; the new token's key and value are copied
into the graph's static inputs between replays (eager work, then a
synchronization).  Every replay's output equals the eager twin's bit for bit
and the oracle within 2e-3, and every cache byte equals the prefill of the
same tokens at the end.
* One-launch steps (kvq_append_decode_attn), plain and progressive layouts.
* Two-call steps (kvq_append, then kvq_decode_attn_noalloc, whose workspace is
  the library's static array).
"""
import numpy as np
import pytest
import torch

import kvq_synth
import oracle
from decode_attention_select_amd import kvq
from tests._gpu_case import SM_SCALE, Case, check_output, compare_cache, dev

pytestmark = pytest.mark.gpu

ATOL = 2e-3

LAYOUTS = [
    kvq_synth.Workload("graph-gqa4", 2, 8, 2, 330, n_qry=8, io_dtype="bf16", outliers="pct2x10",
                       n_pairs_hi=6, residual=64, seed=111),
    kvq_synth.Workload("graph-prog", 1, 8, 2, 32 * 8 + 64 + 40, n_qry=8, io_dtype="fp16",
                       n_pairs_hi=6, residual=64, seed=112, prog_w8=2, prog_w4=5),
]


def _ids(w):
    return w.name


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _twins(w, n_steps):
    T0 = w.tokens - n_steps
    eager = Case(w, T=T0, max_tokens=w.tokens)
    graphed = Case(w, T=T0, max_tokens=w.tokens, data=eager.d)
    return T0, eager, graphed


def _bits(out, io):
    return kvq_synth.bits_to_f64(out.cpu().numpy().view(np.uint16), io)


@pytest.mark.parametrize("w", LAYOUTS, ids=_ids)
def test_one_launch_steps_replayed_from_a_graph(w):
    print("case", w.name, flush=True)
    T0, eager, graphed = _twins(w, 70)
    pairs = eager.oracle_select()[1]
    S = 3
    B, Hq, Hkv = w.batch, w.n_q_heads, w.n_kv_heads
    wsb = kvq.kvq_workspace_bytes(eager.layout, S)
    ws_e = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    ws_g = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    out_e = torch.empty((B, Hq, 128), dtype=torch.int16, device="cuda")
    out_g = torch.empty_like(out_e)
    q_bits = eager.d["q_dec"][:, :, 0]
    q = dev(q_bits)
    kn = torch.empty((B, Hkv, 128), dtype=torch.int16, device="cuda")
    vn = torch.empty_like(kn)

    def step(case, ws, out):
        kvq.kvq_append_decode_attn(case.layout, kn, vn, q, case.cache.struct, SM_SCALE, S, ws,
                                   out)

    packs = 0
    g = None
    for t in range(T0, w.tokens):
        kn.copy_(dev(np.ascontiguousarray(eager.d["k"][:, :, t])))
        vn.copy_(dev(np.ascontiguousarray(eager.d["v"][:, :, t])))
        if g is None:
            # the first step runs eagerly on both (the kernel is loaded before capture)
            step(graphed, ws_g, out_g)
            g = _capture(lambda: step(graphed, ws_g, out_g))
        else:
            g.replay()
        step(eager, ws_e, out_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), t
        before = eager.oracle_quant(T=t, pairs=pairs)
        check_output(_bits(out_g, w.io_dtype), oracle.attention_one_launch(before, q_bits, SM_SCALE),
                     w.io_dtype, ATOL)
        packs += oracle.n_quant(t + 1, w.residual) > oracle.n_quant(t, w.residual)
    assert packs >= 2
    assert kvq.kvq_check(graphed.cache.struct) == 0 and kvq.kvq_check(eager.cache.struct) == 0
    graphed.T = w.tokens
    qz = graphed.oracle_quant(pairs=pairs)
    compare_cache(graphed, qz, qz.nq // 32)


@pytest.mark.parametrize("w", LAYOUTS, ids=_ids)
def test_two_call_steps_replayed_from_a_graph(w):
    print("case", w.name, flush=True)
    T0, eager, graphed = _twins(w, 70)
    pairs = eager.oracle_select()[1]
    S = 5
    B, Hq, Hkv = w.batch, w.n_q_heads, w.n_kv_heads
    out_e = torch.empty((B, Hq, 128), dtype=torch.int16, device="cuda")
    out_g = torch.empty_like(out_e)
    q_bits = eager.d["q_dec"][:, :, 0]
    q = dev(q_bits)
    kn = torch.empty((B, Hkv, 128), dtype=torch.int16, device="cuda")
    vn = torch.empty_like(kn)

    def step(case, out):
        kvq.kvq_append(case.layout, kn, vn, case.cache.struct)
        kvq.kvq_decode_attn_noalloc(case.layout, q, case.cache.struct, SM_SCALE, S, out)

    g = None
    for t in range(T0, w.tokens):
        kn.copy_(dev(np.ascontiguousarray(eager.d["k"][:, :, t])))
        vn.copy_(dev(np.ascontiguousarray(eager.d["v"][:, :, t])))
        if g is None:
            step(graphed, out_g)
            g = _capture(lambda: step(graphed, out_g))
        else:
            g.replay()
        step(eager, out_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), t
        after = eager.oracle_quant(T=t + 1, pairs=pairs)
        check_output(_bits(out_g, w.io_dtype), oracle.attention(after, q_bits, SM_SCALE),
                     w.io_dtype, ATOL)
    assert kvq.kvq_check(graphed.cache.struct) == 0
    graphed.T = w.tokens
    qz = graphed.oracle_quant(pairs=pairs)
    compare_cache(graphed, qz, qz.nq // 32)
