"""GPU parity at the full sizes of the decode workloads, in the launch
configuration the benchmark times:

* the Llama-3-8B-shaped layer at 32K context (B1, 32 q / 8 kv heads, bf16):
  selection, every cache byte and every output element against the oracle,
  at the benchmark's split count;
* the 128K-context layer (B1, 64 q / 8 kv heads, G = 8, 256 splits): every
  cache byte; outputs of two sampled KV heads (16 query heads) against the
  oracle, which computes those heads alone;
* the streaming layer (B16, prefill 4096): 40 appends, which pack one group
  per sequence and head, then every cache byte and every output element;
* the bit-allocation sweep's layer (B4 x 16K) at each of its four key
  precisions: every cache byte and every output element.

Bars as in the small-case tests: bit-exact indices, sums, codes, scales,
zero points and ring bytes; attention within 2e-3, the 16-bit output's own
rounding included (half an output ulp is added only where it exceeds 1e-3,
|o| >= 0.5 in bf16); the fp32 split record of a one-split call within 2e-3
with no allowance."""
import numpy as np
import pytest

import bench
import kvq_synth
import oracle
from tests._gpu_case import (SM_SCALE, Case, check_output, check_single_split, compare_cache,
                              dev)

pytestmark = pytest.mark.gpu

ATOL = 2e-3


def kv_head_slice(qz, heads):
    """The oracle's quantized cache restricted to some KV heads (a view for
    computing only their query heads)."""
    kw = dict(qz.__dict__)
    for n in ("k", "v", "pairs", "kcodes", "ks", "kz", "vcodes", "vs", "vz"):
        kw[n] = np.ascontiguousarray(getattr(qz, n)[:, heads])
    return oracle.Quantized(**kw)


def check_selection(case):
    sums, pairs = case.oracle_select()
    g = case.gpu_bytes()
    assert np.array_equal(g["sums"], sums)
    assert np.array_equal(g["pairs"], pairs)
    return pairs


@pytest.mark.timeout(400)
def test_llama3_8b_32k_full():
    w = kvq_synth.workload("llama3-8b-32k")
    print("case", w.name, flush=True)
    case = Case(w)
    pairs = check_selection(case)
    qz = case.oracle_quant(pairs=pairs)
    compare_cache(case, qz, qz.nq // 32)
    q = case.d["q_dec"][:, :, 0]
    ref = oracle.attention(qz, q, SM_SCALE)
    S = bench.default_splits(w)
    err = check_output(case.decode(q, S), ref, w.io_dtype, ATOL)
    _, part = case.decode(q, 1, partials=True)
    e32 = check_single_split(part, ref, ATOL)
    print("%s S=%d max|err| %.3g max|o| %.3g split-record max|err| %.3g"
          % (w.name, S, err, np.abs(ref).max(), e32))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("qscale", [8, 16])
def test_llama3_8b_32k_large_logits(qscale):
    # PN-Mix (abstract): the error of pairs with large pair-norm products
    # dominates the logits.  Outlier-heavy keys (2 % of pairs x10) met by
    # queries scaled x8 and x16: logits far beyond those of N(0,1) data, every
    # output against the oracle at 2e-3.
    w = kvq_synth.workload("llama3-8b-32k")
    print("case", w.name, "queries x%d" % qscale, flush=True)
    case = Case(w)
    qz = case.oracle_quant()
    qf = kvq_synth.bits_to_f64(case.d["q_dec"][:, :, 0], w.io_dtype) * qscale
    q = kvq_synth.to_bits(qf, w.io_dtype)
    qf = kvq_synth.bits_to_f64(q, w.io_dtype)
    G = w.group_size
    kf = kvq_synth.bits_to_f64(case.d["k"][:, :, :w.tokens], w.io_dtype)
    max_logit = max(float(np.abs(kf[0, h // G] @ qf[0, h]).max()) * SM_SCALE
                    for h in range(w.n_q_heads))
    ref = oracle.attention(qz, q, SM_SCALE)
    S = bench.default_splits(w)
    err = check_output(case.decode(q, S), ref, w.io_dtype, ATOL)
    _, part = case.decode(q, 1, partials=True)
    e32 = check_single_split(part, ref, ATOL)
    print("%s queries x%d: max|logit| %.1f max|err| %.3g max|o| %.3g split-record max|err| %.3g"
          % (w.name, qscale, max_logit, err, np.abs(ref).max(), e32))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("point", kvq_synth.PARETO_POINTS, ids=[p[0] for p in kvq_synth.PARETO_POINTS])
def test_pareto_b4_16k_every_bit_point(point):
    # the bit-allocation sweep's layer (B4 x 16K, 32 q / 8 kv heads, bf16) at
    # each key precision it sweeps: 1.5 (half the pairs at 1 bit), 2.0, 2.26
    # (6 salient pairs at 4 bits), 3.0 (6 salient pairs at 16 bits); every
    # cache byte and every output element, at the benchmark's split count
    label, n_hi, bits_hi, n_lo1 = point
    w = kvq_synth.workload("pareto-b4-16k").replace(n_pairs_hi=n_hi, bits_hi=bits_hi,
                                                    n_pairs_lo1=n_lo1)
    print("case", w.name, "bits", label, flush=True)
    case = Case(w)
    pairs = check_selection(case)
    qz = case.oracle_quant(pairs=pairs)
    compare_cache(case, qz, qz.nq // 32)
    q = case.d["q_dec"][:, :, 0]
    ref = oracle.attention(qz, q, SM_SCALE)
    S = bench.default_splits(w)
    err = check_output(case.decode(q, S), ref, w.io_dtype, ATOL)
    _, part = case.decode(q, 1, partials=True)
    e32 = check_single_split(part, ref, ATOL)
    print("%s %s bits S=%d max|err| %.3g split-record max|err| %.3g"
          % (w.name, label, S, err, e32))


@pytest.mark.timeout(600)
def test_long_128k_sampled_heads():
    w = kvq_synth.workload("long-128k")
    print("case", w.name, flush=True)
    case = Case(w)
    pairs = check_selection(case)
    qz = case.oracle_quant(pairs=pairs)
    compare_cache(case, qz, qz.nq // 32)
    q = case.d["q_dec"][:, :, 0]
    got = case.decode(q, w.n_splits)
    G = w.group_size
    heads = [0, w.n_kv_heads - 1]
    qh = [kh * G + i for kh in heads for i in range(G)]
    ref = oracle.attention(kv_head_slice(qz, heads), np.ascontiguousarray(q[:, qh]), SM_SCALE)
    err = check_output(got[:, qh], ref, w.io_dtype, ATOL)
    _, (ml, o16) = case.decode(q, 1, partials=True)
    e32 = check_single_split((ml[:, qh], o16[:, qh]), ref, ATOL)
    print("%s S=%d heads %s max|err| %.3g max|o| %.3g split-record max|err| %.3g"
          % (w.name, w.n_splits, qh, err, np.abs(ref).max(), e32))


@pytest.mark.timeout(600)
def test_streaming_b16_appends():
    from decode_attention_select_amd import kvq
    w = kvq_synth.workload("streaming-b16")
    print("case", w.name, flush=True)
    n_app = 40
    case = Case(w, T=w.tokens, max_tokens=w.max_tokens)
    pairs = check_selection(case)
    kn = dev(np.ascontiguousarray(case.d["k"][:, :, w.tokens:w.tokens + n_app]))
    vn = dev(np.ascontiguousarray(case.d["v"][:, :, w.tokens:w.tokens + n_app]))
    for i in range(n_app):
        kvq.kvq_append(case.layout, kn[:, :, i].contiguous(), vn[:, :, i].contiguous(),
                       case.cache.struct)
    assert kvq.kvq_check(case.cache.struct) == 0
    T = w.tokens + n_app
    assert oracle.n_quant(T, w.residual) > oracle.n_quant(w.tokens, w.residual)
    qz = case.oracle_quant(T=T, pairs=pairs)
    compare_cache(case, qz, qz.nq // 32)
    q = np.ascontiguousarray(case.d["q_dec"][:, :, n_app - 1])
    ref = oracle.attention(qz, q, SM_SCALE)
    S = bench.default_splits(w)
    err = check_output(case.decode(q, S), ref, w.io_dtype, ATOL)
    _, part = case.decode(q, 1, partials=True)
    e32 = check_single_split(part, ref, ATOL)
    print("%s T=%d S=%d max|err| %.3g max|o| %.3g split-record max|err| %.3g"
          % (w.name, T, S, err, np.abs(ref).max(), e32))


@pytest.mark.timeout(400)
def test_llama3_8b_32k_pruned_and_query_aware_and_shrink():
    # the later calls at the 32K layer's full size: query-aware selection
    # (bit-exact), pruned decode at the benchmark's split count (every output),
    # and the shrink of every quantized group (every byte, then decode)
    from decode_attention_select_amd import kvq
    import torch
    w = kvq_synth.workload("llama3-8b-32k")
    print("case", w.name, "pruned / query-aware / shrink", flush=True)
    case = Case(w)
    pairs = check_selection(case)
    qz = case.oracle_quant(pairs=pairs)
    q = case.d["q_dec"][:, :, 0]
    S = bench.default_splits(w)
    for n_keep in (5, 6):
        ref = oracle.attention_pruned(qz, q, SM_SCALE, n_keep)
        err = check_output(case.decode_pruned(q, S, n_keep), ref, w.io_dtype, ATOL)
        print("%s keep=%d S=%d max|err| %.3g" % (w.name, n_keep, S, err), flush=True)
    kvq.kvq_shrink(case.layout, case.cache.struct, 0, qz.nq // 32)
    torch.cuda.synchronize()
    sh = oracle.shrink(qz, 0, qz.nq // 32)
    compare_cache(case, sh, sh.nq // 32)
    err = check_output(case.decode(q, S), oracle.attention(sh, q, SM_SCALE), w.io_dtype, ATOL)
    print("%s shrunk S=%d max|err| %.3g" % (w.name, S, err), flush=True)
    kvq.kvq_select_pairs_qa(case.layout, case.q_sel, w.n_qry, case.k_sel, w.tokens,
                            case.cache.struct)
    torch.cuda.synchronize()
    Sq, pq = oracle.select_qa(case.d["q_sel"], case.d["k"], w.tokens, w.n_kv_heads, w.io_dtype)
    g = case.gpu_bytes()
    assert np.array_equal(g["sums"][:, :, 0], Sq.view(np.uint64))
    assert np.array_equal(g["pairs"], pq)


@pytest.mark.timeout(400)
def test_llama3_8b_32k_two_value_precisions():
    w = kvq_synth.workload("llama3-8b-32k").replace(n_vblk_hi=2, bits_vhi=4)
    print("case", w.name, "two value precisions", flush=True)
    case = Case(w)
    qz = case.oracle_quant()
    compare_cache(case, qz, qz.nq // 32)
    q = case.d["q_dec"][:, :, 0]
    ref = oracle.attention(qz, q, SM_SCALE)
    S = bench.default_splits(w)
    err = check_output(case.decode(q, S), ref, w.io_dtype, ATOL)
    print("%s v2@4 S=%d max|err| %.3g" % (w.name, S, err))


@pytest.mark.timeout(600)
def test_maximum_context_append_to_capacity():
    # the largest capacity a layout accepts (2^20 tokens per sequence): prefill
    # one token short, append the last one (it completes a group, which is
    # packed from the ring), then one more append must report a full cache
    from decode_attention_select_amd import kvq
    T = 1 << 20
    w = kvq_synth.Workload("max-context-1m", 1, 4, 1, T, n_qry=8, io_dtype="bf16",
                           outliers="pct2x10", n_pairs_hi=6, residual=128, seed=95)
    print("case", w.name, flush=True)
    case = Case(w, T=T - 1, max_tokens=T)
    pairs = check_selection(case)
    assert oracle.n_quant(T, w.residual) > oracle.n_quant(T - 1, w.residual)
    kvq.kvq_append(case.layout, dev(np.ascontiguousarray(case.d["k"][:, :, T - 1])),
                   dev(np.ascontiguousarray(case.d["v"][:, :, T - 1])), case.cache.struct)
    assert kvq.kvq_check(case.cache.struct) == 0
    case.T = T
    qz = case.oracle_quant(pairs=pairs)
    compare_cache(case, qz, qz.nq // 32)
    q = case.d["q_dec"][:, :, 0]
    ref = oracle.attention(qz, q, SM_SCALE)
    S = bench.default_splits(w)
    got = case.decode(q, S)
    err = check_output(got, ref, w.io_dtype, ATOL)
    # the averaged outputs are small here, so also bound the relative error:
    # bf16 output rounding is at most 2^-9 relative, fp16 weights 2^-11
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    assert rel < 5e-3, rel
    print("%s S=%d max|err| %.3g max|o| %.3g rel-L2 %.3g" % (w.name, S, err, np.abs(ref).max(),
                                                           rel), flush=True)
    # a full cache: the next append sets the error bit and leaves len alone
    kvq.kvq_append(case.layout, dev(np.ascontiguousarray(case.d["k"][:, :, T - 1])),
                   dev(np.ascontiguousarray(case.d["v"][:, :, T - 1])), case.cache.struct)
    assert kvq.kvq_check(case.cache.struct) != 0
    assert np.all(case.gpu_bytes()["len"] == T)


@pytest.mark.timeout(400)
def test_llama3_8b_32k_fp16():
    # the same layer with fp16 inputs and outputs: every byte, every output
    w = kvq_synth.workload("llama3-8b-32k").replace(io_dtype="fp16", seed=1096)
    print("case", w.name, "fp16", flush=True)
    case = Case(w)
    pairs = check_selection(case)
    qz = case.oracle_quant(pairs=pairs)
    compare_cache(case, qz, qz.nq // 32)
    q = case.d["q_dec"][:, :, 0]
    ref = oracle.attention(qz, q, SM_SCALE)
    S = bench.default_splits(w)
    err = check_output(case.decode(q, S), ref, w.io_dtype, ATOL)
    print("%s fp16 S=%d max|err| %.3g max|o| %.3g" % (w.name, S, err, np.abs(ref).max()))


@pytest.mark.timeout(600)
def test_batch_with_offsets_beyond_4gib():
    # 32 sequences x 8 KV heads x 128K tokens: the key and value inputs are
    # 8.6 GB each and the cache 3.4 GB, so byte offsets pass 2^32.  Inputs
    # are seeded N(0,1) drawn on the GPU; the oracle checks the first and the
    # last (sequence, KV head) on their own slices (every quantity is per
    # (sequence, KV head)): ranks and sums, every cache byte, the outputs.
    import torch
    from decode_attention_select_amd import kvq
    B, Hq, Hkv, T, NQ, R = 32, 32, 8, 1 << 17, 8, 128
    G, NG, RS = Hq // Hkv, (T - R) // 32, R + 32
    gen = torch.Generator(device="cuda").manual_seed(4242)

    def rnd(shape):
        t = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        for i in range(shape[0]):
            t[i] = torch.randn(shape[1:], generator=gen, device="cuda").to(torch.bfloat16)
        return t.view(torch.int16)

    k, v = rnd((B, Hkv, T, 128)), rnd((B, Hkv, T, 128))
    q_sel, q = rnd((B, Hq, NQ, 128)), rnd((B, Hq, 128))
    layout = kvq.make_layout(B, Hq, Hkv, n_pairs_hi=6, bits_hi=4, residual=R, max_tokens=T,
                             io_dtype="bf16")
    cache = kvq.Cache(layout)
    kvq.kvq_select_pairs(layout, q_sel, NQ, k, T, cache.struct)
    kvq.kvq_quant_keys(layout, k, T, cache.struct)
    kvq.kvq_quant_values(layout, v, T, cache.struct)
    S = bench.default_splits(kvq_synth.Workload("b32", B, Hq, Hkv, T))
    ws = torch.zeros(kvq.kvq_workspace_bytes(layout, S), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, 128), dtype=torch.int16, device="cuda")
    kvq.kvq_decode_attn(layout, q, cache.struct, SM_SCALE, S, ws, out)
    torch.cuda.synchronize()
    print("case b32-128k S=%d" % S, flush=True)

    def host(t, dt):
        return t.contiguous().cpu().numpy().view(dt)

    def buf(name, dt, tdt, *shape):
        n = int(np.prod(shape)) * np.dtype(dt).itemsize
        return cache[name][:n].view(tdt).reshape(*shape)

    for b, kh in ((0, 0), (B - 1, Hkv - 1)):
        ks, vs = host(k[b, kh], np.uint16)[None, None], host(v[b, kh], np.uint16)[None, None]
        qs = host(q_sel[b, kh * G:(kh + 1) * G], np.uint16)[None]
        qd = host(q[b, kh * G:(kh + 1) * G], np.uint16)[None]
        sums, pairs = oracle.select(qs, ks, T, 1, "bf16")
        assert np.array_equal(host(buf("sums", np.uint64, torch.int64, B, Hkv, 2, 64)[b, kh],
                                   np.uint64), sums[0, 0])
        assert np.array_equal(host(buf("pairs", np.int32, torch.int32, B, Hkv, 64)[b, kh],
                                   np.int32), pairs[0, 0])
        qz = oracle.quantize(ks, vs, T, pairs, residual=R, n_pairs_hi=6, bits_hi=4,
                             io_dtype="bf16", ng=NG)
        pk = oracle.pack(qz)
        for name, dt, tdt, w in (("k_lo", np.uint32, torch.int32, 256),
                                 ("k_hi", np.uint8, torch.uint8, 128),
                                 ("k_meta", np.uint16, torch.int16, 256),
                                 ("v_codes", np.uint32, torch.int32, 256),
                                 ("v_meta", np.uint16, torch.int16, 256)):
            got = host(buf(name, dt, tdt, B, Hkv, NG, w)[b, kh], dt)
            assert np.array_equal(got, pk[name][0, 0]), "%s differs at (%d, %d)" % (name, b, kh)
        slots = oracle.live_ring_slots(T, R)
        rk = host(buf("ring_k", np.uint16, torch.int16, B, Hkv, RS, 128)[b, kh], np.uint16)
        rv = host(buf("ring_v", np.uint16, torch.int16, B, Hkv, RS // 32, 128, 32)[b, kh],
                  np.uint16)
        assert np.array_equal(rk[slots], pk["ring_k"][0, 0][slots])
        for s_ in slots:
            assert np.array_equal(rv[s_ // 32, :, s_ % 32], pk["ring_v"][0, 0][s_ // 32, :, s_ % 32])
        ref = oracle.attention(qz, qd, SM_SCALE)
        got = kvq_synth.bits_to_f64(host(out[b, kh * G:(kh + 1) * G], np.uint16)[None], "bf16")
        err = check_output(got, ref, "bf16", ATOL)
        print("b%d kh%d max|err| %.3g" % (b, kh, err), flush=True)


@pytest.mark.timeout(600)
def test_streaming_b16_one_launch_steps():
    # the streaming layer stepped with kvq_append_decode_attn, at the bench's
    # split count: outputs at the step that packs a group and at the last
    # step against the oracle, then every byte against the prefill
    import torch
    from decode_attention_select_amd import kvq
    w = kvq_synth.workload("streaming-b16")
    print("case", w.name, "one launch", flush=True)
    n_app = 40
    case = Case(w, T=w.tokens, max_tokens=w.max_tokens)
    pairs = check_selection(case)
    S = bench.default_splits(w)
    ws = torch.zeros(kvq.kvq_workspace_bytes(case.layout, S), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.int16, device="cuda")
    kn = dev(np.ascontiguousarray(case.d["k"][:, :, w.tokens:w.tokens + n_app]))
    vn = dev(np.ascontiguousarray(case.d["v"][:, :, w.tokens:w.tokens + n_app]))
    packs = [i for i in range(n_app) if oracle.n_quant(w.tokens + i + 1, w.residual) >
             oracle.n_quant(w.tokens + i, w.residual)]
    assert packs
    for i in range(n_app):
        q_bits = np.ascontiguousarray(case.d["q_dec"][:, :, i])
        kvq.kvq_append_decode_attn(case.layout, kn[:, :, i].contiguous(), vn[:, :, i].contiguous(),
                                   dev(q_bits), case.cache.struct, SM_SCALE, S, ws, out)
        if i in (packs[0], n_app - 1):
            qz = case.oracle_quant(T=w.tokens + i + 1, pairs=pairs)
            got = kvq_synth.bits_to_f64(out.cpu().numpy().view(np.uint16), w.io_dtype)
            err = check_output(got, oracle.attention_after_append(qz, q_bits, SM_SCALE),
                               w.io_dtype, ATOL)
            print("step %d max|err| %.3g" % (i, err), flush=True)
    assert kvq.kvq_check(case.cache.struct) == 0
    T = w.tokens + n_app
    case.T = T
    qz = case.oracle_quant(T=T, pairs=pairs)
    compare_cache(case, qz, qz.nq // 32)
