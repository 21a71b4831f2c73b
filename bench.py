"""Decode-step benchmark of the quantized-KV path on one MI355X.

One step = one kvq_decode_attn call (split-K decode attention over the packed
cache plus the split merge) for every query head of the workload, with the
cache already resident in HBM.  Every timed step reads the next of N cache
replicas (N * cache bytes >= 512 MiB) so that the 256 MB Infinity Cache cannot
serve it.  The default workload is the Llama-3-8B-shaped GQA layer at 32K
context (batch 1, 32 query / 8 KV heads, bf16, 6 salient pairs at 4 bits,
residual 128).

Prints one JSON line (rank 0, one GPU):
  value = effective HBM GB/s = algorithmic bytes per step / step time.
Algorithmic bytes per step: for every (sequence, KV head), the n_q quantized
tokens at 35 B of key codes (6 pairs x 4 bits + 116 channels x 2 bits) +
16 B key scale/zero + 32 B value codes + 16 B value scale/zero, the n_r ring
tokens at 256 B key + 256 B value, plus the query and the output.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0
# HBM bytes per launch of the decode kernel on the default workload, from the
# FETCH_SIZE and WRITE_SIZE counters scaled by a plain copy; None when the
# kernel has changed since they were read.
TRAFFIC = 27513237


def algorithmic_bytes(w, T: int, n_keep: int = 4) -> int:
    """Bytes a decode step must move.  With n_keep < 4 (query-channel
    pruning, 2-bit / 4-bit-salient layouts) only the kept chunks' low key
    digits, key scale/zero and ring keys count; the salient high digits are
    one word per token and are read whole."""
    R = w.residual
    nq = 32 * (max(0, T - R) // 32)
    nr = T - nq
    n_hi_ch, n_one_ch = 2 * w.n_pairs_hi, 2 * w.n_pairs_lo1
    n_two_ch = 128 - n_hi_ch - n_one_ch
    bh = w.batch * w.n_kv_heads
    qo = 2 * w.batch * w.n_q_heads * 128 * 2
    if n_keep < 4:
        assert w.bits_hi == 4 and w.n_pairs_lo1 == 0
        per_tok = (2 * 32 * n_keep + 2 * n_hi_ch) / 8 + 4 * n_keep + 32 + 16
        return int(round(bh * (nq * per_tok + nr * (64 * n_keep + 256)) + qo))
    if w.bits_hi == 16:
        k_code_bits = n_hi_ch * 16 + n_two_ch * 2 + n_one_ch
        k_meta = (128 - n_hi_ch) * 4 / 32
    else:
        k_code_bits = n_hi_ch * w.bits_hi + n_two_ch * 2 + n_one_ch
        k_meta = 128 * 4 / 32
    per_tok = k_code_bits / 8 + k_meta + 32 + 16
    if w.n_vblk_hi:  # the high-precision tokens' extra value bits (decode skips the order bytes)
        per_tok += w.n_vblk_hi / 4 * (w.bits_vhi - 2) * 128 / 8
    return int(round(bh * (nq * per_tok + nr * 512) + qo))


def layout_bytes(cache, w, T: int) -> int:
    """Bytes the packed layout actually holds for T tokens (read per step)."""
    R = w.residual
    nq = 32 * (max(0, T - R) // 32)
    nr = T - nq
    ng = nq // 32
    bh = w.batch * w.n_kv_heads
    khi = cache.sizes[1] // max(1, bh * cache_ng(cache, w))
    vhi = cache.sizes[11] // max(1, bh * cache_ng(cache, w))
    per_grp = 1024 + khi + 512 + 1024 + 512 + vhi
    return bh * (ng * per_grp + nr * 512) + 2 * w.batch * w.n_q_heads * 128 * 2


def cache_ng(cache, w):
    return max(cache.layout.max_tokens - w.residual, 0) // 32


def default_splits(w) -> int:
    # one 8-wave workgroup per CU: 256 CUs / (sequences * KV heads)
    return max(1, min(1024, math.ceil(256 / (w.batch * w.n_kv_heads))))


SM_SCALE = 1.0 / math.sqrt(128.0)
METRIC = "quantized-KV decode attn: \u00b5s/step, effective HBM GB/s, % of 8 TB/s peak"


def dev(bits):
    """uint16 bit array -> contiguous int16 tensor on the GPU."""
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def copy_calibration(mib: int, reps: int = 5):
    """Plain device-to-device copies of `mib` MiB (read mib, write mib): the
    reference dispatch for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = mib * 2 ** 20
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_mib": mib, "reps": reps}), flush=True)


def cpu_baseline(w, data, min_s: float = 10.0):
    """The oracle's decode step (all query heads, unsplit fp64) timed on this
    host, single thread, repeated until about `min_s` seconds have passed."""
    import numpy as np
    import oracle
    T = w.tokens
    _, pairs = oracle.select(data["q_sel"], data["k"], T, w.n_kv_heads, w.io_dtype)
    qz = oracle.quantize(data["k"], data["v"], T, pairs, residual=w.residual,
                         n_pairs_hi=w.n_pairs_hi, bits_hi=w.bits_hi, io_dtype=w.io_dtype)
    q = data["q_dec"][:, :, 0]
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.attention(qz, q, float(np.float32(SM_SCALE)))
        n += 1
        el = time.perf_counter() - t0
        if el >= min_s:
            break
    per_step_s = el / n
    return {"value": round(algorithmic_bytes(w, T) / per_step_s / 1e9, 4), "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": "%d full decode steps of the same workload (all %d query heads, %d "
                      "tokens), fp64, 1 thread" % (n, w.batch * w.n_q_heads, T),
            "us_per_step": round(per_step_s * 1e6, 1)}


def streaming_leg(args, w):
    """Long-output decoding: after a prefill of w.tokens tokens, every step
    appends one token per (sequence, KV head) with kvq_append and then decodes
    the next query with kvq_decode_attn, for w.n_app steps.  NL independent
    layer caches (together >= --replica-mib) are stepped in turn, as the
    layers of a model are, so the 256 MB Infinity Cache cannot hold the
    working set.  Two timed passes over the same sequence from the same
    prefilled state: append + decode, then append alone; a third pass runs
    the same steps as one kvq_append_decode_attn launch each."""
    import ctypes

    import numpy as np
    import torch

    import kvq_synth
    from decode_attention_select_amd import kvq

    T0, n = w.tokens, w.n_app
    data = kvq_synth.generate(w)
    layout = kvq.make_layout(w.batch, w.n_q_heads, w.n_kv_heads, n_pairs_hi=w.n_pairs_hi,
                             bits_hi=w.bits_hi, residual=w.residual, max_tokens=T0 + n,
                             io_dtype=w.io_dtype)
    pristine = kvq.Cache(layout)
    kvq.kvq_select_pairs(layout, dev(data["q_sel"]), w.n_qry, dev(data["k"][:, :, :T0]), T0,
                         pristine.struct)
    kvq.kvq_quant_keys(layout, dev(data["k"][:, :, :T0]), T0, pristine.struct)
    kvq.kvq_quant_values(layout, dev(data["v"][:, :, :T0]), T0, pristine.struct)
    torch.cuda.synchronize()
    NL = max(1, math.ceil(args.replica_mib * 2 ** 20 / pristine.nbytes()))
    layers = []
    for _ in range(NL):
        c = kvq.Cache.__new__(kvq.Cache)
        c.layout, c.sizes = pristine.layout, pristine.sizes
        c.bufs = {k: v.clone() for k, v in pristine.bufs.items()}
        c.struct = kvq.kvq_cache(*[c.bufs[nm].data_ptr() for nm in kvq.BUF_NAMES])
        layers.append(c)
    kn = [dev(np.ascontiguousarray(data["k"][:, :, T0 + i])) for i in range(n)]
    vn = [dev(np.ascontiguousarray(data["v"][:, :, T0 + i])) for i in range(n)]
    qd = [dev(np.ascontiguousarray(data["q_dec"][:, :, i])) for i in range(n)]
    S = args.splits or w.n_splits or default_splits(w)
    ws = torch.zeros(kvq.kvq_workspace_bytes(layout, S), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    lib = kvq.lib()
    L, st = ctypes.byref(layout), ctypes.c_void_p(stream.cuda_stream)
    P = ctypes.c_void_p
    scale = ctypes.c_float(float(np.float32(SM_SCALE)))
    wsb = ctypes.c_size_t(ws.numel())
    app_args = [(P(kn[i].data_ptr()), P(vn[i].data_ptr())) for i in range(n)]
    dec_args = [P(qd[i].data_ptr()) for i in range(n)]
    structs = [ctypes.byref(c.struct) for c in layers]

    def restore():
        torch.cuda.synchronize()
        for c in layers:
            for k, v in c.bufs.items():
                v.copy_(pristine.bufs[k])
        torch.cuda.synchronize()

    def run(decode):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for i in range(n):
            a, b = app_args[i]
            for cs in structs:
                assert lib.kvq_append(L, a, b, cs, st) == 0
                if decode:
                    assert lib.kvq_decode_attn(L, dec_args[i], cs, scale, S, P(ws.data_ptr()), wsb,
                                               P(out.data_ptr()), st) == 0
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) * 1e3 / (n * NL)

    # warm-up: decodes leave the caches unchanged
    for i in range(args.warmup):
        assert lib.kvq_decode_attn(L, dec_args[0], structs[0], scale, S, P(ws.data_ptr()), wsb,
                                   P(out.data_ptr()), st) == 0
    def run_fused():
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for i in range(n):
            a, b = app_args[i]
            for cs in structs:
                assert lib.kvq_append_decode_attn(L, a, b, dec_args[i], cs, scale, S,
                                                  P(ws.data_ptr()), wsb, P(out.data_ptr()),
                                                  st) == 0
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) * 1e3 / (n * NL)

    step_us = run(True)
    for c in layers:
        assert kvq.kvq_check(c.struct) == 0
    restore()
    append_us = run(False)
    decode_us = step_us - append_us
    restore()
    fused_us = run_fused()
    for c in layers:
        assert kvq.kvq_check(c.struct) == 0
    alg = sum(algorithmic_bytes(w, T0 + i + 1) for i in range(n)) / n
    gbs = alg / (decode_us * 1e-6) / 1e9
    return {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": n,
        "warmup": args.warmup,
        "ms_per_step": round(step_us * 1e-3, 5),
        "us_per_step": round(step_us, 3),
        "append_us_per_step": round(append_us, 3),
        "decode_us_per_step": round(decode_us, 3),
        "fused_us_per_step": round(fused_us, 3),
        "pct_of_peak": round(100 * gbs / PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 (MFMA) / f32 accumulate",
        "data": "synthetic (seeded N(0,1) + outlier key pairs, RoPE)",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.n_q_heads,
                   "kv_heads": w.n_kv_heads, "prefill": T0, "appended": n,
                   "io_dtype": w.io_dtype, "salient_pairs": w.n_pairs_hi,
                   "salient_bits": w.bits_hi, "residual": w.residual, "n_splits": S,
                   "layer_caches": NL},
        "algorithmic_bytes_per_step": int(alg),
        "note": "one step = kvq_append + kvq_decode_attn on one layer cache; value = "
                "decode bytes / (step time - append time); fused_us_per_step: the same "
                "steps as one kvq_append_decode_attn launch each",
    }


def pareto_leg(args, w):
    """Bit-allocation sweep on one workload: for every point of
    kvq_synth.PARETO_POINTS (key bits) and kvq_synth.VALUE_POINTS (two value
    precisions on the 2.26-bit keys), the decode time and effective GB/s (cache
    replicas beyond the Infinity Cache, as in the main leg) and the attention
    error of the GPU output against plain softmax attention over the
    unquantized 16-bit keys and values (fp64 on the host)."""
    import dataclasses

    import numpy as np
    import torch

    import kvq_synth
    from decode_attention_select_amd import kvq

    T = w.tokens
    data = kvq_synth.generate(w)
    q_bits = data["q_dec"][:, :, 0]
    # unquantized reference, every query head
    qf = kvq_synth.bits_to_f64(q_bits, w.io_dtype)
    G = w.group_size
    ref = np.zeros((w.batch, w.n_q_heads, 128))
    for b in range(w.batch):
        for kh in range(w.n_kv_heads):
            K = kvq_synth.bits_to_f64(data["k"][b, kh, :T], w.io_dtype)
            V = kvq_synth.bits_to_f64(data["v"][b, kh, :T], w.io_dtype)
            lg = (qf[b, kh * G:(kh + 1) * G] @ K.T) * SM_SCALE
            p = np.exp(lg - lg.max(axis=1, keepdims=True))
            ref[b, kh * G:(kh + 1) * G] = (p / p.sum(axis=1, keepdims=True)) @ V
    points = []
    S = args.splits or w.n_splits or default_splits(w)
    pts = [(label, n_hi, bits_hi, n_lo1, 0, 4)
           for label, n_hi, bits_hi, n_lo1 in kvq_synth.PARETO_POINTS]
    pts += [(label, 6, 4, 0, nvb, bvh) for label, nvb, bvh in kvq_synth.VALUE_POINTS]
    for label, n_hi, bits_hi, n_lo1, nvb, bvh in pts:
        wp = dataclasses.replace(w, n_pairs_hi=n_hi, bits_hi=bits_hi, n_pairs_lo1=n_lo1,
                                 n_vblk_hi=nvb, bits_vhi=bvh)
        layout = kvq.make_layout(w.batch, w.n_q_heads, w.n_kv_heads, n_pairs_hi=n_hi,
                                 bits_hi=bits_hi, n_pairs_lo1=n_lo1, residual=w.residual,
                                 max_tokens=T, io_dtype=w.io_dtype, n_vblk_hi=nvb,
                                 bits_vhi=bvh)
        base = kvq.Cache(layout)
        kvq.kvq_select_pairs(layout, dev(data["q_sel"]), w.n_qry, dev(data["k"][:, :, :T]), T,
                             base.struct)
        kvq.kvq_quant_keys(layout, dev(data["k"][:, :, :T]), T, base.struct)
        kvq.kvq_quant_values(layout, dev(data["v"][:, :, :T]), T, base.struct)
        torch.cuda.synchronize()
        n_rep = max(1, math.ceil(args.replica_mib * 2 ** 20 / base.nbytes()))
        reps = [base]
        for _ in range(n_rep - 1):
            r = kvq.Cache.__new__(kvq.Cache)
            r.layout, r.sizes = base.layout, base.sizes
            r.bufs = {k: v.clone() for k, v in base.bufs.items()}
            r.struct = kvq.kvq_cache(*[r.bufs[nm].data_ptr() for nm in kvq.BUF_NAMES])
            reps.append(r)
        q = dev(q_bits)
        out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.int16, device="cuda")
        ws = torch.zeros(kvq.kvq_workspace_bytes(layout, S), dtype=torch.uint8, device="cuda")
        stream = torch.cuda.current_stream()
        sc = float(np.float32(SM_SCALE))
        for i in range(args.warmup):
            kvq.kvq_decode_attn(layout, q, reps[i % n_rep].struct, sc, S, ws, out, stream=stream)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for i in range(args.steps):
            kvq.kvq_decode_attn(layout, q, reps[i % n_rep].struct, sc, S, ws, out, stream=stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        us = ev0.elapsed_time(ev1) * 1e3 / args.steps
        got = kvq_synth.bits_to_f64(out.cpu().numpy().view(np.uint16), w.io_dtype)
        err = np.abs(got - ref)
        alg = algorithmic_bytes(wp, T)
        points.append({"bits": label, "salient_pairs": n_hi, "salient_bits": bits_hi,
                       "one_bit_pairs": n_lo1, "value_blocks_hi": nvb,
                       "value_bits_hi": bvh if nvb else None, "us_per_step": round(us, 3),
                       "GBs": round(alg / (us * 1e-6) / 1e9, 1),
                       "algorithmic_bytes": alg, "layout_bytes": layout_bytes(base, wp, T),
                       "max_abs_err_vs_unquantized": float(err.max()),
                       "mean_abs_err_vs_unquantized": float(err.mean()),
                       "rel_l2_err_vs_unquantized": float(np.linalg.norm(got - ref) /
                                                          np.linalg.norm(ref))})
        del reps, base
        torch.cuda.empty_cache()
    main_pt = [p for p in points if p["bits"] == "2.26"][0]
    return {
        "metric": METRIC,
        "value": main_pt["GBs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_pt["us_per_step"] * 1e-3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 (MFMA) / f32 accumulate",
        "data": "synthetic (seeded N(0,1) + outlier key pairs, RoPE)",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.n_q_heads,
                   "kv_heads": w.n_kv_heads, "context": T, "io_dtype": w.io_dtype,
                   "residual": w.residual, "n_splits": S},
        "pareto": points,
        "note": "value = the 2.26-bit point; errors are against fp64 softmax attention over "
                "the unquantized 16-bit K/V, all query heads",
    }


def prefill_leg(args, w):
    """The calls that build a cache, each timed on its own over the workload:
    pair selection (kvq_select_pairs and the query-aware kvq_select_pairs_qa),
    key and value quantization, and the precision shrink of every quantized
    group.  Inputs rotate over replicas (together >= --replica-mib) so that
    the 256 MB Infinity Cache cannot serve them.  Algorithmic bytes per call:
      select:        queries + keys read, ranks and sums written;
      quant_keys:    keys read; per quantized token the key codes at their
                     bits plus scale/zero, per ring token 256 B, written;
      quant_values:  values read; per quantized token 32 B codes + 16 B
                     scale/zero, per ring token 256 B, written;
      shrink:        the salient channels' 4-bit codes read and written."""
    import numpy as np
    import torch

    import kvq_synth
    from decode_attention_select_amd import kvq

    T = w.tokens
    data = kvq_synth.generate(w)
    layout = kvq.make_layout(w.batch, w.n_q_heads, w.n_kv_heads, n_pairs_hi=w.n_pairs_hi,
                             bits_hi=w.bits_hi, residual=w.residual, max_tokens=T,
                             io_dtype=w.io_dtype, n_vblk_hi=w.n_vblk_hi, bits_vhi=w.bits_vhi)
    cache = kvq.Cache(layout)
    k0, v0, q0 = dev(data["k"][:, :, :T]), dev(data["v"][:, :, :T]), dev(data["q_sel"])
    n_rep = max(1, math.ceil(args.replica_mib * 2 ** 20 / (k0.numel() * 2)))
    ks = [k0] + [k0.clone() for _ in range(n_rep - 1)]
    vs = [v0] + [v0.clone() for _ in range(n_rep - 1)]
    qs = [q0] + [q0.clone() for _ in range(n_rep - 1)]
    stream = torch.cuda.current_stream()
    st = lambda f: (lambda i: f(i % n_rep))
    nq = 32 * (max(0, T - w.residual) // 32)
    nr, bh = T - nq, w.batch * w.n_kv_heads
    kv_in = bh * T * 256
    q_in = w.batch * w.n_q_heads * w.n_qry * 256
    sel_out = bh * (64 * 4 + 2 * 64 * 8)
    n_hi_ch = 2 * w.n_pairs_hi
    if w.bits_hi == 16:
        k_tok = (n_hi_ch * 16 + (128 - n_hi_ch) * 2) / 8 + (128 - n_hi_ch) * 4 / 32
    else:
        k_tok = (n_hi_ch * w.bits_hi + (128 - n_hi_ch) * 2) / 8 + 16
    # two value precisions: the key side writes each group's 32 order bytes,
    # the value side reads them and writes 256 bytes per 8 high-precision tokens
    vhi_k = bh * (nq // 32) * 32 if w.n_vblk_hi else 0
    vhi_v = bh * (nq // 32) * (32 + 256 * w.n_vblk_hi) if w.n_vblk_hi else 0
    calls = [
        ("kvq_select_pairs", q_in + kv_in + sel_out,
         st(lambda i: kvq.kvq_select_pairs(layout, qs[i], w.n_qry, ks[i], T, cache.struct,
                                           stream=stream))),
        ("kvq_select_pairs_qa", q_in + kv_in + sel_out,
         st(lambda i: kvq.kvq_select_pairs_qa(layout, qs[i], w.n_qry, ks[i], T, cache.struct,
                                              stream=stream))),
        ("kvq_quant_keys", kv_in + int(bh * (nq * k_tok + nr * 256)) + vhi_k,
         st(lambda i: kvq.kvq_quant_keys(layout, ks[i], T, cache.struct, stream=stream))),
        ("kvq_quant_values", kv_in + bh * (nq * 48 + nr * 256) + vhi_v,
         st(lambda i: kvq.kvq_quant_values(layout, vs[i], T, cache.struct, stream=stream))),
    ]
    res_calls = []
    for name, alg, f in calls:
        for i in range(args.warmup):
            f(i)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for i in range(args.steps):
            f(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        us = ev0.elapsed_time(ev1) * 1e3 / args.steps
        res_calls.append({"call": name, "us": round(us, 3), "algorithmic_bytes": alg,
                          "GBs": round(alg / (us * 1e-6) / 1e9, 1)})
    # shrink: a fresh quantization before every timed call (outside the timing),
    # so that each call shrinks 4-bit codes of every quantized group
    ng = nq // 32
    sh_alg = 2 * bh * nq * n_hi_ch * 4 // 8
    tot = 0.0
    for i in range(args.warmup + args.steps if w.bits_hi == 4 and w.n_pairs_hi else 0):
        kvq.kvq_quant_keys(layout, ks[i % n_rep], T, cache.struct, stream=stream)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        kvq.kvq_shrink(layout, cache.struct, 0, ng, stream=stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        if i >= args.warmup:
            tot += ev0.elapsed_time(ev1) * 1e3
    us = tot / args.steps
    if tot:
        res_calls.append({"call": "kvq_shrink", "us": round(us, 3), "algorithmic_bytes": sh_alg,
                          "GBs": round(sh_alg / (us * 1e-6) / 1e9, 1),
                          "note": "one launch per call, timed alone; a plain event pair around "
                                  "one launch also holds the launch latency"})
    build = [c for c in res_calls if c["call"] in ("kvq_select_pairs", "kvq_quant_keys",
                                                   "kvq_quant_values")]
    b_us = sum(c["us"] for c in build)
    b_alg = sum(c["algorithmic_bytes"] for c in build)
    gbs = b_alg / (b_us * 1e-6) / 1e9
    return {
        "metric": "cache build (select + quantize keys + quantize values): \u00b5s, "
                  "effective HBM GB/s, % of 8 TB/s peak",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(b_us * 1e-3, 5),
        "pct_of_peak": round(100 * gbs / PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (min/max, codes) / u64 (saliency sums)",
        "data": "synthetic (seeded N(0,1) + outlier key pairs, RoPE)",
        "config": {"workload": w.name + " (cache build)", "batch": w.batch,
                   "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads, "context": T,
                   "selection_queries": w.n_qry, "io_dtype": w.io_dtype,
                   "salient_pairs": w.n_pairs_hi, "salient_bits": w.bits_hi,
                   "residual": w.residual, "input_replicas": n_rep,
                   "value_hi_tokens": 8 * w.n_vblk_hi,
                   "value_hi_bits": w.bits_vhi if w.n_vblk_hi else None},
        "calls": res_calls,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3-8b-32k")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--replica-mib", type=int, default=512)
    ap.add_argument("--prune", type=int, default=4,
                    help="kvq_decode_attn_pruned with this many of the four 32-channel key "
                         "chunks kept (4: kvq_decode_attn)")
    ap.add_argument("--build", action="store_true",
                    help="time the cache-building calls on the workload instead of decode")
    ap.add_argument("--value-hi", default="",
                    help="with --build: N:B, the N*8 tokens of largest key magnitude per group "
                         "get B-bit values (two value precisions)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run the copy-kernel calibration of this size")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_mib:
        copy_calibration(args.copy_mib)
        return

    import numpy as np
    import torch

    import kvq_synth
    from decode_attention_select_amd import kvq

    w = kvq_synth.workload(args.workload)
    if args.value_hi:
        nvb, bvh = (int(x) for x in args.value_hi.split(":"))
        w = w.replace(n_vblk_hi=nvb, bits_vhi=bvh)
    if args.build:
        print(json.dumps(prefill_leg(args, w)), flush=True)
        return
    if w.n_app:
        print(json.dumps(streaming_leg(args, w)), flush=True)
        return
    if w.name.startswith("pareto"):
        print(json.dumps(pareto_leg(args, w)), flush=True)
        return
    S = args.splits or w.n_splits or default_splits(w)
    T = w.tokens
    data = kvq_synth.generate(w)
    layout = kvq.make_layout(w.batch, w.n_q_heads, w.n_kv_heads, n_pairs_hi=w.n_pairs_hi,
                             bits_hi=w.bits_hi, residual=w.residual, max_tokens=T,
                             io_dtype=w.io_dtype)
    base = kvq.Cache(layout)
    kvq.kvq_select_pairs(layout, dev(data["q_sel"]), w.n_qry, dev(data["k"][:, :, :T]), T,
                         base.struct)
    kvq.kvq_quant_keys(layout, dev(data["k"][:, :, :T]), T, base.struct)
    kvq.kvq_quant_values(layout, dev(data["v"][:, :, :T]), T, base.struct)
    torch.cuda.synchronize()

    n_rep = max(1, math.ceil(args.replica_mib * 2 ** 20 / base.nbytes()))
    replicas = [base]
    for _ in range(n_rep - 1):
        r = kvq.Cache.__new__(kvq.Cache)
        r.layout, r.sizes = base.layout, base.sizes
        r.bufs = {k: v.clone() for k, v in base.bufs.items()}
        r.struct = kvq.kvq_cache(*[r.bufs[n].data_ptr() for n in kvq.BUF_NAMES])
        replicas.append(r)
    q = dev(data["q_dec"][:, :, 0])
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.int16, device="cuda")
    ws = torch.zeros(kvq.kvq_workspace_bytes(layout, S), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        if args.prune < 4:
            kvq.kvq_decode_attn_pruned(layout, q, replicas[i % n_rep].struct,
                                       float(np.float32(SM_SCALE)), S, args.prune, ws, out,
                                       stream=stream)
        else:
            kvq.kvq_decode_attn(layout, q, replicas[i % n_rep].struct,
                                float(np.float32(SM_SCALE)), S, ws, out, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ev_ms = ev0.elapsed_time(ev1) / args.steps


    # One step is one launch of the decode kernel, back to back on one stream:
    # the event-timed average over the timed region is its average launch
    # duration (it also holds the short gap between launches).
    alg = algorithmic_bytes(w, T, args.prune)
    gbs = alg / (ev_ms * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ev_ms, 5),
        "us_per_step": round(ev_ms * 1e3, 3),
        "wall_ms_per_step": round(wall_ms, 5),
        "pct_of_peak": round(100 * gbs / PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 (MFMA) / f32 accumulate",
        "data": "synthetic (seeded N(0,1) + outlier key pairs, RoPE)",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.n_q_heads,
                   "kv_heads": w.n_kv_heads, "context": T, "io_dtype": w.io_dtype,
                   "salient_pairs": w.n_pairs_hi, "salient_bits": w.bits_hi,
                   "residual": w.residual, "n_splits": S, "cache_replicas": n_rep,
                   **({"kept_key_chunks": args.prune} if args.prune < 4 else {})},
        "algorithmic_bytes_per_step": alg,
        "layout_bytes_per_step": layout_bytes(base, w, T),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_GBS, 4),
                     "traffic": TRAFFIC if (args.prune == 4 and
                                            w.name == "llama3-8b-32k") else None},
    }
    if args.prune < 4:
        res["note"] = ("query-channel pruning: %d of 4 key chunks kept per KV head; bytes are "
                       "those of the kept chunks" % args.prune)
    if not args.no_cpu_baseline and args.prune == 4:
        res["cpu_baseline"] = cpu_baseline(w, data)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
