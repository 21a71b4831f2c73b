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
import dataclasses
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0
# HBM bytes per launch of the decode kernel on the default workload: a
# committed record of the FETCH_SIZE and WRITE_SIZE counters scaled by a plain
# copy (written by --traffic-from), valid only for the machine code it was
# measured on (a hash of the kernel's bytes in the built library is in the
# record); null once the kernel has changed.
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "decode_traffic_llama3-8b-32k.md")
# the decode kernel instance of the default workload: bf16, 4-bit salient
# digits, quantized groups, unpruned, one value precision, no append, G <= 8
DECODE_KERNEL = "_ZN3kvq13decode_kernelILb1ELi4ELb1ELi0ELb0ELb0ELb1ELb0ELb0EEEv"


def kernel_code_hash(symbol_prefix: str = DECODE_KERNEL, lib_path: str = None):
    """sha256 (16 hex digits) of a kernel's machine code in the gfx950 code
    objects embedded in libkvq.so (the library compiled from these sources), or None."""
    import hashlib
    import struct
    if lib_path is None:
        lib_path = os.path.join(ROOT, "decode_attention_select_amd", "libkvq.so")
    try:
        data = open(lib_path, "rb").read()
    except OSError:
        return None

    def sections(buf, base):
        shoff = struct.unpack_from("<Q", buf, base + 40)[0]
        shentsize, shnum, shstrndx = struct.unpack_from("<HHH", buf, base + 58)
        secs = [struct.unpack_from("<IIQQQQIIQQ", buf, base + shoff + k * shentsize)
                for k in range(shnum)]
        return secs, secs[shstrndx]

    def cstr(buf, at):
        return buf[at:buf.index(b"\0", at)].decode()

    secs, strtab = sections(data, 0)
    fat = [sh for sh in secs if cstr(data, strtab[4] + sh[0]) == ".hip_fatbin"]
    if not fat:
        return None
    blob = data[fat[0][4]:fat[0][4] + fat[0][5]]
    i = 0
    while True:
        i = blob.find(b"\x7fELF", i)
        if i < 0:
            return None
        if struct.unpack_from("<H", blob, i + 18)[0] == 224:  # EM_AMDGPU
            csecs, _ = sections(blob, i)
            for st in [sh for sh in csecs if sh[1] == 2]:  # SHT_SYMTAB
                names = csecs[st[6]]
                for k in range(st[5] // 24):
                    nm, info, _, shndx, val, size = struct.unpack_from("<IBBHQQ", blob,
                                                                       i + st[4] + k * 24)
                    if (info & 15) == 2 and cstr(blob, i + names[4] + nm).startswith(symbol_prefix):
                        sec = csecs[shndx]
                        at = i + sec[4] + (val - sec[3])
                        return hashlib.sha256(blob[at:at + size]).hexdigest()[:16]
        i += 4


def measured_traffic(workload: str):
    """Bytes per launch from the committed counter record, or None when there
    is no record for this workload or the kernel's machine code has changed."""
    try:
        lines = open(TRAFFIC_RECORD).read().splitlines()
    except OSError:
        return None
    for line in lines:
        if line.startswith("record: "):
            rec = json.loads(line[len("record: "):])
            if rec.get("workload") == workload and rec.get("kernel") == kernel_code_hash():
                return int(rec["bytes_per_launch"])
    return None


def counter_means(db_dir: str, kernel_substring: str) -> dict:
    """Per-dispatch means of every counter of the dispatches whose kernel name
    holds `kernel_substring`, from a rocprofv3 --pmc output directory."""
    import glob
    import sqlite3
    out = {}
    for db in glob.glob(os.path.join(db_dir, "**", "*.db"), recursive=True):
        con = sqlite3.connect(db)
        q = ("select s.kernel_name, d.id, p.name, e.value from rocpd_kernel_dispatch d "
             "join rocpd_info_kernel_symbol s on d.kernel_id = s.id "
             "join rocpd_pmc_event e on e.event_id = d.event_id "
             "join rocpd_info_pmc p on e.pmc_id = p.id")
        for name, did, pmc, val in con.execute(q):
            if kernel_substring in name:
                out.setdefault(pmc, {}).setdefault(did, 0.0)
                out[pmc][did] += val
    return {k: sum(v.values()) / len(v) for k, v in out.items()}


def traffic_record(dec_fetch, dec_write, copy_fetch, copy_write, copy_mib=256):
    """The traffic record line from four rocprofv3 --pmc directories: the
    decode kernel's FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled
    by what the same counter reads for a copy of copy_mib MiB."""
    f = counter_means(dec_fetch, "decode_kernel")["FETCH_SIZE"]
    wr = counter_means(dec_write, "decode_kernel")["WRITE_SIZE"]
    cf = counter_means(copy_fetch, "copyBuffer")["FETCH_SIZE"]
    cw = counter_means(copy_write, "copyBuffer")["WRITE_SIZE"]
    kib = copy_mib * 1024.0
    sf, sw = kib / cf, kib / cw
    return {"workload": "llama3-8b-32k", "kernel": kernel_code_hash(),
            "fetch_kib": round(f, 2), "write_kib": round(wr, 2),
            "copy_fetch_kib": round(cf, 2), "copy_write_kib": round(cw, 2),
            "fetch_scale": round(sf, 4), "write_scale": round(sw, 4),
            "bytes_per_launch": int(round((f * sf + wr * sw) * 1024))}


def algorithmic_bytes(w, T: int, n_keep: int = 8) -> int:
    """Bytes a decode step must move.  With n_keep < 8 (query-channel
    pruning, 2-bit / 4-bit-salient layouts) only the kept 16-channel runs'
    low key digits, key scale/zero and ring keys count; the salient high
    digits are one word per token and are read whole."""
    R = w.residual
    nq = 32 * (max(0, T - R) // 32)
    nr = T - nq
    n_hi_ch, n_one_ch = 2 * w.n_pairs_hi, 2 * w.n_pairs_lo1
    n_two_ch = 128 - n_hi_ch - n_one_ch
    bh = w.batch * w.n_kv_heads
    qo = 2 * w.batch * w.n_q_heads * 128 * 2
    if n_keep < 8:
        assert w.bits_hi == 4 and w.n_pairs_lo1 == 0
        per_tok = (2 * 16 * n_keep + 2 * n_hi_ch) / 8 + 2 * n_keep + 32 + 16
        return int(round(bh * (nq * per_tok + nr * (32 * n_keep + 256)) + qo))
    raw = n_hi_ch if w.bits_hi == 16 else 0
    k_meta = (128 - raw) * 4 / 32

    def per_tok_at(width):
        # progressive groups of `width` bits: every non-raw key channel and
        # every value at that width (salient 4-bit channels never below 4)
        kb = raw * 16 + (128 - raw) * width
        return kb / 8 + k_meta + 128 * width / 8 + 16

    if w.prog_w4 > 0:
        ng = nq // 32
        n8 = min(w.prog_w8, ng)
        n4 = min(w.prog_w4, ng) - n8
        tok = 32 * (n8 * per_tok_at(8) + n4 * per_tok_at(4))
        w2 = dataclasses.replace(w, prog_w8=0, prog_w4=0)
        rest = algorithmic_bytes(w2, 32 * (ng - n8 - n4) + R) - (
            bh * R * 512 + qo)  # the 2-bit groups alone
        return int(round(bh * (tok + nr * 512) + rest + qo))
    if w.bits_hi == 16:
        k_code_bits = n_hi_ch * 16 + n_two_ch * 2 + n_one_ch
    else:
        k_code_bits = n_hi_ch * w.bits_hi + n_two_ch * 2 + n_one_ch
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
    klo = cache.sizes[0] // max(1, bh * cache_ng(cache, w))  # 768 in the dense 1-bit layout
    khi = cache.sizes[1] // max(1, bh * cache_ng(cache, w))
    vhi = cache.sizes[11] // max(1, bh * cache_ng(cache, w))
    per_grp = klo + khi + 512 + 1024 + 512 + vhi
    return bh * (ng * per_grp + nr * 512) + 2 * w.batch * w.n_q_heads * 128 * 2


def cache_ng(cache, w):
    return max(cache.layout.max_tokens - w.residual, 0) // 32


def default_splits(w) -> int:
    """One 8-wave workgroup per CU (256 CUs / (sequences * KV heads)), but no
    more splits than give every wave two quantized groups: a short context
    spread over many splits only adds merge work."""
    per_cu = math.ceil(256 / (w.batch * w.n_kv_heads))
    groups = max(0, w.tokens - w.residual) // 32
    return max(1, min(1024, per_cu, math.ceil(groups / 16)))


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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores() -> int:
    """Threads for the all-core leg: the CPUs this process may run on, at most
    16 (one GPU's share of a shared host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(w, data, min_s: float = 10.0):
    """The oracle's decode step (all query heads, unsplit fp64) on this host:
    once on one thread, then on every host core (one thread per core, each
    running whole steps; the oracle is one C call that releases the GIL), each
    leg repeated until about `min_s` seconds have passed."""
    import threading

    import numpy as np
    import oracle
    T = w.tokens
    _, pairs = oracle.select(data["q_sel"], data["k"], T, w.n_kv_heads, w.io_dtype)
    qz = oracle.quantize(data["k"], data["v"], T, pairs, residual=w.residual,
                         n_pairs_hi=w.n_pairs_hi, bits_hi=w.bits_hi, io_dtype=w.io_dtype)
    q = data["q_dec"][:, :, 0]
    sc = float(np.float32(SM_SCALE))

    def leg(n_threads):
        counts = [0] * n_threads
        stop = time.perf_counter() + min_s

        def worker(i):
            while True:
                oracle.attention(qz, q, sc)
                counts[i] += 1
                if time.perf_counter() >= stop:
                    break
        ts = [threading.Thread(target=worker, args=(i,)) for i in range(n_threads)]
        t0 = time.perf_counter()
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        return sum(counts), time.perf_counter() - t0

    alg = algorithmic_bytes(w, T)
    n1, el1 = leg(1)
    cores = host_cores()
    nc, elc = leg(cores)
    return {"value": round(alg * nc / elc / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": "whole decode steps of the same workload (all %d query heads, %d tokens), "
                      "fp64: %d steps on %d threads in %.1f s; single thread: %d steps in %.1f s"
                      % (w.batch * w.n_q_heads, T, nc, cores, elc, n1, el1),
            "us_per_step": round(elc / nc * 1e6, 1),
            "single_thread": {"value": round(alg * n1 / el1 / 1e9, 4), "unit": "GB/s",
                              "us_per_step": round(el1 / n1 * 1e6, 1)},
            "nproc": os.cpu_count(), "cpu_model": cpu_model()}


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
                             io_dtype=w.io_dtype, prog_w8=w.prog_w8, prog_w4=w.prog_w4)
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

    def run_graph(fused):
        # one HIP graph holds a token's step on every layer cache (a model's
        # decode step), captured once with static inputs and replayed n times
        restore()
        kst, vst, qst = kn[0].clone(), vn[0].clone(), qd[0].clone()
        a, b, qq = P(kst.data_ptr()), P(vst.data_ptr()), P(qst.data_ptr())
        wsp, outp = P(ws.data_ptr()), P(out.data_ptr())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cst = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for cs in structs:
                if fused:
                    assert lib.kvq_append_decode_attn(L, a, b, qq, cs, scale, S, wsp, wsb, outp,
                                                      cst) == 0
                else:
                    assert lib.kvq_append(L, a, b, cs, cst) == 0
                    assert lib.kvq_decode_attn(L, qq, cs, scale, S, wsp, wsb, outp, cst) == 0
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(n):
            g.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        for c in layers:
            assert kvq.kvq_check(c.struct) == 0
        return ev0.elapsed_time(ev1) * 1e3 / (n * NL)

    graph_us = run_graph(False)
    graph_fused_us = run_graph(True)
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
        "fused_us_per_step": round(fused_us, 3) if fused_us is not None else None,
        "graph_us_per_step": round(graph_us, 3),
        "graph_fused_us_per_step": round(graph_fused_us, 3),
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
                "steps as one kvq_append_decode_attn launch each; graph_*: the two-call and "
                "one-launch steps of every layer cache captured in one HIP graph per token "
                "and replayed",
    }


def unquantized_reference(w, data):
    """fp64 softmax attention over the unquantized 16-bit keys and values,
    every query head of the workload's first decode query."""
    import numpy as np

    import kvq_synth
    T, G = w.tokens, w.group_size
    qf = kvq_synth.bits_to_f64(data["q_dec"][:, :, 0], w.io_dtype)
    ref = np.zeros((w.batch, w.n_q_heads, 128))
    for b in range(w.batch):
        for kh in range(w.n_kv_heads):
            K = kvq_synth.bits_to_f64(data["k"][b, kh, :T], w.io_dtype)
            V = kvq_synth.bits_to_f64(data["v"][b, kh, :T], w.io_dtype)
            lg = (qf[b, kh * G:(kh + 1) * G] @ K.T) * SM_SCALE
            p = np.exp(lg - lg.max(axis=1, keepdims=True))
            ref[b, kh * G:(kh + 1) * G] = (p / p.sum(axis=1, keepdims=True)) @ V
    return ref


def sweep_point(args, wp, data, S, ref):
    """One layout of a sweep: prefill of the workload's T tokens, then the
    decode time over cache replicas beyond the Infinity Cache (as in the main
    leg), effective GB/s, the cache's bytes and the error of the GPU output
    against `ref` (unquantized fp64 attention)."""
    import numpy as np
    import torch

    import kvq_synth
    from decode_attention_select_amd import kvq

    T = wp.tokens
    layout = kvq.make_layout(wp.batch, wp.n_q_heads, wp.n_kv_heads, n_pairs_hi=wp.n_pairs_hi,
                             bits_hi=wp.bits_hi, n_pairs_lo1=wp.n_pairs_lo1, residual=wp.residual,
                             max_tokens=T, io_dtype=wp.io_dtype, n_vblk_hi=wp.n_vblk_hi,
                             bits_vhi=wp.bits_vhi, prog_w8=wp.prog_w8, prog_w4=wp.prog_w4)
    base = kvq.Cache(layout)
    kvq.kvq_select_pairs(layout, dev(data["q_sel"]), wp.n_qry, dev(data["k"][:, :, :T]), T,
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
    q = dev(data["q_dec"][:, :, 0])
    out = torch.empty((wp.batch, wp.n_q_heads, 128), dtype=torch.int16, device="cuda")
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
    got = kvq_synth.bits_to_f64(out.cpu().numpy().view(np.uint16), wp.io_dtype)
    err = np.abs(got - ref)
    alg = algorithmic_bytes(wp, T)
    pt = {"us_per_step": round(us, 3), "GBs": round(alg / (us * 1e-6) / 1e9, 1),
          "algorithmic_bytes": alg, "cache_bytes": base.nbytes(),
          "max_abs_err_vs_unquantized": float(err.max()),
          "mean_abs_err_vs_unquantized": float(err.mean()),
          "rel_l2_err_vs_unquantized": float(np.linalg.norm(got - ref) / np.linalg.norm(ref))}
    if not wp.prog_w4:
        pt["layout_bytes"] = layout_bytes(base, wp, T)
    del reps, base
    torch.cuda.empty_cache()
    return pt


def sweep_line(args, w, S, value_pt, key, points, note):
    return {
        "metric": METRIC,
        "value": value_pt["GBs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(value_pt["us_per_step"] * 1e-3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 (MFMA) / f32 accumulate",
        "data": "synthetic (seeded N(0,1) + outlier key pairs, RoPE)",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.n_q_heads,
                   "kv_heads": w.n_kv_heads, "context": w.tokens, "io_dtype": w.io_dtype,
                   "residual": w.residual, "n_splits": S},
        key: points,
        "note": note,
    }


def pareto_leg(args, w):
    """Bit-allocation sweep on one workload: for every point of
    kvq_synth.PARETO_POINTS (key bits) and kvq_synth.VALUE_POINTS (two value
    precisions on the 2.26-bit keys), the decode time and effective GB/s (cache
    replicas beyond the Infinity Cache, as in the main leg) and the attention
    error of the GPU output against plain softmax attention over the
    unquantized 16-bit keys and values (fp64 on the host)."""
    import kvq_synth

    data = kvq_synth.generate(w)
    ref = unquantized_reference(w, data)
    S = args.splits or w.n_splits or default_splits(w)
    pts = [(label, n_hi, bits_hi, n_lo1, 0, 4)
           for label, n_hi, bits_hi, n_lo1 in kvq_synth.PARETO_POINTS]
    pts += [(label, 6, 4, 0, nvb, bvh) for label, nvb, bvh in kvq_synth.VALUE_POINTS]
    points = []
    for label, n_hi, bits_hi, n_lo1, nvb, bvh in pts:
        wp = dataclasses.replace(w, n_pairs_hi=n_hi, bits_hi=bits_hi, n_pairs_lo1=n_lo1,
                                 n_vblk_hi=nvb, bits_vhi=bvh)
        pt = {"bits": label, "salient_pairs": n_hi, "salient_bits": bits_hi,
              "one_bit_pairs": n_lo1, "value_blocks_hi": nvb,
              "value_bits_hi": bvh if nvb else None}
        pt.update(sweep_point(args, wp, data, S, ref))
        points.append(pt)
    main_pt = [p for p in points if p["bits"] == "2.26"][0]
    return sweep_line(args, w, S, main_pt, "pareto", points,
                      "value = the 2.26-bit point; errors are against fp64 softmax attention "
                      "over the unquantized 16-bit K/V, all query heads")


def prog_leg(args, w):
    """Progressive precision (PM-KVQ review: groups held at 8, then 4, then
    2 bits as they age): for every window setting of kvq_synth.PROG_POINTS
    (prog_w8, prog_w4: the newest groups held at 8 and at 4 bits or more) the
    decode time, the bytes a step reads, the cache's whole footprint and the
    error against unquantized attention.  The first point is the plain 2-bit
    cache, the last every group (up to 256) at 8 bits: the cache before any
    shrink."""
    import kvq_synth

    data = kvq_synth.generate(w)
    ref = unquantized_reference(w, data)
    S = args.splits or w.n_splits or default_splits(w)
    points = []
    for label, w8, w4 in kvq_synth.PROG_POINTS:
        wp = dataclasses.replace(w, prog_w8=w8, prog_w4=w4)
        pt = {"windows": label, "prog_w8": w8, "prog_w4": w4,
              "groups_at_8": min(w8, (w.tokens - w.residual) // 32) if w4 else 0,
              "groups_at_4": (min(w4, (w.tokens - w.residual) // 32) - min(w8, (w.tokens - w.residual) // 32)) if w4 else 0}
        pt.update(sweep_point(args, wp, data, S, ref))
        points.append(pt)
    main_pt = [p for p in points if p["prog_w4"] == 16][0]
    return sweep_line(args, w, S, main_pt, "progressive", points,
                      "value = windows of 4 (8-bit) and 16 (>= 4-bit) groups; cache_bytes is "
                      "the whole footprint at this capacity; errors against fp64 softmax "
                      "attention over the unquantized 16-bit K/V")


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


STAMP_NAMES = [(0, "entry"), (1, "query in"), (2, "ring blocks done"),
               (11, "first group done"), ("loop", "waves' loop end (last wave)"),
               (23, "every wave done"), (24, "wave results in LDS"),
               (12, "waves merged, records issued"), (13, "records stored"),
               (14, "ticket back"), (18, "last workgroup: records requested"),
               (19, "last workgroup: split weights formed"),
               (20, "last workgroup: weighted sum done"),
               (15, "last workgroup: output issued"), (16, "last workgroup: output stored")]
LAST_WG_SLOTS = (15, 16, 18, 19, 20)


def stamps_leg(args, w):
    """Phase timestamps of the decode kernel (libkvq_stamps.so: the same
    kernel with s_memrealtime stamps at fixed points, 100 MHz): per timed
    call, every workgroup's stamps relative to the earliest workgroup entry;
    reported as the median over calls of each phase's median and maximum
    over workgroups, in microseconds."""
    import numpy as np
    import torch

    import kvq_synth
    from decode_attention_select_amd import kvq
    kvq.use_stamps_library()
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
    reps = [base]
    for _ in range(n_rep - 1):
        r = kvq.Cache.__new__(kvq.Cache)
        r.layout, r.sizes = base.layout, base.sizes
        r.bufs = {k: v.clone() for k, v in base.bufs.items()}
        r.struct = kvq.kvq_cache(*[r.bufs[n].data_ptr() for n in kvq.BUF_NAMES])
        reps.append(r)
    q = dev(data["q_dec"][:, :, 0])
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.int16, device="cuda")
    wsb = kvq.kvq_workspace_bytes(layout, S)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    nwg = w.batch * w.n_kv_heads * S
    st_off = wsb - nwg * 32 * 8
    stream = torch.cuda.current_stream()
    sc = float(np.float32(SM_SCALE))
    for i in range(args.warmup):
        kvq.kvq_decode_attn(layout, q, reps[i % n_rep].struct, sc, S, ws, out, stream=stream)
    torch.cuda.synchronize()
    per_call = []
    for i in range(args.steps):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        kvq.kvq_decode_attn(layout, q, reps[i % n_rep].struct, sc, S, ws, out, stream=stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        st = ws[st_off:].cpu().numpy().view(np.uint64).reshape(nwg, 32).astype(np.int64)
        t0 = st[:, 0].min()
        rel = (st - t0) * 0.01  # 100 MHz ticks -> microseconds
        last = ((st[:, 17] >> 40) & 0xFFFF) == S - 1
        row = {"event_us": ev0.elapsed_time(ev1) * 1e3}
        for slot, name in STAMP_NAMES:
            if slot == "loop":
                v = rel[:, 3:3 + 8].max(axis=1)
            elif slot in LAST_WG_SLOTS:
                v = rel[last, slot]
            else:
                v = rel[:, slot]
            row[name] = (float(np.median(v)), float(v.max()))
        per_call.append(row)
    phases = []
    for slot, name in STAMP_NAMES:
        phases.append({"phase": name,
                       "p50_us": round(float(np.median([r[name][0] for r in per_call])), 3),
                       "max_us": round(float(np.median([r[name][1] for r in per_call])), 3)})
    return {"stamps": w.name, "n_splits": S, "workgroups": nwg, "calls": args.steps,
            "event_us_median": round(float(np.median([r["event_us"] for r in per_call])), 3),
            "phases": phases,
            "note": "medians over calls of each phase's median and maximum over workgroups, "
                    "from the earliest workgroup entry; one call at a time (events around "
                    "each), so the event time holds the launch"}


# kvq_issue_probe's mixes: (name, instructions per loop iteration of one wave)
PROBE_KINDS = [("int_valu", 32), ("cvt_pk_f16_fp4+xor", 32), ("pk_mul_f16", 16),
               ("exp_f32+mul_f32", 32), ("mfma_16x16x32_f16", 4), ("mfma+int_valu", 36),
               ("mfma_16x16x16_f16", 4)]
PROBE_ITERS = 256
ENGINE_GHZ = 2.4


def issue_probe_leg():
    """Issue cost per SIMD of the decode loop's instruction kinds (one launch
    of kvq_issue_probe per kind and occupancy, event-timed, mean of 10)."""
    import torch
    from decode_attention_select_amd import kvq

    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    rows = []
    for wps in (1, 2, 8):
        nb = n_cu * wps
        out = torch.empty(nb * 256, dtype=torch.int32, device="cuda")
        us = []
        for kind in range(len(PROBE_KINDS)):
            for _ in range(3):
                kvq.kvq_issue_probe(kind, nb, out, stream=stream)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(10):
                kvq.kvq_issue_probe(kind, nb, out, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            us.append(e0.elapsed_time(e1) * 1e3 / 10)
        # cycles per loop iteration of one wave, per SIMD (all waves of a SIMD
        # share its issue), at the engine clock
        cyc = [u * 1e-6 * ENGINE_GHZ * 1e9 / (wps * PROBE_ITERS) for u in us]
        per_int = cyc[0] / 32
        rows.append({
            "waves_per_simd": wps,
            "us": {n: round(u, 3) for (n, _), u in zip(PROBE_KINDS, us)},
            "cycles_per_instruction": {
                "int_valu": round(per_int, 2),
                "cvt_scalef32_pk_f16_fp4": round((cyc[1] - 16 * per_int) / 16, 2),
                "pk_mul_f16": round(cyc[2] / 16, 2),
                "exp_f32": round((cyc[3] - 16 * per_int) / 16, 2),
                "mfma_16x16x32_f16": round(cyc[4] / 4, 2),
                "mfma_16x16x16_f16": round(cyc[6] / 4, 2),
            },
            # 1: MFMA and VALU issue serialize on a SIMD; max/sum: they overlap
            "mfma_valu_serial_fraction": round(us[5] / (us[4] + us[0]), 3),
            "full_overlap_would_be": round(max(us[4], us[0]) / (us[4] + us[0]), 3),
        })
    return {"issue_probe": "gfx950", "compute_units": n_cu, "engine_ghz": ENGINE_GHZ,
            "iterations_per_wave": PROBE_ITERS, "rows": rows}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3-8b-32k")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--replica-mib", type=int, default=512)
    ap.add_argument("--prune", type=int, default=8,
                    help="kvq_decode_attn_pruned with this many of the eight 16-channel key "
                         "runs kept (8: kvq_decode_attn)")
    ap.add_argument("--build", action="store_true",
                    help="time the cache-building calls on the workload instead of decode")
    ap.add_argument("--value-hi", default="",
                    help="with --build: N:B, the N*8 tokens of largest key magnitude per group "
                         "get B-bit values (two value precisions)")
    ap.add_argument("--prog", default="",
                    help="W8:W4, progressive precision on the workload (the newest W8 groups "
                         "held at 8 bits, the newest W4 at 4 bits or more)")
    ap.add_argument("--stamps", action="store_true",
                    help="phase timestamps of the decode kernel (libkvq_stamps.so)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run the copy-kernel calibration of this size")
    ap.add_argument("--ceiling", action="store_true",
                    help="time only kvq_read_ceiling (the decode's reads, no arithmetic)")
    ap.add_argument("--issue-probe", action="store_true",
                    help="time kvq_issue_probe: the issue cost per SIMD of the decode loop's "
                         "instruction kinds, and whether MFMA overlaps VALU")
    ap.add_argument("--traffic-from", nargs=4, metavar="DIR",
                    help="print the traffic record from four rocprofv3 --pmc output "
                         "directories: decode FETCH_SIZE, decode WRITE_SIZE, copy FETCH_SIZE, "
                         "copy WRITE_SIZE (the copy of --copy-mib 256)")
    args = ap.parse_args()
    if args.traffic_from:
        print("record: " + json.dumps(traffic_record(*args.traffic_from)), flush=True)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_mib:
        copy_calibration(args.copy_mib)
        return
    if args.issue_probe:
        print(json.dumps(issue_probe_leg()), flush=True)
        return

    import numpy as np
    import torch

    import kvq_synth
    from decode_attention_select_amd import kvq

    w = kvq_synth.workload(args.workload)
    if args.value_hi:
        nvb, bvh = (int(x) for x in args.value_hi.split(":"))
        w = w.replace(n_vblk_hi=nvb, bits_vhi=bvh)
    if args.prog:
        w8, w4 = (int(x) for x in args.prog.split(":"))
        w = w.replace(prog_w8=w8, prog_w4=w4)
    if args.build:
        print(json.dumps(prefill_leg(args, w)), flush=True)
        return
    if args.stamps:
        print(json.dumps(stamps_leg(args, w)), flush=True)
        return
    if w.n_app:
        print(json.dumps(streaming_leg(args, w)), flush=True)
        return
    if w.name.startswith("pareto"):
        print(json.dumps(pareto_leg(args, w)), flush=True)
        return
    if w.name.startswith("prog"):
        print(json.dumps(prog_leg(args, w)), flush=True)
        return
    S = args.splits or w.n_splits or default_splits(w)
    T = w.tokens
    data = kvq_synth.generate(w)
    layout = kvq.make_layout(w.batch, w.n_q_heads, w.n_kv_heads, n_pairs_hi=w.n_pairs_hi,
                             bits_hi=w.bits_hi, residual=w.residual, max_tokens=T,
                             io_dtype=w.io_dtype, prog_w8=w.prog_w8, prog_w4=w.prog_w4)
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

    sink = torch.zeros(16, dtype=torch.uint8, device="cuda")

    def ceiling_us():
        """kvq_read_ceiling over the same replicas, steps and splits."""
        for i in range(args.warmup):
            kvq.kvq_read_ceiling(layout, replicas[i % n_rep].struct, S, sink, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            kvq.kvq_read_ceiling(layout, replicas[i % n_rep].struct, S, sink, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.steps

    if args.ceiling:
        cus = ceiling_us()
        cg = algorithmic_bytes(w, T) / (cus * 1e-6) / 1e9
        print(json.dumps({"ceiling": w.name, "us_per_step": round(cus, 3), "GBs": round(cg, 1),
                          "frac": round(cg / PEAK_GBS, 4), "n_splits": S, "steps": args.steps,
                          "cache_replicas": n_rep}), flush=True)
        return

    def step(i):
        if args.prune < 8:
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
                   **({"kept_key_runs": args.prune} if args.prune < 8 else {})},
        "algorithmic_bytes_per_step": alg,
        "layout_bytes_per_step": layout_bytes(base, w, T) if not w.prog_w4 else None,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_GBS, 4),
                     "traffic": (measured_traffic(w.name)
                                 if args.prune == 8 and not w.prog_w4 else None)},
    }
    if w.prog_w4:
        res["config"].update(prog_w8=w.prog_w8, prog_w4=w.prog_w4)
        res["cache_bytes"] = base.nbytes()
    if args.prune == 8 and not w.prog_w4:
        cus = ceiling_us()
        cg = alg / (cus * 1e-6) / 1e9
        res["ceiling"] = {"us_per_step": round(cus, 3), "GBs": round(cg, 1),
                          "frac": round(cg / PEAK_GBS, 4),
                          "decode_over_ceiling": round(ev_ms * 1e3 / cus, 3),
                          "note": "kvq_read_ceiling: the decode kernel's grid, XCD mapping and "
                                  "group copies over the same cache replicas, reads only"}
    if args.prune < 8:
        res["note"] = ("query-channel pruning: %d of 8 16-channel key runs kept per KV head; "
                       "bytes are those of the kept runs" % args.prune)
    if not args.no_cpu_baseline and args.prune == 8:
        res["cpu_baseline"] = cpu_baseline(w, data)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
