"""The C ABI without a GPU: the built libkvq.so loads, exports every entry
point include/kvq.h declares, reports buffer sizes by their closed forms and
rejects bad arguments on the host before anything is enqueued.

Validation cases pass stand-in device addresses that are never dereferenced:
each call carries exactly one error, which the host checks must catch.  They
are skipped where a GPU is present, so that a validation bug could never turn
into a launch over those addresses."""
import ctypes
import os
import re

import pytest
import torch

from decode_attention_select_amd import kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, EINVAL, ENOTSUP, EALIGN, ECAPACITY = 0, -1, -2, -3, -4

no_gpu = pytest.mark.skipif(torch.cuda.is_available(),
                            reason="host-validation cases run only where no GPU can be reached")


def declared():
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    return re.findall(r"^(?:kvq_status|const char \*)\s*\**(kvq_\w+)\s*\(", text, re.M)


def test_library_exports_every_declared_entry_point():
    names = declared()
    assert set(names) >= {"kvq_select_pairs", "kvq_quant_keys", "kvq_quant_values",
                          "kvq_append", "kvq_decode_attn", "kvq_cache_sizes",
                          "kvq_workspace_bytes", "kvq_check", "kvq_status_str", "kvq_shrink",
                          "kvq_select_pairs_qa", "kvq_decode_attn_pruned",
                          "kvq_append_decode_attn", "kvq_read_ceiling"}
    lib = kvq.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in (OK, EINVAL, ENOTSUP, EALIGN, ECAPACITY, -5):
        assert kvq.kvq_status_str(s) not in ("", "unknown status")
    assert kvq.kvq_status_str(7) == "unknown status"


def L32k(**kw):
    args = dict(n_pairs_hi=6, bits_hi=4, residual=128, max_tokens=32768, io_dtype="bf16")
    args.update(kw)
    return kvq.make_layout(1, 32, 8, **args)


def test_cache_sizes_closed_form():
    # 32K layer: 1020 groups per KV head of 1024 + 128 + 512 + 1024 + 512 B
    s = kvq.kvq_cache_sizes(L32k())
    ng, bh = (32768 - 128) // 32, 8
    assert s == [bh * ng * 1024, bh * ng * 128, bh * ng * 512, bh * ng * 1024, bh * ng * 512,
                 bh * 160 * 256, bh * 160 * 256, bh * 64 * 4, bh * 4, bh * 2 * 64 * 8, 4, 0, 0, 0]
    # two value precisions: 32 order bytes + 256 bytes per 8 high-precision tokens
    for n in (1, 2, 4):
        assert kvq.kvq_cache_sizes(L32k(n_vblk_hi=n, bits_vhi=3))[11] == bh * ng * (32 + 256 * n)
    # raw 16-bit salient channels: 32 tokens x 12 channels x 2 B per group
    s16 = kvq.kvq_cache_sizes(L32k(bits_hi=16))
    assert s16[1] == bh * ng * 32 * 12 * 2 + 32  # + tail slack of the 16-byte row reads
    # no salient pairs: no high-digit section; capacity inside the window: no groups
    assert kvq.kvq_cache_sizes(L32k(n_pairs_hi=0))[1] == 0
    assert kvq.kvq_cache_sizes(L32k(max_tokens=100))[0] == 0


def status_of(name, *args):
    return getattr(kvq.lib(), name)(*args)


@pytest.mark.parametrize("bad,want", [
    (dict(head_dim=64), EINVAL), (dict(group=16), EINVAL), (dict(n_pairs_hi=9), EINVAL),
    (dict(bits_hi=8), ENOTSUP), (dict(n_pairs_lo1=59), EINVAL), (dict(n_pairs_lo1=-1), EINVAL),
    (dict(bits_lo=3), ENOTSUP),
    (dict(residual=48), EINVAL), (dict(residual=0), EINVAL), (dict(max_tokens=0), EINVAL),
    (dict(io_dtype=5), EINVAL), (dict(n_q_heads=30), EINVAL), (dict(n_q_heads=8 * 17), ENOTSUP),
    (dict(batch=0), EINVAL), (dict(n_vblk_hi=5), EINVAL), (dict(n_vblk_hi=-1), EINVAL),
    (dict(n_vblk_hi=2, bits_vhi=2), ENOTSUP), (dict(n_vblk_hi=1, bits_vhi=8), ENOTSUP),
    (dict(prog_w8=-1), EINVAL), (dict(prog_w4=2, prog_w8=3), EINVAL), (dict(prog_w4=257), EINVAL),
    (dict(prog_w4=4, n_pairs_lo1=2), ENOTSUP), (dict(prog_w4=4, n_vblk_hi=1), ENOTSUP),
])
def test_layout_rejected(bad, want):
    L = L32k()
    for k, v in bad.items():
        setattr(L, k, v)
    sizes = (ctypes.c_size_t * kvq.NBUF)()
    assert status_of("kvq_cache_sizes", ctypes.byref(L), sizes) == want
    n = ctypes.c_size_t(0)
    assert status_of("kvq_workspace_bytes", ctypes.byref(L), 4, ctypes.byref(n)) == want


def test_workspace_bytes():
    L = L32k()
    assert kvq.kvq_workspace_bytes(L, 1) < kvq.kvq_workspace_bytes(L, 32)
    rec = 32 * 32  # query heads x splits
    # counters (one 256-byte line per KV head), then twice (a device-coherent
    # copy and an L2-local copy) fp32 (m, l) and fp32 o/l [128]
    want = 8 * 256 + 2 * ((rec * 8 + 255) // 256 * 256 + rec * 512)
    assert kvq.kvq_workspace_bytes(L, 32) == want
    n = ctypes.c_size_t(0)
    for S in (0, 1025, -1):
        assert status_of("kvq_workspace_bytes", ctypes.byref(L), S, ctypes.byref(n)) == EINVAL


FAKE = 1 << 20  # a 16-byte-aligned stand-in device address (never dereferenced)


def fake_cache():
    return kvq.kvq_cache(*[FAKE] * kvq.NBUF)


@no_gpu
def test_decode_validation():
    L = L32k()
    c = fake_cache()
    ws = kvq.kvq_workspace_bytes(L, 8)
    P = ctypes.c_void_p

    def call(q=FAKE, scale=0.088, S=8, wsp=FAKE, wsb=ws, out=FAKE, cache=c):
        return status_of("kvq_decode_attn", ctypes.byref(L), P(q), ctypes.byref(cache),
                         ctypes.c_float(scale), S, P(wsp), ctypes.c_size_t(wsb), P(out), P(0))

    assert call(q=0) == EINVAL
    assert call(out=FAKE + 8) == EALIGN
    assert call(wsp=0) == EINVAL
    assert call(wsb=ws - 1) == ECAPACITY
    assert call(scale=0.0) == EINVAL
    assert call(scale=float("nan")) == EINVAL
    assert call(S=0) == EINVAL
    bad = fake_cache()
    bad.v_meta = FAKE + 4
    assert call(cache=bad) == EALIGN
    bad = fake_cache()
    bad.len = 0
    assert call(cache=bad) == EINVAL
    # the pruned variant: n_keep outside 1..8
    for n_keep, want in ((0, EINVAL), (9, EINVAL), (-1, EINVAL)):
        assert status_of("kvq_decode_attn_pruned", ctypes.byref(L), P(FAKE), ctypes.byref(c),
                         ctypes.c_float(0.088), 8, n_keep, P(FAKE), ctypes.c_size_t(ws), P(FAKE),
                         P(0)) == want
    assert status_of("kvq_decode_attn_pruned", ctypes.byref(L), P(FAKE), ctypes.byref(c),
                     ctypes.c_float(0.088), 8, 2, P(FAKE), ctypes.c_size_t(ws - 1), P(FAKE),
                     P(0)) == ECAPACITY
    # the append-and-decode call: its token pointers, then the decode checks

    def fused(k=FAKE, v=FAKE, sm=0.088, wsb=ws):
        return status_of("kvq_append_decode_attn", ctypes.byref(L), P(k), P(v), P(FAKE),
                         ctypes.byref(c), ctypes.c_float(sm), 8, P(FAKE), ctypes.c_size_t(wsb),
                         P(FAKE), P(0))
    assert fused(k=0) == EINVAL and fused(v=0) == EINVAL
    assert fused(v=FAKE + 4) == EALIGN
    assert fused(sm=0.0) == EINVAL
    assert fused(wsb=ws - 1) == ECAPACITY
    # the read ceiling: its sink and split count
    ceil = lambda sink=FAKE, S=8: status_of("kvq_read_ceiling", ctypes.byref(L), ctypes.byref(c),
                                            S, P(sink), P(0))
    assert ceil(sink=0) == EINVAL and ceil(sink=FAKE + 4) == EALIGN
    assert ceil(S=0) == EINVAL and ceil(S=1025) == EINVAL
    # the issue probe: its kind, block count and output
    probe = lambda kind=0, nb=4, o=FAKE: status_of("kvq_issue_probe", kind, nb, P(o), P(0))
    assert probe(kind=-1) == EINVAL and probe(kind=7) == EINVAL and probe(nb=0) == EINVAL
    assert probe(o=0) == EINVAL and probe(o=FAKE + 4) == EALIGN


@no_gpu
def test_prefill_and_append_validation():
    L = L32k()
    c = fake_cache()
    P = ctypes.c_void_p
    sel = lambda n_qry=64, T=32768, q=FAKE, k=FAKE: status_of(
        "kvq_select_pairs", ctypes.byref(L), P(q), n_qry, P(k), T, ctypes.byref(c), P(0))
    assert sel(n_qry=0) == EINVAL
    assert sel(n_qry=1025) == EINVAL
    assert sel(T=0) == EINVAL
    assert sel(T=32769) == ECAPACITY
    assert sel(k=FAKE + 2) == EALIGN
    for name in ("kvq_quant_keys", "kvq_quant_values"):
        assert status_of(name, ctypes.byref(L), P(FAKE), 32769, ctypes.byref(c), P(0)) == ECAPACITY
        assert status_of(name, ctypes.byref(L), P(FAKE), 0, ctypes.byref(c), P(0)) == EINVAL
        assert status_of(name, ctypes.byref(L), P(0), 100, ctypes.byref(c), P(0)) == EINVAL
    assert status_of("kvq_append", ctypes.byref(L), P(FAKE), P(0), ctypes.byref(c), P(0)) == EINVAL
    assert status_of("kvq_append", ctypes.byref(L), P(FAKE + 1), P(FAKE), ctypes.byref(c),
                     P(0)) == EALIGN
    assert status_of("kvq_check", None, None, P(0)) == EINVAL
    assert status_of("kvq_shrink", ctypes.byref(L), ctypes.byref(c), -1, 4, P(0)) == EINVAL
    assert status_of("kvq_shrink", ctypes.byref(L), ctypes.byref(c), 5, 4, P(0)) == EINVAL
    L16 = L32k(bits_hi=16)
    assert status_of("kvq_shrink", ctypes.byref(L16), ctypes.byref(c), 0, 4, P(0)) == ENOTSUP


def test_prog_plane_sizes():
    # progressive precision: (w4 + 2 w8) KiB of key planes and as much of
    # value planes per (sequence, KV head), whatever the length
    bh = 1 * 8
    for w8, w4 in ((0, 1), (4, 16), (256, 256)):
        s = kvq.kvq_cache_sizes(L32k(prog_w8=w8, prog_w4=w4))
        assert s[12] == s[13] == bh * (w4 + 2 * w8) * 1024
        assert s[:12] == kvq.kvq_cache_sizes(L32k())[:12]
    assert kvq.kvq_cache_sizes(L32k())[12:] == [0, 0]
    assert kvq.kvq_cache_sizes(L32k(prog_w4=4, max_tokens=100))[12] == 0  # no groups


@no_gpu
def test_prog_calls_it_does_not_offer():
    # pruned decode, the explicit salient shrink and the read ceiling return
    # ENOTSUP on a progressive layout, before any launch
    L = L32k(prog_w8=2, prog_w4=8)
    c = fake_cache()
    ws = kvq.kvq_workspace_bytes(L, 8)
    P = ctypes.c_void_p
    assert status_of("kvq_decode_attn_pruned", ctypes.byref(L), P(FAKE), ctypes.byref(c),
                     ctypes.c_float(0.088), 8, 5, P(FAKE), ctypes.c_size_t(ws), P(FAKE),
                     P(0)) == ENOTSUP
    assert status_of("kvq_shrink", ctypes.byref(L), ctypes.byref(c), 0, 4, P(0)) == ENOTSUP
    assert status_of("kvq_read_ceiling", ctypes.byref(L), ctypes.byref(c), 8, P(FAKE),
                     P(0)) == ENOTSUP
    # a plane buffer that is missing is an argument error, for the plain and
    # the one-launch decode (which is offered on progressive layouts)
    c0 = fake_cache()
    c0.k_pl = None
    assert status_of("kvq_decode_attn", ctypes.byref(L), P(FAKE), ctypes.byref(c0),
                     ctypes.c_float(0.088), 8, P(FAKE), ctypes.c_size_t(ws), P(FAKE),
                     P(0)) == EINVAL
    c1 = fake_cache()
    c1.v_pl = None
    assert status_of("kvq_append_decode_attn", ctypes.byref(L), P(FAKE), P(FAKE), P(FAKE),
                     ctypes.byref(c1), ctypes.c_float(0.088), 8, P(FAKE), ctypes.c_size_t(ws),
                     P(FAKE), P(0)) == EINVAL


def test_bench_refuses_more_than_one_gpu():
    # the benchmark measures one GPU; asked for more it says so and exits 2
    # before touching a device
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_record_is_keyed_to_the_kernel_code():
    # roofline.traffic comes from a committed counter record only while the
    # decode kernel's machine code in the built library is the one measured
    import bench
    h = bench.kernel_code_hash()
    assert h is not None and len(h) == 16 and int(h, 16) >= 0
    assert bench.kernel_code_hash() == h
    assert bench.kernel_code_hash("_ZN3kvq_no_such_kernel") is None
    assert bench.measured_traffic("no-such-workload") is None
