"""Guard bands around every buffer the library is handed.

Each cache section, the workspace, the output, the sink and every input sits
between two 4 KiB bands of a fixed byte.  Prefill (pair selection, key and
value quantization), appends across group boundaries, the precision shrink,
every decode entry point and the read ceiling run over the guarded buffers;
afterwards every band must hold its byte still.  The parity tests compare
only the live records (groups [0, n_q/32) and the live ring slots), so a
stray write past a buffer's end or before its start would show up only
here."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kvq_synth
import oracle
from decode_attention_select_amd import kvq
from _gpu_case import SM_SCALE

pytestmark = pytest.mark.gpu

PAD = 4096
BAND = 0xA5


class Guarded:
    """`nbytes` of device memory between two bands; the inner bytes start
    zero (as a cache or workspace must) or as given."""

    def __init__(self, nbytes: int, init: np.ndarray | None = None):
        self.n = max(int(nbytes), 16)
        self.t = torch.full((PAD + self.n + PAD,), BAND, dtype=torch.uint8, device="cuda")
        self.inner = self.t[PAD:PAD + self.n]
        self.inner.zero_()
        if init is not None:
            b = torch.from_numpy(np.ascontiguousarray(init).view(np.uint8).reshape(-1)).cuda()
            self.inner[:b.numel()].copy_(b)

    def ptr(self) -> int:
        return self.inner.data_ptr()

    def bands_intact(self) -> bool:
        t = self.t.cpu().numpy()
        return bool((t[:PAD] == BAND).all() and (t[PAD + self.n:] == BAND).all())


LAYOUTS = [
    # 4-bit salient digits, two value precisions, fp16 io
    dict(name="tiny", n_pairs_hi=8, bits_hi=4, n_vblk_hi=2, bits_vhi=4, io="fp16", Hq=4, Hkv=2),
    # raw 16-bit salient channels, bf16 io
    dict(name="tiny", n_pairs_hi=3, bits_hi=16, n_vblk_hi=0, bits_vhi=4, io="bf16", Hq=8, Hkv=1),
    # 1-bit lowest pairs, no salient pairs
    dict(name="tiny", n_pairs_hi=0, bits_hi=4, n_pairs_lo1=32, n_vblk_hi=0, bits_vhi=4,
         io="bf16", Hq=2, Hkv=2),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("cfg", LAYOUTS, ids=["h4-vhi", "h16", "lo1"])
def test_guard_bands_survive_every_call(cfg):
    T0, n_app, B = 613, 70, 2
    w = kvq_synth.workload(cfg["name"]).replace(
        batch=B, n_q_heads=cfg["Hq"], n_kv_heads=cfg["Hkv"], tokens=T0, n_app=n_app,
        n_pairs_hi=cfg["n_pairs_hi"], bits_hi=cfg["bits_hi"],
        n_pairs_lo1=cfg.get("n_pairs_lo1", 0), io_dtype=cfg["io"], residual=64,
        n_vblk_hi=cfg["n_vblk_hi"], bits_vhi=cfg["bits_vhi"])
    print("case", cfg, flush=True)
    d = kvq_synth.generate(w)
    layout = kvq.make_layout(B, w.n_q_heads, w.n_kv_heads, n_pairs_hi=w.n_pairs_hi,
                             bits_hi=w.bits_hi, n_pairs_lo1=w.n_pairs_lo1, residual=w.residual,
                             max_tokens=T0 + n_app + 8, io_dtype=w.io_dtype,
                             n_vblk_hi=w.n_vblk_hi, bits_vhi=w.bits_vhi)
    sizes = kvq.kvq_cache_sizes(layout)
    cache_bufs = [Guarded(n) for n in sizes]
    cache = kvq.kvq_cache(*[g.ptr() for g in cache_bufs])
    q_sel = Guarded(d["q_sel"].nbytes, d["q_sel"])
    k0 = Guarded(d["k"][:, :, :T0].nbytes, d["k"][:, :, :T0])
    v0 = Guarded(d["v"][:, :, :T0].nbytes, d["v"][:, :, :T0])
    q = Guarded(d["q_dec"][:, :, 0].nbytes, d["q_dec"][:, :, 0])
    out = Guarded(B * w.n_q_heads * 128 * 2)
    sink = Guarded(16)
    S_list = [1, 3, 32]
    ws = Guarded(max(kvq.kvq_workspace_bytes(layout, S) for S in S_list))
    inputs = [q_sel, k0, v0, q]

    kvq.kvq_select_pairs(layout, q_sel.ptr(), w.n_qry, k0.ptr(), T0, cache)
    kvq.kvq_quant_keys(layout, k0.ptr(), T0, cache)
    kvq.kvq_quant_values(layout, v0.ptr(), T0, cache)
    for S in S_list:
        kvq.kvq_decode_attn(layout, q.ptr(), cache, SM_SCALE, S, ws.ptr(), out.ptr(),
                            ws_bytes=ws.n)
        kvq.kvq_read_ceiling(layout, cache, S, sink.ptr())
    if not oracle.dense1(w.n_pairs_hi, w.n_pairs_lo1):  # the dense 1-bit layout: ENOTSUP
        kvq.kvq_decode_attn_pruned(layout, q.ptr(), cache, SM_SCALE, 3, 5, ws.ptr(), out.ptr(),
                                   ws_bytes=ws.n)
    # appends across group boundaries, every other one fused with a decode
    for i in range(n_app):
        kn = Guarded(d["k"][:, :, T0 + i].nbytes, d["k"][:, :, T0 + i])
        vn = Guarded(d["v"][:, :, T0 + i].nbytes, d["v"][:, :, T0 + i])
        if i % 2:
            kvq.kvq_append_decode_attn(layout, kn.ptr(), vn.ptr(), q.ptr(), cache, SM_SCALE, 3,
                                       ws.ptr(), out.ptr(), ws_bytes=ws.n)
        else:
            kvq.kvq_append(layout, kn.ptr(), vn.ptr(), cache)
        inputs += [kn, vn]
    if w.bits_hi == 4 and w.n_pairs_hi > 0:
        ng = max(layout.max_tokens - w.residual, 0) // 32
        kvq.kvq_shrink(layout, cache, 0, ng)
    for S in S_list:
        kvq.kvq_decode_attn(layout, q.ptr(), cache, SM_SCALE, S, ws.ptr(), out.ptr(),
                            ws_bytes=ws.n)
    kvq.kvq_decode_attn_noalloc(layout, q.ptr(), cache, SM_SCALE, 3, out.ptr())
    torch.cuda.synchronize()
    assert kvq.kvq_check(cache) == 0
    bad = [kvq.BUF_NAMES[i] for i, g in enumerate(cache_bufs) if not g.bands_intact()]
    bad += [nm for nm, g in (("workspace", ws), ("out", out), ("sink", sink))
            if not g.bands_intact()]
    bad += ["input %d" % i for i, g in enumerate(inputs) if not g.bands_intact()]
    assert not bad, "guard bands overwritten: %s" % bad
    # the output is finite (the calls did run)
    o = out.inner.cpu().numpy().view(np.uint16)[:B * w.n_q_heads * 128]
    of = kvq_synth.bits_to_f64(o, w.io_dtype)
    assert np.isfinite(of).all()
