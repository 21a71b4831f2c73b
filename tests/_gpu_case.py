"""Shared set-up of GPU parity cases: one seeded workload run through the HIP
library (via the C-ABI binding) and through the CPU oracle on the same data."""
from __future__ import annotations

import math

import numpy as np
import torch

import kvq_synth
import oracle
from decode_attention_select_amd import kvq

SM_SCALE = float(np.float32(1.0 / math.sqrt(128.0)))


def dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bit array -> contiguous int16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def host(t: torch.Tensor, dtype) -> np.ndarray:
    return t.cpu().numpy().view(dtype)


class Case:
    """GPU cache after prefill of `T` tokens, and the oracle's view of it."""

    def __init__(self, w: kvq_synth.Workload, T: int | None = None,
                 max_tokens: int | None = None, data: dict | None = None):
        self.w = w
        self.T = w.tokens if T is None else T
        self.d = kvq_synth.generate(w) if data is None else data
        self.max_tokens = max_tokens or max(w.max_tokens, self.T)
        self.layout = kvq.make_layout(w.batch, w.n_q_heads, w.n_kv_heads,
                                      n_pairs_hi=w.n_pairs_hi, bits_hi=w.bits_hi,
                                      n_pairs_lo1=w.n_pairs_lo1,
                                      residual=w.residual, max_tokens=self.max_tokens,
                                      io_dtype=w.io_dtype, n_vblk_hi=w.n_vblk_hi,
                                      bits_vhi=w.bits_vhi, prog_w8=w.prog_w8,
                                      prog_w4=w.prog_w4)
        self.cache = kvq.Cache(self.layout)
        self.NG = max(self.max_tokens - w.residual, 0) // 32
        # selection always looks at the workload's prefill (once, at prefill)
        Tsel = w.tokens
        self.k_sel = dev(self.d["k"][:, :, :Tsel])
        self.q_sel = dev(self.d["q_sel"])
        kvq.kvq_select_pairs(self.layout, self.q_sel, w.n_qry, self.k_sel, Tsel, self.cache.struct)
        k = dev(self.d["k"][:, :, :self.T])
        v = dev(self.d["v"][:, :, :self.T])
        kvq.kvq_quant_keys(self.layout, k, self.T, self.cache.struct)
        kvq.kvq_quant_values(self.layout, v, self.T, self.cache.struct)
        torch.cuda.synchronize()

    # ----------------------------------------------------------- oracle side
    def oracle_select(self):
        return oracle.select(self.d["q_sel"], self.d["k"], self.w.tokens,
                             self.w.n_kv_heads, self.w.io_dtype)

    def oracle_quant(self, T=None, pairs=None):
        if pairs is None:
            pairs = self.oracle_select()[1]
        return oracle.quantize(self.d["k"], self.d["v"], self.T if T is None else T, pairs,
                               residual=self.w.residual, n_pairs_hi=self.w.n_pairs_hi,
                               bits_hi=self.w.bits_hi, io_dtype=self.w.io_dtype,
                               ng=max(self.NG, 1), n_pairs_lo1=self.w.n_pairs_lo1,
                               n_vblk_hi=self.w.n_vblk_hi, bits_vhi=self.w.bits_vhi,
                               prog_w8=self.w.prog_w8, prog_w4=self.w.prog_w4)

    # -------------------------------------------------------------- GPU side
    def gpu_bytes(self) -> dict:
        B, H, NG = self.w.batch, self.w.n_kv_heads, self.NG
        c = self.cache
        RS = self.w.residual + 32
        khi = oracle.k_hi_words(self.w.n_pairs_hi, self.w.bits_hi) if NG else 0
        out = {
            "k_lo": host(c["k_lo"], np.uint32).reshape(
                B, H, NG, 192 if oracle.dense1(self.w.n_pairs_hi, self.w.n_pairs_lo1) else 256),
            "k_hi": (host(c["k_hi"], np.uint8)[:B * H * NG * khi].reshape(B, H, NG, khi)
                     if khi else np.zeros((B, H, NG, 0), np.uint8)),
            "k_meta": host(c["k_meta"], np.uint16).reshape(B, H, NG, 256),
            "v_codes": host(c["v_codes"], np.uint32).reshape(B, H, NG, 256),
            "v_meta": host(c["v_meta"], np.uint16).reshape(B, H, NG, 256),
            "ring_k": host(c["ring_k"], np.uint16).reshape(B, H, RS, 128),
            "ring_v": host(c["ring_v"], np.uint16).reshape(B, H, RS // 32, 128, 32),
            "pairs": host(c["pairs"], np.int32).reshape(B, H, 64),
            "len": host(c["len"], np.int32).reshape(B, H),
            "sums": host(c["sums"], np.uint64).reshape(B, H, 2, 64),
        }
        vw = 8 + 64 * self.w.n_vblk_hi if self.w.n_vblk_hi else 0
        out["v_hi"] = (host(c["v_hi"], np.uint32)[:B * H * NG * vw].reshape(B, H, NG, vw)
                       if vw and NG else np.zeros((B, H, NG, 0), np.uint32))
        npl = self.w.prog_w4 + 2 * self.w.prog_w8 if NG else 0
        for nm in ("k_pl", "v_pl"):
            out[nm] = (host(c[nm], np.uint32).reshape(B, H, npl, 256) if npl
                       else np.zeros((B, H, 0, 256), np.uint32))
        return out

    def pruned_unsupported(self, n_splits: int = 3, n_keep: int = 5) -> bool:
        """True (after checking that the call returns KVQ_ENOTSUP) when the
        layout offers no pruned decode: the dense 1-bit layout and
        progressive layouts."""
        w = self.w
        if not (oracle.dense1(w.n_pairs_hi, w.n_pairs_lo1) or w.prog_w4):
            return False
        try:
            self.decode_pruned(self.d["q_dec"][:, :, 0], n_splits, n_keep)
        except kvq.KvqError as e:
            assert e.status == -2, e
            return True
        raise AssertionError("pruned decode accepted on a layout that does not offer it")

    def decode_pruned(self, q_bits: np.ndarray, n_splits: int, n_keep: int):
        """kvq_decode_attn_pruned -> GPU output widened to fp64."""
        ws = torch.zeros(kvq.kvq_workspace_bytes(self.layout, n_splits), dtype=torch.uint8,
                         device="cuda")
        out = torch.empty((self.w.batch, self.w.n_q_heads, 128), dtype=torch.int16, device="cuda")
        kvq.kvq_decode_attn_pruned(self.layout, dev(q_bits), self.cache.struct, SM_SCALE,
                                   n_splits, n_keep, ws, out)
        torch.cuda.synchronize()
        return kvq_synth.bits_to_f64(host(out, np.uint16), self.w.io_dtype)

    def decode(self, q_bits: np.ndarray, n_splits: int, partials: bool = False):
        """q_bits [B][Hq][128] -> GPU output widened to fp64; with `partials`
        also the per-split records read back from the workspace: fp32 (m, l)
        [B][Hq][S][2] and the fp32 normalized o/l [B][Hq][S][128] (fp64).
        The workspace holds the split counters first ([B*Hkv] lines of 256
        bytes), then the (m, l) records [B*Hkv][S][G], 256-byte aligned,
        then [B*Hkv][S][G][128] fp32."""
        ws = torch.zeros(kvq.kvq_workspace_bytes(self.layout, n_splits), dtype=torch.uint8,
                         device="cuda")
        out = torch.empty((self.w.batch, self.w.n_q_heads, 128), dtype=torch.int16, device="cuda")
        kvq.kvq_decode_attn(self.layout, dev(q_bits), self.cache.struct, SM_SCALE, n_splits,
                            ws, out)
        torch.cuda.synchronize()
        o = kvq_synth.bits_to_f64(host(out, np.uint16), self.w.io_dtype)
        if not partials:
            return o
        return o, read_partials(host(ws, np.uint8), self.w.batch, self.w.n_kv_heads,
                                self.w.group_size, n_splits)


def read_partials(raw: np.ndarray, B: int, Hkv: int, G: int, S: int):
    """Split records of a decode workspace (layout in include/kvq.h) as fp64:
    (m, l) [B][Hq][S][2] and o/l [B][Hq][S][128]."""
    nrec = B * Hkv * S * G
    t_bytes = B * Hkv * 256
    ml_bytes = (nrec * 8 + 255) // 256 * 256
    ml = raw[t_bytes:t_bytes + nrec * 8].view(np.float32).reshape(B, Hkv, S, G, 2)
    o32 = raw[t_bytes + ml_bytes:t_bytes + ml_bytes + nrec * 512].view(np.float32)
    o32 = o32.reshape(B, Hkv, S, G, 128)
    ml = ml.transpose(0, 1, 3, 2, 4).reshape(B, Hkv * G, S, 2).astype(np.float64)
    o32 = o32.transpose(0, 1, 3, 2, 4).reshape(B, Hkv * G, S, 128).astype(np.float64)
    return ml, o32


def lse_merge(part) -> np.ndarray:
    """The log-sum-exp combine of a call's split records, in fp64 on the
    host: o = sum_s 2^(m_s - M) l_s o_s / sum_s 2^(m_s - M) l_s."""
    ml, o = part
    m, l = ml[..., 0], ml[..., 1]
    M = np.max(np.where(l > 0, m, -np.inf), axis=-1, keepdims=True)
    w = np.where(l > 0, np.exp2(np.where(l > 0, m, 0.0) - M) * l, 0.0)
    return np.einsum("bhs,bhsc->bhc", w, o) / w.sum(axis=-1)[..., None]


def half_ulp(x: np.ndarray, io_dtype: str) -> np.ndarray:
    """Half a unit in the last place of the 16-bit output dtype at |x|: the
    rounding error of storing an exact result in that dtype."""
    mant = 7 if io_dtype == "bf16" else 10
    emin = -126 if io_dtype == "bf16" else -14
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** emin)))
    return 2.0 ** (e - mant - 1)


def check_output(got, ref, io_dtype, atol):
    """|got - ref| <= atol elementwise: the budget holds the output's own
    rounding to the 16-bit dtype.  Only where that rounding alone can take
    more than half the budget (half an output ulp above 1e-3: |o| >= 0.5 in
    bf16) is the half ulp added on top; the number of such elements and the
    largest |o| are printed.  Returns the largest error."""
    err = np.abs(got - ref)
    hu = half_ulp(ref, io_dtype)
    wide = hu > 1e-3
    bound = atol + np.where(wide, hu, 0.0)
    if np.any(wide):
        print("check_output: %d of %d elements with |o| where half an %s ulp exceeds 1e-3 "
              "(max |o| %.3g)" % (int(wide.sum()), wide.size, io_dtype, float(np.abs(ref).max())))
    assert np.all(err <= bound), "max err %.3g (bound there %.3g)" % (
        err.max(), bound.flat[np.argmax(err - bound)])
    return float(err.max())


def single_split(part) -> np.ndarray:
    """Attention result of a one-split call before the 16-bit output
    rounding: the split record's o/l, computed and stored in fp32."""
    ml, o32 = part
    assert o32.shape[2] == 1
    return o32[:, :, 0]


def check_single_split(part, ref, atol):
    """The fp32 result of a one-split call, read from its record: within
    `atol` of the oracle (no rounding allowance)."""
    got = single_split(part)
    err = np.abs(got - ref)
    assert np.all(err <= atol), "max err %.3g" % err.max()
    return float(err.max())


def compare_cache(case: Case, qz, ng: int):
    """Asserts the GPU cache bytes equal the oracle's packing for groups
    [0, ng) and the live ring slots."""
    g = case.gpu_bytes()
    o = oracle.pack(qz)
    for name in ("k_lo", "k_meta", "v_codes", "v_meta"):
        a, b = g[name][:, :, :ng], o[name][:, :, :ng]
        assert np.array_equal(a, b), "%s differs at %s" % (name, np.argwhere(a != b)[:5])
    if o["k_hi"].shape[-1] and ng:
        a, b = g["k_hi"][:, :, :ng], o["k_hi"][:, :, :ng]
        assert np.array_equal(a, b), "k_hi differs at %s" % np.argwhere(a != b)[:5]
    if case.w.n_vblk_hi and ng:
        a, b = g["v_hi"][:, :, :ng], o["v_hi"][:, :, :ng]
        assert np.array_equal(a, b), "v_hi differs at %s" % np.argwhere(a != b)[:5]
    if case.w.prog_w4 and ng:
        # the digit planes of the live wide groups (other slots hold stale bytes)
        assert ng == qz.nq // 32
        for grp, sl in oracle.live_plane_slots(qz.T, qz.R, case.w.prog_w8, case.w.prog_w4):
            for nm in ("k_pl", "v_pl"):
                a, b = g[nm][:, :, sl], o[nm][:, :, sl]
                assert np.array_equal(a, b), "%s slot %d (group %d) differs at %s" % (
                    nm, sl, grp, np.argwhere(a != b)[:5])
    slots = oracle.live_ring_slots(qz.T, qz.R)
    assert np.array_equal(g["ring_k"][:, :, slots], o["ring_k"][:, :, slots])
    rv_g = g["ring_v"].reshape(*g["ring_v"].shape[:2], -1, 128, 32)
    for s in slots:
        assert np.array_equal(rv_g[:, :, s // 32, :, s % 32], o["ring_v"][:, :, s // 32, :, s % 32])
    assert np.all(g["len"] == qz.T)
