"""CPU oracle of the quantized-KV decode path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the GPU library
(``decode_attention_select_amd``) and neither imports the other; both read
their inputs from ``kvq_synth``.

The arithmetic lives in ``kvq_oracle.c`` (plain loops, IEEE fp32/fp64, built
with ``-O2 -ffp-contract=off``); this module builds it with gcc and wraps it
with numpy.  ``oracle.brute`` holds independent brute-force checks used to pin
the oracle itself.

Pinned by (see tests/test_oracle_*.py): 16-bit conversions against numpy and
torch casts over every bit pattern; the quantizer against nearest-level
search, its error bound, min/max codes, idempotence and constant groups; the
selection against an exhaustive mean over all query/key combinations, planted
outliers, RoPE invariance and token-order invariance; packing against an
independent bit-level unpacker; attention against textbook softmax attention
(all-16-bit cache), T = 1, q = 0 and a brute-force pass over the dequantized
cache.

Parity unpinned: the query-aware pair score (select_qa), the kept key runs
of pruned decode (prune_chunks) and the token order of two value precisions
(order in quantize) follow rules the pages describe without a formula; their
tests pin each to its own rule (float sums, invariances, planted cases), not
to values the pages fix.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

GS = 32
D = 128


_LIB_SAN = os.path.join(_HERE, "liboracle_san.so")
# set (to any value) in a process started with the sanitizer runtime
# preloaded: the oracle is then loaded from its address- and
# undefined-behaviour-checked build
SANITIZED_ENV = "KVQ_ORACLE_SANITIZED"


def build(force: bool = True, sanitized: bool = False) -> str:
    """Compile liboracle.so with gcc (IEEE arithmetic, no FMA contraction).
    sanitized: the same source into liboracle_san.so under AddressSanitizer
    and UndefinedBehaviorSanitizer (any finding aborts)."""
    lib = _LIB_SAN if sanitized else _LIB
    if force or not os.path.exists(lib):
        tmp = lib + ".tmp%d" % os.getpid()
        opt = (["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                "-fno-sanitize-recover=all"] if sanitized else ["-O2"])
        subprocess.check_call(["gcc"] + opt + ["-std=c11", "-fPIC", "-shared",
                               "-ffp-contract=off", "-fno-fast-math",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, lib)
    return lib


def _load():
    global _lib
    if _lib is None:
        if os.environ.get(SANITIZED_ENV):
            if not os.path.exists(_LIB_SAN):
                build(force=True, sanitized=True)
            _lib = ctypes.CDLL(_LIB_SAN)
        else:
            if not os.path.exists(_LIB):
                build(force=True)
            _lib = ctypes.CDLL(_LIB)
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _bf(io_dtype: str) -> int:
    return 1 if io_dtype == "bf16" else 0


def n_quant(T: int, R: int) -> int:
    """Quantized tokens held when T tokens are cached with residual R."""
    return int(_load().orc_n_quant(int(T), int(R)))


def half_to_f64(bits) -> np.ndarray:
    lib = _load()
    lib.orc_half_to_f64.restype = ctypes.c_double
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.orc_half_to_f64(ctypes.c_uint16(int(x))) for x in b])


def bf16_to_f64(bits) -> np.ndarray:
    lib = _load()
    lib.orc_bf16_to_f64.restype = ctypes.c_double
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.orc_bf16_to_f64(ctypes.c_uint16(int(x))) for x in b])


def f32_to_half(x) -> np.ndarray:
    lib = _load()
    lib.orc_f32_to_half.restype = ctypes.c_uint16
    lib.orc_f32_to_half.argtypes = [ctypes.c_float]
    a = np.asarray(x, dtype=np.float32).ravel()
    return np.array([lib.orc_f32_to_half(float(v)) for v in a], dtype=np.uint16)


def quant_group(x, bits: int):
    """Quantize one group of 32 values (fp32-exact) at `bits` bits.
    Returns (codes uint8[32], s_bits, z_bits)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.shape == (GS,)
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.uint16)
    c = np.zeros(GS, np.uint8)
    lib.orc_quant_group(_p(x), ctypes.c_int((1 << bits) - 1), _p(s), _p(z), _p(c))
    return c, int(s[0]), int(z[0])


def select(q_sel, k, T: int, n_kv_heads: int, io_dtype: str):
    """Pair ranking.  q_sel [B][Hq][n_qry][128], k [B][Hkv][Tstride][128]
    bits.  Returns (sums uint64 [B][Hkv][2][64], pairs int32 [B][Hkv][64])."""
    q_sel = np.ascontiguousarray(q_sel, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    B, Hq, n_qry, _ = q_sel.shape
    Hkv = n_kv_heads
    sums = np.zeros((B, Hkv, 2, 64), np.uint64)
    pairs = np.zeros((B, Hkv, 64), np.int32)
    rc = _load().orc_select(B, Hq, Hkv, _bf(io_dtype), _p(q_sel), n_qry, _p(k),
                            k.shape[2], int(T), _p(sums), _p(pairs))
    assert rc == 0
    return sums, pairs


class Quantized:
    """Logical (unpacked) quantized cache of the oracle."""

    def __init__(self, **kw):
        self.__dict__.update(kw)


def quantize(k, v, T: int, pairs, *, residual: int, n_pairs_hi: int,
             bits_hi: int, io_dtype: str, ng: int | None = None,
             n_pairs_lo1: int = 0, n_vblk_hi: int = 0, bits_vhi: int = 4,
             prog_w8: int = 0, prog_w4: int = 0) -> Quantized:
    """Quantize keys and values of the first T tokens (k, v
    [B][Hkv][Tstride][128] bits) with the given rank table.  With n_vblk_hi >
    0 each group's tokens are ordered by descending key magnitude (``order``
    [B][Hkv][NG][32]: slot -> position; identity otherwise) and the values of
    the first 8 n_vblk_hi tokens in that order get bits_vhi bits, the rest 2
    bits (the SemKV reading).  Codes, scales and zeros stay in position
    order.  prog_w4 > 0: progressive precision (the PM-KVQ reading of
    orc_prog_keys): every group quantized at 8 bits, then shrunk to 4 and 2
    bits by its age, the newest prog_w8 groups held at 8 bits and the newest
    prog_w4 at 4 bits or more (no 1-bit pairs, one value precision)."""
    lib = _load()
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    pairs = np.ascontiguousarray(pairs, dtype=np.int32)
    B, Hkv, Tstride, _ = k.shape
    nq = n_quant(T, residual)
    NG = ng if ng is not None else max(nq // GS, 1)
    kc = np.zeros((B, Hkv, NG, D, GS), np.uint8)
    ks = np.zeros((B, Hkv, NG, D), np.uint16)
    kz = np.zeros((B, Hkv, NG, D), np.uint16)
    vc = np.zeros((B, Hkv, NG, GS, D), np.uint8)
    vs = np.zeros((B, Hkv, NG, GS, 4), np.uint16)
    vz = np.zeros((B, Hkv, NG, GS, 4), np.uint16)
    prog = prog_w4 > 0
    assert not prog or (n_pairs_lo1 == 0 and n_vblk_hi == 0 and 0 <= prog_w8 <= prog_w4)
    if prog:
        rc = lib.orc_prog_keys(B, Hkv, _bf(io_dtype), _p(k), Tstride, int(T), int(residual),
                               int(n_pairs_hi), int(bits_hi), _p(pairs), NG, int(prog_w8),
                               int(prog_w4), _p(kc), _p(ks), _p(kz))
    else:
        rc = lib.orc_quant_keys(B, Hkv, _bf(io_dtype), _p(k), Tstride, int(T),
                                int(residual), int(n_pairs_hi), int(bits_hi),
                                int(n_pairs_lo1), _p(pairs), NG, _p(kc), _p(ks), _p(kz))
    assert rc == 0
    order = np.zeros((B, Hkv, NG, GS), np.uint8)
    rc = lib.orc_token_order(B, Hkv, _bf(io_dtype), _p(k), Tstride, int(T), int(residual),
                             NG, int(n_vblk_hi), _p(order))
    assert rc == 0
    if prog:
        rc = lib.orc_prog_values(B, Hkv, _bf(io_dtype), _p(v), Tstride, int(T), int(residual),
                                 NG, int(prog_w8), int(prog_w4), _p(vc), _p(vs), _p(vz))
    else:
        rc = lib.orc_quant_values(B, Hkv, _bf(io_dtype), _p(v), Tstride, int(T),
                                  int(residual), 2, NG, int(n_vblk_hi), int(bits_vhi),
                                  _p(order), _p(vc), _p(vs), _p(vz))
    assert rc == 0
    return Quantized(k=k, v=v, T=int(T), R=int(residual), n_hi=int(n_pairs_hi),
                     bits_hi=int(bits_hi), n_lo1=int(n_pairs_lo1), io_dtype=io_dtype,
                     pairs=pairs,
                     NG=NG, nq=nq, kcodes=kc, ks=ks, kz=kz, vcodes=vc, vs=vs,
                     vz=vz, n_vblk_hi=int(n_vblk_hi), bits_vhi=int(bits_vhi), order=order,
                     prog_w8=int(prog_w8), prog_w4=int(prog_w4))


def attention(qz: Quantized, q, sm_scale: float, with_lse: bool = False):
    """Decode attention over the oracle's quantized cache.  q [B][Hq][128]
    bits.  Returns fp64 [B][Hq][128] (and lse [B][Hq] if asked)."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    B, Hq, _ = q.shape
    Hkv = qz.k.shape[1]
    out = np.zeros((B, Hq, D), np.float64)
    lse = np.zeros((B, Hq), np.float64)
    rc = _load().orc_attention(
        B, Hq, Hkv, _bf(qz.io_dtype), _p(q), _p(qz.k), _p(qz.v), qz.k.shape[2],
        qz.T, qz.R, qz.n_hi, qz.bits_hi, qz.n_lo1, _p(qz.pairs), qz.NG, _p(qz.kcodes),
        _p(qz.ks), _p(qz.kz), _p(qz.vcodes), _p(qz.vs), _p(qz.vz),
        ctypes.c_double(float(np.float32(sm_scale))), _p(out), _p(lse))
    assert rc == 0
    return (out, lse) if with_lse else out


def attention_after_append(qz: Quantized, q, sm_scale: float, with_lse: bool = False):
    """Decode attention of a call that appends token T-1 and decodes in one
    step (qz holds the cache after the append, T tokens): every token is
    attended, but the quantized prefix is the one from before the append,
    n_q(T-1).  A group that the append packs is attended at 16 bits in that
    call (it is still in the ring), and quantized from the next call on
    (PM-KVQ, key_machinery: new tokens are held at 16 bits first and
    quantized later).  Since n_q(T, R+1) = n_q(T-1, R) for every T, this is
    the attention above with the residual window one token longer."""
    kw = dict(qz.__dict__)
    kw["R"] = qz.R + 1
    return attention(Quantized(**kw), q, sm_scale, with_lse=with_lse)


def attention_one_launch(qz_before: Quantized, q, sm_scale: float, with_lse: bool = False):
    """Decode attention of a call that finds the cache as qz_before holds it
    (qz_before.T tokens, every group at the width of its age then), appends
    token qz_before.T from the inputs (present in qz_before.k / .v) and
    decodes in the same step: the quantized prefix and its widths are the
    ones from before the append, and every token past it, the new one
    included, is attended at 16 bits (PM-KVQ, key_machinery: new tokens are
    held at 16 bits first and quantized later).  With n_q(T+1, R+1) =
    n_q(T, R) this is the attention above over T + 1 tokens with the
    residual window one token longer.  Without progressive precision it
    equals attention_after_append of the cache after the append; with it,
    a step that packs a group also shrinks the groups crossing the window
    edges, which this call still reads at their former widths."""
    assert qz_before.k.shape[2] > qz_before.T, "the appended token must be in qz_before.k"
    kw = dict(qz_before.__dict__)
    kw["T"] = qz_before.T + 1
    kw["R"] = qz_before.R + 1
    return attention(Quantized(**kw), q, sm_scale, with_lse=with_lse)


def k_hi_words(n_pairs_hi: int, bits_hi: int) -> int:
    """Bytes of the salient-key section of one group record."""
    if n_pairs_hi == 0:
        return 0
    return 128 if bits_hi == 4 else 32 * 2 * n_pairs_hi * 2


def pack(qz: Quantized) -> dict:
    """Byte records of the oracle's quantized cache (layout of include/kvq.h)
    for groups [0, n_q/32); plus the live ring slots."""
    lib = _load()
    B, Hkv, Tstride, _ = qz.k.shape
    NG = qz.NG
    k_lo = np.zeros((B, Hkv, NG, 192 if dense1(qz.n_hi, qz.n_lo1) else 256), np.uint32)
    k_hi = np.zeros((B, Hkv, NG, max(k_hi_words(qz.n_hi, qz.bits_hi), 1)), np.uint8)
    k_meta = np.zeros((B, Hkv, NG, 256), np.uint16)
    v_codes = np.zeros((B, Hkv, NG, 256), np.uint32)
    v_meta = np.zeros((B, Hkv, NG, 256), np.uint16)
    RS = qz.R + GS
    ring_k = np.zeros((B, Hkv, RS, D), np.uint16)
    ring_v = np.zeros((B, Hkv, RS // GS, D, GS), np.uint16)
    lib.orc_pack_keys(B, Hkv, _p(qz.k), Tstride, qz.T, qz.R, qz.n_hi,
                      qz.bits_hi, qz.n_lo1, _p(qz.pairs), NG, _p(qz.order), _p(qz.kcodes),
                      _p(qz.ks), _p(qz.kz), _p(k_lo), _p(k_hi), _p(k_meta))
    nvb = qz.n_vblk_hi
    v_hi = np.zeros((B, Hkv, NG, 8 + 64 * nvb if nvb else 0), np.uint32)
    lib.orc_pack_values(B, Hkv, qz.T, qz.R, NG, _p(qz.vcodes), _p(qz.vs),
                        _p(qz.vz), int(nvb), _p(qz.order), _p(v_codes),
                        _p(v_meta), _p(v_hi) if nvb else None)
    lib.orc_ring(B, Hkv, _p(qz.k), _p(qz.v), Tstride, qz.T, qz.R, _p(ring_k),
                 _p(ring_v))
    if k_hi_words(qz.n_hi, qz.bits_hi) == 0:
        k_hi = k_hi[..., :0]
    w8, w4 = getattr(qz, "prog_w8", 0), getattr(qz, "prog_w4", 0)
    nslot = w4 + 2 * w8
    k_pl = np.zeros((B, Hkv, nslot, 256), np.uint32)
    v_pl = np.zeros((B, Hkv, nslot, 256), np.uint32)
    if w4 > 0:
        lib.orc_pack_planes(B, Hkv, qz.T, qz.R, NG, w8, w4, _p(qz.kcodes), _p(qz.vcodes),
                            _p(k_pl), _p(v_pl))
    return dict(k_lo=k_lo, k_hi=k_hi, k_meta=k_meta, v_codes=v_codes,
                v_meta=v_meta, ring_k=ring_k, ring_v=ring_v, v_hi=v_hi, k_pl=k_pl, v_pl=v_pl)


def prog_width(age: int, w8: int, w4: int) -> int:
    """Bits of a progressive group of the given age (0 = newest)."""
    return int(_load().orc_prog_width(int(age), int(w8), int(w4)))


def live_plane_slots(T: int, R: int, w8: int, w4: int):
    """(group, plane slot) of every digit plane a progressive cache holds
    with T tokens: digit 1 of the groups younger than w4 at slot g % w4,
    digits 2 and 3 of those younger than w8 at w4 + 2 (g % w8) and the next."""
    ng = n_quant(T, R) // GS
    out = []
    for g in range(max(ng - w4, 0), ng):
        out.append((g, g % w4))
        if ng - 1 - g < w8:
            out += [(g, w4 + 2 * (g % w8)), (g, w4 + 2 * (g % w8) + 1)]
    return out


def dense1(n_pairs_hi: int, n_pairs_lo1: int) -> bool:
    """The dense 1-bit layout (the 1.5-bit point): half of the pairs at one
    bit, none salient; k_lo holds 768 bytes per group in plane order."""
    return bool(_load().orc_dense1(int(n_pairs_hi), int(n_pairs_lo1)))


def live_ring_slots(T: int, R: int) -> np.ndarray:
    """Ring slots that hold tokens when T tokens are cached."""
    RS = R + GS
    return np.array([p % RS for p in range(n_quant(T, R), T)], dtype=np.int64)


def shrink_code(x: int, b: int) -> int:
    """round(x / (2^b + 1)): the b-bit code of a 2b-bit code after the shrink."""
    return int(_load().orc_shrink_code(int(x), int(b)))


def ers(x: int, b: int) -> int:
    """The review's shift form of the same map, as written there."""
    lib = _load()
    lib.orc_ers.restype = ctypes.c_longlong
    lib.orc_ers.argtypes = [ctypes.c_longlong, ctypes.c_int]
    return int(lib.orc_ers(int(x), int(b)))


def shrink(qz: Quantized, g0: int, g1: int) -> Quantized:
    """Copy of qz with the 4-bit salient key channels of groups [g0, g1)
    shrunk to the 2-bit grid of step 5 s (zero kept): 4-bit code 5 * round(X/5)
    under the unchanged scale s."""
    assert qz.bits_hi == 4
    kw = dict(qz.__dict__)
    kw["kcodes"] = qz.kcodes.copy()
    kw["ks"] = qz.ks.copy()
    B, Hkv = qz.kcodes.shape[:2]
    rc = _load().orc_shrink_keys(B, Hkv, qz.n_hi, _p(qz.pairs), qz.NG, qz.nq // GS, int(g0),
                                 int(g1), _p(kw["kcodes"]), _p(kw["ks"]))
    assert rc == 0
    return Quantized(**kw)


def select_qa(q_sel, k, T: int, n_kv_heads: int, io_dtype: str):
    """Query-aware channel score (the MixKVQ reading): returns (score
    [B][Hkv][64] float64, pairs [B][Hkv][64] int32)."""
    q_sel = np.ascontiguousarray(q_sel, dtype=np.uint16)
    k = np.ascontiguousarray(np.asarray(k)[:, :, :T], dtype=np.uint16)
    B, Hq, n_qry, _ = q_sel.shape
    bits = np.zeros((B, n_kv_heads, 64), np.uint64)
    pairs = np.zeros((B, n_kv_heads, 64), np.int32)
    rc = _load().orc_select_qa(B, Hq, n_kv_heads, _bf(io_dtype), _p(q_sel), n_qry, _p(k),
                               int(T), _p(bits), _p(pairs))
    assert rc == 0
    return bits.view(np.float64), pairs


def prune_chunks(q, n_kv_heads: int, io_dtype: str, n_keep: int) -> np.ndarray:
    """Query-channel pruning (the Dual-QK reading): bool [B][Hkv][8], True
    for the n_keep 16-channel key runs of largest summed fixed-point |q|
    over the group's heads (ties to the lower run)."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    B, Hq, _ = q.shape
    keep = np.zeros((B, n_kv_heads, 8), np.uint8)
    rc = _load().orc_prune_chunks(B, Hq, n_kv_heads, _bf(io_dtype), _p(q), int(n_keep), _p(keep))
    assert rc == 0
    return keep.astype(bool)


def attention_pruned(qz: Quantized, q, sm_scale: float, n_keep: int, with_lse: bool = False):
    """Decode attention with pruned query channels: every logit sums q_c k^_c
    over the kept runs' channels only (quantized and ring tokens alike),
    written as attention over the query with the pruned channels set to 0."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    B, Hq, _ = q.shape
    Hkv = qz.kcodes.shape[1]
    keep = prune_chunks(q, Hkv, qz.io_dtype, n_keep)
    qm = q.copy()
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            for s in range(8):
                if not keep[b, h // G, s]:
                    qm[b, h, 16 * s:16 * s + 16] = 0
    return attention(qz, qm, sm_scale, with_lse=with_lse)
