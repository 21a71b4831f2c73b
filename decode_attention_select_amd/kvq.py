"""Python binding of libkvq's C ABI (include/kvq.h).

Argument marshalling only: every function forwards to the entry point of the
same name in libkvq.so (HIP kernels for gfx950).  Tensors must be CUDA (HIP)
tensors; the work is enqueued on torch's current stream unless a stream is
given.  There is no CPU path: if the library is not built, or no GPU is
present, calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvq.so")
_lib = None

KVQ_FP16, KVQ_BF16 = 0, 1
NBUF = 14
BUF_NAMES = ["k_lo", "k_hi", "k_meta", "v_codes", "v_meta", "ring_k", "ring_v",
             "pairs", "len", "sums", "err", "v_hi", "k_pl", "v_pl"]


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s failed: %s (%d)" % (where, kvq_status_str(status), status))
        self.status = status


class kvq_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_q_heads", "n_kv_heads", "head_dim", "group", "n_pairs_hi",
        "bits_hi", "n_pairs_lo1", "bits_lo", "bits_v", "residual", "max_tokens",
        "io_dtype", "n_vblk_hi", "bits_vhi", "prog_w8", "prog_w4")]


class kvq_cache(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BUF_NAMES]


# The same library with the decode kernel's phase timestamps compiled in
# (measurement builds only: its workspace holds the timestamps after the
# records, so kvq_workspace_bytes reports more).
STAMPS_LIB_PATH = os.path.join(_PKG, "libkvq_stamps.so")


def lib():
    """The loaded libkvq.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libkvq.so is not built (run __graft_entry__.build())")
        _lib = ctypes.CDLL(LIB_PATH)
        _lib.kvq_status_str.restype = ctypes.c_char_p
    return _lib


def use_stamps_library():
    """Binds every call of this module to libkvq_stamps.so instead of
    libkvq.so (before any call has loaded the library)."""
    global _lib, LIB_PATH
    if _lib is not None and LIB_PATH != STAMPS_LIB_PATH:
        raise RuntimeError("kvq: libkvq.so is already loaded")
    LIB_PATH = STAMPS_LIB_PATH


def make_layout(batch, n_q_heads, n_kv_heads, *, n_pairs_hi=6, bits_hi=4,
                residual=128, max_tokens, io_dtype="bf16", n_pairs_lo1=0,
                bits_lo=2, bits_v=2, n_vblk_hi=0, bits_vhi=4, prog_w8=0,
                prog_w4=0) -> kvq_layout:
    return kvq_layout(batch, n_q_heads, n_kv_heads, 128, 32, n_pairs_hi, bits_hi,
                      n_pairs_lo1, bits_lo, bits_v, residual, max_tokens,
                      KVQ_BF16 if io_dtype == "bf16" else KVQ_FP16, n_vblk_hi, bits_vhi,
                      prog_w8, prog_w4)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t):
    if t is None:
        return ctypes.c_void_p(0)
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    if not t.is_cuda:
        raise ValueError("kvq: tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("kvq: tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise KvqError(st, name)


def kvq_status_str(status: int) -> str:
    return lib().kvq_status_str(ctypes.c_int32(status)).decode()


def kvq_cache_sizes(layout: kvq_layout) -> list:
    sizes = (ctypes.c_size_t * NBUF)()
    _call("kvq_cache_sizes", ctypes.byref(layout), sizes)
    return list(sizes)


def kvq_workspace_bytes(layout: kvq_layout, n_splits: int) -> int:
    n = ctypes.c_size_t(0)
    _call("kvq_workspace_bytes", ctypes.byref(layout), ctypes.c_int32(n_splits), ctypes.byref(n))
    return n.value


def kvq_select_pairs(layout, q_sel, n_qry, k, T, cache: kvq_cache, stream=None):
    _call("kvq_select_pairs", ctypes.byref(layout), _ptr(q_sel), ctypes.c_int32(n_qry),
          _ptr(k), ctypes.c_int32(T), ctypes.byref(cache), _stream(stream))


def kvq_select_pairs_qa(layout, q_sel, n_qry, k, T, cache: kvq_cache, stream=None):
    _call("kvq_select_pairs_qa", ctypes.byref(layout), _ptr(q_sel), ctypes.c_int32(n_qry),
          _ptr(k), ctypes.c_int32(T), ctypes.byref(cache), _stream(stream))


def kvq_quant_keys(layout, k, T, cache: kvq_cache, stream=None):
    _call("kvq_quant_keys", ctypes.byref(layout), _ptr(k), ctypes.c_int32(T),
          ctypes.byref(cache), _stream(stream))


def kvq_quant_values(layout, v, T, cache: kvq_cache, stream=None):
    _call("kvq_quant_values", ctypes.byref(layout), _ptr(v), ctypes.c_int32(T),
          ctypes.byref(cache), _stream(stream))


def kvq_append(layout, k_new, v_new, cache: kvq_cache, stream=None):
    _call("kvq_append", ctypes.byref(layout), _ptr(k_new), _ptr(v_new),
          ctypes.byref(cache), _stream(stream))


def kvq_shrink(layout, cache: kvq_cache, g0: int, g1: int, stream=None):
    _call("kvq_shrink", ctypes.byref(layout), ctypes.byref(cache), ctypes.c_int32(g0),
          ctypes.c_int32(g1), _stream(stream))


def kvq_decode_attn(layout, q, cache: kvq_cache, sm_scale, n_splits, workspace, out,
                    stream=None, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _call("kvq_decode_attn", ctypes.byref(layout), _ptr(q), ctypes.byref(cache),
          ctypes.c_float(sm_scale), ctypes.c_int32(n_splits), _ptr(workspace),
          ctypes.c_size_t(ws_bytes), _ptr(out), _stream(stream))


def kvq_decode_attn_pruned(layout, q, cache: kvq_cache, sm_scale, n_splits, n_keep, workspace,
                           out, stream=None, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _call("kvq_decode_attn_pruned", ctypes.byref(layout), _ptr(q), ctypes.byref(cache),
          ctypes.c_float(sm_scale), ctypes.c_int32(n_splits), ctypes.c_int32(n_keep),
          _ptr(workspace), ctypes.c_size_t(ws_bytes), _ptr(out), _stream(stream))


def kvq_append_decode_attn(layout, k_new, v_new, q, cache: kvq_cache, sm_scale, n_splits,
                           workspace, out, stream=None, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _call("kvq_append_decode_attn", ctypes.byref(layout), _ptr(k_new), _ptr(v_new), _ptr(q),
          ctypes.byref(cache), ctypes.c_float(sm_scale), ctypes.c_int32(n_splits),
          _ptr(workspace), ctypes.c_size_t(ws_bytes), _ptr(out), _stream(stream))


NOALLOC_WORKSPACE_BYTES = 4 << 20


def kvq_decode_attn_noalloc(layout, q, cache: kvq_cache, sm_scale, n_splits, out, stream=None):
    _call("kvq_decode_attn_noalloc", ctypes.byref(layout), _ptr(q), ctypes.byref(cache),
          ctypes.c_float(sm_scale), ctypes.c_int32(n_splits), _ptr(out), _stream(stream))


def kvq_read_ceiling(layout, cache: kvq_cache, n_splits, sink, stream=None):
    _call("kvq_read_ceiling", ctypes.byref(layout), ctypes.byref(cache),
          ctypes.c_int32(n_splits), _ptr(sink), _stream(stream))


def kvq_issue_probe(kind, n_blocks, out, stream=None):
    _call("kvq_issue_probe", ctypes.c_int32(kind), ctypes.c_int32(n_blocks), _ptr(out),
          _stream(stream))


def kvq_check(cache: kvq_cache, stream=None) -> int:
    err = ctypes.c_int32(0)
    _call("kvq_check", ctypes.byref(cache), ctypes.byref(err), _stream(stream))
    return err.value


class Cache:
    """Device buffers of one cache (torch uint8 tensors, sizes from
    kvq_cache_sizes) and the kvq_cache struct that points at them."""

    def __init__(self, layout: kvq_layout, device="cuda"):
        self.layout = layout
        self.sizes = kvq_cache_sizes(layout)
        self.bufs = {}
        for name, n in zip(BUF_NAMES, self.sizes):
            # zero-size sections still get a valid, aligned pointer
            self.bufs[name] = torch.zeros(max(n, 16), dtype=torch.uint8, device=device)
        self.struct = kvq_cache(*[self.bufs[n].data_ptr() for n in BUF_NAMES])

    def __getitem__(self, name):
        return self.bufs[name][:self.sizes[BUF_NAMES.index(name)]]

    def nbytes(self) -> int:
        return sum(self.sizes)
