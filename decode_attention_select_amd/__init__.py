"""decode_attention_select_amd — MI355X-native quantized-KV decode path.

libkvq.so (HIP, gfx950) implements pair-norm-selected mixed-precision key
quantization, per-token value quantization, the 16-bit ring of recent tokens
and split-K decode attention over the packed cache; ``kvq`` is its ctypes
binding (same entry-point names as include/kvq.h).
"""
from . import kvq  # noqa: F401

__all__ = ["kvq"]
