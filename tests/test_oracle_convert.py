"""Pins of the oracle's own 16-bit conversions against numpy's and torch's
casts (library routines), over every bit pattern where that is cheap."""
import numpy as np
import torch

import oracle


def test_half_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.half_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    got = oracle.bf16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_f32_to_half_rne():
    rng = np.random.default_rng(7)
    # normal range, subnormal range, around the overflow threshold, exact ties
    x = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * 10,
        (rng.standard_normal(2000) * 2.0 ** -16).astype(np.float32),
        (rng.standard_normal(1000) * 2.0 ** -22).astype(np.float32),
        np.float32([65504, 65519.99, 65520, 65536, -65520, 1e6, 0.0, -0.0]),
        # midpoints between adjacent halves: ties must go to even
        ((np.arange(2048, 4096, dtype=np.float64) + 0.5) * 2.0 ** -10).astype(np.float32),
        ((np.arange(1, 1024, dtype=np.float64) + 0.5) * 2.0 ** -24).astype(np.float32),
    ])
    ref = x.astype(np.float16).view(np.uint16)
    got = oracle.f32_to_half(x)
    assert np.array_equal(got, ref)
