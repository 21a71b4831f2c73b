"""Pins of the oracle's affine quantizer (SemKV abstract: scale + zero
point; PN-Mix abstract: 2-bit and higher-precision codes) by properties that
hold for any correct min/max grid quantizer, and by nearest-level search."""
import numpy as np
import pytest

import kvq_synth
import oracle
from oracle import brute


def _groups(io_dtype, n, seed):
    rng = np.random.default_rng(seed)
    scales = rng.choice([1e-3, 0.1, 1.0, 10.0, 300.0], size=(n, 1))
    x = rng.standard_normal((n, 32)) * scales + rng.standard_normal((n, 1)) * scales
    bits = kvq_synth.to_bits(x, io_dtype)
    return kvq_synth.bits_to_f64(bits, io_dtype)


def _f16(b):
    return float(np.uint16(b).view(np.float16))


@pytest.mark.parametrize("io_dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("bits", [1, 2, 4])
def test_codes_are_nearest_levels(io_dtype, bits):
    L = (1 << bits) - 1
    xs = _groups(io_dtype, 300, 11 + bits)
    checked = 0
    for x in xs:
        codes, sb, zb = oracle.quant_group(x, bits)
        s, z = _f16(sb), _f16(zb)
        assert s > 0
        q, margin = brute.nearest_level(x, s, z, L)
        # skip inputs within 1e-4 of a level spacing of a rounding boundary:
        # there the fp32 product (x - z) * (1/s) may legitimately round across
        ok = margin > 1e-4 * s
        assert np.array_equal(codes[ok], q[ok])
        checked += ok.sum()
    assert checked > 0.95 * xs.size


@pytest.mark.parametrize("io_dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("bits", [2, 4])
def test_error_bound_and_extremes(io_dtype, bits):
    L = (1 << bits) - 1
    for x in _groups(io_dtype, 300, 5 + bits):
        codes, sb, zb = oracle.quant_group(x, bits)
        s, z = _f16(sb), _f16(zb)
        xhat = z + s * codes.astype(np.float64)
        # z is the min rounded to fp16; s is the range / L rounded to fp16
        slack = abs(x.min() - z) + L * abs(s - (x.max() - z) / L) + 1e-12
        assert np.all(np.abs(x - xhat) <= s / 2 + slack)
        assert codes[np.argmax(x)] == L
        if io_dtype == "fp16":
            assert z == x.min() and codes[np.argmin(x)] == 0


def test_scale_is_nearest_half_of_range_over_levels():
    for bits in (1, 2, 4):
        L = (1 << bits) - 1
        for x in _groups("bf16", 200, 3):
            _, sb, zb = oracle.quant_group(x, bits)
            z = _f16(zb)
            target = (x.max() - z) / L
            cand = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float64)
            cand = cand[np.isfinite(cand) & (cand >= 0)]
            err = np.abs(cand - target)
            best = err.min()
            assert abs(_f16(sb) - target) <= best * (1 + 1e-6) + 1e-30


def test_constant_group():
    for v in (0.0, 1.5, -3.25, 1000.0):
        codes, sb, zb = oracle.quant_group(np.full(32, v), 2)
        assert sb == 0 and not codes.any() and _f16(zb) == v


def test_idempotent():
    for bits in (2, 4):
        L = (1 << bits) - 1
        for x in _groups("fp16", 200, 9):
            codes, sb, zb = oracle.quant_group(x, bits)
            s, z = _f16(sb), _f16(zb)
            xhat = z + s * codes.astype(np.float64)
            if not np.array_equal(xhat.astype(np.float32).astype(np.float64), xhat):
                continue
            c2, sb2, zb2 = oracle.quant_group(xhat, bits)
            assert (sb2, zb2) == (sb, zb)
            assert np.array_equal(c2, codes)
