"""Pins for the oracle's binary16 codec (the Q8_0 scale format).

The Q8_0 block stores its scale as fp16 ("Ember packed Q8 decode" post,
row-contiguous source diagram and the "16 fp16 scales" of a packed record).
The oracle's converter is written from the IEEE 754 bit definitions; here it
is compared, exhaustively, with numpy's independent float16 conversion (round
to nearest even with subnormals), and with textbook boundary cases.
"""
import os

import numpy as np
import pytest

import oracle


def _golden_pairs(golden_dir):
    pairs = []
    with open(os.path.join(golden_dir, "fp16_boundaries.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split()[:2]
            pairs.append((int(a, 16), int(b, 16)))
    return pairs


def test_f32_to_f16_boundaries(golden_dir):
    pairs = _golden_pairs(golden_dir)
    assert len(pairs) >= 20
    src = np.array([p[0] for p in pairs], dtype=np.uint32).view(np.float32)
    want = np.array([p[1] for p in pairs], dtype=np.uint16)
    got = oracle.f32_to_f16_bits(src)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(pairs[i][0]), hex(int(got[i])), hex(pairs[i][1])) for i in bad]


def _low_patterns():
    """Low 13 mantissa bits that decide rounding: for every bit position p the
    patterns just below, at and just above 2^p (this covers the rounding bit of
    the normal range, p = 12, and every rounding position of the subnormal
    range), plus all-ones and zero."""
    pats = {0, 0x1FFF}
    for p in range(13):
        for v in ((1 << p) - 1, 1 << p, (1 << p) + 1, (1 << p) | 0x1000, ((1 << p) - 1) | 0x1000):
            pats.add(v & 0x1FFF)
    return np.array(sorted(pats), dtype=np.uint32)


def test_f32_to_f16_stratified_exhaustive():
    """Every (sign, exponent, top-10 mantissa bits) combination of fp32 with
    every rounding class of the low 13 bits, plus 2^24 random bit patterns,
    against numpy's float16 conversion."""
    low = _low_patterns()
    hi = (np.arange(1 << 19, dtype=np.uint32) << 13)  # sign, exponent and top 10 mantissa bits
    for lo in low:
        _compare(hi | lo)
    rng = np.random.default_rng(20261202)
    _compare(rng.integers(0, 1 << 32, size=1 << 24, dtype=np.uint64).astype(np.uint32))


def _compare(bits):
    f = bits.view(np.float32)
    got = oracle.f32_to_f16_bits(f)
    with np.errstate(all="ignore"):
        ref = f.astype(np.float16).view(np.uint16)
    nan_src = np.isnan(f)
    ok = (got == ref) | nan_src
    if not ok.all():
        i = int(np.nonzero(~ok)[0][0])
        pytest.fail(f"fp32 0x{int(bits[i]):08x}: oracle 0x{int(got[i]):04x} numpy 0x{int(ref[i]):04x}")
    # every NaN input must stay a NaN
    got_nan = got[nan_src]
    assert np.all(((got_nan & 0x7c00) == 0x7c00) & ((got_nan & 0x03ff) != 0))


def test_f16_to_f32_exhaustive():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_bits_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    both_nan = np.isnan(got) & np.isnan(ref)
    assert np.all((got.view(np.uint32) == ref.view(np.uint32)) | both_nan)
    # round trip for every non-NaN fp16 value
    back = oracle.f32_to_f16_bits(got)
    finite = ~np.isnan(ref)
    assert np.array_equal(back[finite], h[finite])


def test_fp16_products_exact_in_fp32():
    """The block term relies on fp16 x fp16 being exact in fp32: check it on
    every positive normal/subnormal fp16 against fp64 for a sample grid."""
    rng = np.random.default_rng(7)
    a = rng.integers(1, 0x7c00, size=200000, dtype=np.uint16)
    b = rng.integers(1, 0x7c00, size=200000, dtype=np.uint16)
    fa, fb = oracle.f16_bits_to_f32(a), oracle.f16_bits_to_f32(b)
    p32 = fa * fb
    p64 = fa.astype(np.float64) * fb.astype(np.float64)
    assert np.array_equal(p32.astype(np.float64), p64)
