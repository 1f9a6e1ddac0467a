"""Pins for the oracle's Q8_0 block quantizer.

Definition (pages): per 32-value block, scale d = amax / 127 and values
rounded to the nearest integer ("ferro" README, "How the iGPU path is fast",
item 1, activations quantized per 32-block; weights converted to Q8_0 at load,
"Using LFM2.5"); the block is an fp16 scale followed by 32 int8 values, 34
bytes ("Ember packed Q8 decode" post, row-contiguous diagram).  Readings taken
where the pages are silent: ties away from zero, one correctly rounded fp32
division x / d by the fp32 d, stored scale fp16(d).

Pins used: hand-worked examples (tests/golden/q8_quant_hand.txt), the zero
block, invariants that hold for any correct quantizer (range, sign symmetry,
power-of-two scale invariance, reconstruction bound), and agreement with an
fp64 evaluation of round-half-away(x / d) away from near-ties.
"""
import os

import numpy as np
import pytest

import oracle


def _hand_examples(golden_dir):
    ex, cur = [], {}
    with open(os.path.join(golden_dir, "q8_quant_hand.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            cur[key.strip()] = val.strip()
            if key.strip() == "d_bits":
                ex.append(cur)
                cur = {}
    return ex


def test_hand_examples(golden_dir):
    ex = _hand_examples(golden_dir)
    assert len(ex) == 5
    for e in ex:
        xs = [float(v) for v in e["x"].split()]
        qs = [int(v) for v in e["q"].split()]
        x = np.zeros(32, np.float32)
        x[: len(xs)] = np.array(xs, np.float32)
        want = np.zeros(32, np.int8)
        want[: len(qs)] = qs
        q, dbits, _ = oracle.quantize_block(x)
        assert np.array_equal(q, want), (e["name"], q, want)
        assert dbits == int(e["d_bits"], 16), (e["name"], hex(dbits))


def test_zero_block_positive_zero_scale():
    for x in (np.zeros(32, np.float32), -np.zeros(32, np.float32)):
        q, dbits, d = oracle.quantize_block(x)
        assert not q.any() and dbits == 0 and d == 0.0


def _random_blocks(n, seed=1):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 32)).astype(np.float32)
    # mix magnitudes: 1e-3 .. 1e3, and a few outlier entries
    x *= (10.0 ** rng.uniform(-3, 3, size=(n, 1))).astype(np.float32)
    out = rng.random((n, 32)) < 0.02
    x[out] *= np.float32(20.0)
    return x


def _quant_all(x):
    buf = oracle.quantize_rows(x.reshape(1, -1), oracle.LAYOUT_ROWS)
    q, d = oracle.rows_planes(buf, 1, x.size)
    return q.reshape(-1, 32), d.reshape(-1)


def test_invariants_range_and_amax():
    x = _random_blocks(20000)
    q, dbits = _quant_all(x)
    assert np.abs(q.astype(np.int32)).max() <= 127
    i = np.abs(x).argmax(axis=1)
    qa = q[np.arange(len(q)), i].astype(np.int32)
    assert np.array_equal(qa, np.where(x[np.arange(len(x)), i] > 0, 127, -127))


def test_invariant_sign_symmetry():
    x = _random_blocks(20000, seed=2)
    q1, d1 = _quant_all(x)
    q2, d2 = _quant_all(-x)
    assert np.array_equal(q1.astype(np.int32), -q2.astype(np.int32))
    assert np.array_equal(d1, d2)


def test_invariant_power_of_two_scaling():
    """x * 2^e gives the same q and the scale times 2^e: exact in fp32 and, as
    long as the fp32 scale before and after scaling lies in fp16's normal
    range, exact in fp16 too (rounding to fp16 commutes with 2^e there)."""
    x = _random_blocks(20000, seed=3)
    q0, d0 = _quant_all(x)
    d32 = np.abs(x).max(axis=1) / np.float32(127)
    for e in (-3, 1, 4):
        qe, de = _quant_all(x * np.float32(2.0 ** e))
        assert np.array_equal(q0, qe)
        f0 = d0.view(np.float16).astype(np.float64) * 2.0 ** e
        fe = de.view(np.float16).astype(np.float64)
        lo = np.minimum(d32, d32 * 2.0 ** e)
        hi = np.maximum(d32, d32 * 2.0 ** e)
        normal = (lo >= 2.0 ** -14) & (hi <= 65504)
        assert normal.sum() > 10000
        assert np.array_equal(f0[normal], fe[normal])


def test_reconstruction_bound_and_fp64_agreement():
    """|x - q d| <= d (1/2 + 2^-18) with the fp32 d (x / d < 128 in magnitude,
    whose fp32 rounding error is at most 2^-18), and q equals
    round-half-away(x / d) evaluated in fp64 wherever x / d is not within
    2^-17 of a half-integer."""
    x = _random_blocks(5000, seed=4)
    for blk in x[:5000]:
        q, _, d = oracle.quantize_block(blk)
        r64 = blk.astype(np.float64) / np.float64(d)
        err = np.abs(blk.astype(np.float64) - q.astype(np.float64) * d)
        assert np.all(err <= d * (0.5 + 2.0 ** -18))
        frac = np.abs(r64 - np.trunc(r64))
        far = np.abs(frac - 0.5) > 2.0 ** -17
        ref = np.trunc(r64 + np.copysign(0.5, r64))
        assert np.array_equal(q[far].astype(np.float64), ref[far])


def test_scale_is_fp16_of_amax_over_127():
    """The stored scale is the fp16 rounding of amax/127; checked against
    numpy's own fp32 division and fp16 conversion."""
    x = _random_blocks(20000, seed=5)
    _, dbits = _quant_all(x)
    amax = np.abs(x).max(axis=1)
    d = (amax / np.float32(127)).astype(np.float32)
    assert np.array_equal(dbits, d.astype(np.float16).view(np.uint16))


def test_layouts_rows_and_act():
    """ROWS is [fp16 d][32 int8] per block, rows of k/32 blocks; ACT is the
    int8 plane [rows][k] then the fp16 plane [rows][k/32]; the row stride of
    the fp32 input is honoured."""
    rng = np.random.default_rng(9)
    base = rng.standard_normal((3, 100)).astype(np.float32)
    x = base[:, :96]  # row stride 100 elements, k = 96 (3 blocks)
    rows = oracle.quantize_rows(x, oracle.LAYOUT_ROWS)
    act = oracle.quantize_rows(x, oracle.LAYOUT_ACT)
    assert rows.size == act.size == 3 * 3 * 34
    qa, da = oracle.act_planes(act, 3, 96)
    for r in range(3):
        for b in range(3):
            q, dbits, _ = oracle.quantize_block(x[r, 32 * b: 32 * b + 32])
            blk = rows[(r * 3 + b) * 34: (r * 3 + b + 1) * 34]
            assert int(blk[0]) | (int(blk[1]) << 8) == dbits
            assert np.array_equal(blk[2:].view(np.int8), q)
            assert np.array_equal(qa[r, 32 * b: 32 * b + 32], q)
            assert da[r, b] == dbits
