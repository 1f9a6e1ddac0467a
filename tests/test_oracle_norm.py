"""Pins of the oracle's fused residual + RMSNorm + Q8_0 producer
(q8ref_rmsnorm_quantize; "ferro" README, "How the iGPU path is fast", item 3)
against things other than itself: numpy's fp32 addition, an fp64 evaluation
with an exactly rounded sum (math.fsum), closed forms and exact scaling
invariants."""
import math

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

EPS = 1e-5


def _rng(seed):
    return np.random.default_rng(1000 + seed)


def _case(rows, k, seed, scale=1.0):
    g = _rng(seed)
    x = (g.standard_normal((rows, k)) * scale).astype(np.float32)
    r = (g.standard_normal((rows, k)) * scale).astype(np.float32)
    w = (1.0 + 0.1 * g.standard_normal(k)).astype(np.float32)
    return x, r, w


def _codes(q, rows, k):
    return oracle.act_planes(q, rows, k)


@pytest.mark.parametrize("rows,k", [(1, 32), (3, 256), (2, 2048), (1, 8192), (4, 7168), (2, 2080)])
def test_residual_is_numpy_fp32_sum(rows, k):
    x, r, w = _case(rows, k, rows + k)
    ro, _ = oracle.rmsnorm_quantize(x, r, w, EPS)
    assert np.array_equal(ro.view(np.uint32), (r + x).astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("rows,k", [(1, 32), (3, 256), (2, 2048), (1, 8192), (4, 7168), (2, 2080)])
def test_against_exactly_rounded_fp64_evaluation(rows, k):
    """The scale r from an exactly rounded sum (math.fsum) of the fp64 squares,
    then the fp32 normalize and the block quantizer: codes and scales must
    equal the oracle's (the fixed fp64 summation order can only differ from
    the exactly rounded sum by a few fp64 ulps, far below fp32 resolution)."""
    x, r, w = _case(rows, k, 7 * rows + k)
    _, q = oracle.rmsnorm_quantize(x, r, w, EPS)
    h = (r + x).astype(np.float32)
    n = np.empty_like(h)
    for i in range(rows):
        ss = math.fsum(float(v) * float(v) for v in h[i])
        rs = np.float32(1.0 / math.sqrt(ss / k + EPS))
        n[i] = (h[i] * rs).astype(np.float32) * w
    q_ref = oracle.quantize_rows(n.astype(np.float32), oracle.LAYOUT_ACT)
    assert np.array_equal(q, q_ref)


def test_fp64_brute_force_within_one_code():
    """Against a pure fp64 evaluation n = h / sqrt(mean + eps) * w: every code
    within one step, and equal wherever the fp64 quotient is not within 1e-4
    of a rounding boundary."""
    rows, k = 8, 2048
    x, r, w = _case(rows, k, 99)
    _, q = oracle.rmsnorm_quantize(x, r, w, EPS)
    qi, _ = _codes(q, rows, k)
    h = (r.astype(np.float64) + x.astype(np.float64))
    h = h.astype(np.float32).astype(np.float64)  # the residual sum is an fp32 value by definition
    n = h / np.sqrt((h * h).mean(axis=1, keepdims=True) + EPS) * w.astype(np.float64)
    nb = n.reshape(rows, k // 32, 32)
    d = np.abs(nb).max(axis=2, keepdims=True) / 127.0
    v = nb / d
    q64 = np.sign(v) * np.floor(np.abs(v) + 0.5)
    qi = qi.reshape(rows, k // 32, 32).astype(np.float64)
    assert np.abs(qi - q64).max() <= 1
    frac = np.abs(np.abs(v) - np.floor(np.abs(v)) - 0.5)
    safe = frac > 1e-4
    assert np.array_equal(qi[safe], q64[safe])


def test_constant_row_closed_form():
    """Every h equal: r = 1/sqrt(c^2 + eps), all normalized values equal, so
    every code is +-127 and every block scale is fp16(|n| / 127)."""
    k = 512
    for c in (0.75, -3.0, 100.0):
        x = np.full((1, k), c, np.float32)
        r = np.zeros((1, k), np.float32)
        w = np.ones(k, np.float32)
        _, q = oracle.rmsnorm_quantize(x, r, w, EPS)
        qi, sc = _codes(q, 1, k)
        assert (qi == (127 if c > 0 else -127)).all()
        rs = np.float32(1.0 / math.sqrt(float(c) * float(c) + EPS))
        nv = np.float32(np.float32(c) * rs)
        d = np.float32(abs(nv) / np.float32(127.0))
        assert (sc == oracle.f32_to_f16_bits(np.array([d], np.float32))[0]).all()


def test_zero_row_gives_zero_blocks():
    k = 256
    z = np.zeros((2, k), np.float32)
    ro, q = oracle.rmsnorm_quantize(z, z, np.ones(k, np.float32), EPS)
    qi, sc = _codes(q, 2, k)
    assert (qi == 0).all() and (sc == 0).all() and (ro == 0).all()


def test_power_of_two_scaling_is_exact_without_eps():
    """With eps = 0, scaling h by 2^j scales ss by 4^j, the mean and its root
    exactly, so r scales by 2^-j and the normalized row -- hence every code
    and scale -- is unchanged."""
    rows, k = 3, 1024
    x, r, w = _case(rows, k, 5)
    _, q0 = oracle.rmsnorm_quantize(x, r, w, 0.0)
    for j in (-3, 1, 4):
        f = np.float32(2.0 ** j)
        _, q1 = oracle.rmsnorm_quantize(x * f, r * f, w, 0.0)
        assert np.array_equal(q0, q1)


def test_weight_doubling_doubles_scales_only():
    rows, k = 2, 2048
    x, r, w = _case(rows, k, 6)
    _, q0 = oracle.rmsnorm_quantize(x, r, w, EPS)
    _, q1 = oracle.rmsnorm_quantize(x, r, w * np.float32(2.0), EPS)
    qa, sa = _codes(q0, rows, k)
    qb, sb = _codes(q1, rows, k)
    assert np.array_equal(qa, qb)
    fa = oracle.f16_bits_to_f32(sa)
    fb = oracle.f16_bits_to_f32(sb)
    assert np.array_equal(fb, 2 * fa)


def test_residual_in_place_and_bad_shape():
    x, r, w = _case(2, 64, 8)
    ro, _ = oracle.rmsnorm_quantize(x, r, w, EPS)
    assert np.array_equal(ro, (r + x).astype(np.float32))
    with pytest.raises(ValueError):
        oracle.rmsnorm_quantize(np.zeros((1, 40), np.float32), np.zeros((1, 40), np.float32),
                                np.ones(40, np.float32), EPS)


def test_no_residual_equals_zero_residual():
    """Without a residual the normalized row is that of x itself: identical to
    passing an all-zero residual (fp32 0 + x == x exactly)."""
    x, _, w = _case(3, 2048, 9)
    ro0, q0 = oracle.rmsnorm_quantize(x, None, w, EPS)
    ro1, q1 = oracle.rmsnorm_quantize(x, np.zeros_like(x), w, EPS)
    assert np.array_equal(q0, q1) and np.array_equal(ro0, x) and np.array_equal(ro1, x)
