"""The arithmetic shortcuts of the GPU's fused activation quantizer, checked on
the host against the correctly rounded operations they replace (fp32 numpy
arithmetic is IEEE round-to-nearest-even).  The device code is compared with the
standalone quantizer bit for bit by the GPU tests; these tests pin the methods.

- Block scale: d = amax / 127 as q = RN(amax * y), y = RN(1/127), then one
  correction RN(q + RN(amax - 127 q) * y) (Markstein's theorem: with y the
  correctly rounded reciprocal and q faithful, the corrected quotient is the
  correctly rounded one).  Checked for every fp32 significand at several
  exponents; the fma steps are emulated exactly (the products fit fp64, and
  the last sum is checked never to sit on an fp32 midpoint, where a second
  rounding could differ).
- Rounding: round half away from zero as trunc(q + copysign(0.5 - 2^-25, q)),
  on every half-integer up to 128 and the fp32 values next to it (an
  exhaustive run over all |q| <= 128 is recorded in the design notes)."""
import numpy as np
import pytest



def _fast_scale(amax: np.ndarray):
    y = np.float32(1) / np.float32(127)
    q = (amax * y).astype(np.float32)
    # fma(-127, q, amax): exact in fp64 (31 significant bits), one rounding to fp32
    r = (amax.astype(np.float64) - 127.0 * q.astype(np.float64)).astype(np.float32)
    # fma(r, y, q): r * y is exact in fp64; the sum is rounded once in fp64, so
    # the fp32 cast is exact unless that fp64 sum is an fp32 midpoint
    s = q.astype(np.float64) + r.astype(np.float64) * np.float64(y)
    d = s.astype(np.float32)
    up = np.nextafter(d, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(d, np.float32(-np.inf)).astype(np.float64)
    mid = (s == (d.astype(np.float64) + up) / 2) | (s == (d.astype(np.float64) + dn) / 2)
    return d, int(mid.sum())


@pytest.mark.parametrize("exp", [0, -89, 95])
def test_block_scale_by_constant_reciprocal_is_correctly_rounded(exp):
    sig = np.arange(1 << 23, 1 << 24, dtype=np.float64)
    amax = (sig * 2.0 ** (exp - 23)).astype(np.float32)
    d, mids = _fast_scale(amax)
    assert mids == 0
    assert np.array_equal(d, amax / np.float32(127))


def _round_half_away_fast(q: np.ndarray) -> np.ndarray:
    c = np.float32(0.5 - 2.0 ** -25)
    return np.trunc(q + np.copysign(c, q)).astype(np.int64)


def test_round_half_away_near_every_half_integer():
    half = np.arange(0, 128, dtype=np.float32) + np.float32(0.5)
    vals = [half]
    up, dn = half.copy(), half.copy()
    for _ in range(4):
        up = np.nextafter(up, np.float32(np.inf)); dn = np.nextafter(dn, np.float32(-np.inf))
        vals += [up, dn]
    vals += [np.float32(0.5 - 2.0 ** -25) * np.ones(1, np.float32), np.arange(0, 129, dtype=np.float32),
             np.random.default_rng(0).uniform(0, 128, 100000).astype(np.float32)]
    q = np.concatenate(vals)
    q = np.concatenate([q, -q])
    ref = (np.sign(q.astype(np.float64)) * np.floor(np.abs(q.astype(np.float64)) + 0.5)).astype(np.int64)
    assert np.array_equal(_round_half_away_fast(q), ref)
