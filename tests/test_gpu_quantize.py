"""GPU quantizer (q8_quantize_rows) against the oracle: bit-exact int8 values
and fp16 scales, in both output layouts, on ragged, crafted and full-size
inputs."""
import os

import numpy as np
import pytest

import oracle
import workloads as wl
from decode_q8_amd import q8
from tests.gpu_helpers import down, quantize, require_gpu, up

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _check(x, layout):
    got = down(quantize(x, layout))
    ref = oracle.quantize_rows(x, layout)
    assert got.shape == ref.shape
    if not np.array_equal(got, ref):
        i = int(np.nonzero(got != ref)[0][0])
        pytest.fail(f"byte {i} of {ref.size}: gpu {got[i]} oracle {ref[i]}")


@pytest.mark.parametrize("rows,k", [(1, 32), (3, 96), (17, 2048), (5, 7168), (64, 8192), (1, 128256 // 32 * 32)])
@pytest.mark.parametrize("layout", [q8.Q8_LAYOUT_ACT, q8.Q8_LAYOUT_ROWS])
def test_random_rows(rows, k, layout):
    rng = np.random.default_rng(rows * 7 + k)
    x = rng.standard_normal((rows, k)).astype(np.float32)
    x *= (10.0 ** rng.uniform(-4, 4, size=(rows, 1))).astype(np.float32)
    _check(x, layout)


def test_row_stride():
    rng = np.random.default_rng(3)
    base = rng.standard_normal((7, 260)).astype(np.float32)
    xt = up(base)
    view = xt[:, :256]
    got = down(q8.quantize(view, q8.Q8_LAYOUT_ACT))
    assert np.array_equal(got, oracle.quantize_rows(base[:, :256], oracle.LAYOUT_ACT))


def _hand_blocks():
    path = os.path.join(os.path.dirname(__file__), "golden", "q8_quant_hand.txt")
    blocks = []
    for line in open(path):
        if line.startswith("x:"):
            v = np.zeros(32, np.float32)
            vals = np.array([float(t) for t in line[2:].split()], np.float32)
            v[: vals.size] = vals
            blocks.append(v)
    return blocks


def test_crafted_blocks():
    """Hand examples (ties, near-ties, subnormal fp16 scale, zero block), exact
    ties at many scales, +-0, one-hot blocks, and fp16-subnormal scales."""
    rng = np.random.default_rng(5)
    blocks = _hand_blocks()
    for e in range(-20, 12):
        d = np.float32(2.0 ** e)
        b = (rng.integers(-127, 127, 32).astype(np.float32) + np.float32(0.5)) * d
        b[0] = np.float32(127) * d
        blocks.append(b)
    blocks.append(-np.zeros(32, np.float32))
    oh = np.zeros(32, np.float32)
    oh[7] = -3.0
    blocks.append(oh)
    for amax in (1e-4, 3e-5, 6.1e-5, 8e-6):
        b = rng.uniform(-1, 1, 32).astype(np.float32) * np.float32(amax)
        blocks.append(b)
    x = np.stack(blocks).reshape(1, -1)
    for layout in (q8.Q8_LAYOUT_ACT, q8.Q8_LAYOUT_ROWS):
        _check(x, layout)


def test_full_size_inputs():
    """The single-GEMV weight and activation, and the largest prefill
    activation (2048 x 8192 with outlier channels)."""
    w = wl.weight(wl.SINGLE, 0, 2048, 2048)
    _check(w, q8.Q8_LAYOUT_ROWS)
    x = wl.activation(wl.SINGLE, 0, 1, 2048)
    _check(x, q8.Q8_LAYOUT_ACT)
    xp = wl.activation(wl.PREFILL, 2, 2048, 8192, outliers=True)
    _check(xp, q8.Q8_LAYOUT_ACT)
