"""The seeded input generator: determinism, shapes and the routing recipe."""
import numpy as np

import workloads as wl


def test_determinism_and_independence():
    a = wl.weight(wl.SINGLE, 0, 64, 256)
    b = wl.weight(wl.SINGLE, 0, 64, 256)
    c = wl.weight(wl.SINGLE, 1, 64, 256)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert a.dtype == np.float32 and abs(float(a.std()) - 0.02) < 0.002


def test_outliers():
    x = wl.activation(wl.PREFILL, 0, 4, 2048, outliers=True)
    base = wl.activation(wl.PREFILL, 0, 4, 2048)
    cols = wl.outlier_channels(wl.PREFILL, 0, 2048)
    assert cols.size == 20 and np.unique(cols).size == 20
    ratio = x[:, cols] / base[:, cols]
    assert np.allclose(ratio, 20.0)
    rest = np.setdiff1d(np.arange(2048), cols)
    assert np.array_equal(x[:, rest], base[:, rest])
    assert wl.outlier_channels(wl.PREFILL, 0, 8192).size == 82


def test_routing_is_topk_of_uniform_logits():
    ids = wl.routing(wl.MOE, wl.MOE_TOKENS, wl.MOE_EXPERTS, wl.MOE_TOPK)
    assert ids.shape == (16, 8) and ids.dtype == np.int32
    logits = wl.generator(wl.MOE, (wl.TAG_ROUTE, 0, 0)).random((16, 256), dtype=np.float32)
    for t in range(16):
        full = sorted(range(256), key=lambda e: (-logits[t, e], e))[:8]
        assert list(ids[t]) == full
    # expected number of distinct experts under uniform routing: 256 (1 - (1 - 8/256)^16)
    expect = 256 * (1 - (1 - 8 / 256) ** 16)
    assert abs(expect - 101.96) < 0.01
    assert 70 <= np.unique(ids).size <= 128


def test_decode_byte_count():
    assert wl.decode_weight_bytes() == 1312980992
    assert len(wl.decode_matrices()) == 16 * 4 + 1
