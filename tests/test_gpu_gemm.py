"""Prefill GEMM (q8_matmul with m > 8, int8 MFMA) against the oracle, and its
row invariance: a row's output does not depend on m or on the row order."""
import os

import numpy as np
import pytest

import oracle
import workloads as wl
from decode_q8_amd import q8
from tests.gpu_helpers import bits_equal, check_tol, down, quantize, ref_quantize, require_gpu, weights_packed

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _gemm(xq, m, wp, n, k):
    return down(q8.matmul(xq, m, wp, q8.Q8_LAYOUT_PACKED, n, k))


@pytest.mark.parametrize("m,n,k", [(9, 64, 256), (32, 128, 256), (40, 192, 512), (24, 64, 768), (130, 256, 2048),
                                   (136, 128, 1280), (188, 320, 1024), (257, 128, 7168)])
def test_parity(m, n, k):
    x = wl.activation(wl.PREFILL, 50 + m, m, k, outliers=True)
    w = wl.weight(wl.PREFILL, 50 + n, n, k)
    xq = quantize(x, q8.Q8_LAYOUT_ACT)
    wr, wp = weights_packed(w)
    y_ref, S = oracle.matmul(ref_quantize(x, oracle.LAYOUT_ACT), m, ref_quantize(w, oracle.LAYOUT_ROWS), n, k,
                             threads=8)
    check_tol(_gemm(xq, m, wp, n, k), y_ref, S, f"gemm m={m} n={n} k={k}")


def test_row_invariance_across_m_and_order():
    n, k = 256, 2048
    x = wl.activation(wl.PREFILL, 60, 752, k, outliers=True)
    _, wp = weights_packed(wl.weight(wl.PREFILL, 60, n, k))
    y752 = _gemm(quantize(x, q8.Q8_LAYOUT_ACT), 752, wp, n, k)
    y188 = _gemm(quantize(x[:188], q8.Q8_LAYOUT_ACT), 188, wp, n, k)
    assert bits_equal(y188, y752[:188])
    y9 = _gemm(quantize(x[100:109], q8.Q8_LAYOUT_ACT), 9, wp, n, k)
    assert bits_equal(y9, y752[100:109])
    perm = wl.permutation(wl.PREFILL, 188)
    yp = _gemm(quantize(x[:188][perm], q8.Q8_LAYOUT_ACT), 188, wp, n, k)
    assert bits_equal(yp, y188[perm])


def test_row_invariance_across_tile_shapes():
    """m = 1024 on n = 4096 runs 128 x 128 workgroups, m = 100 the k-split
    strip kernel: the rows they share are still bit-identical."""
    n, k = 4096, 512
    x = wl.activation(wl.PREFILL, 61, 1024, k, outliers=True)
    _, wp = weights_packed(wl.weight(wl.PREFILL, 61, n, k))
    y_big = _gemm(quantize(x, q8.Q8_LAYOUT_ACT), 1024, wp, n, k)
    y_small = _gemm(quantize(x[900:1000], q8.Q8_LAYOUT_ACT), 100, wp, n, k)
    assert bits_equal(y_small, y_big[900:1000])


THREADS = min(16, os.cpu_count() or 1)


@pytest.mark.parametrize("m", wl.PREFILL_M)
@pytest.mark.parametrize("n,k", wl.PREFILL_NK)
def test_prefill_full_size_whole_output(m, n, k):
    """Every prefill configuration at full size, every output against the
    oracle.  m = 2048 and 752 x 8192 run the 128 x 128 tiled kernel, the rest
    the k-split strip kernel."""
    x = wl.activation(wl.PREFILL, m, m, k, outliers=True)
    w = wl.weight(wl.PREFILL, n + k, n, k)
    xq = quantize(x, q8.Q8_LAYOUT_ACT)
    wr, wp = weights_packed(w)
    y = _gemm(xq, m, wp, n, k)
    y_ref, S = oracle.matmul(ref_quantize(x, oracle.LAYOUT_ACT), m, ref_quantize(w, oracle.LAYOUT_ROWS), n, k,
                             threads=THREADS)
    check_tol(y, y_ref, S, f"prefill m={m} n={n} k={k}")


@pytest.mark.parametrize("m,n,k", [(2048, 2112, 2048), (1100, 4160, 512)])
def test_tiled_ragged_n_whole_output(m, n, k):
    """Tiled kernel with an odd number of 64-row weight tiles (n / 64 = 33 and
    65): the last workgroup column holds one real tile and reloads it for its
    second; every output against the oracle, and the columns past n are never
    written (checked through a wider output stride)."""
    import torch
    x = wl.activation(wl.PREFILL, 70 + m, m, k, outliers=True)
    w = wl.weight(wl.PREFILL, 70 + n, n, k)
    xq = quantize(x, q8.Q8_LAYOUT_ACT)
    _, wp = weights_packed(w)
    ld = n + 64
    yt = torch.full((m, ld), 7.0, dtype=torch.float32, device="cuda")
    q8.q8_matmul(xq, m, wp, q8.Q8_LAYOUT_PACKED, n, k, yt, ld)
    yfull = down(yt)
    assert np.all(yfull[:, n:] == 7.0), "columns past n were written"
    y_ref, S = oracle.matmul(ref_quantize(x, oracle.LAYOUT_ACT), m, ref_quantize(w, oracle.LAYOUT_ROWS), n, k,
                             threads=THREADS)
    check_tol(yfull[:, :n], y_ref, S, f"ragged tiled m={m} n={n} k={k}")


@pytest.mark.parametrize("m,n,k", [(2048, 2048, 256), (2048, 2048, 768), (2053, 2048, 1280)])
def test_tiled_short_and_odd_k_whole_output(m, n, k):
    """Tiled kernel with fewer stages than its four stage buffers (k = 256: two
    stages, so the first wait is for every load issued) and with an odd number
    of 256-value groups (k = 768, 1280: the loop leaves after the first group of
    its two-group body), and a row count that is not a multiple of 128: every
    output against the oracle, and the rows are bit-identical to the strip
    kernel's (the same rows computed inside a small problem)."""
    x = wl.activation(wl.PREFILL, 90 + k, m, k, outliers=True)
    w = wl.weight(wl.PREFILL, 90 + n, n, k)
    xq = quantize(x, q8.Q8_LAYOUT_ACT)
    _, wp = weights_packed(w)
    y = _gemm(xq, m, wp, n, k)
    y_ref, S = oracle.matmul(ref_quantize(x, oracle.LAYOUT_ACT), m, ref_quantize(w, oracle.LAYOUT_ROWS), n, k,
                             threads=THREADS)
    check_tol(y, y_ref, S, f"tiled m={m} n={n} k={k}")
    rows = [0, 1, 2, 127, 128, 129, 500, 1000, 1500, 2000, m - 2, m - 1]
    ys = _gemm(quantize(x[rows], q8.Q8_LAYOUT_ACT), len(rows), wp, n, k)  # 12 rows (> 8: GEMM): strip kernel
    assert bits_equal(ys, y[rows]), "tiled and strip kernels differ"
