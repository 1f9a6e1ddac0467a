"""Decode GEMV (q8_matmul with m <= 8) against the oracle, and the invariance
contract: a row's output is bit-identical alone or in any batch of up to 8
rows, in any row order, in either weight layout, inside a larger (fused)
matrix, and across repeated calls ("ferro" README, "Exactness contract")."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from decode_q8_amd import q8
from tests.gpu_helpers import bits_equal, check_tol, down, quantize, ref_quantize, require_gpu, up, weights_packed

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _gemv(xq, m, w, layout, n, k):
    return down(q8.matmul(xq, m, w, layout, n, k))


def _case(m, n, k, seed):
    x = wl.activation(wl.BATCHED, seed, m, k)
    w = wl.weight(wl.BATCHED, seed, n, k)
    return x, w


# (n, k): one tile; several tiles and groups (split by group); ragged group
# count k = 7168; a matrix wide enough to run whole rows per wave.
SHAPES = [(64, 256), (192, 512), (512, 2048), (640, 7168), (65536, 256)]


@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("m", [1, 2, 3, 5, 8])
def test_parity_packed_and_rows(m, n, k):
    x, w = _case(m, n, k, seed=n + m)
    xq = quantize(x, q8.Q8_LAYOUT_ACT)
    wr, wp = weights_packed(w)
    y_ref, S = oracle.matmul(ref_quantize(x, oracle.LAYOUT_ACT), m, ref_quantize(w, oracle.LAYOUT_ROWS), n, k,
                             threads=8)
    yp = _gemv(xq, m, wp, q8.Q8_LAYOUT_PACKED, n, k)
    check_tol(yp, y_ref, S, f"packed m={m} n={n} k={k}")
    yr = _gemv(xq, m, wr, q8.Q8_LAYOUT_ROWS, n, k)
    assert bits_equal(yp, yr), "packed and row-contiguous layouts differ"


@pytest.mark.parametrize("n,k", [(1, 512), (50, 512), (100, 512), (1000, 512), (100, 4096), (1, 7168)])
def test_rows_layout_ragged_n(n, k):
    x, w = _case(3, n, k, seed=n)
    xq = quantize(x, q8.Q8_LAYOUT_ACT)
    wr = quantize(w, q8.Q8_LAYOUT_ROWS)
    y_ref, S = oracle.matmul(ref_quantize(x, oracle.LAYOUT_ACT), 3, ref_quantize(w, oracle.LAYOUT_ROWS), n, k)
    check_tol(_gemv(xq, 3, wr, q8.Q8_LAYOUT_ROWS, n, k), y_ref, S, f"rows n={n}")


@pytest.mark.parametrize("n,k", [(512, 2048), (65536, 256), (2048, 8192)])
def test_batch_invariance_and_permutation(n, k):
    x, w = _case(8, n, k, seed=7)
    _, wp = weights_packed(w)
    singles = np.stack([_gemv(quantize(x[i:i + 1], q8.Q8_LAYOUT_ACT), 1, wp, 1, n, k)[0] for i in range(8)])
    for m in (2, 4, 6, 8):
        ym = _gemv(quantize(x[:m], q8.Q8_LAYOUT_ACT), m, wp, 1, n, k)
        assert bits_equal(ym, singles[:m]), f"m={m}"
        perm = wl.permutation(wl.BATCHED, m)
        yp = _gemv(quantize(x[:m][perm], q8.Q8_LAYOUT_ACT), m, wp, 1, n, k)
        assert bits_equal(yp, ym[perm]), f"permuted m={m}"


def test_fused_matrix_rows_equal_parts():
    """Rows of a fused [W1; W2] matrix equal those of W1 and W2 alone, although
    the fused matrix runs whole rows per wave and the parts split by group."""
    k = 256
    x, w1 = _case(2, 512, k, seed=11)
    _, w2 = _case(2, 65536, k, seed=12)
    xq = quantize(x, q8.Q8_LAYOUT_ACT)
    _, p1 = weights_packed(w1)
    _, p2 = weights_packed(w2)
    _, pf = weights_packed(np.concatenate([w1, w2]))
    yf = _gemv(xq, 2, pf, 1, 512 + 65536, k)
    assert bits_equal(yf[:, :512], _gemv(xq, 2, p1, 1, 512, k))
    assert bits_equal(yf[:, 512:], _gemv(xq, 2, p2, 1, 65536, k))


def test_long_rows_wide_matrix_m8():
    """m = 8 with k = 8448 (33 groups, 5 segments) on a wide matrix: the group
    sums of a whole tile exceed 64 KB of LDS, so tiles are spread over two
    workgroups even though n / 64 >= 256."""
    m, n, k = 8, 16384, 8448
    assert q8.q8_matmul_workspace_bytes(m, n, k) > 0
    x, w = _case(m, n, k, seed=21)
    wr, wp = weights_packed(w)
    xq = quantize(x, q8.Q8_LAYOUT_ACT)
    y = _gemv(xq, m, wp, 1, n, k)
    rng = np.random.default_rng(21)
    mi, ni = rng.integers(0, m, 2048), rng.integers(0, n, 2048)
    y_ref, S = oracle.matmul_points(ref_quantize(x, oracle.LAYOUT_ACT), m, ref_quantize(w, oracle.LAYOUT_ROWS), n, k,
                                    mi, ni)
    check_tol(y[mi, ni], y_ref, S, "m=8 k=8448")
    for i in (0, 5):
        yi = _gemv(quantize(x[i:i + 1], q8.Q8_LAYOUT_ACT), 1, wp, 1, n, k)
        assert bits_equal(y[i:i + 1], yi)


def test_repeatable():
    x, w = _case(4, 2048, 8192, seed=13)
    xq = quantize(x, q8.Q8_LAYOUT_ACT)
    _, wp = weights_packed(w)
    a = _gemv(xq, 4, wp, 1, 2048, 8192)
    b = _gemv(xq, 4, wp, 1, 2048, 8192)
    assert bits_equal(a, b)


@pytest.mark.parametrize("n,k", [(64, 256), (512, 2048), (640, 7168), (2048, 8192), (65536, 256)])
@pytest.mark.parametrize("m", [1, 3, 4, 6, 7, 8])
def test_fused_quantization_bit_identical(m, n, k):
    """q8_quantize_matmul (quantization inside the GEMV) equals
    q8_quantize_rows + q8_matmul bitwise, in both layouts, with a row stride."""
    x, w = _case(m, n, k, seed=3 * n + m)
    wr, wp = weights_packed(w)
    xs = up(np.concatenate([x, np.zeros((m, 4), np.float32)], axis=1))
    ref = _gemv(quantize(x, q8.Q8_LAYOUT_ACT), m, wp, 1, n, k)
    for layout, wt in ((q8.Q8_LAYOUT_PACKED, wp), (q8.Q8_LAYOUT_ROWS, wr)):
        y = torch.empty((m, n), dtype=torch.float32, device="cuda")
        ws = q8.workspace(m, n, k)
        q8.q8_quantize_matmul(xs, k + 4, m, wt, layout, n, k, y, n, ws, 0 if ws is None else ws.numel())
        assert bits_equal(down(y), ref), f"layout {layout}"


def _half_integer_activations(m, k, seed):
    """Rows whose quotients x / d sit on or next to half-integers: per 32-value
    block a scale d0, the block maximum 127 * d0, and values (j + 0.5) * d0,
    (j + 0.5 +- 1e-4) * d0 and (j + 0.5 +- 3e-4) * d0 mixed with random ones --
    the cases where a fast reciprocal could round differently from the
    correctly rounded quotient."""
    rng = np.random.default_rng(seed)
    x = np.empty((m, k), np.float32)
    offs = np.array([0.0, 1e-4, -1e-4, 3e-4, -3e-4, 2.44140625e-4, -2.44140625e-4], np.float64)
    for r in range(m):
        for b in range(k // 32):
            d0 = float(rng.uniform(1e-3, 4.0))
            j = rng.integers(-127, 127, size=32)
            o = offs[rng.integers(0, len(offs), size=32)]
            v = (j + 0.5 + o) * d0
            v[rng.random(32) < 0.25] = rng.uniform(-127, 127, size=1) * d0
            v[rng.integers(0, 32)] = 127.0 * d0 * (1 if rng.random() < 0.5 else -1)
            x[r, 32 * b:32 * b + 32] = v.astype(np.float32)
    return x


@pytest.mark.parametrize("m", [1, 2, 4, 8])
def test_fused_quantization_half_integer_quotients(m):
    """The fused quantization equals the standalone quantizer bitwise where the
    quotients are exact or near half-integers (ties away from zero)."""
    n, k = 512, 2048
    x = _half_integer_activations(m, k, seed=77 + m)
    _, w = _case(m, n, k, seed=5 * m)
    _, wp = weights_packed(w)
    ref = _gemv(quantize(x, q8.Q8_LAYOUT_ACT), m, wp, 1, n, k)
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    ws = q8.workspace(m, n, k)
    q8.q8_quantize_matmul(up(x), k, m, wp, q8.Q8_LAYOUT_PACKED, n, k, y, n, ws, 0 if ws is None else ws.numel())
    assert bits_equal(down(y), ref)
    # and the standalone codes are the oracle's (ties away from zero)
    assert np.array_equal(down(quantize(x, q8.Q8_LAYOUT_ACT)), ref_quantize(x, q8.Q8_LAYOUT_ACT))


def _tie_neighbour_activations(m, k, seed):
    """Per 32-value block a scale d0 of 2^-120 .. 2^-90 (across the lower end
    2^-96 of the range where the fused path divides by a shared refined
    reciprocal; such blocks add 0 to y, since their fp16 scale is 0) or 2^-30
    .. 2^14 (inside it, where every code shows in y), the block maximum
    127 * d0, and values at the exact fp32 ties (j + 0.5) * d and 1 or 2 ulps
    to either side, where d = fp32(amax / 127) is the scale the quantizer
    computes: quotients that a division one ulp off would round the other way.
    (Larger scales overflow the fp16 scale and turn outputs into inf / NaN.)"""
    rng = np.random.default_rng(seed)
    x = np.empty((m, k), np.float32)
    exps = np.concatenate([np.arange(-120, -90), np.arange(-30, 15), np.arange(-30, 15)])
    for r in range(m):
        for b in range(k // 32):
            d0 = np.float32(rng.uniform(1.0, 2.0) * 2.0 ** int(rng.choice(exps)))
            amax = np.float32(127) * d0
            d = amax / np.float32(127)
            j = rng.integers(-127, 127, size=32).astype(np.float32)
            v = ((j + np.float32(0.5)) * d).astype(np.float32)
            for _ in range(2):
                step = rng.integers(-1, 2, size=32)
                v = np.where(step > 0, np.nextafter(v, np.float32(np.inf)),
                             np.where(step < 0, np.nextafter(v, np.float32(-np.inf)), v)).astype(np.float32)
            v = np.clip(v, -amax, amax)
            v[rng.integers(0, 32)] = amax if rng.random() < 0.5 else -amax
            x[r, 32 * b:32 * b + 32] = v
    return x


@pytest.mark.parametrize("m", [1, 2, 3, 8])
def test_fused_quantization_tie_neighbours_and_scale_range(m):
    """The fused quantization equals the standalone quantizer (IEEE division)
    bitwise on exact ties and their 1- and 2-ulp neighbours, at scales inside
    and outside the range where the fused path divides by a shared refined
    reciprocal; the standalone codes are the oracle's."""
    n, k = 256, 4096
    x = _tie_neighbour_activations(m, k, seed=91 + m)
    _, w = _case(m, n, k, seed=7 * m)
    _, wp = weights_packed(w)
    xq = quantize(x, q8.Q8_LAYOUT_ACT)
    assert np.array_equal(down(xq), ref_quantize(x, q8.Q8_LAYOUT_ACT))
    ref = _gemv(xq, m, wp, 1, n, k)
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    ws = q8.workspace(m, n, k)
    q8.q8_quantize_matmul(up(x), k, m, wp, q8.Q8_LAYOUT_PACKED, n, k, y, n, ws, 0 if ws is None else ws.numel())
    assert bits_equal(down(y), ref)


def test_ld_y_and_workspace_reuse():
    """Output row stride larger than n; one zeroed workspace reused by calls of
    different shapes and m leaves its tile counters at zero and gives the same
    bits as fresh workspaces."""
    k = 8192
    need = max(q8.q8_matmul_workspace_bytes(m, n, k) for m in (1, 3, 8) for n in (512, 2048))
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for m, n in ((3, 512), (1, 2048), (8, 512), (3, 2048)):
        x, w = _case(m, n, k, seed=14 + m + n)
        xq = quantize(x, q8.Q8_LAYOUT_ACT)
        _, wp = weights_packed(w)
        y = torch.full((m, n + 64), 7.0, dtype=torch.float32, device="cuda")
        q8.q8_matmul(xq, m, wp, 1, n, k, y, n + 64, ws, ws.numel())
        got = down(y)
        assert np.all(got[:, n:] == 7.0)
        assert bits_equal(got[:, :n], _gemv(xq, m, wp, 1, n, k))
        tiles = (n + 63) // 64
        assert not down(ws[: tiles * 4]).any(), "tile counters not left at zero"


def test_single_gemv_full_size():
    """The 2048 x 2048 single GEMV: every output against the oracle."""
    n = k = 2048
    w = wl.weight(wl.SINGLE, 0, n, k)
    x = wl.activation(wl.SINGLE, 0, 1, k)
    xq = quantize(x, q8.Q8_LAYOUT_ACT)
    wr, wp = weights_packed(w)
    y_ref, S = oracle.matmul(ref_quantize(x, oracle.LAYOUT_ACT), 1, ref_quantize(w, oracle.LAYOUT_ROWS), n, k,
                             threads=8)
    yp = _gemv(xq, 1, wp, 1, n, k)
    check_tol(yp, y_ref, S, "single 2048x2048")
    assert bits_equal(yp, _gemv(xq, 1, wr, 0, n, k))


@pytest.mark.parametrize("name,n,k", [m[:3] for m in wl.LLAMA_LAYER_MATS] + [wl.LLAMA_HEAD])
def test_decode_shapes_full_size_whole_output(name, n, k):
    """Full decode-step shapes (fused QKV, O, gate||up, down, LM head) at m = 1
    and m = 8: every output against the oracle; every row of the m = 8 batch
    bit-identical to its m = 1 run; both layouts bit-identical."""
    import os
    w = wl.weight(wl.BATCHED, 1000 + n + k, n, k)
    x = wl.activation(wl.BATCHED, 1000 + n + k, 8, k)
    wr, wp = weights_packed(w)
    wr_h = ref_quantize(w, oracle.LAYOUT_ROWS)
    y1 = None
    for m in (1, 8):
        xq = quantize(x[:m], q8.Q8_LAYOUT_ACT)
        y = _gemv(xq, m, wp, 1, n, k)
        y_ref, S = oracle.matmul(ref_quantize(x[:m], oracle.LAYOUT_ACT), m, wr_h, n, k,
                                 threads=min(16, os.cpu_count() or 1))
        check_tol(y, y_ref, S, f"{name} m={m}")
        if m == 1:
            y1 = y
            assert bits_equal(y, _gemv(xq, 1, wr, 0, n, k)), f"{name}: layouts differ"
        else:
            assert bits_equal(y[:1], y1)
            for i in range(1, 8):
                yi = _gemv(quantize(x[i:i + 1], q8.Q8_LAYOUT_ACT), 1, wp, 1, n, k)
                assert bits_equal(y[i:i + 1], yi), f"{name}: row {i} differs alone"
