"""q8_rmsnorm_quantize (residual add + RMSNorm + Q8_0 quantization in one
pass) against the oracle: codes, scales and the updated residual bit-exact,
for every residual mode, ragged and maximum k, edge-case rows, and the full
prefill row counts; the codes feed q8_matmul like any quantized input."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from decode_q8_amd import q8
from tests.gpu_helpers import bits_equal, check_tol, dev, down, ref_quantize, require_gpu, up, weights_packed

pytestmark = pytest.mark.gpu

EPS = wl.NORM_EPS


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _gpu_norm(x, res, gain, eps=EPS, mode="out"):
    """mode: 'out' (separate residual_out), 'in_place' (residual updated),
    'on_x' (result written over x), 'none' (residual_out NULL)."""
    rows, k = x.shape
    xt = up(x)
    rt = None if res is None else up(res)
    gt = up(gain)
    q = torch.full((q8.q8_quantized_bytes(rows, k),), 0xAB, dtype=torch.uint8, device=dev())
    ro = {"out": torch.full((rows, k), float("nan"), dtype=torch.float32, device=dev()),
          "in_place": rt, "on_x": xt, "none": None}[mode]
    print(f"q8_rmsnorm_quantize rows={rows} k={k} mode={mode} residual={res is not None}", flush=True)
    q8.q8_rmsnorm_quantize(xt, rt, ro, gt, rows, k, eps, q)
    return down(q), (None if ro is None else down(ro))


def _check(x, res, gain, eps=EPS, mode="out"):
    q, ro = _gpu_norm(x, res, gain, eps, mode)
    ro_ref, q_ref = oracle.rmsnorm_quantize(x, res, gain, eps)
    rows, k = x.shape
    if not np.array_equal(q, q_ref):
        qi, sc = oracle.act_planes(q, rows, k)
        qi_r, sc_r = oracle.act_planes(q_ref, rows, k)
        bad_rows = np.nonzero((qi != qi_r).any(axis=1) | (sc != sc_r).any(axis=1))[0]
        pytest.fail(f"codes/scales differ in {bad_rows.size} rows, first {bad_rows[:5]}")
    if ro is not None:
        assert bits_equal(ro, ro_ref), "residual_out"
    return q


@pytest.mark.parametrize("rows,k", [(1, 32), (1, 2048), (3, 2080), (2, 1056), (5, 7168), (2, 16384), (64, 4096),
                                    (7, 1024), (9, 15360)])
def test_parity_with_residual(rows, k):
    x, res, gain = wl.norm_inputs(wl.NORM, rows + k, rows, k)
    _check(x, res, gain)


@pytest.mark.parametrize("mode", ["in_place", "on_x", "none"])
def test_residual_modes(mode):
    rows, k = 6, 2048
    x, res, gain = wl.norm_inputs(wl.NORM, 77, rows, k)
    _check(x, res, gain, mode=mode)


def test_no_residual():
    rows, k = 4, 7168
    x, _, gain = wl.norm_inputs(wl.NORM, 78, rows, k)
    _check(x, None, gain)
    _check(x, None, gain, mode="on_x")


def test_edge_rows():
    """Zero rows (all blocks zero, +0 scales), a constant row (all +-127), tiny
    values (subnormal fp16 scales after the norm's gain is tiny), a row with
    one huge value, and eps = 0."""
    k = 2048
    x = np.zeros((6, k), np.float32)
    res = np.zeros((6, k), np.float32)
    x[1] = 3.0
    x[2] = np.linspace(-1, 1, k, dtype=np.float32)
    x[3, 17] = 1e30
    x[3, 18] = -1.0
    x[4] = np.float32(1e-30)
    x[5] = wl.activation(wl.NORM, 90, 1, k)[0]
    gain = np.ones(k, np.float32)
    gain[:32] = np.float32(1e-4)   # block 0: scales in fp16's subnormal range
    gain[32:64] = np.float32(1e-6)  # block 1: scales that round to zero in fp16
    gain[100::7] = np.float32(1e-6)
    _check(x, res, gain)
    # eps = 0 (not on the zero row, whose norm would divide by zero)
    _check(x[1:], res[1:], gain, eps=0.0)


def test_prefill_rows_full():
    """The full prefill row counts, every code and scale compared."""
    for rows in wl.NORM_ROWS:
        x, res, gain = wl.norm_inputs(wl.NORM, rows, rows, wl.LLAMA_HIDDEN)
        _check(x, res, gain)
    x, res, gain = wl.norm_inputs(wl.NORM, 9, 128, wl.MOE_HIDDEN)
    _check(x, res, gain)


def test_row_independent_of_batch():
    """A row's codes and residual do not depend on the other rows."""
    rows, k = 40, 2048
    x, res, gain = wl.norm_inputs(wl.NORM, 41, rows, k)
    q_all, ro_all = _gpu_norm(x, res, gain)
    qi, sc = oracle.act_planes(q_all, rows, k)
    for i in (0, 17, 39):
        q1, ro1 = _gpu_norm(x[i:i + 1], res[i:i + 1], gain)
        qi1, sc1 = oracle.act_planes(q1, 1, k)
        assert np.array_equal(qi1[0], qi[i]) and np.array_equal(sc1[0], sc[i])
        assert bits_equal(ro1[0], ro_all[i])


def test_codes_feed_the_gemv():
    """The producer's output is a q8_matmul input: the decode GEMV on it meets
    the oracle bound against the oracle's own codes."""
    rows, k, n = 4, 2048, 3072
    x, res, gain = wl.norm_inputs(wl.NORM, 55, rows, k)
    xt, rt, gt = up(x), up(res), up(gain)
    qt = q8.rmsnorm_quantize(xt, rt, gt, EPS)
    w = wl.weight(wl.NORM, 55, n, k)
    _, wp = weights_packed(w)
    y = down(q8.matmul(qt, rows, wp, q8.Q8_LAYOUT_PACKED, n, k))
    _, q_ref = oracle.rmsnorm_quantize(x, res, gain, EPS)
    y_ref, S = oracle.matmul(q_ref, rows, ref_quantize(w, oracle.LAYOUT_ROWS), n, k)
    check_tol(y, y_ref, S, "norm -> GEMV")
    assert bits_equal(down(rt), (res + x).astype(np.float32))
