"""Pins for the oracle's Q8_0 matmul (block terms, outputs, grouped experts).

Definition (pages): each block dot is an exact int32 sum of 32 int8 products,
scaled by the weight block's fp16 scale and the activation block's fp16
scale; block results are reduced per output row ("ferro" README, "How the iGPU
path is fast", item 1; "Ember packed Q8 decode" post: 32-value blocks with one
fp16 scale).  The oracle rounds each term once to fp32 and sums the terms in
fp64, rounding the sum once.

Pins: (1) the block-term identity t == fp32(s * Dw * Dx) evaluated in fp64,
with s from numpy's integer dot; (2) brute force: fp64 dequantize-then-matmul
on tiny shapes must lie within 2^-23 * sum|t| of the oracle; (3) closed forms:
a one-block row equals its term, one-hot weight rows pick one activation value
times a known factor, constant rows quantize to +-127; (4) permuting weight
rows permutes outputs; (5) grouped experts equal the single-row matmul of the
routed expert.
"""
import numpy as np
import pytest

import oracle


def _quant(x, layout):
    return oracle.quantize_rows(np.ascontiguousarray(x, np.float32), layout)


def _dequant(q, d, k):
    f = d.view(np.float16).astype(np.float64)
    return q.astype(np.float64) * np.repeat(f, 32, axis=1)


def _case(m, n, k, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k)).astype(np.float32)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    return _quant(x, oracle.LAYOUT_ACT), _quant(w, oracle.LAYOUT_ROWS)


@pytest.mark.parametrize("m,n,k", [(1, 8, 32), (3, 17, 64), (8, 64, 256), (5, 33, 96)])
def test_block_term_identity(m, n, k):
    xa, wr = _case(m, n, k, seed=m * 100 + n)
    s, t = oracle.block_terms(xa, m, wr, n, k)
    qx, dx = oracle.act_planes(xa, m, k)
    qw, dw = oracle.rows_planes(wr, n, k)
    nb = k // 32
    s_np = np.einsum("mbj,nbj->mnb", qx.reshape(m, nb, 32).astype(np.int64), qw.reshape(n, nb, 32).astype(np.int64))
    assert np.array_equal(s, s_np)
    fx = dx.view(np.float16).astype(np.float64)
    fw = dw.view(np.float16).astype(np.float64)
    t64 = s_np.astype(np.float64) * fw[None, :, :] * fx[:, None, :]  # exact: < 2^53
    assert np.array_equal(t, t64.astype(np.float32))


@pytest.mark.parametrize("m,n,k", [(1, 64, 32), (4, 40, 64), (8, 64, 256), (7, 9, 512)])
def test_bruteforce_fp64(m, n, k):
    xa, wr = _case(m, n, k, seed=7 + k)
    y, S = oracle.matmul(xa, m, wr, n, k)
    qx, dx = oracle.act_planes(xa, m, k)
    qw, dw = oracle.rows_planes(wr, n, k)
    X = _dequant(qx, dx, k)
    W = _dequant(qw, dw, k)
    y64 = X @ W.T
    mag = np.abs(X) @ np.abs(W).T
    err = np.abs(y.astype(np.float64) - y64)
    assert np.all(err <= 2.0 ** -23 * S + 2.0 ** -45 * mag)
    # S is the sum of |block terms|
    _, t = oracle.block_terms(xa, m, wr, n, k)
    assert np.allclose(S, np.abs(t.astype(np.float64)).sum(axis=2), rtol=1e-12, atol=0)
    # threads do not change results
    y4, S4 = oracle.matmul(xa, m, wr, n, k, threads=4)
    assert np.array_equal(y, y4) and np.array_equal(S, S4)


def test_single_block_equals_term():
    m, n, k = 6, 50, 32
    xa, wr = _case(m, n, k, seed=11)
    y, _ = oracle.matmul(xa, m, wr, n, k)
    _, t = oracle.block_terms(xa, m, wr, n, k)
    assert np.array_equal(y, t[:, :, 0])


def test_one_hot_rows():
    """W[n][c] = 1 if c == n else 0: each weight row has one non-zero block
    whose amax is 1, so d1 = fp32(1/127), the value quantizes to 127 and the
    stored scale is fp16(d1) = 0x2008 (tests/golden/fp16_boundaries.txt).
    Output n is then fp32(127 * qx[n] * 0x2008 * Dx[block of n]) exactly."""
    m, n, k = 3, 96, 128
    w = np.zeros((n, k), np.float32)
    w[np.arange(n), np.arange(n)] = 1.0
    rng = np.random.default_rng(12)
    x = rng.standard_normal((m, k)).astype(np.float32)
    xa, wr = _quant(x, oracle.LAYOUT_ACT), _quant(w, oracle.LAYOUT_ROWS)
    y, _ = oracle.matmul(xa, m, wr, n, k)
    qx, dx = oracle.act_planes(xa, m, k)
    d1 = float(np.array([0x2008], np.uint16).view(np.float16)[0])
    cols = np.arange(n)
    expect = (127.0 * qx[:, cols].astype(np.float64) * d1 * dx[:, cols // 32].view(np.float16).astype(np.float64))
    assert np.array_equal(y, expect.astype(np.float32))


def test_constant_rows():
    """W[n][:] = c_n != 0: every weight block quantizes to sign(c) * 127 with
    scale fp16(|c|/127), so output = sum_b fp32(127 sign(c) * sum_j qx_bj *
    Dw * Dx_b), each term exact in fp64 before its one rounding."""
    m, n, k = 4, 8, 256
    c = np.array([0.5, -0.02, 3.0, -7.25, 1e-3, 0.125, -0.375, 2.0], np.float32)
    w = np.repeat(c[:, None], k, axis=1)
    rng = np.random.default_rng(13)
    x = rng.standard_normal((m, k)).astype(np.float32)
    xa, wr = _quant(x, oracle.LAYOUT_ACT), _quant(w, oracle.LAYOUT_ROWS)
    qw, dw = oracle.rows_planes(wr, n, k)
    assert np.array_equal(np.abs(qw.astype(np.int32)), np.full((n, k), 127))
    assert np.array_equal(np.sign(qw[:, 0]), np.sign(c).astype(np.int8))
    assert np.array_equal(dw[:, 0], (np.abs(c) / np.float32(127)).astype(np.float16).view(np.uint16))
    y, _ = oracle.matmul(xa, m, wr, n, k)
    qx, dx = oracle.act_planes(xa, m, k)
    sx = qx.reshape(m, k // 32, 32).astype(np.int64).sum(axis=2)  # [m][b]
    fw = dw[:, 0].view(np.float16).astype(np.float64)
    fx = dx.view(np.float16).astype(np.float64)
    terms = (127.0 * np.sign(c).astype(np.float64)[None, :, None] * sx[:, None, :] * fw[None, :, None]
             * fx[:, None, :]).astype(np.float32)
    expect = terms.astype(np.float64).sum(axis=2).astype(np.float32)
    assert np.array_equal(y, expect)


def test_permuting_weight_rows_permutes_outputs():
    m, n, k = 5, 64, 256
    xa, wr = _case(m, n, k, seed=14)
    perm = np.random.default_rng(15).permutation(n)
    wp = wr.reshape(n, -1)[perm].reshape(-1)
    y, _ = oracle.matmul(xa, m, wr, n, k)
    yp, _ = oracle.matmul(xa, m, wp, n, k)
    assert np.array_equal(yp, y[:, perm])


def test_points_match_full():
    m, n, k = 4, 64, 512
    xa, wr = _case(m, n, k, seed=16)
    y, S = oracle.matmul(xa, m, wr, n, k)
    mi = np.array([0, 3, 2, 1, 3])
    ni = np.array([0, 63, 17, 5, 40])
    yp, Sp = oracle.matmul_points(xa, m, wr, n, k, mi, ni)
    assert np.array_equal(yp, y[mi, ni]) and np.array_equal(Sp, S[mi, ni])


@pytest.mark.parametrize("x_per_pair", [False, True])
def test_grouped_routes_each_pair(x_per_pair):
    tokens, topk, E, n, k = 5, 3, 7, 16, 64
    rng = np.random.default_rng(17)
    ids = np.stack([rng.permutation(E)[:topk] for _ in range(tokens)]).astype(np.int32)
    rows = tokens * topk if x_per_pair else tokens
    x = rng.standard_normal((rows, k)).astype(np.float32)
    xa = _quant(x, oracle.LAYOUT_ACT)
    ws = [(rng.standard_normal((n, k)) * 0.02).astype(np.float32) for _ in range(E)]
    wr = np.concatenate([_quant(w, oracle.LAYOUT_ROWS) for w in ws])
    stride = n * (k // 32) * 34
    y, S = oracle.grouped_matmul(xa, rows, x_per_pair, ids, wr, E, stride, n, k)
    qx, dx = oracle.act_planes(xa, rows, k)
    X = _dequant(qx, dx, k)
    for t in range(tokens):
        for j in range(topk):
            p = t * topk + j
            e = ids[t, j]
            xr = p if x_per_pair else t
            one = _quant(x[xr:xr + 1], oracle.LAYOUT_ACT)
            y1, _ = oracle.matmul(one, 1, wr[e * stride:(e + 1) * stride], n, k)
            assert np.array_equal(y[p], y1[0])
            qw, dw = oracle.rows_planes(wr[e * stride:(e + 1) * stride], n, k)
            y64 = _dequant(qw, dw, k) @ X[xr]
            assert np.all(np.abs(y[p] - y64) <= 2.0 ** -23 * S[p] + 1e-12)
