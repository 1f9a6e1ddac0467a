"""Pins of the oracle's router, SwiGLU and combine (the steps either side of the
routed-expert GEMVs) and of its fixed exp algorithm, against things other than
themselves: Python's math.exp, brute-force orderings with sorted(), numpy fp64
softmax and SwiGLU, closed forms."""
import math

import numpy as np
import pytest

import oracle

F32_ULP = 2.0 ** -23


def _rng(seed):
    return np.random.default_rng(5000 + seed)


# ---- exp ---------------------------------------------------------------------

def test_exp_against_math_exp():
    """Within 4 fp64 ulps of math.exp over [-745, 0] (normal results), exact
    at 0, and within a few units of the last place for subnormal results."""
    xs = np.concatenate([-np.geomspace(1e-300, 708.0, 4000), -_rng(1).random(4000) * 708.0,
                         -np.arange(0, 709) * math.log(2.0), [0.0, -0.0, -1e-17, -0.5 * math.log(2.0)]])
    for x in xs:
        a, b = oracle.exp_nonpos(float(x)), math.exp(float(x))
        assert abs(a - b) <= 4 * math.ulp(b), (x, a, b)
    assert oracle.exp_nonpos(0.0) == 1.0
    for x in (-709.5, -720.0, -740.0, -745.0):
        a, b = oracle.exp_nonpos(x), math.exp(x)
        assert abs(a - b) <= 4 * 5e-324 + 4 * math.ulp(b), (x, a, b)
    assert oracle.exp_nonpos(-746.0) == 0.0 and oracle.exp_nonpos(-1e6) == 0.0


def test_exp_functional_equation():
    """e^(a+b) = e^a * e^b to a few fp64 ulps (independent of any library)."""
    g = _rng(2)
    for _ in range(2000):
        a, b = -g.random() * 300, -g.random() * 300
        lhs = oracle.exp_nonpos(a + b)
        rhs = oracle.exp_nonpos(a) * oracle.exp_nonpos(b)
        assert abs(lhs - rhs) <= 1e-13 * rhs + 1e-300


# ---- router ------------------------------------------------------------------

def _brute_topk(row, k):
    order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
    return order[:k]


@pytest.mark.parametrize("tokens,E,k", [(16, 256, 8), (5, 64, 6), (3, 7, 7), (4, 1000, 1), (2, 300, 13)])
def test_route_selection_is_topk(tokens, E, k):
    logits = _rng(tokens + E).random((tokens, E), dtype=np.float32)
    ids, _ = oracle.moe_route(logits, k)
    for t in range(tokens):
        assert list(ids[t]) == _brute_topk(logits[t], k)


def test_route_ties_go_to_lower_id():
    logits = np.zeros((2, 16), np.float32)
    logits[0, [3, 9, 12]] = 1.0          # a tie at the top
    logits[0, [1, 4]] = 0.5
    logits[1, :] = 0.25                  # everything tied
    ids, w = oracle.moe_route(logits, 5)
    assert list(ids[0]) == [3, 9, 12, 1, 4]
    assert list(ids[1]) == [0, 1, 2, 3, 4]
    assert np.all(w[1] == np.float32(0.2))  # equal weights: exp(0) / 5


def _softmax64(x):
    z = np.exp(x - x.max())
    return z / z.sum()


@pytest.mark.parametrize("normalize", [True, False])
def test_route_weights_against_numpy_softmax(normalize):
    tokens, E, k = 32, 256, 8
    logits = (_rng(7).standard_normal((tokens, E)) * 2.0).astype(np.float32)
    ids, w = oracle.moe_route(logits, k, normalize)
    for t in range(tokens):
        l64 = logits[t].astype(np.float64)
        if normalize:
            ref = _softmax64(l64[ids[t]])
        else:
            ref = _softmax64(l64)[ids[t]]
        # one fp32 rounding of a value correct to ~1e-15: within one fp32 ulp,
        # equal to numpy's rounding wherever it is not close to a tie
        r32 = ref.astype(np.float32)
        assert np.all(np.abs(w[t].astype(np.float64) - ref) <= np.spacing(r32).astype(np.float64))
        frac = np.abs(ref / np.spacing(r32).astype(np.float64) % 1.0 - 0.5)
        safe = frac < 0.49
        assert np.array_equal(w[t][safe], r32[safe])
        if normalize:
            assert abs(float(w[t].astype(np.float64).sum()) - 1.0) <= k * F32_ULP
        # slots in descending weight order
        assert np.all(np.diff(w[t]) <= 0)


def test_route_uniform_logits_closed_form():
    """Equal logits: normalize over k gives 1/k; over all experts gives 1/E."""
    logits = np.full((1, 128), 0.37, np.float32)
    _, w1 = oracle.moe_route(logits, 4, True)
    _, w0 = oracle.moe_route(logits, 4, False)
    assert np.all(w1 == np.float32(0.25)) and np.all(w0 == np.float32(1.0 / 128))


# ---- SwiGLU + quantization ----------------------------------------------------

def test_swiglu_against_fp64_numpy():
    """h = fp32(silu(g) * u) from numpy's fp64 exp, then the pinned quantizer:
    codes equal wherever h agrees; every h within one fp32 ulp of the fp64
    value, so every code within one step."""
    rows, n = 16, 2048
    g = _rng(11)
    gate = (g.standard_normal((rows, n)) * 3.0).astype(np.float32)
    up = g.standard_normal((rows, n)).astype(np.float32)
    q = oracle.swiglu_quantize(gate, up)
    g64, u64 = gate.astype(np.float64), up.astype(np.float64)
    h64 = g64 / (1.0 + np.exp(-g64)) * u64
    h32 = h64.astype(np.float32)
    q_ref = oracle.quantize_rows(h32, oracle.LAYOUT_ACT)
    qi, sc = oracle.act_planes(q, rows, n)
    qi_r, sc_r = oracle.act_planes(q_ref, rows, n)
    assert np.abs(qi.astype(int) - qi_r.astype(int)).max() <= 1
    # blocks whose fp32 values are all far from rounding ties must match exactly
    near = np.abs(h64 / np.spacing(h32).astype(np.float64) % 1.0 - 0.5) > 0.499
    blocks_safe = ~near.reshape(rows, n // 32, 32).any(axis=2)
    assert blocks_safe.mean() > 0.9
    qb, qb_r = qi.reshape(rows, n // 32, 32), qi_r.reshape(rows, n // 32, 32)
    assert np.array_equal(qb[blocks_safe], qb_r[blocks_safe])
    assert np.array_equal(sc[blocks_safe], sc_r[blocks_safe])


def test_swiglu_closed_forms():
    n = 64
    gate = np.zeros((3, n), np.float32)
    up = np.ones((3, n), np.float32)
    gate[1] = 1000.0       # e^-g underflows: silu(g) = g exactly
    up[1] = np.linspace(-2, 2, n, dtype=np.float32)
    gate[2] = -1000.0      # e^g underflows: silu(g) = -0
    q = oracle.swiglu_quantize(gate, up)
    qi, sc = oracle.act_planes(q, 3, n)
    assert (qi[0] == 0).all() and (sc[0] == 0).all()
    assert (qi[2] == 0).all() and (sc[2] == 0).all()
    assert np.array_equal(q[n:2 * n].view(np.int8),
                          oracle.act_planes(oracle.quantize_rows(gate[1:2] * up[1:2], oracle.LAYOUT_ACT), 1, n)[0][0])


def test_swiglu_sign_identity():
    """silu(g) - silu(-g) = g: with u = 1, h(g) - h(-g) equals g to fp32
    rounding; checked through the codes of paired rows with a shared scale."""
    n = 256
    g = _rng(12).standard_normal((1, n)).astype(np.float32)
    q_pos = oracle.swiglu_quantize(g, np.ones_like(g))
    q_neg = oracle.swiglu_quantize(-g, np.ones_like(g))
    qp, sp = oracle.act_planes(q_pos, 1, n)
    qn, sn = oracle.act_planes(q_neg, 1, n)
    dp, dn = oracle.f16_bits_to_f32(sp)[0], oracle.f16_bits_to_f32(sn)[0]
    recon = (qp[0].reshape(-1, 32) * dp[:, None]) - (qn[0].reshape(-1, 32) * dn[:, None])
    bound = 0.5 * (dp + dn)[:, None] * 1.01 + 1e-6
    assert np.all(np.abs(recon - g[0].reshape(-1, 32)) <= bound)


# ---- combine -----------------------------------------------------------------

def test_combine_against_fp64_and_one_hot():
    tokens, k, n = 6, 4, 96
    g = _rng(13)
    y = g.standard_normal((tokens * k, n)).astype(np.float32)
    w = g.random((tokens, k)).astype(np.float32)
    out, S = oracle.moe_combine(y, w)
    ref = (w.astype(np.float64)[:, :, None] * y.reshape(tokens, k, n).astype(np.float64)).sum(axis=1)
    assert np.all(np.abs(out - ref) <= np.abs(np.spacing(ref.astype(np.float32))))
    assert np.allclose(S, np.abs(w.astype(np.float64)[:, :, None] * y.reshape(tokens, k, n)).sum(axis=1))
    one = np.zeros((tokens, k), np.float32)
    one[np.arange(tokens), np.arange(tokens) % k] = 1.0
    out1, _ = oracle.moe_combine(y, one)
    assert np.array_equal(out1, y.reshape(tokens, k, n)[np.arange(tokens), np.arange(tokens) % k])
