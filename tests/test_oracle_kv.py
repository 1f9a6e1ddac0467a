"""Pins of the oracle's Q8 KV cache: the fused norm + rope + cache write and
the decode attention over the quantized cache, against numpy fp64 rotation,
norm and softmax attention, closed forms and the pinned block quantizer."""
import math

import numpy as np
import pytest

import oracle
import workloads as wl

U = 2.0 ** -24


def _rng(seed):
    return np.random.default_rng(7000 + seed)


def _identity_tables(P, hd):
    return np.ones((P, hd // 2), np.float32), np.zeros((P, hd // 2), np.float32)


def _write(qkv, H, Hk, hd, pos, tabs, qg=None, kg=None, slots=None, n_slots=None, eps=1e-6):
    T = qkv.shape[0]
    slots = np.arange(T, dtype=np.int32) if slots is None else slots
    n_slots = T if n_slots is None else n_slots
    return oracle.kv_write(qkv, H, Hk, hd, pos, tabs[0], tabs[1], qg, kg, eps, slots, n_slots)


@pytest.mark.parametrize("hd", [64, 128])
def test_write_identity_rotation_quantizes_raw_rows(hd):
    """cos = 1, sin = 0 and no norm: q passes through; K and V codes are the
    pinned quantizer's codes of the raw rows, scales fp32(amax / 127)."""
    H, Hk, T = 4, 2, 5
    qkv = _rng(hd).standard_normal((T, (H + 2 * Hk) * hd)).astype(np.float32)
    q, kc, ks, vc, vs = _write(qkv, H, Hk, hd, np.zeros(T, np.int32), _identity_tables(1, hd))
    assert np.array_equal(q.reshape(T, -1), qkv[:, :H * hd])
    for cache, scale, off in ((kc, ks, H * hd), (vc, vs, (H + Hk) * hd)):
        rows = qkv[:, off:off + Hk * hd].reshape(T, Hk, hd).transpose(1, 0, 2).reshape(Hk * T, hd)
        codes, _ = oracle.act_planes(oracle.quantize_rows(rows, oracle.LAYOUT_ACT), T * Hk, hd)
        assert np.array_equal(cache.reshape(Hk * T, hd), codes)
        amax = np.abs(rows.reshape(T * Hk, hd // 32, 32)).max(axis=2)
        assert np.array_equal(scale.reshape(Hk * T, hd // 32), (amax / np.float32(127.0)).astype(np.float32))


def test_write_rope_against_fp64_rotation():
    """Rotation in the half-split layout: within 2 fp32 ulps of numpy's fp64
    rotation by the same fp32 table entries; pair norms preserved."""
    H, Hk, hd, T = 2, 1, 64, 9
    cos_t, sin_t = wl.rope_tables(4096, hd)
    pos = np.array([0, 1, 2, 17, 100, 1000, 2047, 3000, 4095], np.int32)
    qkv = _rng(1).standard_normal((T, (H + 2 * Hk) * hd)).astype(np.float32)
    q, *_ = _write(qkv, H, Hk, hd, pos, (cos_t, sin_t))
    x = qkv[:, :H * hd].reshape(T, H, hd).astype(np.float64)
    c = cos_t[pos].astype(np.float64)[:, None, :]
    s = sin_t[pos].astype(np.float64)[:, None, :]
    a, b = x[..., :hd // 2], x[..., hd // 2:]
    ref = np.concatenate([a * c - b * s, b * c + a * s], axis=-1)
    tol = 2 * np.abs(np.spacing(ref.astype(np.float32))).astype(np.float64) + 4 * U * (np.abs(a) + np.abs(b)).repeat(2, -1).reshape(ref.shape)
    assert np.all(np.abs(q - ref) <= tol)
    qa, qb = q[..., :hd // 2].astype(np.float64), q[..., hd // 2:].astype(np.float64)
    assert np.allclose(qa * qa + qb * qb, a * a + b * b, rtol=1e-5, atol=1e-6)
    assert np.array_equal(q[0].reshape(-1), qkv[0, :H * hd])  # position 0: cos 1, sin 0


def test_write_head_norm_against_fp64():
    H, Hk, hd, T = 3, 1, 128, 4
    g = _rng(2)
    qkv = (g.standard_normal((T, (H + 2 * Hk) * hd)) * 3).astype(np.float32)
    qg = (1 + 0.1 * g.standard_normal(hd)).astype(np.float32)
    q, *_ = _write(qkv, H, Hk, hd, np.zeros(T, np.int32), _identity_tables(1, hd), qg=qg, eps=1e-6)
    x = qkv[:, :H * hd].reshape(T, H, hd).astype(np.float64)
    ref = x / np.sqrt((x * x).mean(-1, keepdims=True) + 1e-6) * qg.astype(np.float64)
    assert np.all(np.abs(q - ref) <= 3 * np.abs(np.spacing(ref.astype(np.float32))))
    # power-of-two scaling with eps = 0 leaves the normalized head unchanged
    q0, *_ = _write(qkv, H, Hk, hd, np.zeros(T, np.int32), _identity_tables(1, hd), qg=qg, eps=0.0)
    q1, *_ = _write(qkv * np.float32(8.0), H, Hk, hd, np.zeros(T, np.int32), _identity_tables(1, hd), qg=qg, eps=0.0)
    assert np.array_equal(q0, q1)


def test_write_layout_and_slots():
    """Head h of the qkv row lands in head h of q_out; key head j and value
    head j of token t land in cache slot slots[t]; other slots stay zero."""
    H, Hk, hd, T = 4, 2, 64, 3
    qkv = np.zeros((T, (H + 2 * Hk) * hd), np.float32)
    for t in range(T):
        for h in range(H + 2 * Hk):
            qkv[t, h * hd:(h + 1) * hd] = 10 * t + h + 1
    slots = np.array([5, 0, 9], np.int32)
    q, kc, ks, vc, vs = _write(qkv, H, Hk, hd, np.zeros(T, np.int32), _identity_tables(1, hd), slots=slots,
                               n_slots=12)
    for t in range(T):
        for h in range(H):
            assert np.all(q[t, h] == 10 * t + h + 1)
        for j in range(Hk):
            assert np.all(kc[j, slots[t]] == 127) and np.all(vc[j, slots[t]] == 127)
            assert np.all(ks[j, slots[t]] == np.float32(10 * t + H + j + 1) / np.float32(127))
            assert np.all(vs[j, slots[t]] == np.float32(10 * t + H + Hk + j + 1) / np.float32(127))
    unused = [i for i in range(12) if i not in slots]
    assert not kc[:, unused].any() and not vs[:, unused].any()


def _cache(seed, slots, Hk, hd, scale_v=1.0):
    """A random head-major cache: int8 [Hk][slots][hd], fp32 scales [Hk][slots][hd/32]."""
    g = _rng(seed)
    kc = g.integers(-127, 128, (Hk, slots, hd)).astype(np.int8)
    vc = g.integers(-127, 128, (Hk, slots, hd)).astype(np.int8)
    ks = (g.random((Hk, slots, hd // 32)) * 0.02).astype(np.float32)
    vs = (g.random((Hk, slots, hd // 32)) * 0.02 * scale_v).astype(np.float32)
    return kc, ks, vc, vs


def _numpy_attention(q, kc, ks, vc, vs, base, length, scale):
    S, H, hd = q.shape
    G = H // kc.shape[0]
    out = np.empty((S, H, hd))
    for s in range(S):
        sl = slice(base[s], base[s] + length[s])
        for h in range(H):
            k = kc[h // G, sl].astype(np.float64) * np.repeat(ks[h // G, sl].astype(np.float64), 32, axis=1)
            v = vc[h // G, sl].astype(np.float64) * np.repeat(vs[h // G, sl].astype(np.float64), 32, axis=1)
            sc = scale * (k @ q[s, h].astype(np.float64))
            p = np.exp(sc - sc.max())
            out[s, h] = (p[:, None] * v).sum(0) / p.sum()
    return out


@pytest.mark.parametrize("hd,H,Hk", [(64, 8, 2), (128, 4, 4), (64, 32, 8)])
def test_attention_against_numpy(hd, H, Hk):
    S = 3
    length = np.array([1, 37, 300], np.int32)
    base = np.array([0, 1, 38], np.int32)
    kc, ks, vc, vs = _cache(hd + H, 400, Hk, hd)
    q = _rng(hd).standard_normal((S, H, hd)).astype(np.float32)
    out, bound = oracle.attention_decode(q, kc, ks, vc, vs, base, length, 1 / math.sqrt(hd))
    ref = _numpy_attention(q, kc, ks, vc, vs, base, length, float(np.float32(1 / math.sqrt(hd))))  # the fp32 scale
    assert np.all(np.abs(out - ref) <= np.abs(np.spacing(ref.astype(np.float32))))
    assert np.all(bound >= 0) and np.all(bound[out != 0] > 0)


def test_attention_closed_forms():
    hd, H, Hk = 64, 4, 2
    kc, ks, vc, vs = _cache(5, 64, Hk, hd)
    q = _rng(5).standard_normal((2, H, hd)).astype(np.float32)
    # one key: the output is that key's value row, dequantized
    out, _ = oracle.attention_decode(q, kc, ks, vc, vs, np.array([10, 20], np.int32), np.array([1, 1], np.int32), 0.125)
    for s, slot in ((0, 10), (1, 20)):
        for h in range(H):
            v = (vc[h // 2, slot].astype(np.float64) * np.repeat(vs[h // 2, slot], 32)).astype(np.float32)
            assert np.array_equal(out[s, h], v)
    # scale 0: uniform weights, the mean of the value rows
    out0, _ = oracle.attention_decode(q, kc, ks, vc, vs, np.array([0, 0], np.int32), np.array([64, 7], np.int32), 0.0)
    for s, L in ((0, 64), (1, 7)):
        v = vc[:, :L].astype(np.float64) * np.repeat(vs[:, :L], 32, axis=2)
        for h in range(H):
            assert np.allclose(out0[s, h], v[h // 2].mean(0), rtol=1e-6, atol=1e-9)


def test_attention_fp32_evaluation_within_bound():
    """A straightforward fp32 evaluation (fp32 dots, exp, sequential fp32 sums)
    stays inside the oracle's error budget."""
    hd, H, Hk, L = 64, 4, 1, 700
    kc, ks, vc, vs = _cache(9, L, Hk, hd)
    q = (_rng(9).standard_normal((1, H, hd)) * 4).astype(np.float32)
    scale = np.float32(1 / 8)
    out, bound = oracle.attention_decode(q, kc, ks, vc, vs, np.array([0], np.int32), np.array([L], np.int32), scale)
    k = (kc[0].astype(np.float32) * np.repeat(ks[0], 32, axis=1)).astype(np.float32)
    v = (vc[0].astype(np.float32) * np.repeat(vs[0], 32, axis=1)).astype(np.float32)
    for h in range(H):
        sc = np.array([np.float32(scale) * np.float32(np.dot(k[j], q[0, h])) for j in range(L)], np.float32)
        p = np.exp(sc - sc.max()).astype(np.float32)
        acc = np.zeros(hd, np.float32)
        l = np.float32(0)
        for j in range(L):
            acc = (acc + p[j] * v[j]).astype(np.float32)
            l = np.float32(l + p[j])
        o32 = acc / l
        assert np.all(np.abs(o32.astype(np.float64) - out[0, h].astype(np.float64)) <= bound[0, h] + np.abs(np.spacing(out[0, h])))
