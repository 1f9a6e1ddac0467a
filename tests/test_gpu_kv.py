"""Q8 KV cache on the device against the oracle: the fused norm + rope +
cache write (rotated queries, int8 codes and fp32 scales bit-exact) and the
decode attention over the quantized cache (within the oracle's fp32 error
budget, bit-identical whatever the other sequences of the batch)."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from decode_q8_amd import q8
from tests.gpu_helpers import bits_equal, dev, down, require_gpu, up

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _i32(a):
    return up(np.ascontiguousarray(a, np.int32))


def _gpu_write(qkv, H, Hk, hd, pos, tabs, qg, kg, eps, slots, n_slots, caches=None):
    T = qkv.shape[0]
    if caches is None:
        caches = (torch.zeros((Hk, n_slots, hd), dtype=torch.int8, device=dev()),
                  torch.zeros((Hk, n_slots, hd // 32), dtype=torch.float32, device=dev()),
                  torch.zeros((Hk, n_slots, hd), dtype=torch.int8, device=dev()),
                  torch.zeros((Hk, n_slots, hd // 32), dtype=torch.float32, device=dev()))
    kc, ks, vc, vs = caches
    q_out = torch.full((T, H, hd), float("nan"), dtype=torch.float32, device=dev())
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    print(f"q8_kv_write tokens={T} heads={H}/{Hk} head_dim={hd} gains={qg is not None}", flush=True)
    q8.q8_kv_write(up(qkv), T, H, Hk, hd, _i32(pos), tabs[0].shape[0], up(tabs[0]), up(tabs[1]),
                   None if qg is None else up(qg), None if kg is None else up(kg), eps, _i32(slots), n_slots, q_out,
                   kc, ks, vc, vs, status)
    return q_out, caches, int(down(status)[0])


def _check_write(T, H, Hk, hd, gains, seed, n_slots=None, P=4096):
    qkv, qg, kg = wl.kv_inputs(wl.KV, seed, T, H, Hk, hd)
    if not gains:
        qg = kg = None
    tabs = wl.rope_tables(P, hd)
    g = np.random.default_rng(seed)
    pos = g.integers(0, P, T).astype(np.int32)
    n_slots = n_slots or 2 * T + 3
    slots = g.permutation(n_slots)[:T].astype(np.int32)
    q_out, caches, status = _gpu_write(qkv, H, Hk, hd, pos, tabs, qg, kg, 1e-6, slots, n_slots)
    assert status == 0
    ref = oracle.kv_write(qkv, H, Hk, hd, pos, tabs[0], tabs[1], qg, kg, 1e-6, slots, n_slots)
    assert bits_equal(down(q_out), ref[0]), "rotated queries"
    for name, got, want in zip(("k codes", "k scales", "v codes", "v scales"), caches, ref[1:]):
        got = down(got)
        if got.dtype == np.float32:
            assert bits_equal(got, want), name
        else:
            assert np.array_equal(got, want), name


@pytest.mark.parametrize("gains", [False, True])
@pytest.mark.parametrize("T,H,Hk,hd", [(5, 4, 2, 64), (3, 8, 8, 128), (2, 4, 1, 256), (16, 32, 8, 64), (7, 6, 3, 128)])
def test_write_parity(T, H, Hk, hd, gains):
    _check_write(T, H, Hk, hd, gains, seed=T * 31 + hd)


def test_write_prefill_rows():
    """A prefill-sized write: 2048 tokens of the Llama-3.2-1B shape."""
    _check_write(2048, 32, 8, 64, True, seed=2048, n_slots=4096)


def test_write_out_of_range_position_and_slot():
    H, Hk, hd, T, n_slots = 4, 2, 64, 3, 8
    qkv, _, _ = wl.kv_inputs(wl.KV, 5, T, H, Hk, hd)
    tabs = wl.rope_tables(16, hd)
    pos = np.array([1, 16, 2], np.int32)     # 16 is outside the 16-row table
    slots = np.array([0, 1, 9], np.int32)    # 9 is outside the 8-slot cache
    q_out, caches, status = _gpu_write(qkv, H, Hk, hd, pos, tabs, None, None, 0.0, slots, n_slots)
    assert status == q8.Q8_ERR_ARG
    ref = oracle.kv_write(qkv[:1], H, Hk, hd, pos[:1], tabs[0], tabs[1], None, None, 0.0, slots[:1], n_slots)
    assert bits_equal(down(q_out)[0], ref[0][0])
    assert np.isnan(down(q_out)[1:]).all()          # the bad tokens are not written
    kc = down(caches[0])
    assert np.array_equal(kc, ref[1]) and not kc[:, 1:].any()


def _cache_from_oracle(seed, Hk, hd, n_slots):
    """A filled cache: every slot written by the oracle's own kv_write from
    seeded fused-QKV rows (H = Hk query heads, discarded)."""
    qkv, _, kg = wl.kv_inputs(wl.KV, seed, n_slots, Hk, Hk, hd)
    tabs = wl.rope_tables(n_slots, hd)
    pos = np.arange(n_slots, dtype=np.int32)
    _, kc, ks, vc, vs = oracle.kv_write(qkv, Hk, Hk, hd, pos, tabs[0], tabs[1], None, kg, 1e-6, pos, n_slots)
    return kc, ks, vc, vs


def _gpu_attention(q, caches, base, length, max_len, scale):
    S, H, hd = q.shape
    kc, ks, vc, vs = caches
    Hk, n_slots = kc.shape[0], kc.shape[1]
    need = q8.q8_attention_workspace_bytes(S, H, Hk, hd, max_len)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=dev())
    out = torch.full((S, H, hd), float("nan"), dtype=torch.float32, device=dev())
    print(f"q8_attention_decode seqs={S} heads={H}/{Hk} head_dim={hd} max_len={max_len}", flush=True)
    q8.q8_attention_decode(up(q), S, H, Hk, hd, kc, ks, vc, vs, n_slots, _i32(base), _i32(length), max_len, scale,
                           out, ws, need)
    return down(out), int(down(ws[:4].view(torch.int32))[0])


def _check_attention(S, H, Hk, hd, lengths, seed):
    lengths = np.asarray(lengths, np.int32)
    base = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int32)
    n_slots = int(lengths.sum()) + 5
    kc, ks, vc, vs = _cache_from_oracle(seed, Hk, hd, n_slots)
    q = np.random.default_rng(seed).standard_normal((S, H, hd)).astype(np.float32)
    scale = 1.0 / math.sqrt(hd)
    caches = tuple(up(a) for a in (kc, ks, vc, vs))
    out, status = _gpu_attention(q, caches, base, lengths, int(lengths.max()), scale)
    assert status == 0
    ref, bound = oracle.attention_decode(q, kc, ks, vc, vs, base, lengths, scale)
    err = np.abs(out.astype(np.float64) - ref.astype(np.float64))
    bad = err > bound
    if bad.any():
        i = np.unravel_index(int(np.argmax(err - bound)), err.shape)
        pytest.fail(f"{int(bad.sum())} outputs outside the error budget; worst {i}: {out[i]!r} vs {ref[i]!r}, "
                    f"budget {bound[i]!r}")
    return q, caches, base, lengths, out


@pytest.mark.parametrize("hd", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_attention_parity(hd, G):
    Hk = 2
    _check_attention(3, G * Hk, Hk, hd, [1, 37, 300], seed=hd + G)


@pytest.mark.parametrize("lengths", [[255, 256, 257], [511, 512, 513, 1], [4096]])
def test_attention_chunk_boundaries(lengths):
    _check_attention(len(lengths), 32, 8, 64, lengths, seed=sum(lengths))


def test_attention_batch_invariance():
    """A sequence's output does not depend on the rest of the batch or on
    max_len (beyond its own length)."""
    q, caches, base, lengths, out = _check_attention(4, 32, 8, 64, [700, 3, 1500, 256], seed=77)
    for s in (0, 2):
        o1, st = _gpu_attention(q[s:s + 1], caches, base[s:s + 1], lengths[s:s + 1], int(lengths[s]), 0.125)
        assert st == 0 and bits_equal(o1[0], out[s])
        o2, _ = _gpu_attention(q[s:s + 1], caches, base[s:s + 1], lengths[s:s + 1], 4000, 0.125)
        assert bits_equal(o2[0], out[s])


def test_attention_invalid_length_reports():
    kc, ks, vc, vs = _cache_from_oracle(3, 2, 64, 600)
    caches = tuple(up(a) for a in (kc, ks, vc, vs))
    q = np.random.default_rng(3).standard_normal((3, 4, 64)).astype(np.float32)
    base = np.array([0, 100, 590], np.int32)
    lengths = np.array([50, 0, 20], np.int32)   # a zero length and a range past the cache
    out, status = _gpu_attention(q, caches, base, lengths, 64, 0.125)
    assert status == q8.Q8_ERR_ARG
    assert np.isnan(out[1]).all() and np.isnan(out[2]).all() and not np.isnan(out[0]).any()
    ref, bound = oracle.attention_decode(q[:1], kc, ks, vc, vs, base[:1], lengths[:1], 0.125)
    assert np.all(np.abs(out[0].astype(np.float64) - ref[0]) <= bound[0])


def test_write_then_attend_full_size():
    """The Llama-3.2-1B decode shape at full size: 16 sequences x 4096 cached
    positions written by the device (2048 tokens per call), then attention;
    every output within the oracle's budget of the oracle's own chain."""
    S, H, Hk, hd, L = wl.KV_SEQS, wl.LLAMA_HEADS, wl.LLAMA_KV_HEADS, wl.LLAMA_HEAD_DIM, wl.KV_CONTEXT
    n_slots = S * L
    tabs = wl.rope_tables(L, hd)
    kc_d = torch.zeros((Hk, n_slots, hd), dtype=torch.int8, device=dev())
    ks_d = torch.zeros((Hk, n_slots, hd // 32), dtype=torch.float32, device=dev())
    vc_d = torch.zeros_like(kc_d)
    vs_d = torch.zeros_like(ks_d)
    kc = np.zeros((Hk, n_slots, hd), np.int8)
    ks = np.zeros((Hk, n_slots, hd // 32), np.float32)
    vc = np.zeros_like(kc)
    vs = np.zeros_like(ks)
    chunk = 2048
    for c0 in range(0, n_slots, chunk):
        qkv, qg, kg = wl.kv_inputs(wl.KV, 1000 + c0 // chunk, chunk, H, Hk, hd)
        slots = np.arange(c0, c0 + chunk, dtype=np.int32)
        pos = (slots % L).astype(np.int32)
        _, _, st = _gpu_write(qkv, H, Hk, hd, pos, tabs, qg, kg, 1e-6, slots, n_slots, (kc_d, ks_d, vc_d, vs_d))
        assert st == 0
        _, kc1, ks1, vc1, vs1 = oracle.kv_write(qkv, H, Hk, hd, pos, tabs[0], tabs[1], qg, kg, 1e-6,
                                                np.arange(chunk, dtype=np.int32), chunk)
        kc[:, c0:c0 + chunk], ks[:, c0:c0 + chunk], vc[:, c0:c0 + chunk], vs[:, c0:c0 + chunk] = kc1, ks1, vc1, vs1
    assert np.array_equal(down(kc_d), kc) and bits_equal(down(vs_d), vs)
    q = np.random.default_rng(8).standard_normal((S, H, hd)).astype(np.float32)
    base = (np.arange(S) * L).astype(np.int32)
    lengths = np.full(S, L, np.int32)
    out, status = _gpu_attention(q, (kc_d, ks_d, vc_d, vs_d), base, lengths, L, 0.125)
    assert status == 0
    ref, bound = oracle.attention_decode(q, kc, ks, vc, vs, base, lengths, 0.125)
    assert np.all(np.abs(out.astype(np.float64) - ref.astype(np.float64)) <= bound)
