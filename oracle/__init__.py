"""Python access to the CPU oracle (oracle/q8ref.c).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may use it; the HIP library never does.  The
oracle is plain scalar C with no code shared with the HIP path; this module
only marshals numpy arrays into it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "q8ref.c")
# Q8REF_LIB names another build of q8ref.c (the sanitizer build of the tests).
LIB = os.environ.get("Q8REF_LIB") or os.path.join(HERE, "libq8ref.so")
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra"]

LAYOUT_ROWS = 0
LAYOUT_PACKED = 1
LAYOUT_ACT = 2
QK = 32
BLOCK_BYTES = 34


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (always recompiles)."""
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm", "-lpthread"]
    out = subprocess.run(cmd, capture_output=True, text=True)
    if out.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + out.stderr)
    if verbose and out.stderr:
        print(out.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.q8ref_f32_to_f16.argtypes = [ctypes.c_float]
        L.q8ref_f32_to_f16.restype = ctypes.c_uint16
        L.q8ref_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.q8ref_f16_to_f32.restype = ctypes.c_float
        L.q8ref_f32_to_f16_n.argtypes = [P, P, I64]
        L.q8ref_f16_to_f32_n.argtypes = [P, P, I64]
        L.q8ref_quantize_block.argtypes = [P, P, P]
        L.q8ref_quantize_block.restype = ctypes.c_uint16
        L.q8ref_quantize_rows.argtypes = [P, I64, I64, I64, I, P]
        L.q8ref_pack.argtypes = [P, I64, I64, P]
        L.q8ref_unpack.argtypes = [P, I64, I64, P]
        L.q8ref_block_terms.argtypes = [P, I64, P, I64, I64, P, P]
        L.q8ref_matmul.argtypes = [P, I64, P, I64, I64, P, I64, P, I]
        L.q8ref_matmul_points.argtypes = [P, I64, P, I64, I64, P, P, I64, P, P]
        L.q8ref_grouped_matmul.argtypes = [P, I64, I, P, I64, I, P, I64, I64, I64, I64, P, P, I]
        L.q8ref_rmsnorm_quantize.argtypes = [P, P, P, I64, I64, ctypes.c_float, P, P]
        L.q8ref_exact_sum.argtypes = [P, I64]
        L.q8ref_exact_sum.restype = ctypes.c_double
        L.q8ref_exp_nonpos.argtypes = [ctypes.c_double]
        L.q8ref_exp_nonpos.restype = ctypes.c_double
        L.q8ref_moe_route.argtypes = [P, I64, I64, I, I, P, P]
        L.q8ref_swiglu_quantize.argtypes = [P, I64, P, I64, I64, I64, P]
        L.q8ref_moe_combine.argtypes = [P, I64, P, I64, I, I64, P, P]
        L.q8ref_kv_write.argtypes = [P, I64, I, I, I, P, P, P, P, P, ctypes.c_float, P, I64, P, P, P, P, P]
        L.q8ref_attention_decode.argtypes = [P, I64, I, I, I, P, P, P, P, I64, P, P, ctypes.c_float, P, P]
        for name in ("q8ref_kv_write", "q8ref_attention_decode",
                     "q8ref_quantize_rows", "q8ref_pack", "q8ref_unpack", "q8ref_block_terms",
                     "q8ref_matmul", "q8ref_matmul_points", "q8ref_grouped_matmul", "q8ref_rmsnorm_quantize",
                     "q8ref_moe_route", "q8ref_swiglu_quantize", "q8ref_moe_combine"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} returned {rc}")


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().q8ref_f32_to_f16_n(_p(x), _p(out), x.size)
    return out


def f16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().q8ref_f16_to_f32_n(_p(h), _p(out), h.size)
    return out


def quantize_block(x: np.ndarray):
    """-> (q int8[32], stored fp16 bits, fp32 d)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.size == QK
    q = np.empty(QK, dtype=np.int8)
    d = np.empty(1, dtype=np.float32)
    bits = lib().q8ref_quantize_block(_p(x), _p(q), _p(d))
    return q, int(bits), float(d[0])


def quantized_bytes(rows: int, k: int) -> int:
    return rows * (k // QK) * BLOCK_BYTES


def quantize_rows(x: np.ndarray, layout: int = LAYOUT_ACT) -> np.ndarray:
    """fp32 [rows][k] (any row stride) -> uint8 buffer in layout ROWS or ACT."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    if x.strides[1] != 4:
        x = np.ascontiguousarray(x)
    rows, k = x.shape
    ld = x.strides[0] // 4
    out = np.empty(quantized_bytes(rows, k), dtype=np.uint8)
    _check(lib().q8ref_quantize_rows(_p(x), ld, rows, k, layout, _p(out)), "quantize_rows")
    return out


def rmsnorm_quantize(x: np.ndarray, res_in: np.ndarray, w: np.ndarray, eps: float):
    """Fused residual + RMSNorm + Q8_0 quantization (q8ref_rmsnorm_quantize):
    fp32 [rows][k] x and residual (None: no residual add), fp32 [k] weight ->
    (new residual fp32 [rows][k], ACT buffer of the normalized rows)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    rows, k = x.shape
    r = None if res_in is None else np.ascontiguousarray(res_in, dtype=np.float32).reshape(rows, k)
    w = np.ascontiguousarray(w, dtype=np.float32).reshape(k)
    res_out = np.empty((rows, k), dtype=np.float32)
    q = np.empty(quantized_bytes(rows, k), dtype=np.uint8)
    _check(lib().q8ref_rmsnorm_quantize(_p(x), None if r is None else _p(r), _p(w), rows, k, float(eps),
                                        _p(res_out), _p(q)),
           "rmsnorm_quantize")
    return res_out, q


def exact_sum(v) -> float:
    """Sum of non-negative finite doubles rounded once to fp64 (q8ref_exact_sum)."""
    a = np.ascontiguousarray(v, dtype=np.float64)
    return float(lib().q8ref_exact_sum(_p(a), a.size))


def exp_nonpos(x: float) -> float:
    """e^x for x <= 0 by the fixed fp64 algorithm (q8ref_exp_nonpos)."""
    return lib().q8ref_exp_nonpos(float(x))


def moe_route(logits: np.ndarray, topk: int, normalize: bool = True):
    """fp32 [tokens][experts] router logits -> (int32 ids [tokens][topk], fp32 weights [tokens][topk])."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    tokens, E = logits.shape
    ids = np.empty((tokens, topk), np.int32)
    w = np.empty((tokens, topk), np.float32)
    _check(lib().q8ref_moe_route(_p(logits), tokens, E, int(topk), int(bool(normalize)), _p(ids), _p(w)), "moe_route")
    return ids, w


def swiglu_quantize(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """fp32 [rows][n] gate and up -> ACT buffer of silu(gate) * up."""
    gate = np.ascontiguousarray(gate, dtype=np.float32)
    up = np.ascontiguousarray(up, dtype=np.float32)
    rows, n = gate.shape
    assert up.shape == (rows, n)
    q = np.empty(quantized_bytes(rows, n), np.uint8)
    _check(lib().q8ref_swiglu_quantize(_p(gate), n, _p(up), n, rows, n, _p(q)), "swiglu_quantize")
    return q


def moe_combine(y: np.ndarray, w: np.ndarray):
    """fp32 y [tokens*topk][n] and weights [tokens][topk] -> (fp32 out [tokens][n], fp64 S [tokens][n])."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    tokens, topk = w.shape
    n = y.shape[1]
    assert y.shape[0] == tokens * topk
    out = np.empty((tokens, n), np.float32)
    S = np.empty((tokens, n), np.float64)
    _check(lib().q8ref_moe_combine(_p(y), n, _p(w), tokens, topk, n, _p(out), _p(S)), "moe_combine")
    return out, S


def kv_write(qkv, n_heads: int, n_kv: int, head_dim: int, positions, cos_tab, sin_tab, q_gain, k_gain, eps: float,
             slots, n_slots: int):
    """Fused norm + rope + Q8 KV cache write.  Returns (q_out fp32 [tokens][n_heads][head_dim],
    k_cache int8 [n_kv][n_slots][head_dim], k_scale fp32 [n_kv][n_slots][head_dim/32], v_cache, v_scale);
    cache slots not written hold zeros."""
    qkv = np.ascontiguousarray(qkv, dtype=np.float32)
    tokens = qkv.shape[0]
    positions = np.ascontiguousarray(positions, dtype=np.int32)
    slots = np.ascontiguousarray(slots, dtype=np.int32)
    cos_tab = np.ascontiguousarray(cos_tab, dtype=np.float32)
    sin_tab = np.ascontiguousarray(sin_tab, dtype=np.float32)
    qg = None if q_gain is None else np.ascontiguousarray(q_gain, dtype=np.float32)
    kg = None if k_gain is None else np.ascontiguousarray(k_gain, dtype=np.float32)
    q_out = np.empty((tokens, n_heads, head_dim), np.float32)
    kc = np.zeros((n_kv, n_slots, head_dim), np.int8)
    vc = np.zeros((n_kv, n_slots, head_dim), np.int8)
    ks = np.zeros((n_kv, n_slots, head_dim // 32), np.float32)
    vs = np.zeros((n_kv, n_slots, head_dim // 32), np.float32)
    _check(lib().q8ref_kv_write(_p(qkv), tokens, n_heads, n_kv, head_dim, _p(positions), _p(cos_tab), _p(sin_tab),
                                None if qg is None else _p(qg), None if kg is None else _p(kg), float(eps),
                                _p(slots), n_slots, _p(q_out), _p(kc), _p(ks), _p(vc), _p(vs)), "kv_write")
    return q_out, kc, ks, vc, vs


def attention_decode(q, k_cache, k_scale, v_cache, v_scale, base, length, scale: float):
    """q fp32 [seqs][n_heads][head_dim]; caches as kv_write returns them (head-major) ->
    (out fp32 [seqs][n_heads][head_dim], fp64 error budget of an fp32 evaluation)."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    seqs, n_heads, head_dim = q.shape
    n_kv, n_slots = k_cache.shape[0], k_cache.shape[1]
    base = np.ascontiguousarray(base, dtype=np.int32)
    length = np.ascontiguousarray(length, dtype=np.int32)
    out = np.empty_like(q)
    bound = np.empty(q.shape, np.float64)
    _check(lib().q8ref_attention_decode(_p(q), seqs, n_heads, n_kv, head_dim, _p(np.ascontiguousarray(k_cache)),
                                        _p(np.ascontiguousarray(k_scale)), _p(np.ascontiguousarray(v_cache)),
                                        _p(np.ascontiguousarray(v_scale)), n_slots, _p(base), _p(length), float(scale),
                                        _p(out), _p(bound)), "attention_decode")
    return out, bound


def act_planes(buf: np.ndarray, rows: int, k: int):
    """Split an ACT buffer into (int8 [rows][k], fp16 bits [rows][k/32])."""
    q = buf[: rows * k].view(np.int8).reshape(rows, k)
    d = buf[rows * k: rows * k + rows * (k // QK) * 2].view(np.uint16).reshape(rows, k // QK)
    return q, d


def rows_planes(buf: np.ndarray, n: int, k: int):
    """Split a ROWS buffer into (int8 [n][k], fp16 bits [n][k/32])."""
    blocks = buf.reshape(n, k // QK, BLOCK_BYTES)
    d = np.ascontiguousarray(blocks[:, :, :2]).view(np.uint16).reshape(n, k // QK)
    q = np.ascontiguousarray(blocks[:, :, 2:]).view(np.int8).reshape(n, k)
    return q, d


def pack(w_rows: np.ndarray, n: int, k: int) -> np.ndarray:
    w_rows = np.ascontiguousarray(w_rows, dtype=np.uint8)
    out = np.empty(quantized_bytes(n, k), dtype=np.uint8)
    _check(lib().q8ref_pack(_p(w_rows), n, k, _p(out)), "pack")
    return out


def unpack(w_packed: np.ndarray, n: int, k: int) -> np.ndarray:
    w_packed = np.ascontiguousarray(w_packed, dtype=np.uint8)
    out = np.empty(quantized_bytes(n, k), dtype=np.uint8)
    _check(lib().q8ref_unpack(_p(w_packed), n, k, _p(out)), "unpack")
    return out


def block_terms(x_act: np.ndarray, m: int, w_rows: np.ndarray, n: int, k: int):
    """-> (s int32 [m][n][k/32], t float32 [m][n][k/32])."""
    nb = k // QK
    s = np.empty((m, n, nb), dtype=np.int32)
    t = np.empty((m, n, nb), dtype=np.float32)
    _check(lib().q8ref_block_terms(_p(np.ascontiguousarray(x_act)), m, _p(np.ascontiguousarray(w_rows)),
                                   n, k, _p(s), _p(t)), "block_terms")
    return s, t


def matmul(x_act: np.ndarray, m: int, w_rows: np.ndarray, n: int, k: int, threads: int = 1):
    """-> (y float32 [m][n], S float64 [m][n] = sum of |block terms|)."""
    y = np.empty((m, n), dtype=np.float32)
    S = np.empty((m, n), dtype=np.float64)
    _check(lib().q8ref_matmul(_p(np.ascontiguousarray(x_act)), m, _p(np.ascontiguousarray(w_rows)),
                              n, k, _p(y), n, _p(S), threads), "matmul")
    return y, S


def matmul_points(x_act: np.ndarray, m: int, w_rows: np.ndarray, n: int, k: int, mi, ni):
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    y = np.empty(mi.size, dtype=np.float32)
    S = np.empty(mi.size, dtype=np.float64)
    _check(lib().q8ref_matmul_points(_p(np.ascontiguousarray(x_act)), m, _p(np.ascontiguousarray(w_rows)),
                                     n, k, _p(mi), _p(ni), mi.size, _p(y), _p(S)), "matmul_points")
    return y, S


def grouped_matmul(x_act: np.ndarray, x_rows: int, x_per_pair: bool, ids: np.ndarray, w_rows: np.ndarray,
                   n_experts: int, expert_stride: int, n: int, k: int, threads: int = 1):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    tokens, topk = ids.shape
    y = np.empty((tokens * topk, n), dtype=np.float32)
    S = np.empty((tokens * topk, n), dtype=np.float64)
    _check(lib().q8ref_grouped_matmul(_p(np.ascontiguousarray(x_act)), x_rows, int(bool(x_per_pair)), _p(ids),
                                      tokens, topk, _p(np.ascontiguousarray(w_rows)), n_experts, expert_stride,
                                      n, k, _p(y), _p(S), threads), "grouped_matmul")
    return y, S
