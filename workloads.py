"""Seeded synthetic inputs for the Q8_0 matmul workloads.

This module only draws random numbers and names shapes.  It holds none of the
method's arithmetic (no quantization, no dot products): both the CPU oracle
(`oracle/`) and the HIP library (`decode_q8_amd/`) are fed from here, and
neither of them is imported by it.

Recipe (every tensor is independent of every other one):
  * bit generator: numpy Philox (a counter-based generator) keyed by
    ``SeedSequence(base_seed, spawn_key=tag)``; ``tag`` is a tuple of small
    integers naming the tensor (see ``TAG_*`` below), so each tensor can be
    regenerated alone, in any order, on any machine;
  * weights: fp32 standard normal times 0.02 (the "N(0, 0.02)" weights of the
    Llama-3.2-1B Q8_0 decode workload and of the MoE workload);
  * activations: fp32 standard normal; the prefill workload additionally picks
    round(0.01 * K) outlier channels without replacement and multiplies those
    columns by 20 in every row;
  * routing: uniform(0, 1) logits [tokens x experts]; each token takes the
    top-k experts by logit (ties go to the lower expert id), slots ordered by
    descending logit.
  * norm (the fused residual + RMSNorm + quantize producer): the residual
    stream N(0, 1) with the prefill outlier recipe (round(0.01 * K) channels
    x 20), the layer output added to it N(0, 1), the per-channel gain
    1 + 0.1 * N(0, 1);
  * base seed of workload i is 20261202 + i.

Shapes (out x in = N x K):
  * single:  W 2048x2048, one activation row.
  * decode:  Llama-3.2-1B, 16 layers of QKV fused [3072x2048] (Q 2048 + K 512
    + V 512 rows), O [2048x2048], gate||up fused [16384x2048], down
    [2048x8192], then the LM head [128256x2048]; one independent activation
    row per distinct input (attention input, O input, MLP input, down input,
    LM-head input).
  * batched: the decode shapes with M in {1, 2, 4, 6, 8} activation rows.
  * prefill: M in {188, 752, 2048} x (N, K) in {(2048, 2048), (8192, 2048),
    (2048, 8192)}.
  * moe:     256 experts, gate and up [2048x7168], down [7168x2048]; 16 tokens,
    top-8 routing, token rows [16x7168], down inputs [128x2048].
  * norm:    rows in {1, 188, 752, 2048} (decode and prefill tokens) x hidden
    2048 (Llama-3.2-1B), plus hidden 7168 (the MoE model).
  * kv:      Llama-3.2-1B attention (32 query heads, 8 KV heads of 64) over a
    Q8 KV cache: 16 sequences x 4096 cached positions, fused QKV rows N(0, 1).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

BASE_SEED = 20261202

W_STD = np.float32(0.02)
OUTLIER_FRACTION = 0.01
OUTLIER_SCALE = np.float32(20.0)

# Tensor tags: (kind, layer-or-expert, index).  kind values:
TAG_WEIGHT = 1
TAG_ACT = 2
TAG_ROUTE = 3
TAG_PERM = 4
TAG_OUTLIER = 5
TAG_GAIN = 6

# Workload indices (offsets from BASE_SEED).
SINGLE, DECODE, BATCHED, PREFILL, MOE, NORM, KV = 0, 1, 2, 3, 4, 5, 6

LLAMA_HIDDEN = 2048
LLAMA_LAYERS = 16
LLAMA_VOCAB = 128256
LLAMA_FFN = 8192
# Decode-step matrices of one layer: (name, N, K).  Q/K/V and gate/up share
# their input, so each pair is one fused matrix fed by one quantized row.
LLAMA_LAYER_MATS = (
    ("qkv", 2048 + 512 + 512, LLAMA_HIDDEN),
    ("o", LLAMA_HIDDEN, LLAMA_HIDDEN),
    ("gate_up", 2 * LLAMA_FFN, LLAMA_HIDDEN),
    ("down", LLAMA_HIDDEN, LLAMA_FFN),
)
LLAMA_HEAD = ("lm_head", LLAMA_VOCAB, LLAMA_HIDDEN)

BATCHED_M = (1, 2, 4, 6, 8)
PREFILL_M = (188, 752, 2048)
PREFILL_NK = ((2048, 2048), (8192, 2048), (2048, 8192))

MOE_EXPERTS = 256
MOE_HIDDEN = 7168
MOE_FFN = 2048
MOE_TOKENS = 16
MOE_TOPK = 8
# (name, N, K) of one expert's matrices.
MOE_MATS = (("gate", MOE_FFN, MOE_HIDDEN), ("up", MOE_FFN, MOE_HIDDEN), ("down", MOE_HIDDEN, MOE_FFN))

NORM_ROWS = (1, 188, 752, 2048)
NORM_EPS = 1e-5

# Llama-3.2-1B attention: 32 query heads, 8 key/value heads of 64.
LLAMA_HEADS = 32
LLAMA_KV_HEADS = 8
LLAMA_HEAD_DIM = 64
KV_SEQS = 16
KV_CONTEXT = 4096


def generator(workload: int, tag: tuple) -> np.random.Generator:
    """Independent generator for one tensor of one workload."""
    ss = np.random.SeedSequence(BASE_SEED + workload, spawn_key=tuple(int(t) for t in tag))
    return np.random.Generator(np.random.Philox(ss))


def normal(workload: int, tag: tuple, shape, scale=None) -> np.ndarray:
    a = generator(workload, tag).standard_normal(shape, dtype=np.float32)
    if scale is not None:
        a *= np.float32(scale)
    return a


def weight(workload: int, index: int, n: int, k: int, group: int = 0) -> np.ndarray:
    """fp32 [n][k] weight, N(0, 0.02^2).  ``group`` is the layer or expert."""
    return normal(workload, (TAG_WEIGHT, group, index), (n, k), W_STD)


def activation(workload: int, index: int, m: int, k: int, group: int = 0,
               outliers: bool = False) -> np.ndarray:
    """fp32 [m][k] activation rows, N(0, 1), optionally with outlier channels."""
    x = normal(workload, (TAG_ACT, group, index), (m, k))
    if outliers:
        cols = outlier_channels(workload, index, k, group)
        x[:, cols] *= OUTLIER_SCALE
    return x


def outlier_channels(workload: int, index: int, k: int, group: int = 0) -> np.ndarray:
    count = int(round(OUTLIER_FRACTION * k))
    g = generator(workload, (TAG_OUTLIER, group, index))
    return np.sort(g.choice(k, size=count, replace=False))


def norm_inputs(workload: int, index: int, rows: int, k: int):
    """(x, residual, gain) for the residual + RMSNorm + quantize producer:
    fp32 [rows][k] layer output N(0, 1), fp32 [rows][k] residual stream N(0, 1)
    with outlier channels, fp32 [k] gain 1 + 0.1 * N(0, 1)."""
    x = activation(workload, 2 * index, rows, k)
    res = activation(workload, 2 * index + 1, rows, k, outliers=True)
    gain = np.float32(1.0) + normal(workload, (TAG_GAIN, 0, index), (k,), 0.1)
    return x, res, gain.astype(np.float32)


def router_logits(workload: int, tokens: int, n_experts: int, group: int = 0) -> np.ndarray:
    """fp32 [tokens][n_experts] router logits, uniform(0, 1)."""
    return generator(workload, (TAG_ROUTE, group, 0)).random((tokens, n_experts), dtype=np.float32)


def rope_tables(max_pos: int, head_dim: int, theta: float = 500000.0):
    """Rotary-embedding tables, a model constant handed to both sides as an
    input: fp32 cos and sin [max_pos][head_dim/2] of pos * theta^(-2i/head_dim),
    evaluated by numpy in fp64 and rounded once (Llama 3 uses theta = 500000)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * theta ** (-2.0 * i / head_dim)[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def kv_inputs(workload: int, index: int, tokens: int, n_heads: int, n_kv: int, head_dim: int):
    """(qkv fp32 [tokens][(n_heads + 2 n_kv) head_dim] N(0, 1), q gain, k gain
    fp32 [head_dim] 1 + 0.1 N(0, 1)) for the KV-cache write."""
    qkv = normal(workload, (TAG_ACT, 50, index), (tokens, (n_heads + 2 * n_kv) * head_dim))
    qg = np.float32(1.0) + normal(workload, (TAG_GAIN, 50, index), (head_dim,), 0.1)
    kg = np.float32(1.0) + normal(workload, (TAG_GAIN, 51, index), (head_dim,), 0.1)
    return qkv, qg.astype(np.float32), kg.astype(np.float32)


def kv_cache(workload: int, layer: int, n_kv: int, n_slots: int, head_dim: int):
    """A filled Q8 KV cache for one layer (head-major): int8 codes uniform in
    [-127, 127] and fp32 block scales |N(0, 1)| * 0.02 / 127, for K and V."""
    g = generator(workload, (TAG_WEIGHT, 60 + layer, 0))
    kc = g.integers(-127, 128, (n_kv, n_slots, head_dim), dtype=np.int8)
    vc = g.integers(-127, 128, (n_kv, n_slots, head_dim), dtype=np.int8)
    ks = (np.abs(g.standard_normal((n_kv, n_slots, head_dim // 32), dtype=np.float32)) * np.float32(0.02 / 127))
    vs = (np.abs(g.standard_normal((n_kv, n_slots, head_dim // 32), dtype=np.float32)) * np.float32(0.02 / 127))
    return kc, ks.astype(np.float32), vc, vs.astype(np.float32)


def routing(workload: int, tokens: int, n_experts: int, topk: int, group: int = 0) -> np.ndarray:
    """int32 [tokens][topk] expert ids: top-k of uniform logits per token
    (input generation for the routed-expert GEMV alone; the library's router
    computes the same selection on the device)."""
    logits = router_logits(workload, tokens, n_experts, group)
    # Stable sort of the negated logits: descending logit, ties to the lower id.
    order = np.argsort(-logits, axis=1, kind="stable")
    return np.ascontiguousarray(order[:, :topk].astype(np.int32))


def permutation(workload: int, m: int, index: int = 0) -> np.ndarray:
    return generator(workload, (TAG_PERM, m, index)).permutation(m).astype(np.int64)


def many(fn, args_list, threads: int = 8):
    """Run independent generator calls in a thread pool (numpy releases the GIL
    while filling large arrays); results come back in argument order."""
    with ThreadPoolExecutor(max(1, threads)) as ex:
        return list(ex.map(lambda a: fn(*a), args_list))


@dataclass(frozen=True)
class Matrix:
    name: str
    n: int
    k: int
    layer: int
    index: int  # weight index within the layer
    act: int    # which activation row feeds it (index within the layer)


def decode_matrices() -> list:
    """The decode step's matrices in execution order, with their inputs."""
    mats = []
    for layer in range(LLAMA_LAYERS):
        for i, (name, n, k) in enumerate(LLAMA_LAYER_MATS):
            mats.append(Matrix(name, n, k, layer, i, i))
    name, n, k = LLAMA_HEAD
    mats.append(Matrix(name, n, k, LLAMA_LAYERS, 0, 0))
    return mats


def decode_weight_bytes() -> int:
    return sum(m.n * (m.k // 32) * 34 for m in decode_matrices())
