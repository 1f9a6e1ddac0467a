"""Routed-expert GEMV (q8_grouped_matmul) against the oracle, bit-identical to
the single-row GEMV of each (token, slot) pair, plus the device-side check of
expert ids."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from decode_q8_amd import q8
from tests.gpu_helpers import bits_equal, check_tol, down, quantize, ref_quantize, require_gpu, up

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _experts(E, n, k, seed, only=None):
    """Packed experts laid out back to back; returns (device buffer, stride,
    the oracle's own row-contiguous quantization of each generated expert)."""
    stride = q8.q8_quantized_bytes(n, k)
    buf = torch.zeros(E * stride, dtype=torch.uint8, device="cuda")
    rows = {}
    for e in range(E):
        if only is not None and e not in only:
            continue
        w = wl.weight(wl.MOE, e, n, k, group=seed)
        wr = quantize(w, q8.Q8_LAYOUT_ROWS)
        q8.q8_repack_weights(wr, n, k, buf[e * stride:(e + 1) * stride])
        rows[e] = ref_quantize(w, oracle.LAYOUT_ROWS)
    return buf, stride, rows


def _grouped(xq, x_rows, per_pair, ids, E, buf, stride, n, k):
    tokens, topk = ids.shape
    y = torch.full((tokens * topk, n), float("nan"), dtype=torch.float32, device="cuda")
    need = q8.q8_grouped_workspace_bytes(tokens, topk, E, n, k)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    q8.q8_grouped_matmul(xq, x_rows, per_pair, up(ids), tokens, topk, buf, E, stride, n, k, y, ws, need)
    status = int(down(ws[:4].view(torch.int32))[0])
    return down(y), status


@pytest.mark.parametrize("per_pair", [0, 1])
@pytest.mark.parametrize("tokens,topk,E,n,k", [(5, 3, 7, 128, 512), (16, 8, 32, 64, 256), (40, 2, 4, 192, 768)])
def test_parity_and_single_gemv_equality(tokens, topk, E, n, k, per_pair):
    rng = np.random.default_rng(tokens * 100 + E)
    ids = np.stack([rng.permutation(E)[:topk] for _ in range(tokens)]).astype(np.int32)
    rows = tokens * topk if per_pair else tokens
    x = wl.activation(wl.MOE, 7, rows, k)
    xq = quantize(x, q8.Q8_LAYOUT_ACT)
    buf, stride, wrows = _experts(E, n, k, seed=tokens)
    y, status = _grouped(xq, rows, per_pair, ids, E, buf, stride, n, k)
    assert status == 0
    w_all = np.concatenate([wrows[e] for e in range(E)])
    y_ref, S = oracle.grouped_matmul(ref_quantize(x, oracle.LAYOUT_ACT), rows, per_pair, ids, w_all, E, stride, n, k,
                                     threads=8)
    check_tol(y, y_ref, S, "grouped")
    for t in range(tokens):
        for j in range(topk):
            p = t * topk + j
            xr = p if per_pair else t
            y1 = down(q8.matmul(quantize(x[xr:xr + 1], q8.Q8_LAYOUT_ACT), 1, buf[ids[t, j] * stride:], 1, n, k))
            assert bits_equal(y[p:p + 1], y1), f"pair {p}"


def test_bad_expert_id_sets_status():
    tokens, topk, E, n, k = 4, 2, 8, 64, 256
    ids = np.array([[0, 1], [2, 9], [3, -1], [4, 5]], np.int32)
    x = wl.activation(wl.MOE, 8, tokens, k)
    xq = quantize(x, q8.Q8_LAYOUT_ACT)
    buf, stride, _ = _experts(E, n, k, seed=99)
    y, status = _grouped(xq, tokens, 0, ids, E, buf, stride, n, k)
    assert status == q8.Q8_ERR_ARG
    assert np.isnan(y[3]).all() and np.isnan(y[5]).all()      # pairs with bad ids are left unwritten
    assert not np.isnan(y[[0, 1, 2, 4, 6, 7]]).any()


@pytest.mark.parametrize("mat", [0, 2])
def test_moe_full_size_whole_output(mat):
    """The MoE workload at full size: 256 experts (only routed ones generated),
    16 tokens, top-8 routing; gate (token rows, K = 7168) or down (per-pair
    rows, K = 2048).  Every output of all 128 pairs against the oracle (the
    pairs of each routed expert in one oracle call), the device-quantized
    activations equal to the oracle's, and every pair bit-identical to its
    single-row GEMV."""
    import os
    name, n, k = wl.MOE_MATS[mat]
    T, K8, E = wl.MOE_TOKENS, wl.MOE_TOPK, wl.MOE_EXPERTS
    ids = wl.routing(wl.MOE, T, E, K8)
    used = set(int(e) for e in np.unique(ids))
    per_pair = 1 if name == "down" else 0
    rows = T * K8 if per_pair else T
    x = wl.activation(wl.MOE, 100 + mat, rows, k)
    xq = quantize(x, q8.Q8_LAYOUT_ACT)
    buf, stride, wrows = _experts(E, n, k, seed=mat, only=used)
    y, status = _grouped(xq, rows, per_pair, ids, E, buf, stride, n, k)
    assert status == 0 and not np.isnan(y).any()
    xa = ref_quantize(x, oracle.LAYOUT_ACT)
    assert np.array_equal(down(xq), xa), "activation quantization"
    threads = min(16, os.cpu_count() or 1)
    for e in sorted(used):
        pairs = [p for p in range(T * K8) if int(ids[p // K8, p % K8]) == e]
        xr = np.array([p if per_pair else p // K8 for p in pairs])
        sub = ref_quantize(x[xr], oracle.LAYOUT_ACT)
        y_ref, S = oracle.matmul(sub, len(pairs), wrows[e], n, k, threads=threads)
        check_tol(y[pairs], y_ref, S, f"moe {name} expert {e}")
    for p in range(T * K8):
        t, j = divmod(p, K8)
        xr = p if per_pair else t
        y1 = down(q8.matmul(quantize(x[xr:xr + 1], q8.Q8_LAYOUT_ACT), 1, buf[int(ids[t, j]) * stride:], 1, n, k))
        assert bits_equal(y[p:p + 1], y1), f"pair {p}"
