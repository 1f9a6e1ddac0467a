"""The steps either side of the routed-expert GEMVs against the oracle: the
router (expert ids and weights bit-exact), SwiGLU + quantization (codes and
scales bit-exact) and the weighted combine (within its rounding bound); then
a whole mixture-of-experts layer on the device (route -> gate||up -> SwiGLU
-> down -> combine), whose stages equal the stages run alone and whose output
stays within the quantization bound of the oracle's layer."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from decode_q8_amd import q8
from tests.gpu_helpers import bits_equal, dev, down, quantize, ref_quantize, require_gpu, up

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _route(logits, topk, normalize):
    T, E = logits.shape
    ids = torch.full((T, topk), -7, dtype=torch.int32, device=dev())
    w = torch.full((T, topk), float("nan"), dtype=torch.float32, device=dev())
    print(f"q8_moe_route tokens={T} experts={E} topk={topk} normalize={normalize}", flush=True)
    q8.q8_moe_route(up(logits), T, E, topk, normalize, ids, w)
    return down(ids), down(w)


def _check_route(logits, topk, normalize):
    ids, w = _route(logits, topk, normalize)
    ids_r, w_r = oracle.moe_route(logits, topk, normalize)
    assert np.array_equal(ids, ids_r), "expert ids"
    assert bits_equal(w, w_r), "expert weights"


@pytest.mark.parametrize("normalize", [True, False])
@pytest.mark.parametrize("T,E,k", [(16, 256, 8), (5, 64, 6), (3, 7, 7), (4, 1000, 1), (2, 1024, 32), (130, 256, 8),
                                   (9, 65, 3)])
def test_route_parity(T, E, k, normalize):
    _check_route(wl.router_logits(wl.MOE, T, E, group=E + k), k, normalize)


def test_route_spread_ties_and_signed_zero():
    g = np.random.default_rng(3)
    logits = (g.standard_normal((6, 256)) * 100.0).astype(np.float32)  # e^x underflows for most experts
    logits[1, :] = 0.25                          # all tied
    logits[2, [5, 77, 200]] = 1e9                # a tie at the top
    logits[3, :] = -0.0
    logits[3, [0, 9]] = 0.0                      # -0 and +0 are the same logit: ties by id
    logits[4] = -np.abs(logits[4])
    for normalize in (True, False):
        _check_route(logits, 8, normalize)


def test_route_matches_workload_routing():
    """The device router picks the same experts as the host routing the
    routed-expert benchmarks use for the same uniform logits."""
    T, E, k = wl.MOE_TOKENS, wl.MOE_EXPERTS, wl.MOE_TOPK
    ids, _ = _route(wl.router_logits(wl.MOE, T, E), k, True)
    assert np.array_equal(ids, wl.routing(wl.MOE, T, E, k))


def _swiglu(gate_up, rows, n, ld):
    q = torch.full((q8.q8_quantized_bytes(rows, n),), 0xCD, dtype=torch.uint8, device=dev())
    print(f"q8_swiglu_quantize rows={rows} n={n} ld={ld}", flush=True)
    q8.q8_swiglu_quantize(gate_up, ld, gate_up[:, n:] if ld >= 2 * n else gate_up, ld, rows, n, q)
    return down(q)


@pytest.mark.parametrize("rows,n,scale", [(128, 2048, 1.7), (3, 32, 1.0), (5, 7168, 30.0), (1, 2048, 0.01),
                                          (130, 1024, 1.7)])
def test_swiglu_parity(rows, n, scale):
    """gate and up as the two halves of one fused gate||up output row."""
    g = np.random.default_rng(rows + n)
    gu = (g.standard_normal((rows, 2 * n)) * scale).astype(np.float32)
    got = _swiglu(up(gu), rows, n, 2 * n)
    ref = oracle.swiglu_quantize(gu[:, :n], gu[:, n:])
    if not np.array_equal(got, ref):
        qi, sc = oracle.act_planes(got, rows, n)
        qr, sr = oracle.act_planes(ref, rows, n)
        bad = np.nonzero((qi != qr).any(axis=1) | (sc != sr).any(axis=1))[0]
        pytest.fail(f"SwiGLU codes differ in {bad.size} rows, first {bad[:5]}")


def test_swiglu_closed_forms_and_separate_buffers():
    n = 64
    gate = np.zeros((4, n), np.float32)
    upv = np.ones((4, n), np.float32)
    gate[1] = 1000.0
    upv[1] = np.linspace(-2, 2, n, dtype=np.float32)
    gate[2] = -1000.0
    gate[3] = np.linspace(-40, 40, n, dtype=np.float32)
    q = torch.empty(q8.q8_quantized_bytes(4, n), dtype=torch.uint8, device=dev())
    q8.q8_swiglu_quantize(up(gate), n, up(upv), n, 4, n, q)
    assert np.array_equal(down(q), oracle.swiglu_quantize(gate, upv))


@pytest.mark.parametrize("T,k,n,pad", [(16, 8, 7168, 32), (3, 1, 64, 0), (5, 6, 2048, 4)])
def test_combine_within_rounding_bound(T, k, n, pad):
    g = np.random.default_rng(T * k)
    y = g.standard_normal((T * k, n + pad)).astype(np.float32)
    w = g.random((T, k)).astype(np.float32)
    out = torch.full((T, n), float("nan"), dtype=torch.float32, device=dev())
    print(f"q8_moe_combine tokens={T} topk={k} n={n}", flush=True)
    q8.q8_moe_combine(up(y), n + pad, up(w), T, k, n, out, n)
    ref, S = oracle.moe_combine(np.ascontiguousarray(y[:, :n]), w)
    err = np.abs(down(out).astype(np.float64) - ref.astype(np.float64))
    assert np.all(err <= 2 * k * 2.0 ** -24 * S + np.abs(np.spacing(ref))), "combine outside its rounding bound"
    one = np.zeros((T, k), np.float32)
    one[:, k - 1] = 1.0
    q8.q8_moe_combine(up(y), n + pad, up(one), T, k, n, out, n)
    assert bits_equal(down(out), y.reshape(T, k, n + pad)[:, k - 1, :n])


def _experts_fused(E, H, F, seed):
    """Per expert: gate||up [2F x H] (gate rows first) and down [H x F], packed
    on the device; the oracle's own row-contiguous bytes of both."""
    s_gu, s_d = q8.q8_quantized_bytes(2 * F, H), q8.q8_quantized_bytes(H, F)
    gu = torch.empty(E * s_gu, dtype=torch.uint8, device=dev())
    dn = torch.empty(E * s_d, dtype=torch.uint8, device=dev())
    ref_gu, ref_d = [], []
    for e in range(E):
        w_gu = np.concatenate([wl.weight(wl.MOE, e, F, H, group=100 + seed),
                               wl.weight(wl.MOE, e, F, H, group=200 + seed)])
        w_d = wl.weight(wl.MOE, e, H, F, group=300 + seed)
        q8.q8_repack_weights(quantize(w_gu, q8.Q8_LAYOUT_ROWS), 2 * F, H, gu[e * s_gu:(e + 1) * s_gu])
        q8.q8_repack_weights(quantize(w_d, q8.Q8_LAYOUT_ROWS), H, F, dn[e * s_d:(e + 1) * s_d])
        ref_gu.append(ref_quantize(w_gu, oracle.LAYOUT_ROWS))
        ref_d.append(ref_quantize(w_d, oracle.LAYOUT_ROWS))
    return gu, s_gu, dn, s_d, np.concatenate(ref_gu), np.concatenate(ref_d)


def _abs_codes_rows(w_rows, n, k):
    """Row-contiguous Q8_0 bytes with every code replaced by its magnitude."""
    b = w_rows.reshape(n * (k // 32), 34).copy()
    b[:, 2:] = np.abs(b[:, 2:].view(np.int8).astype(np.int16)).astype(np.uint8)
    return b.reshape(-1)


@pytest.mark.parametrize("normalize", [True, False])
def test_moe_layer(normalize):
    """route -> gate||up grouped GEMV -> SwiGLU + quantize -> down grouped GEMV
    -> combine, all on the device.  Checks: ids and weights bit-exact; the
    device chain equals its stages run one by one (bitwise); the output within
    the bound a different rounding of the gate/up sums can cause downstream --
    a code of h may move by one step, so each output may move by at most
    sum_j w_j * sum_b d_h(b) * sum_i |W_down| (a full quantization step per
    value) plus the GEMV tolerance."""
    E, H, F, T, k = 16, 512, 256, 16, 4
    logits = wl.router_logits(wl.MOE, T, E, group=7)
    x = wl.activation(wl.MOE, 40, T, H)
    gu, s_gu, dn, s_d, ref_gu, ref_d = _experts_fused(E, H, F, seed=1)
    P = T * k
    ids = torch.empty((T, k), dtype=torch.int32, device=dev())
    wts = torch.empty((T, k), dtype=torch.float32, device=dev())
    y_gu = torch.empty((P, 2 * F), dtype=torch.float32, device=dev())
    hq = torch.empty(q8.q8_quantized_bytes(P, F), dtype=torch.uint8, device=dev())
    y_d = torch.empty((P, H), dtype=torch.float32, device=dev())
    out = torch.empty((T, H), dtype=torch.float32, device=dev())
    need = max(q8.q8_grouped_workspace_bytes(T, k, E, 2 * F, H), q8.q8_grouped_workspace_bytes(T, k, E, H, F))
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    xq = quantize(x, q8.Q8_LAYOUT_ACT)
    lg = up(logits)

    def layer():
        q8.q8_moe_route(lg, T, E, k, normalize, ids, wts)
        q8.q8_grouped_matmul(xq, T, 0, ids, T, k, gu, E, s_gu, 2 * F, H, y_gu, ws, need)
        q8.q8_swiglu_quantize(y_gu, 2 * F, y_gu[:, F:], 2 * F, P, F, hq)
        q8.q8_grouped_matmul(hq, P, 1, ids, T, k, dn, E, s_d, H, F, y_d, ws, need)
        q8.q8_moe_combine(y_d, H, wts, T, k, H, out, H)

    print("moe layer on the device", flush=True)
    layer()
    ids_h, w_h, y_gu_h, hq_h, y_d_h, out_h = (down(t) for t in (ids, wts, y_gu, hq, y_d, out))
    assert int(down(ws[:4].view(torch.int32))[0]) == 0
    # the oracle's layer
    ids_r, w_r = oracle.moe_route(logits, k, normalize)
    assert np.array_equal(ids_h, ids_r) and bits_equal(w_h, w_r)
    y_gu_r, _ = oracle.grouped_matmul(ref_quantize(x, oracle.LAYOUT_ACT), T, False, ids_r, ref_gu, E, s_gu, 2 * F,
                                      H)
    h_r = oracle.swiglu_quantize(y_gu_r[:, :F], y_gu_r[:, F:])
    y_d_r, S_d = oracle.grouped_matmul(h_r, P, True, ids_r, ref_d, E, s_d, H, F)
    out_r, _ = oracle.moe_combine(y_d_r, w_r)
    # a full quantization step of h per value, through |W_down|
    _, sc_r = oracle.act_planes(h_r, P, F)
    steps = np.zeros(oracle.quantized_bytes(P, F), np.uint8)
    steps[: P * F] = 1
    steps[P * F:] = sc_r.reshape(-1).view(np.uint8)
    absd = np.concatenate([_abs_codes_rows(ref_d[e * s_d:(e + 1) * s_d], H, F) for e in range(E)])
    B, _ = oracle.grouped_matmul(steps, P, True, ids_r, absd, E, s_d, H, F)
    bound = (w_r.astype(np.float64)[:, :, None] * (1.01 * B + 2e-5 * S_d + 2 * k * 2.0 ** -24 * np.abs(y_d_r))
             .reshape(T, k, H)).sum(axis=1)
    assert np.all(np.abs(out_h.astype(np.float64) - out_r) <= bound + 1e-30)
    # the chain equals its stages run alone, bit for bit
    out1 = torch.empty_like(out)
    q8.q8_moe_combine(up(y_d_h), H, up(w_h), T, k, H, out1, H)
    assert bits_equal(down(out1), out_h)
    hq1 = torch.empty_like(hq)
    q8.q8_swiglu_quantize(up(y_gu_h), 2 * F, up(np.ascontiguousarray(y_gu_h[:, F:])), F, P, F, hq1)
    assert np.array_equal(down(hq1), hq_h)
    # and the second call (same workspace) repeats the first
    layer()
    assert bits_equal(down(out), out_h)
