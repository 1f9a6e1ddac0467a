"""q8_quantize_matmul_sequence: a chain of decode GEMVs in one persistent
launch.  Every step's output must be bit-identical to q8_quantize_matmul on
that step alone (the same arithmetic, only the scheduling differs), sampled
outputs must meet the oracle's bound, the workspace must come back zero, and
repeated calls and graph replays must reproduce the eager result."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from decode_q8_amd import q8
from tests.gpu_helpers import bits_equal, check_tol, dev, down, ref_quantize, require_gpu, up, weights_packed

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _chain(shapes, m, seed):
    """Weights (packed, plus the rows layout for the oracle), fp32 inputs and
    output buffers for a chain of (n, k) steps."""
    steps = []
    for i, (n, k) in enumerate(shapes):
        w = wl.weight(wl.BATCHED, seed + 7 * i, n, k)
        _, wp = weights_packed(w)
        xh = wl.activation(wl.BATCHED, seed + 7 * i + 1, m, k)
        y = torch.full((m, n), float("nan"), dtype=torch.float32, device=dev())
        steps.append(dict(n=n, k=k, w=wp, w_host=w, x_host=xh, x=up(xh), y=y))
    return steps


def _tuples(steps):
    return [(s["x"], s["k"], s["w"], s["n"], s["k"], s["y"], s["n"]) for s in steps]


def _run(steps, m, ws=None):
    t = _tuples(steps)
    need = q8.q8_sequence_workspace_bytes(t, m)
    if ws is None:
        ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    q8.q8_quantize_matmul_sequence(t, m, ws, ws.numel())
    q8.check_sequence(ws)
    return ws


def _single(s, m):
    return down(q8.quantize_matmul(s["x"], s["w"], q8.Q8_LAYOUT_PACKED, s["n"]))


LAYER = [(3072, 2048), (2048, 2048), (16384, 2048), (2048, 8192)]  # fused QKV, O, gate||up, down


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 6, 7, 8])
def test_decode_layers_bit_identical_to_single_launches(m):
    """Two decode layers plus a head: every step equals its own launch bit for
    bit, sampled outputs meet the oracle bound, the workspace returns to zero."""
    shapes = LAYER * 2 + [(8192, 2048)]
    steps = _chain(shapes, m, seed=300 + m)
    ws = _run(steps, m)
    assert int(down(ws).astype(np.uint8).any()) == 0, "workspace not returned to zero"
    rng = np.random.default_rng(m)
    for i, s in enumerate(steps):
        y = down(s["y"])
        assert bits_equal(y, _single(s, m)), f"step {i} ({s['n']}x{s['k']}) differs from its own launch"
        if i in (0, 3, len(steps) - 1):
            mi = rng.integers(0, m, 256)
            ni = rng.integers(0, s["n"], 256)
            y_ref, S = oracle.matmul_points(ref_quantize(s["x_host"], oracle.LAYOUT_ACT), m,
                                            ref_quantize(s["w_host"], oracle.LAYOUT_ROWS), s["n"], s["k"], mi, ni)
            check_tol(y[mi, ni], y_ref, S, f"sequence step {i} m={m}")


def test_general_path_many_groups_per_wave():
    """A step whose workgroups hold more groups than waves (k = 8448 on a wide
    matrix) runs the general kernel; it still equals its own launch."""
    shapes = [(2048, 2048), (16384, 8448), (2048, 8192), (64, 256)]
    steps = _chain(shapes, 2, seed=400)
    ws = _run(steps, 2)
    assert int(down(ws).astype(np.uint8).any()) == 0
    for i, s in enumerate(steps):
        assert bits_equal(down(s["y"]), _single(s, 2)), f"step {i}"


@pytest.mark.parametrize("m", [1, 3, 8])
def test_split_steps_back_to_back_and_last(m):
    """Steps whose tiles are split over several workgroups (long rows, few
    tiles): two in a row (the second chains the first's segment sums while
    handing over its own), one followed by a single-unit step (that unit
    chains every tile of it), and one as the last step (chained inside the
    step itself).  Every step equals its own launch; the workspace returns to
    zero."""
    shapes = [(2048, 8192), (1024, 16384), (64, 256), (2048, 8192), (512, 2048), (1024, 8192)]
    steps = _chain(shapes, m, seed=700 + m)
    ws = _run(steps, m)
    assert int(down(ws).astype(np.uint8).any()) == 0, "workspace not returned to zero"
    for i, s in enumerate(steps):
        assert bits_equal(down(s["y"]), _single(s, m)), f"step {i} ({s['n']}x{s['k']}) differs from its own launch"


def test_maximum_length_and_repeat():
    """Q8_SEQUENCE_MAX_STEPS small steps (the longest argument block), called
    twice on one workspace: identical results, workspace zero after each."""
    shapes = [(64 * (1 + i % 3), 256 * (1 + i % 2)) for i in range(q8.Q8_SEQUENCE_MAX_STEPS)]
    steps = _chain(shapes, 1, seed=500)
    ws = _run(steps, 1)
    first = [down(s["y"]).copy() for s in steps]
    assert int(down(ws).astype(np.uint8).any()) == 0
    for s in steps:
        s["y"].fill_(float("nan"))
    _run(steps, 1, ws)
    assert int(down(ws).astype(np.uint8).any()) == 0
    for i, s in enumerate(steps):
        assert bits_equal(down(s["y"]), first[i]), f"step {i} changed on the second call"
        if i % 9 == 0:
            assert bits_equal(first[i], _single(s, 1)), f"step {i}"


def test_graph_replay():
    """Captured once, replayed several times with eager work in between: every
    replay reproduces the eager outputs and leaves the workspace zero."""
    steps = _chain(LAYER + [(4096, 2048)], 1, seed=600)
    t = _tuples(steps)
    ws = torch.zeros(q8.q8_sequence_workspace_bytes(t, 1), dtype=torch.uint8, device=dev())
    q8.q8_quantize_matmul_sequence(t, 1, ws, ws.numel())
    eager = [down(s["y"]).copy() for s in steps]
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        q8.q8_quantize_matmul_sequence(t, 1, ws, ws.numel(), stream)
    for r in range(4):
        for s in steps:
            s["y"].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(down(ws).astype(np.uint8).any()) == 0, f"replay {r}: workspace"
        for i, s in enumerate(steps):
            assert bits_equal(down(s["y"]), eager[i]), f"replay {r} step {i}"


def test_no_device_queries_after_the_first_call():
    """The grid size (resident workgroups per CU, CU count) is discovered once
    per device and kernel variant and cached: repeated calls make no further
    device queries."""
    steps = _chain(LAYER, 1, seed=650)
    ws = _run(steps, 1)
    torch.cuda.synchronize()
    after_first = q8.q8_device_queries()
    assert after_first >= 1
    for _ in range(5):
        _run(steps, 1, ws)
    torch.cuda.synchronize()
    assert q8.q8_device_queries() == after_first
    assert int(down(ws).astype(np.uint8).any()) == 0
