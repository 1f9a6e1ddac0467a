"""q8_quantize_matmul_sequence_noalloc, the allocation-free decode-step
sequence (its workspace is the library's own per-GPU array), against
q8_quantize_matmul_sequence with a caller-allocated workspace: outputs
bit-identical on consecutive calls, the second with a smaller input (fewer
steps, fewer rows, narrower matrices), the status word delivered, a large
call after the small one still exact, and sampled outputs within the
oracle's bound."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from decode_q8_amd import q8
from tests.gpu_helpers import bits_equal, check_tol, dev, down, ref_quantize, require_gpu, up, weights_packed

pytestmark = pytest.mark.gpu

LAYER = [(3072, 2048), (2048, 2048), (16384, 2048), (2048, 8192)]  # fused QKV, O, gate||up, down


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _chain(shapes, m, seed):
    steps = []
    for i, (n, k) in enumerate(shapes):
        w = wl.weight(wl.BATCHED, seed + 7 * i, n, k)
        _, wp = weights_packed(w)
        xh = wl.activation(wl.BATCHED, seed + 7 * i + 1, m, k)
        steps.append(dict(n=n, k=k, w=wp, w_host=w, x_host=xh, x=up(xh)))
    return steps


def _tuples(steps, ys):
    return [(s["x"], s["k"], s["w"], s["n"], s["k"], y, s["n"]) for s, y in zip(steps, ys)]


def _outputs(steps, m):
    return [torch.full((m, s["n"]), float("nan"), dtype=torch.float32, device=dev()) for s in steps]


def _compare(steps, m, what):
    """One no-alloc call and one call with a caller workspace on the same
    inputs: every output bit-identical, status 0, workspace back to zero."""
    y_na = _outputs(steps, m)
    status = torch.full((1,), -1, dtype=torch.int32, device=dev())
    q8.q8_quantize_matmul_sequence_noalloc(_tuples(steps, y_na), m, status)
    y_ws = _outputs(steps, m)
    t = _tuples(steps, y_ws)
    ws = torch.zeros(q8.q8_sequence_workspace_bytes(t, m), dtype=torch.uint8, device=dev())
    q8.q8_quantize_matmul_sequence(t, m, ws, ws.numel())
    assert int(down(status)[0]) == 0, f"{what}: status"
    assert int(down(ws[:4].view(torch.int32))[0]) == 0
    for i, s in enumerate(steps):
        a, b = down(y_na[i]), down(y_ws[i])
        assert not np.isnan(a).any(), f"{what}: step {i} not written"
        assert bits_equal(a, b), f"{what}: step {i} ({s['n']}x{s['k']}) differs from the workspace entry point"
    return y_na


def test_two_calls_in_a_row_second_smaller():
    big = _chain(LAYER * 2 + [(8192, 2048)], 4, seed=810)       # split down steps hand their sums over
    small = _chain([(2048, 2048), (1024, 8192), (128, 256)], 2, seed=820)
    y_big = _compare(big, 4, "first call (9 steps, m = 4)")
    _compare(small, 2, "second call (3 steps, m = 2)")
    # a large call after the small one: its leftovers must not leak in
    _compare(big, 4, "third call (9 steps, m = 4)")
    rng = np.random.default_rng(5)
    for i in (0, 3, len(big) - 1):
        s = big[i]
        mi, ni = rng.integers(0, 4, 256), rng.integers(0, s["n"], 256)
        y_ref, S = oracle.matmul_points(ref_quantize(s["x_host"], oracle.LAYOUT_ACT), 4,
                                        ref_quantize(s["w_host"], oracle.LAYOUT_ROWS), s["n"], s["k"], mi, ni)
        check_tol(down(y_big[i])[mi, ni], y_ref, S, f"no-alloc step {i}")


def test_without_status_pointer_and_in_a_graph():
    """status may be NULL; the call captures into a graph (no allocation, the
    scratch cleared by a kernel) and every replay reproduces the eager run."""
    steps = _chain(LAYER + [(4096, 2048)], 1, seed=830)
    ys = _outputs(steps, 1)
    t = _tuples(steps, ys)
    q8.q8_quantize_matmul_sequence_noalloc(t, 1)
    eager = [down(y).copy() for y in ys]
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        q8.q8_quantize_matmul_sequence_noalloc(t, 1, None, stream)
    for r in range(3):
        for y in ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, y in enumerate(ys):
            assert bits_equal(down(y), eager[i]), f"replay {r} step {i}"
