"""Helpers for the GPU parity tests: device transfers, quantization through the
library, and the acceptance bound |y - y_ref| <= 1e-5 * sum_b |t_b|."""
import numpy as np
import pytest
import torch

from decode_q8_amd import q8

TOL = 1e-5  # acceptance bound, relative to the sum of |block terms| of the output


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev():
    return torch.device("cuda", 0)


def up(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def down(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def quantize(x: np.ndarray, layout: int) -> torch.Tensor:
    """Host fp32 -> device quantized buffer, quantized by the library."""
    xt = up(np.ascontiguousarray(x, np.float32))
    return q8.quantize(xt, layout)


def ref_quantize(a: np.ndarray, layout: int) -> np.ndarray:
    """The oracle's own quantization of host fp32 rows (expected values and
    oracle inputs never come from the GPU); large inputs split over threads
    by row ranges."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    a = np.ascontiguousarray(a, np.float32)
    rows, k = a.shape
    if rows * k < (1 << 22):
        return oracle.quantize_rows(a, layout)
    step = (rows + 7) // 8
    parts = list(ThreadPoolExecutor(8).map(lambda r0: oracle.quantize_rows(a[r0:r0 + step], layout),
                                           range(0, rows, step)))
    if layout == oracle.LAYOUT_ROWS:
        return np.concatenate(parts)
    codes = np.concatenate([p[: p.size // 34 * 32] for p in parts])
    scales = np.concatenate([p[p.size // 34 * 32:] for p in parts])
    return np.concatenate([codes, scales])


def weights_packed(w: np.ndarray):
    """Host fp32 [n][k] -> (rows-layout device buffer, packed device buffer)."""
    n, k = w.shape
    wr = quantize(w, q8.Q8_LAYOUT_ROWS)
    wp = q8.repack(wr, n, k)
    return wr, wp


def check_tol(y: np.ndarray, y_ref: np.ndarray, S: np.ndarray, what: str = ""):
    y = np.asarray(y, np.float64)
    err = np.abs(y - np.asarray(y_ref, np.float64))
    bound = TOL * np.asarray(S, np.float64)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(int(np.argmax(err - bound)), err.shape)
        pytest.fail(f"{what}: {int(bad.sum())} outputs outside 1e-5*S; worst at {i}: got {y[i]!r} "
                    f"ref {y_ref[i]!r} S {S[i]!r}")


def bits_equal(a, b) -> bool:
    a = np.ascontiguousarray(a, np.float32)
    b = np.ascontiguousarray(b, np.float32)
    return a.shape == b.shape and np.array_equal(a.view(np.uint32), b.view(np.uint32))
