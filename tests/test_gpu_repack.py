"""GPU weight repack (q8_repack_weights) against the oracle's pack: bytewise
equal, same size, and a pure permutation of the source bytes."""
import numpy as np
import pytest

import oracle
import workloads as wl
from decode_q8_amd import q8
from tests.gpu_helpers import down, quantize, ref_quantize, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("n,k", [(64, 256), (128, 512), (192, 7168), (2048, 2048), (7168, 2048)])
def test_repack_matches_oracle(n, k):
    w = wl.weight(wl.SINGLE, 100 + n, n, k)
    wr = quantize(w, q8.Q8_LAYOUT_ROWS)
    wp = q8.repack(wr, n, k)
    rows_ref = ref_quantize(w, oracle.LAYOUT_ROWS)
    assert np.array_equal(down(wr), rows_ref)
    got = down(wp)
    assert got.size == rows_ref.size == n * k // 32 * 34
    assert np.array_equal(got, oracle.pack(rows_ref, n, k))
