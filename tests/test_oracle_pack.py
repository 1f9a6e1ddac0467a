"""Pins for the oracle's packed-tile layout.

The pages' packed layout keeps the weight bytes and only changes which bytes
arrive together: one 16-row tile/block record is 544 bytes, exactly the size
of 16 ordinary 34-byte Q8_0 blocks ("Ember packed Q8 decode" post, packed
16-row tile diagram and the paragraph after it).  This project's gfx950 layout
uses records of 64 rows x 8 blocks = 17,408 bytes = 32 x 544, with 16-byte
chunks of one row's values interleaved across the 64 rows, and each row's 8
scales together in one 16-byte chunk.

Pins: the size identity, the bytewise round trip, and that packing is a pure
permutation of the bytes (sorted multisets equal).  The placement test spells
out the documented byte positions of one record.
"""
import numpy as np
import pytest

import oracle


def _rows(n, k, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    return oracle.quantize_rows(w, oracle.LAYOUT_ROWS)


def test_size_identity():
    assert 16 * 34 == 544
    assert 64 * 8 * 34 == 17408 == 32 * 544
    for n, k in [(64, 256), (128, 2048), (2048, 2048), (128256, 2048), (7168, 2048), (2048, 7168)]:
        assert oracle.quantized_bytes(n, k) == n * (k // 32) * 34
        assert oracle.quantized_bytes(n, k) % 17408 == 0


@pytest.mark.parametrize("n,k", [(64, 256), (128, 512), (192, 1792)])
def test_round_trip_and_permutation(n, k):
    wr = _rows(n, k, seed=n + k)
    wp = oracle.pack(wr, n, k)
    assert wp.size == wr.size == n * k // 32 * 34
    assert np.array_equal(oracle.unpack(wp, n, k), wr)
    assert np.array_equal(np.sort(wp), np.sort(wr))
    assert not np.array_equal(wp, wr)


def test_record_placement():
    n, k = 128, 512  # 2 row tiles x 2 column groups
    wr = _rows(n, k, seed=3)
    wp = oracle.pack(wr, n, k)
    q, d = oracle.rows_planes(wr, n, k)
    groups = k // 256
    for T in range(2):
        for G in range(groups):
            rec = wp[(T * groups + G) * 17408:(T * groups + G + 1) * 17408]
            vals = rec[:16384].view(np.int8).reshape(8, 2, 64, 16)      # [bb][h][r][j]
            scales = rec[16384:].view(np.uint16).reshape(64, 8)          # [r][bb]
            for r in (0, 1, 31, 63):
                row = 64 * T + r
                for bb in range(8):
                    col = 256 * G + 32 * bb
                    assert np.array_equal(vals[bb, 0, r], q[row, col:col + 16])
                    assert np.array_equal(vals[bb, 1, r], q[row, col + 16:col + 32])
                    assert scales[r, bb] == d[row, 8 * G + bb]


def test_pack_rejects_unsupported_shapes():
    wr = _rows(64, 256, seed=4)
    with pytest.raises(ValueError):
        oracle.pack(wr[: 32 * 8 * 34], 32, 256)
    with pytest.raises(ValueError):
        oracle.pack(_rows(64, 96, seed=5), 64, 96)
