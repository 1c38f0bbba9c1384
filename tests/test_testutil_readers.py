"""The GPU tests read packed codes back with their own bit readers; pin those
readers to the oracle's packers (round trip on random indices)."""
import numpy as np

import oracle as O
import tq_testutil as U


def test_row_and_tile32_readers_invert_oracle_packers():
    rng = np.random.default_rng(0)
    for b in (1, 2, 3, 4, 5, 8):
        idx = rng.integers(0, 1 << b, (7, 40))
        assert np.array_equal(U.read_rows(O.pack_rows(idx, b), 40, b), idx)
        idx2 = rng.integers(0, 1 << b, (70, 6))
        assert np.array_equal(U.read_tile32(O.pack_tile32(idx2, b, 3), 6, b, 70), idx2)


def test_boundary_distance():
    c, t = O.lloyd_max(16, 3)
    y = np.random.default_rng(1).uniform(-0.6, 0.6, (50, 16))
    d1 = U.boundary_distance(t, y, O.coord_index(y, t))
    assert np.array_equal(d1, np.min(np.abs(y[..., None] - t), axis=-1))
