"""The tests' tiled-scale reshape against the byte-offset formula that
include/mxq.h states for MXQ_SCALES_TILED, element by element (CPU)."""
import numpy as np
import pytest

from tests.scale_order import tile_scales, untile_scales


@pytest.mark.parametrize("R,J,P", [(128, 24, 4), (64, 8, 8), (192, 40, 8)])
def test_tile_scales_matches_header_formula(R, J, P):
    s = np.arange(R * J, dtype=np.int64).reshape(R, J)
    t = tile_scales(s, P).reshape(-1)
    for r in range(R):
        for j in range(J):
            assert t[((r // 64) * (J // P) + j // P) * 64 * P + (r % 64) * P + j % P] == s[r, j]


def test_untile_inverts_tile():
    s = np.arange(128 * 40, dtype=np.int64).reshape(128, 40)
    for P in (4, 8):
        np.testing.assert_array_equal(untile_scales(tile_scales(s, P), P), s)
