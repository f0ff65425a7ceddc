"""The GEMM-tiled byte order of block scales, written independently of the
library (a reshape), for comparing the library's tiled scales with the oracle's
row-major ones."""
import numpy as np


def tile_scales(s, per_step):
    """Row-major [R, J] block scales -> the tiled byte order: rows in blocks of 64,
    scales in steps of per_step (one step = 128 K values), each (row block, step)
    one run of 64 rows x per_step bytes.  Returns the same shape [R, J]."""
    R, J = s.shape
    return np.ascontiguousarray(
        s.reshape(R // 64, 64, J // per_step, per_step).transpose(0, 2, 1, 3)).reshape(R, J)


def untile_scales(t, per_step):
    """Inverse of tile_scales: tiled-order scales [R, J] -> row-major [R, J]."""
    R, J = t.shape
    return np.ascontiguousarray(
        t.reshape(R // 64, J // per_step, 64, per_step).transpose(0, 2, 1, 3)).reshape(R, J)
