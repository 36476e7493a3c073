"""CPU check of how the prefill grouped GEMMs deal their tiles to
workgroups: the grid is sized on the host for the largest possible number
of route tiles (rounded up to a whole multiple of 8 columns), the tiles that
exist are counted on the device, and each workgroup b maps to logical tile
L = x*q + i (XCD x = b mod 8, i = b div 8, q = ceil(valid / 8)) or exits.
Every existing (route tile, weight tile) pair must run exactly once, for
any count of existing route tiles up to the maximum."""
import numpy as np
import pytest


def remap(b, nvalid):
    """Logical tile of workgroup b, or -1 (the kernels' XCD dealing)."""
    x, i = b & 7, b >> 3
    q = (nvalid + 7) >> 3
    L = x * q + i
    return np.where((i < q) & (L < nvalid), L, -1)


def grid_columns(max_tiles, round_to_8=True):
    """Columns of the GEMM grid for max_tiles route tiles (the host rule)."""
    return (max_tiles + 7) // 8 * 8 if round_to_8 else max_tiles


def tiles_run(max_tiles, n_tiles, nnt, round_to_8=True):
    nb = grid_columns(max_tiles, round_to_8) * nnt  # blockIdx.y * gridDim.x + blockIdx.x
    L = remap(np.arange(nb), n_tiles * nnt)
    return np.sort(L[L >= 0])


@pytest.mark.parametrize("nnt", [1, 2, 3, 4, 8, 16, 28])
def test_every_existing_tile_runs_exactly_once(nnt):
    for max_tiles in range(1, 260):
        for n_tiles in sorted({1, max(1, max_tiles // 3), max(1, max_tiles // 2),
                               max(1, max_tiles - 1), max_tiles}):
            got = tiles_run(max_tiles, n_tiles, nnt)
            assert np.array_equal(got, np.arange(n_tiles * nnt)), (max_tiles, n_tiles, nnt)


def test_a_grid_of_max_tiles_columns_misses_tiles():
    # without rounding the columns up to a multiple of 8, the last XCDs'
    # ranges run short and some existing tiles never run (the check above
    # would catch the rule going back)
    misses = [(m, n) for m in range(1, 200) for n in (m,)
              if tiles_run(m, n, 1, round_to_8=False).size < n]
    assert misses, "expected the unrounded grid to drop tiles somewhere"
    # 17 tiles in a grid of 17 columns: q = 3, but only XCD 0 gets a third workgroup
    assert (17, 17) in misses
