"""Subsequence index maps (Skiparse, block) from the library's host path
equal the oracle's membership-predicate maps bit for bit.  CPU only."""
import numpy as np
import pytest

import oracle
import spatiotemporal_attention_amd as osp

CASES = [
    (n, k) for n in (16, 48, 64, 320, 720, 4096, 28800) for k in (1, 2, 3, 4, 8)
] + [(86400, 4), (17550, 3), (1 << 20, 16), (9, 3), (1, 1)]


@pytest.mark.parametrize("n,k", CASES)
def test_host_maps_bitexact(n, k):
    for mode in ("full", "skiparse_single", "skiparse_group", "block"):
        div = k * k if mode == "skiparse_group" else (1 if mode == "full" else k)
        if n % div:
            with pytest.raises(osp.OspError):
                osp.osp_skiparse_index(mode, k, n)
            continue
        perm, inv = osp.osp_skiparse_index(mode, k, n)
        want_perm, want_inv = oracle.skiparse_index(mode, k, n)
        assert perm.dtype == np.int32 and inv.dtype == np.int32
        assert np.array_equal(perm, want_perm), (mode, n, k)
        assert np.array_equal(inv, want_inv), (mode, n, k)


def test_large_ratio_division_paths():
    # the library divides by k with multiply-high; exercise many divisors
    for k in list(range(1, 40)) + [63, 64, 65, 127, 255, 256]:
        n = k * k * (3 if k < 64 else 1)
        perm, _ = osp.osp_skiparse_index("skiparse_group", k, n)
        assert np.array_equal(perm, oracle.skiparse_index("skiparse_group", k, n)[0]), k
    for k in list(range(1, 40)) + [63, 64, 65, 127, 255, 256, 1000, 4096]:
        perm, _ = osp.osp_skiparse_index("skiparse_single", k, k * 7)
        assert np.array_equal(perm, oracle.skiparse_index("skiparse_single", k, k * 7)[0]), k


GRIDS_2D = [(1, 2, 2), (2, 4, 4), (3, 6, 9), (5, 8, 8), (2, 12, 12), (24, 30, 40), (16, 36, 64),
            (1, 9, 27), (2, 3, 5), (4, 16, 8)]


@pytest.mark.parametrize("grid", GRIDS_2D)
def test_host_maps_bitexact_2d(grid):
    n = int(np.prod(grid))
    for mode in ("skiparse2d_single", "skiparse2d_group"):
        for k in (1, 4, 9, 16):
            s = int(round(k ** 0.5))
            step = s if mode == "skiparse2d_single" else s * s
            if grid[1] % step or grid[2] % step:
                with pytest.raises(osp.OspError):
                    osp.osp_skiparse_index3d(mode, k, grid)
                continue
            perm, inv = osp.osp_skiparse_index3d(mode, k, grid)
            want_perm, want_inv = oracle.skiparse_index(mode, k, n, grid)
            assert np.array_equal(perm, want_perm), (mode, grid, k)
            assert np.array_equal(inv, want_inv), (mode, grid, k)
    # the grid form agrees with the plain form on the 1D modes
    for mode, k in (("full", 1), ("skiparse_single", 2), ("block", grid[0])):
        if n % k == 0:
            assert np.array_equal(osp.osp_skiparse_index3d(mode, k, grid)[0],
                                  osp.osp_skiparse_index(mode, k, n)[0])


def test_2d_modes_need_the_grid():
    for mode in ("skiparse2d_single", "skiparse2d_group"):
        with pytest.raises(osp.OspError) as e:
            osp.osp_skiparse_index(mode, 4, 64)
        assert e.value.code == 3 and "grid" in e.value.message
    with pytest.raises(osp.OspError):
        osp.osp_skiparse_index3d("skiparse2d_single", 4, (0, 4, 4))
