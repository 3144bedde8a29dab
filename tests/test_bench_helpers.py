"""Host-side reporting helpers of bench.py, checked against the oracle."""
import numpy as np

import bench
import oracle
import workloads


def _geoms():
    rng = np.random.default_rng(21)
    out = [(5, 48, 1, 1, 0, 16, 16, 0, 0), (3, 80, 0, 0, -1, 16, 16, 0, 0), (9, 16, 2, 0, 8, 16, 16, 0, 0),
           (4, 112, 3, 3, 1, 16, 16, 0, 0), (6, 80, 0, 1, 1, 16, 16, 1, 2), (7, 48, 1, 0, 0, 16, 16, 0, 3)]
    for _ in range(12):
        T = 16 * int(rng.integers(1, 12))
        F_ = int(rng.integers(1, 10))
        r, nr = int(rng.integers(-1, F_)), int(rng.integers(0, 3))
        if r + max(1, nr) > F_:
            nr = 0
        out.append((F_, T, int(rng.integers(0, 4)), int(rng.integers(0, 4)), r, 16, 16, int(rng.integers(0, 2)), nr))
    return out


def test_partial_tile_share_matches_bruteforce():
    """bench.partial_tile_share (frame-level prefix sums) equals the oracle's
    token-level count of live and partly live tiles, for several tile sizes."""
    for g in _geoms():
        w = workloads.make_workload("t", 1, 1, g[0], g[1], 64, "bf16", g[2], g[3], g[4], g[5], g[6],
                                    ref_queries_global=g[7], ref_count=g[8])
        for tile in (32, 48, 128):
            got = bench.partial_tile_share(w, tile)
            partial, live = oracle.partial_blocks_if_tiled(oracle.MaskGeometry(*g), tile)
            assert (got["partial_tiles"], got["live_tiles"]) == (partial, live), (g, tile)


def test_partial_tile_share_on_the_workloads():
    for i in (1, 2, 4):
        w = workloads.workload(i)
        got = bench.partial_tile_share(w)
        partial, live = oracle.partial_blocks_if_tiled(oracle.MaskGeometry(*w.mask_tuple()), 128)
        assert (got["partial_tiles"], got["live_tiles"]) == (partial, live), i
    assert bench.partial_tile_share(workloads.workload(4))["partial_tiles"] == 0   # dense mask, T = 8 tiles
