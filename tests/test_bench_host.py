"""Host-side arithmetic of the benchmark: the exact (query, key) pair counts
behind the windowed branches' algorithmic FLOPs, against a brute-force count
of the key sets J(i) defined in the oracle (frame residues, group positions,
causal or centred band)."""
import numpy as np
import pytest

import bench
from oracle import frame_index_maps


def _brute_pairs(T, L, w, dil, fo, centered):
    _, r, p = frame_index_maps(T, L, dil, fo)
    same = r[:, None] == r[None, :]
    dp = p[None, :] - p[:, None]                    # key position - query position
    band = (np.abs(dp) <= w // 2) if centered else ((dp > -w) & (dp <= 0))
    return int(np.count_nonzero(same & band))


@pytest.mark.parametrize("T,L,w,dil,fo", [(60, 6, 7, 1, 0), (60, 6, 14, 4, 0), (67, 6, 9, 4, 3),
                                          (96, 8, 40, 6, 0), (96, 8, 5, 12, 1), (50, 50, 200, 1, 0),
                                          (84, 4, 1, 6, 0)])
@pytest.mark.parametrize("centered", [False, True])
def test_window_pairs_match_bruteforce(T, L, w, dil, fo, centered):
    assert bench.window_pairs(T, L, w, dil, fo, centered) == _brute_pairs(T, L, w, dil, fo, centered)


def _brute_sets(T, L, w, dil, fo, centered):
    """Boolean [query, key] membership of the SWA and DSWA windows."""
    sets = []
    for dl in (1, dil):
        _, r, p = frame_index_maps(T, L, dl, fo)
        same = r[:, None] == r[None, :]
        dp = p[None, :] - p[:, None]
        band = (np.abs(dp) <= w // 2) if centered else ((dp > -w) & (dp <= 0))
        sets.append(same & band)
    return sets


@pytest.mark.parametrize("T,L,w,dil", [(60, 6, 7, 4), (60, 6, 6, 4), (67, 6, 9, 3), (96, 8, 8, 6),
                                        (96, 8, 17, 3), (50, 7, 1, 2), (70, 10, 10, 2)])
@pytest.mark.parametrize("centered", [False, True])
def test_shared_frame_pairs_match_bruteforce(T, L, w, dil, centered):
    """The own-frame pairs are exactly the pairs both windows hold (within the
    stated window sizes), and the hybrid pair count is the union's size."""
    fits = (w // 2 < L) if centered else (w <= (dil - 1) * L + 1)
    if not fits:
        pytest.skip("window reaches a shared frame of the other branch")
    swa, dswa = _brute_sets(T, L, w, dil, 0, centered)
    assert bench.shared_frame_pairs(T, L, w, centered) == int(np.count_nonzero(swa & dswa))
    assert bench.hybrid_pairs(T, L, w, dil, centered) == int(np.count_nonzero(swa | dswa))
