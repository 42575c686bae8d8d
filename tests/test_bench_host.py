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
