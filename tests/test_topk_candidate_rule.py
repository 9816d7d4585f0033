"""The candidate-tile rule of the top-k path without stored logits, checked by
brute force on the CPU (numpy only; no oracle, no GPU).

Rule (m* = the k-th largest of a row's 128-wide tile maxima, NaN entries
ignored): when m* is above -inf, the exact top-k under the order (value
descending, id ascending, NaN never) lies in the tiles whose maximum exceeds
m* together with the first k - |A| tiles, by index, whose maximum equals m*;
there are exactly k such tiles.  When m* is -inf every tile is needed, and
rows exist where the first k tied tiles do not suffice.  A wrong reading of
the rule (taking the last tied tiles, taking only the k tiles with the
largest maxima by value and index, or a strict/loose comparison swapped)
fails the checks below on the tie-heavy rows.
"""

import numpy as np
import pytest

TILE = 128


def _tile_max(z):
    V = z.size
    nst = (V + TILE - 1) // TILE
    zz = np.full(nst * TILE, -np.inf)
    zz[:V] = np.where(np.isnan(z), -np.inf, z)
    return zz.reshape(nst, TILE).max(axis=1)


def _exact_topk(z, k, among=None):
    ids = np.arange(z.size) if among is None else np.asarray(among)
    ids = ids[~np.isnan(z[ids])]
    order = np.lexsort((ids, -z[ids]))       # value descending, then id ascending
    return ids[order][:k].tolist()


def _candidates(tm, k):
    srt = np.sort(tm)[::-1]
    mstar = srt[k - 1] if tm.size >= k else -np.inf
    if not mstar > -np.inf:
        return None
    a = [j for j in range(tm.size) if tm[j] > mstar]
    b = [j for j in range(tm.size) if tm[j] == mstar][:k - len(a)]
    return a + b


def _rows(seed, n):
    g = np.random.Generator(np.random.PCG64(seed))
    for trial in range(n):
        V = int(g.integers(1, 12000))
        k = min(int(g.integers(1, 65)), V)
        kind = trial % 4
        if kind == 0:
            z = g.integers(-3, 4, V).astype(np.float64)           # heavy ties
        elif kind == 1:
            z = g.standard_normal(V)
        elif kind == 2:
            z = g.integers(-2, 3, V).astype(np.float64)
            z[g.random(V) < 0.3] = np.nan
        else:
            z = g.choice(np.array([-np.inf, np.inf, np.nan, 0.0, 1.0]), V)
        yield z, k


def test_candidate_tiles_hold_the_exact_topk():
    checked = 0
    for z, k in _rows(11, 600):
        tm = _tile_max(z)
        cand = _candidates(tm, k)
        if cand is None:
            continue
        assert len(cand) == k and len(set(cand)) == k
        inside = np.concatenate([np.arange(j * TILE, min((j + 1) * TILE, z.size)) for j in cand])
        assert _exact_topk(z, k, inside) == _exact_topk(z, k)
        checked += 1
    assert checked > 300


def test_last_tied_tiles_would_be_wrong():
    """Tied tiles taken from the end instead of the start lose the smaller
    ids: a row of 8 tiles that all hold the value 1.0 once, k = 3."""
    z = np.zeros(8 * TILE)
    z[np.arange(8) * TILE + 5] = 1.0
    tm = _tile_max(z)
    cand = _candidates(tm, 3)
    assert cand == [0, 1, 2]
    assert _exact_topk(z, 3) == [5, TILE + 5, 2 * TILE + 5]


def test_minus_inf_rows_need_every_tile():
    """m* = -inf: the first k tiles can hold only NaN, the -inf entries that
    make the cut sit further on, so all tiles are candidates."""
    z = np.full(6 * TILE, np.nan)
    z[4 * TILE + 7] = -np.inf
    z[5 * TILE + 1] = 2.0
    k = 3
    assert _candidates(_tile_max(z), k) is None
    assert _exact_topk(z, k) == [5 * TILE + 1, 4 * TILE + 7]
