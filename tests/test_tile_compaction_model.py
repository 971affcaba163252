"""Host model of the tile-parallel compaction's ordering (CPU).

The kernel (compact.hip, compact_tiles_kernel) moves one tile of T destination rows per block:
it loads the tile's source rows kept[i] into registers, publishes a flag, waits until every
earlier tile of its stream has published, then writes rows [qT, qT + T).  Blocks take their tiles
from a counter in order.  This model replays that protocol over many random interleavings, with a
bounded number of resident blocks, and checks that
  * every schedule ends (no wait can block forever), and
  * the result equals indexing the original rows by kept (row i takes row kept[i], kept
    ascending; chenxutan.com/d/2624 section 4.2),
and that the same replay without the wait does produce wrong rows, so the model can see the
hazard the wait removes.
"""
import numpy as np
import pytest


def _kept(rng, N, B):
    return np.sort(rng.choice(N, size=B, replace=False)).astype(np.int64)


def _replay(rows, kept, T, rng, slots, wait=True):
    """One random interleaving of the tile protocol on a copy of `rows`; returns the result, or
    None if the schedule could not finish."""
    out = rows.copy()
    B = len(kept)
    tiles = (B + T - 1) // T
    published = [False] * tiles
    next_tile = 0                      # the counter
    running = {}                       # tile -> state: 0 = to load, 1 = waiting, 2 = to write
    held = {}
    done = 0
    steps = 0
    while done < tiles:
        steps += 1
        if steps > 100 * tiles + 1000:
            return None
        # a free slot takes the next tile from the counter
        if next_tile < tiles and len(running) < slots and (not running or rng.random() < 0.5):
            running[next_tile] = 0
            next_tile += 1
            continue
        q = list(running)[rng.integers(len(running))]
        st = running[q]
        lo, hi = q * T, min(B, q * T + T)
        if st == 0:
            held[q] = out[kept[lo:hi]].copy()          # the tile's sources, in registers
            published[q] = True
            running[q] = 1
        elif st == 1:
            if not wait or all(published[:q]):
                running[q] = 2
        else:
            out[lo:hi] = held.pop(q)
            del running[q]
            done += 1
    return out


@pytest.mark.parametrize("N,B,T", [(3200, 3072, 128), (400, 300, 16), (1000, 100, 16), (257, 256, 32),
                                   (500, 499, 8), (64, 1, 8), (129, 64, 8)])
def test_every_interleaving_ends_with_the_indexed_rows(N, B, T):
    rng = np.random.default_rng(N * 7 + B)
    rows = np.arange(N, dtype=np.int64) * 10 + 3
    for trial in range(40):
        kept = _kept(rng, N, B)
        want = rows.copy()
        want[:B] = rows[kept]
        slots = int(rng.integers(1, 6))
        got = _replay(rows, kept, T, rng, slots)
        assert got is not None, f"schedule did not end (trial {trial}, {slots} slots)"
        assert np.array_equal(got, want), f"trial {trial}"


def test_without_the_wait_rows_are_lost():
    """Planted in the model: tiles write as soon as they hold their own sources."""
    rng = np.random.default_rng(5)
    N, B, T = 400, 300, 16
    rows = np.arange(N, dtype=np.int64)
    wrong = 0
    for trial in range(40):
        kept = _kept(rng, N, B)
        want = rows.copy()
        want[:B] = rows[kept]
        got = _replay(rows, kept, T, rng, slots=4, wait=False)
        wrong += not np.array_equal(got, want)
    assert wrong > 0
