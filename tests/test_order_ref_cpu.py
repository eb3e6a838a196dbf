"""The definition of the query tiles' processing order as the GPU tests state it
(gpu_util.tile_order_ref), checked on the CPU against a plain sort of tuples, so that the
GPU test of veda_tile_order rests on a definition checked by other means."""
import itertools

import numpy as np

from gpu_util import tile_order_ref


def _rows(g, Tq, T, K, pad_every=0):
    idx = np.full((Tq, K), -1, np.int32)
    for i in range(Tq):
        n = K if not pad_every or i % pad_every else int(g.integers(0, K + 1))
        idx[i, :n] = np.sort(g.choice(T, size=n, replace=False))
    return idx


def _by_tuples(rows, T):
    """Sort tile ids by (their first E entries, -1 and later as the all-ones id, then id)."""
    bits = max(4, (T - 1).bit_length())
    E = min(50 // bits, rows.shape[1])
    ones = (1 << bits) - 1

    def key(i):
        ent, ended = [], False
        for t in rows[i, :E]:
            ended = ended or t < 0
            ent.append(ones if ended else int(t))
        return (tuple(ent), i)
    return sorted(range(rows.shape[0]), key=key)


def test_sorted_like_tuples():
    g = np.random.default_rng(7)
    for T, K, Tq, pad in ((1008, 50, 200, 0), (6, 3, 40, 0), (300, 9, 101, 3), (5000, 20, 64, 2)):
        rows = _rows(g, Tq, T, K, pad)
        got = tile_order_ref(rows[None, None], [T], [K])[0, 0]
        assert sorted(got.tolist()) == list(range(Tq))
        assert got.tolist() == _by_tuples(rows, T)


def test_first_selecting_segment_and_identity():
    g = np.random.default_rng(8)
    # the first segment selects every tile (K == T): the key comes from the second one
    ref_part = np.broadcast_to(np.arange(4, dtype=np.int32), (30, 4))
    vid = _rows(g, 30, 200, 6)
    rows = np.concatenate([ref_part, vid], axis=1)
    got = tile_order_ref(rows[None, None], [4, 200], [4, 6])[0, 0]
    assert got.tolist() == _by_tuples(vid, 200)
    # no selecting segment, or more tiles than the cap: identity
    assert tile_order_ref(ref_part[None, None].copy(), [4], [4])[0, 0].tolist() == list(range(30))
    assert tile_order_ref(vid[None, None], [200], [6], cap=29)[0, 0].tolist() == list(range(30))


def test_equal_rows_keep_tile_order():
    rows = np.array([[3, 5, 7]] * 5 + [[1, 2, 3]] * 3, np.int32)
    got = tile_order_ref(rows[None, None], [10], [3])[0, 0].tolist()
    assert got == [5, 6, 7, 0, 1, 2, 3, 4]
    # permuting equal rows never reorders them
    for p in itertools.permutations(range(3)):
        r = np.array([[4, 6, 8]] * 3, np.int32)[list(p)]
        assert tile_order_ref(r[None, None], [10], [3])[0, 0].tolist() == [0, 1, 2]
