"""Pins of the oracle's fixed window pattern (VDN article, "The mechanism: solving
instead of stepping": chunks of five consecutive latent frames attend to themselves
and the chunks on either side; every frame also attends the first and last frames,
which attend every frame).  Expected values come from hand-written lists read off
that description, closed forms, and a token-by-token brute force."""
import itertools

import numpy as np
import pytest

from oracle import veda_oracle as O


def test_frame_mask_hand_lists_page_setting():
    """Chunks of 5, one neighbour chunk on each side, anchors, 20 frames."""
    m = O.window_frame_mask(20, 5, 1, True)
    assert m.shape == (20, 20)
    assert list(np.flatnonzero(m[0])) == list(range(20))          # first frame: everything
    assert list(np.flatnonzero(m[19])) == list(range(20))         # last frame: everything
    assert list(np.flatnonzero(m[7])) == list(range(0, 15)) + [19]   # chunk 1: chunks 0..2 + last
    assert list(np.flatnonzero(m[12])) == [0] + list(range(5, 20))   # chunk 2: chunks 1..3 (incl. last)
    assert list(np.flatnonzero(m[3])) == list(range(0, 10)) + [19]   # chunk 0: chunks 0..1 + last
    assert list(np.flatnonzero(m[16])) == [0] + list(range(10, 20))  # chunk 3: chunks 2..3
    # without anchors the window alone
    w = O.window_frame_mask(20, 5, 1, False)
    assert list(np.flatnonzero(w[0])) == list(range(0, 10))
    assert list(np.flatnonzero(w[7])) == list(range(0, 15))
    assert list(np.flatnonzero(w[19])) == list(range(10, 20))


def test_frame_mask_closed_forms():
    for F in (1, 2, 7, 23):
        # one frame per chunk: a band of half-width h
        for h in (0, 1, 3):
            i, j = np.meshgrid(np.arange(F), np.arange(F), indexing="ij")
            assert np.array_equal(O.window_frame_mask(F, 1, h, False), np.abs(i - j) <= h)
        # a chunk as long as the clip: dense
        assert O.window_frame_mask(F, F, 0, False).all()
        # halo beyond the last chunk: dense
        assert O.window_frame_mask(F, 2, F, True).all()
    # anchors only (one frame per chunk, no neighbours): identity plus the borders
    F = 9
    expect = np.eye(F, dtype=bool)
    expect[:, [0, F - 1]] = True
    expect[[0, F - 1], :] = True
    assert np.array_equal(O.window_frame_mask(F, 1, 0, True), expect)
    # the pattern is symmetric: the window by construction, the anchors by the text
    for F, c, h, a in itertools.product((5, 11, 32), (1, 3, 5), (0, 1, 2), (False, True)):
        m = O.window_frame_mask(F, c, h, a)
        assert np.array_equal(m, m.T)
        assert m.diagonal().all()                    # every frame attends itself
    with pytest.raises(ValueError):
        O.window_frame_mask(0, 5, 1, True)
    with pytest.raises(ValueError):
        O.window_frame_mask(4, 0, 1, True)


def _brute_tile_rows(L, tile, ft, c, h, anchors):
    """Token-by-token: query tile a takes key tile b when some token i of a may attend
    some token j of b.  Frame of a token is i // ft; chunk of a frame is f // c."""
    F = -(-L // ft)
    T = -(-L // tile)

    def may(i, j):
        fi, fj = i // ft, j // ft
        if abs(fi // c - fj // c) <= h:
            return True
        return anchors and (fi in (0, F - 1) or fj in (0, F - 1))

    rows = []
    for a in range(T):
        take = []
        for b in range(T):
            if any(may(i, j) for i in range(a * tile, min((a + 1) * tile, L))
                   for j in range(b * tile, min((b + 1) * tile, L))):
                take.append(b)
        rows.append(np.array(take, dtype=np.int32))
    return rows


@pytest.mark.parametrize("L,tile,ft,c,h,anchors", [
    (96, 8, 8, 1, 0, False),          # frames = tiles: identity
    (96, 8, 8, 2, 1, True),
    (100, 8, 6, 3, 1, True),          # frames straddle tiles, ragged last tile and frame
    (100, 8, 6, 3, 1, False),
    (77, 16, 5, 5, 1, True),          # several frames per tile
    (64, 4, 9, 2, 0, True),           # several tiles per frame
    (50, 64, 7, 1, 0, True),          # one tile
    (131, 12, 13, 5, 1, True),
])
def test_tile_rows_match_token_brute_force(L, tile, ft, c, h, anchors):
    got = O.window_tile_rows(L, tile, ft, c, h, anchors)
    ref = _brute_tile_rows(L, tile, ft, c, h, anchors)
    assert len(got) == len(ref)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)


def test_tile_rows_closed_forms():
    # frames coincide with tiles, one frame per chunk: the tile band
    rows = O.window_tile_rows(80, 8, 8, 1, 2, False)
    for t, r in enumerate(rows):
        assert list(r) == list(range(max(0, t - 2), min(10, t + 3)))
    # with anchors: first and last rows full, others band + tiles 0 and 9
    rows = O.window_tile_rows(80, 8, 8, 1, 0, True)
    assert list(rows[0]) == list(range(10)) and list(rows[9]) == list(range(10))
    for t in range(1, 9):
        assert list(rows[t]) == sorted({0, t, 9})


def test_window_indices_padding():
    rows = [np.array([0, 1], np.int32), np.array([0, 1, 2, 3], np.int32), np.array([3], np.int32)]
    idx = O.window_indices(rows)
    assert idx.dtype == np.int32
    assert idx.tolist() == [[0, 1, -1, -1], [0, 1, 2, 3], [3, -1, -1, -1]]
    assert O.window_indices(rows, 6).shape == (3, 6)
    with pytest.raises(ValueError):
        O.window_indices(rows, 3)
