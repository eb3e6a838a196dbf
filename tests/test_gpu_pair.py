"""GPU parity of the paired two-group kernel (64-row tiles: one workgroup takes two
neighbouring query tiles, each half of every group streams its own tile's 32-key blocks)
against the fp64 oracle.  Aimed at its control flow: the two tiles of a pair with
different block counts (0, 1, 2, ... per row, odd and even, so one stream runs out before
the other), -1 padding, partial last tiles and dense blocks, an odd number of query tiles
(the last pair has one tile), d = 64 and 128, and the size limit of its per-tile table
(1536 32-key blocks) on both sides, where the launcher switches to the single-pipeline
kernel.

Oracle: oracle.veda_oracle.attend.  Bar: max-abs <= 1e-2, mean-abs <= 1e-3, lse within 2^-9.
"""
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_predictor_amd import binding as Bnd
from oracle import veda_oracle as O
from gpu_util import bf16_to_f64, check_attn, to_dev, to_dev_bf16
from test_gpu_twogroup import _inputs, _padded_rows

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    Bnd._load()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("with_dense", [True, False])
def test_pair_block_counts_padding_and_ragged_tiles(d, with_dense):
    """15 query tiles of 64 rows (the last one 40 rows; the last pair holds one tile);
    segment tiles of 64 with a partial last tile (40 tokens: two 32-key blocks, the second
    partial) and a 20-token one; every row a different number of blocks."""
    _need_gpu()
    B, H, tile = 1, 2, 64
    segs = [(0, 936, 5), (936, 212, 3)]
    dense = [(1148, 45)] if with_dense else []
    N = 1193
    query = (0, 936)
    Tq = -(-query[1] // tile)
    assert Tq % 2 == 1
    q, k, v = _inputs(71 + d, B, N, H, d)
    g = np.random.default_rng(8)
    idx = _padded_rows(g, B, H, Tq, segs, tile)
    if not with_dense:
        for h in range(H):
            for i in range(Tq):
                if idx[0, h, i, 0] < 0 and idx[0, h, i, 5] < 0 and (h, i) != (1, 4):
                    idx[0, h, i, 0] = i % 9
        idx[0, 1, 4, :] = -1                        # no key at all: zero rows
        idx[0, 0, 6, :] = [-1, -1, -1, -1, -1, 3, -1, -1]   # one block: the 20-token tile
    L = Bnd.make_layer(B=B, H=H, d=d, p=16, tile=tile, n_tokens=N, query=query, segments=segs,
                       strides=(N * H * d, H * d, d))
    qd, kd, vd = (to_dev_bf16(x) for x in (q, k, v))
    out, lse = Bnd.sparse_attn(L, qd, kd, vd, to_dev(idx), dense, want_lse=True)
    torch.cuda.synchronize()
    o = bf16_to_f64(out)
    lse = lse.cpu().numpy()
    pairs, empty = [], []
    for h in range(H):
        for i in range(Tq):
            (empty if O.attended_tokens(idx[0, h, i], tile, segs, dense).size == 0 else pairs).append((0, h, i))
    res = O.attend(q, k, v, idx, tile, query, segs, dense, pairs=pairs)
    for (b, h, i), (ref, l_ref) in res.items():
        r0, r1 = i * tile, min((i + 1) * tile, query[1])
        check_attn(o[b, r0:r1, h], ref)
        assert np.abs(lse[b, h, r0:r1] - l_ref).max() <= 2.0 ** -9
    assert empty == ([] if with_dense else [(0, 1, 4)])
    for (b, h, i) in empty:
        assert np.all(o[b, i * tile:(i + 1) * tile, h] == 0)
    # rows outside the query segment are never written
    assert np.all(o[:, query[1]:] == 0)


@pytest.mark.parametrize("n_dense_blocks", [1536 - 8, 1536 - 8 + 1])
def test_pair_table_limit(n_dense_blocks):
    """4 selected tiles (8 blocks of 32) plus a dense range of n 32-key blocks: 1536 blocks
    in all is the per-tile table capacity, one more takes the single-pipeline kernel."""
    _need_gpu()
    B, H, d, tile = 1, 1, 64, 64
    seg_len = 6 * tile
    dense_len = n_dense_blocks * 32 - 3
    N = seg_len + dense_len
    q, k, v = _inputs(31, B, N, H, d)
    segs = [(0, seg_len, 4)]
    dense = [(seg_len, dense_len)]
    query = (0, 2 * tile)
    idx = np.array([[[[0, 2, 3, 5], [1, 2, 4, 5]]]], dtype=np.int32)
    L = Bnd.make_layer(B=B, H=H, d=d, p=16, tile=tile, n_tokens=N, query=query, segments=segs,
                       strides=(N * H * d, H * d, d))
    qd, kd, vd = (to_dev_bf16(x) for x in (q, k, v))
    out = Bnd.sparse_attn(L, qd, kd, vd, to_dev(idx), dense)
    torch.cuda.synchronize()
    o = bf16_to_f64(out)
    res = O.attend(q, k, v, idx, tile, query, segs, dense)
    for (b, h, i), (ref, _) in res.items():
        check_attn(o[b, i * tile:(i + 1) * tile, h], ref)


def test_pair_batches_heads_and_full_budget_rows():
    """B = 2, H = 5, d = 128, every tile selected (no index: the dense-query launch form, whole
    heads per XCD) against dense attention computed directly."""
    _need_gpu()
    B, H, d, tile = 2, 5, 128, 64
    segs = [(0, 700, 10 ** 6), (700, 150, 10 ** 6)]
    dense = [(850, 77)]
    N = 927
    query = (0, 700)
    q, k, v = _inputs(47, B, N, H, d)
    L = Bnd.make_layer(B=B, H=H, d=d, p=32, tile=tile, n_tokens=N, query=query, segments=segs,
                       strides=(N * H * d, H * d, d))
    qd, kd, vd = (to_dev_bf16(x) for x in (q, k, v))
    out = Bnd.sparse_attn(L, qd, kd, vd, None, dense)
    torch.cuda.synchronize()
    o = bf16_to_f64(out)
    qf, kf, vf = (O.bf16_bits_to_f64(x) for x in (q, k, v))
    for b in range(B):
        for h in range(H):
            ref, _ = O.attend_rows(qf[b, :700, h], kf[b, :, h], vf[b, :, h], 1 / math.sqrt(d))
            check_attn(o[b, :700, h], ref)
