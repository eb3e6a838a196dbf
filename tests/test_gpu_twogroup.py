"""GPU parity of the attention kernels at 128-row tiles against the fp64 oracle, aimed at
the control flow of the two-group kernel: rows with 0, 1, 2, 3 ... key blocks (the
two groups take the even and odd blocks, so odd counts leave one group a block short),
-1 padding inside segment blocks, partial last tiles and partial dense blocks, d = 64
and d = 128, and the size limit of its LDS block table (3072 blocks) on both sides,
where the launcher switches to the single-pipeline kernel.

Oracle: oracle.veda_oracle.attend (plain two-pass softmax in float64 over the tokens of
the selected tiles and the dense ranges).  Bar: max-abs <= 1e-2, mean-abs <= 1e-3.
"""
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_predictor_amd import binding as Bnd
from block_sparse_attention_predictor_amd import inputs as I
from oracle import veda_oracle as O
from gpu_util import bf16_to_f64, check_attn, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    Bnd._load()


def _inputs(seed, B, N, H, d):
    g = np.random.default_rng(seed)
    ramp = np.sin(np.arange(N) / 23.0)[None, :, None, None]
    q = g.standard_normal((B, N, H, d)) + 0.5 * ramp * g.standard_normal((1, 1, H, d))
    k = g.standard_normal((B, N, H, d)) + 0.5 * ramp * g.standard_normal((1, 1, H, d))
    v = g.standard_normal((B, N, H, d))
    return tuple(I.f32_to_bf16_bits(x.astype(np.float32)) for x in (q, k, v))


def _padded_rows(g, B, H, Tq, segs, tile):
    """Index rows where the number of real entries per segment cycles through 0 .. K and
    the rest of each segment block is -1; ids are distinct and ascending."""
    rows = np.full((B, H, Tq, sum(min(b, -(-ln // tile)) for (_, ln, b) in segs)), -1, np.int32)
    r = 0
    for b in range(B):
        for h in range(H):
            for i in range(Tq):
                kc = 0
                for si, (_, ln, bud) in enumerate(segs):
                    T = -(-ln // tile)
                    K = min(bud, T)
                    n = (r + si) % (K + 1)
                    ids = np.sort(g.choice(T, size=n, replace=False)).astype(np.int32)
                    if n and r % 3 == 0:
                        ids[-1] = T - 1          # the partial last tile
                        ids = np.unique(ids)
                    rows[b, h, i, kc:kc + len(ids)] = ids
                    kc += K
                r += 1
    return rows


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("with_dense", [True, False])
def test_block_counts_padding_and_ragged_tiles(d, with_dense):
    """Every row gets a different number of key blocks, from none (when dense keys exist)
    upward, odd and even; the last tile of each segment is partial (104 tokens, two blocks;
    42 tokens, one block), the dense range ends in a 6-token block."""
    _need_gpu()
    B, H, tile = 1, 2, 128
    segs = [(0, 1000, 3), (1000, 170, 2)]
    dense = [(1170, 70)] if with_dense else []
    N = 1240
    query = (0, 1000)
    Tq = -(-query[1] // tile)
    q, k, v = _inputs(11 + d, B, N, H, d)
    g = np.random.default_rng(5)
    idx = _padded_rows(g, B, H, Tq, segs, tile)
    if not with_dense:
        # keep one key somewhere in every row, except row (0, 0, 1): no key at all
        for h in range(H):
            for i in range(Tq):
                if idx[0, h, i, 0] < 0 and idx[0, h, i, 3] < 0 and (h, i) != (0, 1):
                    idx[0, h, i, 0] = i % 8
        idx[0, 0, 1, :] = -1
        idx[0, 1, 2, :] = [-1, -1, -1, 1, -1]       # one block: the 42-token tile
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
    # a row with no key at all is written as zeros
    assert empty == ([] if with_dense else [(0, 0, 1)])
    for (b, h, i) in empty:
        assert np.all(o[b, i * tile:(i + 1) * tile, h] == 0)


@pytest.mark.parametrize("n_dense_blocks", [3072 - 16, 3072 - 16 + 1])
def test_block_table_limit(n_dense_blocks):
    """16 selected blocks plus a dense range of n 64-token blocks: 3072 blocks in all is the
    two-group kernel's table capacity, one more takes the single-pipeline kernel.  Both
    match the oracle on the rows of one query tile."""
    _need_gpu()
    B, H, d, tile = 1, 1, 64, 128
    seg_len = 8 * tile
    dense_len = n_dense_blocks * 64 - 5          # the last dense block is partial
    N = seg_len + dense_len
    q, k, v = _inputs(29, B, N, H, d)
    segs = [(0, seg_len, 8)]
    dense = [(seg_len, dense_len)]
    query = (0, tile)
    idx = np.arange(8, dtype=np.int32).reshape(1, 1, 1, 8)
    L = Bnd.make_layer(B=B, H=H, d=d, p=16, tile=tile, n_tokens=N, query=query, segments=segs,
                       strides=(N * H * d, H * d, d))
    qd, kd, vd = (to_dev_bf16(x) for x in (q, k, v))
    out = Bnd.sparse_attn(L, qd, kd, vd, to_dev(idx), dense)
    torch.cuda.synchronize()
    o = bf16_to_f64(out)
    (ref, _), = O.attend(q, k, v, idx, tile, query, segs, dense, pairs=[(0, 0, 0)]).values()
    check_attn(o[0, :tile, 0], ref)


def test_batches_heads_and_full_budget_rows():
    """B = 2, H = 3 with full-budget index rows (every tile of both segments, so the two
    groups split long block lists) against dense attention computed directly."""
    _need_gpu()
    B, H, d, tile = 2, 3, 128, 128
    segs = [(0, 900, 10 ** 6), (900, 300, 10 ** 6)]
    dense = [(1200, 131)]
    N = 1331
    query = (0, 900)
    q, k, v = _inputs(41, B, N, H, d)
    Tq = -(-query[1] // tile)
    T = [-(-ln // tile) for (_, ln, _) in segs]
    idx = np.concatenate([np.broadcast_to(np.arange(t, dtype=np.int32), (B, H, Tq, t)) for t in T], axis=-1)
    L = Bnd.make_layer(B=B, H=H, d=d, p=32, tile=tile, n_tokens=N, query=query, segments=segs,
                       strides=(N * H * d, H * d, d))
    qd, kd, vd = (to_dev_bf16(x) for x in (q, k, v))
    out = Bnd.sparse_attn(L, qd, kd, vd, to_dev(np.ascontiguousarray(idx)), dense)
    torch.cuda.synchronize()
    o = bf16_to_f64(out)
    keys = np.arange(N)
    qf, kf, vf = (O.bf16_bits_to_f64(x) for x in (q, k, v))
    for b in range(B):
        for h in range(H):
            ref, _ = O.attend_rows(qf[b, :900, h], kf[b, keys, h], vf[b, keys, h], 1 / math.sqrt(d))
            check_attn(o[b, :900, h], ref)
