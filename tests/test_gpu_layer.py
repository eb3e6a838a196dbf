"""GPU parity of the full-layer call and of the attention call's index conventions
(no index = every tile; -1 entries = padding), against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_predictor_amd import binding as Bnd
from block_sparse_attention_predictor_amd import inputs as I
from oracle import veda_oracle as O

from gpu_util import bf16_to_f64, check_attn, check_indices, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _case(seed, d=128, tile=64, H=3, B=1):
    """video 640 | reference 200 | text 37 | audio 90: the reference is a key segment
    and, with text and audio, a dense query range."""
    g = np.random.default_rng(seed)
    N = 640 + 200 + 37 + 90
    ramp = np.sin(np.arange(N) / 23.0)[None, :, None, None].astype(np.float32)
    qf = g.standard_normal((B, N, H, d)).astype(np.float32) + ramp * g.standard_normal((1, 1, H, d)).astype(np.float32)
    kf = g.standard_normal((B, N, H, d)).astype(np.float32) + ramp * g.standard_normal((1, 1, H, d)).astype(np.float32)
    vf = g.standard_normal((B, N, H, d)).astype(np.float32)
    wq = I.f32_to_bf16_bits(g.standard_normal((H, 32, d)).astype(np.float32) / math.sqrt(d))
    wk = I.f32_to_bf16_bits(g.standard_normal((H, 32, d)).astype(np.float32) / math.sqrt(d))
    q, k, v = (I.f32_to_bf16_bits(x) for x in (qf, kf, vf))
    segments = [(640, 200, 2), (0, 640, 3)]
    dense = [(840, 37), (877, 90)]
    dense_queries = [(640, 200), (840, 37), (877, 90)]
    L = Bnd.make_layer(B=B, H=H, d=d, p=32, tile=tile, n_tokens=N, query=(0, 640), segments=segments,
                       strides=(N * H * d, H * d, d))
    return L, q, k, v, wq, wk, segments, dense, dense_queries


@pytest.mark.parametrize("d,tile", [(128, 64), (128, 128), (64, 64)])
def test_layer_attn_matches_oracle(d, tile):
    L, q, k, v, wq, wk, segments, dense, dq = _case(5, d=d, tile=tile, B=2 if d == 64 else 1)
    qd, kd, vd, wqd, wkd = (to_dev_bf16(x) for x in (q, k, v, wq, wk))
    out, idx = Bnd.layer_attn(L, qd, kd, vd, wqd, wkd, dense, dq)
    torch.cuda.synchronize()
    o = bf16_to_f64(out)
    idx_np = idx.cpu().numpy()
    idx_ref, S_ref, _, _ = O.select(q, k, wq, wk, tile, (0, 640), segments)
    seg_T = [-(-ln // tile) for (_, ln, _) in segments]
    seg_K = [min(bud, T) for (_, _, bud), T in zip(segments, seg_T)]
    check_indices(idx_np, idx_ref, S_ref, seg_T, seg_K)
    # video rows: sparse attention over the very index sets the GPU chose
    res = O.attend(q, k, v, idx_np, tile, (0, 640), segments, dense)
    got = np.concatenate([o[b, t * tile:min((t + 1) * tile, 640), h] for (b, h, t) in res])
    check_attn(got, np.concatenate([r[0] for r in res.values()]))
    # every other query row: dense over all keys
    for b in range(L.B):
        for h in range(L.H):
            for (st, ln) in dq:
                ref, _ = O.attend_all_keys(q, k, v, b, h, (st, ln), segments, dense)
                check_attn(o[b, st:st + ln, h], ref)


@pytest.mark.parametrize("H,tile", [(3, 64), (8, 64), (8, 128)])
def test_no_index_equals_every_tile(H, tile):
    """No index = an index row listing every tile.  With 8 or more (b, h) pairs the no-index
    launch maps whole heads to XCDs instead of slicing each head's tiles over them; the
    mapping changes which workgroup computes an item, not the arithmetic, so the outputs
    are bit-identical."""
    L, q, k, v, wq, wk, segments, dense, dq = _case(7, tile=tile, H=H)
    full = [(st, ln, 10 ** 6) for (st, ln, _) in segments]
    Lf = Bnd.make_layer(B=1, H=L.H, d=L.d, p=L.p, tile=L.tile, n_tokens=L.n_tokens, query=(0, 640),
                        segments=full, strides=(L.stride_b, L.stride_n, L.stride_h))
    qd, kd, vd = (to_dev_bf16(x) for x in (q, k, v))
    Tq = -(-640 // L.tile)
    idx = np.concatenate([np.broadcast_to(np.arange(-(-ln // L.tile), dtype=np.int32), (1, L.H, Tq, -(-ln // L.tile)))
                          for (_, ln, _) in segments], axis=-1)
    a = Bnd.sparse_attn(Lf, qd, kd, vd, to_dev(np.ascontiguousarray(idx)), dense)
    b_ = Bnd.sparse_attn(Lf, qd, kd, vd, None, dense)
    torch.cuda.synchronize()
    assert torch.equal(a, b_)
    # without an index, budgets below the tile count are rejected
    with pytest.raises(Bnd.VedaError):
        Bnd.sparse_attn(L, qd, kd, vd, None, dense)


def test_padding_entries():
    L, q, k, v, wq, wk, segments, dense, dq = _case(9)
    qd, kd, vd = (to_dev_bf16(x) for x in (q, k, v))
    Tq = -(-640 // L.tile)
    g = np.random.default_rng(3)
    idx = np.full((1, L.H, Tq, L.Ktot), -1, dtype=np.int32)
    for h in range(L.H):
        for t in range(Tq):
            n_ref = int(g.integers(0, 3))              # 0..2 reference tiles, rest padding
            n_vid = int(g.integers(1, 4))              # 1..3 video tiles
            idx[0, h, t, :n_ref] = np.sort(g.choice(4, n_ref, replace=False))
            idx[0, h, t, 2:2 + n_vid] = np.sort(g.choice(10, n_vid, replace=False))
    out = Bnd.sparse_attn(L, qd, kd, vd, to_dev(idx), dense)
    torch.cuda.synchronize()
    o = bf16_to_f64(out)
    res = O.attend(q, k, v, idx, L.tile, (0, 640), segments, dense)
    got = np.concatenate([o[b, t * L.tile:(t + 1) * L.tile, h] for (b, h, t) in res])
    check_attn(got, np.concatenate([r[0] for r in res.values()]))


def test_all_padding_without_dense_gives_zero_rows():
    L, q, k, v, wq, wk, segments, dense, dq = _case(11)
    qd, kd, vd = (to_dev_bf16(x) for x in (q, k, v))
    Tq = -(-640 // L.tile)
    idx = np.broadcast_to(np.array([0, 1, 0, 1, 2], dtype=np.int32), (1, L.H, Tq, L.Ktot)).copy()
    idx[0, 1, 4, :] = -1                               # one query tile with nothing to attend
    out = torch.full_like(qd, 7.0)
    Bnd.sparse_attn(L, qd, kd, vd, to_dev(idx), [], out=out)
    torch.cuda.synchronize()
    o = bf16_to_f64(out)
    assert np.all(o[0, 4 * L.tile:5 * L.tile, 1] == 0.0)
    assert np.all(np.isfinite(o[0, :640]))


def test_layer_attn_heads_mapping_and_adjacent_dense_query_ranges():
    """B x H = 8: the dense query rows run with whole heads per XCD; the three touching
    dense query ranges (reference, text, audio) run as one launch, in whatever order the
    caller lists them.  Against the oracle, and bit-identical across orders."""
    L, q, k, v, wq, wk, segments, dense, dq = _case(11, d=128, tile=128, H=4, B=2)
    qd, kd, vd, wqd, wkd = (to_dev_bf16(x) for x in (q, k, v, wq, wk))
    out, idx = Bnd.layer_attn(L, qd, kd, vd, wqd, wkd, dense, dq)
    out_r, idx_r = Bnd.layer_attn(L, qd, kd, vd, wqd, wkd, dense, list(reversed(dq)))
    torch.cuda.synchronize()
    assert torch.equal(out, out_r) and torch.equal(idx, idx_r)
    o = bf16_to_f64(out)
    res = O.attend(q, k, v, idx.cpu().numpy(), L.tile, (0, 640), segments, dense)
    got = np.concatenate([o[b, t * L.tile:min((t + 1) * L.tile, 640), h] for (b, h, t) in res])
    check_attn(got, np.concatenate([r[0] for r in res.values()]))
    st, ln = dq[0][0], sum(n for _, n in dq)          # one merged run of rows
    for b in range(L.B):
        for h in range(L.H):
            ref, _ = O.attend_all_keys(q, k, v, b, h, (st, ln), segments, dense)
            check_attn(o[b, st:st + ln, h], ref)
