"""The query tiles' processing order (veda_tile_order) and the attention kernels run in it.

* The order equals its definition (gpu_util.tile_order_ref: index rows sorted on the first
  selecting segment, ties to the lower tile id) on rows with shared prefixes, -1 padding,
  several segments with the first one full, B > 1, odd and single-tile layers, a segment
  of 6 tiles (ids at the 4-bit floor), a layer
  with no selecting segment and one beyond the kernel's 16384-tile LDS array (identity).
* Attention output and lse do not depend on the order: bit-identical to the natural
  order under the sorted, reversed and a random order, for the two-group kernel, the
  paired 64-row kernel, the single-pipeline kernel (block lists past the two-group
  table) and both FP8 kernels.
* An order entry outside [0, Tq) is skipped: the rows of the tile no entry names keep
  their previous contents, every other tile is as in the natural order.
* Small indexed layers run whole heads per XCD in the caller's order: oracle parity on
  every tile with padding head slots and an odd tile count, for both 128- and 64-row tiles.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_predictor_amd import binding as Bnd
from gpu_util import tile_order_ref, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    Bnd._load()


def _rows(g, B, H, Tq, segs, tile, pool=None, pad_every=0):
    """Ascending distinct ids per segment block; ids drawn from a small pool for the first
    selecting segment (so rows share prefixes and whole keys), -1 tails on some rows."""
    ks = [min(bud, -(-ln // tile)) for (_, ln, bud) in segs]
    idx = np.full((B, H, Tq, sum(ks)), -1, np.int32)
    r = 0
    for b in range(B):
        for h in range(H):
            for i in range(Tq):
                kc = 0
                for (_, ln, bud), K in zip(segs, ks):
                    T = -(-ln // tile)
                    src = np.arange(T) if pool is None or K >= T else pool[pool < T]
                    n = K if not pad_every or r % pad_every else int(g.integers(0, K + 1))
                    ids = np.sort(g.choice(src, size=min(n, len(src)), replace=False))
                    idx[b, h, i, kc:kc + len(ids)] = ids
                    kc += K
                r += 1
    return idx


def _layer(B, H, d, tile, N, query, segs):
    return Bnd.make_layer(B=B, H=H, d=d, p=16, tile=tile, n_tokens=N, query=query, segments=segs,
                          strides=(N * H * d, H * d, d))


def _check_order(L, idx, segs, tile):
    seg_T = [-(-ln // tile) for (_, ln, _) in segs]
    seg_K = [min(b, T) for (_, _, b), T in zip(segs, seg_T)]
    order = Bnd.tile_order(L, to_dev(idx))
    torch.cuda.synchronize()
    got = order.cpu().numpy()
    ref = tile_order_ref(idx, seg_T, seg_K)
    assert np.array_equal(got, ref)
    return order


@pytest.mark.parametrize("case", ["prefixes", "padding", "first_full", "batch", "single", "none", "small_T"])
def test_tile_order_matches_definition(case):
    _need_gpu()
    g = np.random.default_rng(3)
    tile = 128
    B, H = (2, 3) if case == "batch" else (1, 2)
    if case == "first_full":          # reference segment fully selected: the key is the video's
        segs = [(0, 4 * tile, 8), (4 * tile, 600 * tile, 5)]
        query = (4 * tile, 600 * tile - 50)
    elif case == "single":
        segs = [(0, 40 * tile, 3)]
        query = (0, 100)
    elif case == "small_T":           # 6 key tiles: ids packed at the 4-bit floor
        segs = [(0, 6 * tile, 3)]
        query = (0, 6 * tile)
    elif case == "none":              # every budget covers its segment: identity
        segs = [(0, 20 * tile, 20), (20 * tile, 3 * tile, 9)]
        query = (0, 20 * tile)
    else:
        segs = [(0, 1100 * tile, 7)]
        query = (0, 777 * tile - 3)   # odd tile count, ragged last tile
    N = segs[-1][0] + segs[-1][1]
    Tq = -(-query[1] // tile)
    pool = np.array([0, 1, 2, 5, 9, 17, 64, 100, 511, 512, 599, 1023, 1024, 1099])
    idx = _rows(g, B, H, Tq, segs, tile, pool=pool, pad_every=3 if case == "padding" else 0)
    L = _layer(B, H, 64, tile, N, query, segs)
    _check_order(L, idx, segs, tile)


def test_tile_order_identity_beyond_the_lds_array():
    _need_gpu()
    tile, Tq = 64, 16385
    segs = [(0, Tq * tile, 1)]
    L = _layer(1, 1, 64, tile, Tq * tile, (0, Tq * tile), [(0, Tq * tile, 1)])
    idx = np.ascontiguousarray((np.arange(Tq, dtype=np.int32)[::-1] % 97).reshape(1, 1, Tq, 1))
    order = _check_order(L, idx, [(0, Tq * tile, 1)], tile)
    assert np.array_equal(order.cpu().numpy()[0, 0], np.arange(Tq))


def _qkv(g, B, N, H, d):
    x = [g.standard_normal((B, N, H, d)).astype(np.float32) for _ in range(3)]
    from block_sparse_attention_predictor_amd import inputs as I
    return tuple(to_dev_bf16(I.f32_to_bf16_bits(a)) for a in x)


def _orders(L, idx_dev, g):
    B, H, Tq = L.B, L.H, L.Tq
    sorted_ = Bnd.tile_order(L, idx_dev)
    rev = torch.flip(torch.arange(Tq, dtype=torch.int32, device="cuda"), [0]).expand(B, H, Tq).contiguous()
    rnd = torch.from_numpy(np.stack([g.permutation(Tq) for _ in range(B * H)]).astype(np.int32)
                           .reshape(B, H, Tq)).cuda()
    return {"sorted": sorted_, "reversed": rev, "random": rnd}


@pytest.mark.parametrize("kind", ["two_group", "pair", "single_pipeline"])
def test_attention_does_not_depend_on_the_order(kind):
    _need_gpu()
    g = np.random.default_rng(17)
    if kind == "pair":
        B, H, d, tile = 1, 3, 128, 64
        segs = [(0, 300 * tile, 9)]
        dense = [(300 * tile, 100)]
        query = (0, 300 * tile - 10)
    elif kind == "two_group":
        B, H, d, tile = 2, 2, 128, 128
        segs = [(0, 6 * tile, 6), (6 * tile, 200 * tile, 7)]
        dense = [(206 * tile, 300)]
        query = (6 * tile, 200 * tile - 70)
    else:                              # 16 selected blocks + 3057 dense blocks > the 3072-entry table
        B, H, d, tile = 1, 2, 64, 128
        segs = [(0, 40 * tile, 8)]
        dense = [(40 * tile, 3057 * 64)]
        query = (0, 40 * tile)
    N = max(segs[-1][0] + segs[-1][1], dense[-1][0] + dense[-1][1])
    Tq = -(-query[1] // tile)
    idx = to_dev(_rows(g, B, H, Tq, segs, tile, pad_every=4))
    L = _layer(B, H, d, tile, N, query, segs)
    q, k, v = _qkv(g, B, N, H, d)
    ref, lse_ref = Bnd.sparse_attn(L, q, k, v, idx, dense, want_lse=True)
    for name, order in _orders(L, idx, g).items():
        out, lse = Bnd.sparse_attn(L, q, k, v, idx, dense, want_lse=True, order=order)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), name
        assert torch.equal(lse, lse_ref), name


def test_fp8_attention_does_not_depend_on_the_order():
    _need_gpu()
    g = np.random.default_rng(23)
    B, H, d, tile = 1, 3, 128, 128
    segs = [(0, 150 * tile, 6)]
    dense = [(150 * tile, 512)]
    query = (0, 150 * tile)
    N = 150 * tile + 512
    Tq = 150
    idx = to_dev(_rows(g, B, H, Tq, segs, tile, pad_every=5))
    L = _layer(B, H, d, tile, N, query, segs)
    q, k, v = _qkv(g, B, N, H, d)
    q8, qs = Bnd.quantize_fp8(L, q)
    k8, ks = Bnd.quantize_fp8(L, k)
    vt, vs = Bnd.quantize_fp8_vt(L, v)
    ref_qk, lse_qk = Bnd.sparse_attn_fp8qk(L, q8, k8, v, qs, ks, idx, dense, want_lse=True)
    ref_v8, lse_v8 = Bnd.sparse_attn_fp8(L, q8, k8, vt, qs, ks, vs, idx, dense, want_lse=True)
    for name, order in _orders(L, idx, g).items():
        o1, l1 = Bnd.sparse_attn_fp8qk(L, q8, k8, v, qs, ks, idx, dense, want_lse=True, order=order)
        o2, l2 = Bnd.sparse_attn_fp8(L, q8, k8, vt, qs, ks, vs, idx, dense, want_lse=True, order=order)
        torch.cuda.synchronize()
        assert torch.equal(o1, ref_qk) and torch.equal(l1, lse_qk), name
        assert torch.equal(o2, ref_v8) and torch.equal(l2, lse_v8), name


@pytest.mark.parametrize("tile", [128, 64])
def test_order_entries_outside_the_tiles_are_skipped(tile):
    _need_gpu()
    g = np.random.default_rng(31)
    B, H, d = 1, 2, 64
    segs = [(0, 64 * tile, 5)]
    query = (0, 64 * tile - 5)
    N = 64 * tile
    Tq = 64
    idx = to_dev(_rows(g, B, H, Tq, segs, tile))
    L = _layer(B, H, d, tile, N, query, segs)
    q, k, v = _qkv(g, B, N, H, d)
    ref = Bnd.sparse_attn(L, q, k, v, idx, [])
    order = torch.arange(Tq, dtype=torch.int32, device="cuda").expand(B, H, Tq).contiguous()
    order[0, 0, 7] = -3               # tile 7 of head 0: never named
    order[0, 1, 11] = Tq              # tile 11 of head 1: never named
    order[0, 1, 12] = 13              # tile 12 of head 1: never named, tile 13 twice
    sentinel = torch.full_like(q, 7.0)
    out = Bnd.sparse_attn(L, q, k, v, idx, [], out=sentinel.clone(), order=order)
    torch.cuda.synchronize()
    skipped = {(0, 7), (1, 11), (1, 12)}
    for h in range(H):
        for t in range(Tq):
            r0, r1 = t * tile, min((t + 1) * tile, query[1])
            want = sentinel if (h, t) in skipped else ref
            assert torch.equal(out[0, r0:r1, h], want[0, r0:r1, h]), (h, t)


@pytest.mark.parametrize("tile", [128, 64])
def test_whole_heads_per_xcd_matches_oracle(tile):
    """Indexed layers whose eight heads' K and V fit the Infinity Cache together run whole
    heads per XCD, in the caller's order.  Here B * H = 10, so the grid's last head slots
    are padding workgroups, and 9 query tiles (the last one partial), so at tile 64 the last
    paired workgroup has one tile; every tile is compared with the oracle, in the sorted
    order and in the natural one."""
    _need_gpu()
    from block_sparse_attention_predictor_amd import inputs as I
    from oracle import veda_oracle as O
    from gpu_util import bf16_to_f64, check_attn
    g = np.random.default_rng(23)
    B, H, d = 2, 5, 64
    qlen = 9 * tile - 17
    segs = [(0, qlen, 3)]
    dense = [(qlen, 70)]
    query = (0, qlen)
    N = qlen + 70
    Tq = -(-qlen // tile)
    idx = _rows(g, B, H, Tq, segs, tile, pad_every=4)
    q, k, v = (I.f32_to_bf16_bits(g.standard_normal((B, N, H, d)).astype(np.float32)) for _ in range(3))
    L = _layer(B, H, d, tile, N, query, segs)
    qd, kd, vd = (to_dev_bf16(x) for x in (q, k, v))
    idx_dev = to_dev(idx)
    order = Bnd.tile_order(L, idx_dev)
    out = Bnd.sparse_attn(L, qd, kd, vd, idx_dev, dense, order=order)
    nat = Bnd.sparse_attn(L, qd, kd, vd, idx_dev, dense)
    torch.cuda.synchronize()
    assert torch.equal(out, nat)
    o = bf16_to_f64(out)
    res = O.attend(q, k, v, idx, tile, query, segs, dense)
    assert len(res) == B * H * Tq
    for (b, h, i), (ref, _) in res.items():
        r0, r1 = i * tile, min((i + 1) * tile, qlen)
        check_attn(o[b, r0:r1, h], ref)
