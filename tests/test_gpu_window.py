"""GPU parity of the fixed window-pattern producer (rows bit-exact against the
oracle's tile rows) and of block-sparse attention fed its -1-padded rows."""
import gc

import numpy as np
import pytest
import torch

from block_sparse_attention_predictor_amd import binding as Bnd
from block_sparse_attention_predictor_amd import inputs as I
from oracle import veda_oracle as O

from gpu_util import bf16_to_f64, check_attn, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _layer(L, tile, d, H=2, B=1, extra=0):
    N = L + extra
    return Bnd.make_layer(B=B, H=H, d=d, p=32, tile=tile, n_tokens=N, query=(0, L),
                          segments=[(0, L, 1)], strides=(N * H * d, H * d, d))


CASES = [  # L, tile, d, frame tokens, chunk frames, halo chunks, anchors
    (1000, 64, 64, 70, 3, 1, True),
    (1000, 64, 128, 70, 3, 1, False),
    (640, 64, 64, 64, 1, 0, False),        # frames = tiles, one frame per chunk: identity
    (1300, 128, 128, 96, 5, 1, True),      # ragged last tile and frame
    (700, 128, 64, 150, 2, 0, True),
]


@pytest.mark.parametrize("L,tile,d,ft,c,h,anchors", CASES)
def test_window_indices_bit_exact(L, tile, d, ft, c, h, anchors):
    lay = _layer(L, tile, d, H=3, B=2)
    idx, att = Bnd.window_indices(lay, ft, c, h, anchors)
    torch.cuda.synchronize()
    ref = O.window_indices(O.window_tile_rows(L, tile, ft, c, h, anchors))
    assert idx.shape[-1] == ref.shape[-1] == att.budget[0]
    got = idx.cpu().numpy()
    for b in range(2):
        for hh in range(3):
            assert np.array_equal(got[b, hh], ref)
    # a wider row than needed pads further
    idx2, _ = Bnd.window_indices(lay, ft, c, h, anchors, width=-(-L // tile))
    torch.cuda.synchronize()
    assert np.array_equal(idx2.cpu().numpy()[1, 2], O.window_indices(
        O.window_tile_rows(L, tile, ft, c, h, anchors), -(-L // tile)))


@pytest.mark.parametrize("L,tile,d,ft,c,h,anchors", CASES)
def test_window_attention_matches_oracle(L, tile, d, ft, c, h, anchors):
    g = np.random.default_rng(L + tile + d)
    H, extra = 2, 45                                    # a dense range after the video
    N = L + extra
    ramp = 0.5 * np.sin(np.arange(N) / 17.0)[None, :, None, None]   # z + 0.5 F, as the workloads
    q = I.f32_to_bf16_bits((g.standard_normal((1, N, H, d)) + ramp).astype(np.float32))
    k = I.f32_to_bf16_bits((g.standard_normal((1, N, H, d)) + ramp).astype(np.float32))
    v = I.f32_to_bf16_bits(g.standard_normal((1, N, H, d)).astype(np.float32))
    lay = _layer(L, tile, d, H=H, extra=extra)
    idx, att = Bnd.window_indices(lay, ft, c, h, anchors)
    qd, kd, vd = (to_dev_bf16(x) for x in (q, k, v))
    dense = [(L, extra)]
    out = Bnd.sparse_attn(att, qd, kd, vd, idx, dense)
    torch.cuda.synchronize()
    o = bf16_to_f64(out)
    idx_np = idx.cpu().numpy()
    res = O.attend(q, k, v, idx_np, tile, (0, L), [(0, L, att.budget[0])], dense)
    got = np.concatenate([o[b, t * tile:min((t + 1) * tile, L), hh] for (b, hh, t) in res])
    check_attn(got, np.concatenate([r[0] for r in res.values()]))


@pytest.mark.parametrize("name", ["t2v5s", "t2v14s"])
def test_window_full_size(name):
    """The VDN setting (chunks of five latent frames, one neighbour chunk each side,
    boundary anchors) on a full layer: every head's rows bit-exact, and attention on
    sampled query tiles (both anchor tiles, a window tile, a frame-straddling tile)."""
    wl = I.WORKLOADS[name]
    ft = wl.grid[1] * wl.grid[2]
    lay = Bnd.layer_from_workload(wl)
    print(f"[{name}] window rows", flush=True)
    idx, att = Bnd.window_indices(lay, ft, 5, 1, True)
    torch.cuda.synchronize()
    ref = torch.from_numpy(O.window_indices(O.window_tile_rows(wl.query.length, wl.tile, ft, 5, 1, True)))
    assert idx.shape == (1, wl.H, wl.n_query_tiles, ref.shape[1])
    ref_d = ref.to(idx.device)
    for hh in range(wl.H):
        assert torch.equal(idx[0, hh], ref_d), f"head {hh}"
    if name != "t2v5s":
        return
    q, k, v = I.make_qkv(wl)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    dense = [(r.start, r.length) for r in wl.dense]
    print(f"[{name}] window attention", flush=True)
    out = Bnd.sparse_attn(att, qd, kd, vd, idx, dense)
    torch.cuda.synchronize()
    Tq = wl.n_query_tiles
    tiles = sorted({0, Tq - 1, Tq // 2, ft // wl.tile})
    pairs = [(0, hh, t) for hh in (0, wl.H - 1) for t in tiles]
    res = O.attend(q, k, v, idx.cpu().numpy(), wl.tile, (0, wl.query.length),
                   [(0, wl.query.length, att.budget[0])], dense, pairs=pairs)
    got = [out[b, t * wl.tile:min((t + 1) * wl.tile, wl.query.length), hh].to(torch.float64).cpu().numpy()
           for (b, hh, t) in res]
    mx, mean = check_attn(np.concatenate(got), np.concatenate([r[0] for r in res.values()]))
    print(f"[{name}] window attention ok: max-abs {mx:.2e} mean-abs {mean:.2e}", flush=True)
