"""GPU parity at the full layer sizes, in the launch configuration the benchmark
times: the GPU runs the whole layer; the oracle checks every row of sampled
heads for selection, and sampled (head, query tile) pairs for attention (first
tile, last tile, a tile that straddles a frame boundary, and random ones)."""
import gc

import numpy as np
import pytest
import torch

from block_sparse_attention_predictor_amd import binding as Bnd
from block_sparse_attention_predictor_amd import inputs as I
from oracle import veda_oracle as O

from gpu_util import bf16_to_f64, check_attn, check_indices, check_scores, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def sampled_tiles(wl, rng, extra=2):
    Tq = wl.n_query_tiles
    frame = wl.grid[1] * wl.grid[2]
    straddle = (frame // wl.tile)            # the tile holding the first frame boundary
    tiles = {0, Tq - 1, straddle}
    tiles |= set(rng.integers(1, Tq - 1, extra).tolist())
    return sorted(tiles)


@pytest.mark.parametrize("name", ["t2v5s", "r2va", "t2v14s"])
def test_full_layer_parity(name):
    wl = I.WORKLOADS[name]
    print(f"[{name}] generating inputs", flush=True)
    q, k, v = I.make_qkv(wl)
    w = I.make_weights(wl)
    rng = np.random.default_rng(wl.index)
    if w.fp8:
        # the path as it runs: FP8 weights dequantised on the GPU at load
        wq = Bnd.dequant_fp8_e4m3(to_dev(w.wq), w.pow2_exp)
        wk = Bnd.dequant_fp8_e4m3(to_dev(w.wk), w.pow2_exp)
        wq_bits = O.dequant_e4m3fn_to_bf16_bits(w.wq, w.pow2_exp)
        wk_bits = O.dequant_e4m3fn_to_bf16_bits(w.wk, w.pow2_exp)
        assert np.array_equal(wq.view(torch.int16).cpu().numpy().view(np.uint16), wq_bits)
        assert np.array_equal(wk.view(torch.int16).cpu().numpy().view(np.uint16), wk_bits)
    else:
        wq_bits, wk_bits = w.wq, w.wk
        wq, wk = to_dev_bf16(w.wq), to_dev_bf16(w.wk)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    L = Bnd.layer_from_workload(wl)
    segs = [(s.start, s.length, s.budget) for s in wl.segments]
    dense = [(r.start, r.length) for r in wl.dense]
    print(f"[{name}] GPU select", flush=True)
    idx, sc = Bnd.select(L, qd, kd, wq, wk, want_scores=True)
    torch.cuda.synchronize()
    heads = [0, wl.H // 2, wl.H - 1]
    print(f"[{name}] oracle select on heads {heads}", flush=True)
    idx_ref, S_ref, _, _ = O.select(q, k, wq_bits, wk_bits, wl.tile, (wl.query.start, wl.query.length),
                                    segs, heads=heads)
    idx_np = idx.cpu().numpy()
    sc_np = sc[:, heads].cpu().numpy().astype(np.float64)
    del sc
    seg_T = [wl.seg_tiles(s) for s in wl.segments]
    seg_K = [min(s.budget, T) for s, T in zip(wl.segments, seg_T)]
    check_scores(sc_np, S_ref[:, heads])
    ties = check_indices(idx_np[:, heads], idx_ref[:, heads], S_ref[:, heads], seg_T, seg_K)
    print(f"[{name}] selection ok ({ties} rows decided inside the tie window)", flush=True)

    # attention with the oracle's indices on the sampled heads
    idx_np[:, heads] = idx_ref[:, heads]
    out = Bnd.sparse_attn(L, qd, kd, vd, to_dev(idx_np), dense)
    torch.cuda.synchronize()
    tiles = sampled_tiles(wl, rng)
    pairs = [(0, h, t) for h in heads for t in tiles]
    print(f"[{name}] oracle attention on {len(pairs)} (head, tile) pairs", flush=True)
    res = O.attend(q, k, v, idx_np, wl.tile, (wl.query.start, wl.query.length), segs, dense,
                   pairs=pairs)
    got = []
    for (b, h, t) in res:
        r0 = wl.query.start + t * wl.tile
        r1 = wl.query.start + min((t + 1) * wl.tile, wl.query.length)
        got.append(out[b, r0:r1, h].to(torch.float64).cpu().numpy())
    mx, mean = check_attn(np.concatenate(got), np.concatenate([r[0] for r in res.values()]))
    print(f"[{name}] attention ok: max-abs {mx:.2e} mean-abs {mean:.2e}", flush=True)
