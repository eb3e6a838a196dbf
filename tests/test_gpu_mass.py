"""GPU parity of the teacher block attention mass and of the recall of index sets
under it, against the fp64 oracle.

Bars: mass rows row-normwise (max_j |dM| <= 1e-4 * max_j M, the selection scores'
bar: both are fp32 reductions of exact bf16 products), dense mass and lse within
1e-4 absolute, recall within 1e-4 absolute."""
import gc

import numpy as np
import pytest
import torch

from block_sparse_attention_predictor_amd import binding as Bnd
from block_sparse_attention_predictor_amd import inputs as I
from oracle import veda_oracle as O

from gpu_util import to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

MASS_RTOL = 1e-4
ABS_TOL = 1e-4


@pytest.fixture(autouse=True)
def _free():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _case(seed, d, tile, n_video=640, n_ref=200, H=3, B=1):
    """video | reference | text 37 | audio 90; the reference is a key segment listed first."""
    g = np.random.default_rng(seed)
    N = n_video + n_ref + 37 + 90
    field = 0.5 * np.sin(np.arange(N) / 23.0)[None, :, None, None] * g.standard_normal((1, 1, H, d))
    q = I.f32_to_bf16_bits((g.standard_normal((B, N, H, d)) + field).astype(np.float32))
    k = I.f32_to_bf16_bits((g.standard_normal((B, N, H, d)) + field).astype(np.float32))
    segments = [(n_video, n_ref, 2), (0, n_video, 3)]
    dense = [(n_video + n_ref, 37), (n_video + n_ref + 37, 90)]
    L = Bnd.make_layer(B=B, H=H, d=d, p=32, tile=tile, n_tokens=N, query=(0, n_video), segments=segments,
                       strides=(N * H * d, H * d, d))
    return L, q, k, segments, dense


def check_mass(m_gpu, m_ref):
    scale = np.abs(m_ref).max(axis=-1, keepdims=True)
    worst = float((np.abs(m_gpu - m_ref).max(axis=-1, keepdims=True) / scale).max())
    assert worst <= MASS_RTOL, f"row-normwise mass error {worst:.3e}"
    return worst


def _random_idx(g, L, seg_T, seg_K, pad=True):
    Tq = L.Tq
    idx = np.full((L.B, L.H, Tq, sum(seg_K)), -1, dtype=np.int32)
    for b in range(L.B):
        for h in range(L.H):
            for t in range(Tq):
                kc = 0
                for T, K in zip(seg_T, seg_K):
                    n = int(g.integers(0 if pad else K, K + 1))
                    idx[b, h, t, kc:kc + n] = np.sort(g.choice(T, n, replace=False))
                    kc += K
    return idx


@pytest.mark.parametrize("d,tile,n_video,n_ref", [(128, 64, 640, 200), (128, 128, 640, 200),
                                                   (64, 64, 610, 150), (64, 128, 700, 129)])
def test_block_mass_matches_oracle(d, tile, n_video, n_ref):
    L, q, k, segments, dense = _case(d + tile, d, tile, n_video, n_ref, B=2 if d == 64 else 1)
    qd, kd = to_dev_bf16(q), to_dev_bf16(k)
    mass, dm, lse = Bnd.block_mass(L, qd, kd, dense)
    torch.cuda.synchronize()
    mass, dm, lse = mass.cpu().numpy(), dm.cpu().numpy(), lse.cpu().numpy()
    assert np.allclose(mass.sum(-1) + dm, 1.0, rtol=0, atol=ABS_TOL)
    for b in range(L.B):
        for h in range(L.H):
            m_ref, d_ref, l_ref = O.block_mass(q, k, b, h, tile, (0, n_video), segments, dense)
            check_mass(mass[b, h], m_ref)
            assert np.abs(dm[b, h] - d_ref).max() <= ABS_TOL
            l_ref = np.concatenate([l_ref[i] for i in sorted(l_ref)])
            assert np.abs(lse[b, h] - l_ref).max() <= ABS_TOL


def test_block_recall_matches_oracle():
    L, q, k, segments, dense = _case(31, 128, 64)
    qd, kd = to_dev_bf16(q), to_dev_bf16(k)
    mass, _, _ = Bnd.block_mass(L, qd, kd, dense)
    g = np.random.default_rng(2)
    seg_T = L.seg_tiles
    seg_K = [min(L.budget[s], T) for s, T in enumerate(seg_T)]
    idx = _random_idx(g, L, seg_T, seg_K)
    rec = Bnd.block_recall(L, mass, to_dev(idx))
    torch.cuda.synchronize()
    rec = rec.cpu().numpy()
    for h in range(L.H):
        m_ref, _, _ = O.block_mass(q, k, 0, h, L.tile, (0, 640), segments, dense)
        for t in range(L.Tq):
            r_ref = O.block_recall(m_ref[t], idx[0, h, t], L.tile, segments)
            assert abs(rec[0, h, t] - r_ref) <= ABS_TOL, (h, t)
    # every tile selected: recall one
    full = [(st, ln, 10 ** 6) for (st, ln, _) in segments]
    Lf = Bnd.make_layer(B=1, H=L.H, d=L.d, p=L.p, tile=L.tile, n_tokens=L.n_tokens, query=(0, 640),
                        segments=full, strides=(L.stride_b, L.stride_n, L.stride_h))
    idx_full = np.concatenate([np.broadcast_to(np.arange(T, dtype=np.int32), (1, L.H, L.Tq, T)) for T in seg_T], -1)
    rec_full = Bnd.block_recall(Lf, mass, to_dev(np.ascontiguousarray(idx_full)))
    torch.cuda.synchronize()
    assert np.allclose(rec_full.cpu().numpy(), 1.0, rtol=0, atol=1e-6)


def test_selector_recall_beats_nothing_and_is_consistent():
    """The learned selector's indices (GPU) through the GPU recall, against the oracle
    recall of the same indices."""
    L, q, k, segments, dense = _case(37, 128, 128)
    g = np.random.default_rng(4)
    wq = I.f32_to_bf16_bits((g.standard_normal((L.H, 32, 128)) / np.sqrt(128)).astype(np.float32))
    wk = I.f32_to_bf16_bits((g.standard_normal((L.H, 32, 128)) / np.sqrt(128)).astype(np.float32))
    qd, kd = to_dev_bf16(q), to_dev_bf16(k)
    idx = Bnd.select(L, qd, kd, to_dev_bf16(wq), to_dev_bf16(wk))
    mass, _, _ = Bnd.block_mass(L, qd, kd, dense)
    rec = Bnd.block_recall(L, mass, idx)
    torch.cuda.synchronize()
    rec, idx_np = rec.cpu().numpy(), idx.cpu().numpy()
    assert np.all((rec > 0) & (rec <= 1 + 1e-6))
    for h in range(L.H):
        m_ref, _, _ = O.block_mass(q, k, 0, h, L.tile, (0, 640), segments, dense)
        for t in range(L.Tq):
            assert abs(rec[0, h, t] - O.block_recall(m_ref[t], idx_np[0, h, t], L.tile, segments)) <= ABS_TOL


@pytest.mark.parametrize("name", ["t2v5s", "r2va"])
def test_block_mass_full_size(name):
    """The whole layer on the GPU; the oracle checks sampled (head, query tile) rows."""
    wl = I.WORKLOADS[name]
    print(f"[{name}] inputs", flush=True)
    q, k, _ = I.make_qkv(wl)
    qd, kd = to_dev_bf16(q), to_dev_bf16(k)
    L = Bnd.layer_from_workload(wl)
    segs = [(s.start, s.length, s.budget) for s in wl.segments]
    dense = [(r.start, r.length) for r in wl.dense]
    print(f"[{name}] GPU teacher mass", flush=True)
    mass, dm, lse = Bnd.block_mass(L, qd, kd, dense)
    w = I.make_weights(wl)
    idx = Bnd.select(L, qd, kd, to_dev_bf16(w.wq), to_dev_bf16(w.wk))
    rec = Bnd.block_recall(L, mass, idx)
    torch.cuda.synchronize()
    tot = (mass.sum(-1) + dm).cpu().numpy()
    assert np.abs(tot - 1.0).max() <= ABS_TOL
    Tq = wl.n_query_tiles
    tiles = [0, Tq // 3, Tq - 1]
    idx_np = idx.cpu().numpy()
    for h in (0, wl.H - 1):
        print(f"[{name}] oracle mass, head {h}", flush=True)
        m_ref, d_ref, l_ref = O.block_mass(q, k, 0, h, wl.tile, (wl.query.start, wl.query.length), segs,
                                           dense, qtiles=tiles)
        m_gpu = mass[0, h, tiles].cpu().numpy()
        check_mass(m_gpu, m_ref)
        assert np.abs(dm[0, h, tiles].cpu().numpy() - d_ref).max() <= ABS_TOL
        for r, t in enumerate(tiles):
            r0 = t * wl.tile
            assert np.abs(lse[0, h, r0:r0 + len(l_ref[t])].cpu().numpy() - l_ref[t]).max() <= ABS_TOL
            assert abs(float(rec[0, h, t]) - O.block_recall(m_ref[r], idx_np[0, h, t], wl.tile, segs)) <= ABS_TOL
    print(f"[{name}] mean recall of the selection: {float(rec.mean()):.4f}", flush=True)
