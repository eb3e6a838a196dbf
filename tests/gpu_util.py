"""Helpers shared by the GPU tests: device upload and the parity criteria.

Parity criteria (the tolerances of the method's target):
  * scores: row-normwise,  max_j |s_gpu - s_ref| <= 1e-4 * max_j |s_ref|
  * indices: identical except tiles whose oracle score lies within 1e-4 (same
    row-normwise scale) of the k-th score of their segment; the GPU list must
    still hold exactly k distinct ascending in-range ids
  * attention fed the oracle's indices: max-abs <= 1e-2 and mean-abs <= 1e-3
    against the fp64 oracle
"""
import numpy as np
import torch

SCORE_RTOL = 1e-4
ATTN_MAX_ABS = 1e-2
ATTN_MEAN_ABS = 1e-3


def to_dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_dev(x: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def check_scores(s_gpu: np.ndarray, s_ref: np.ndarray):
    scale = np.abs(s_ref).max(axis=-1, keepdims=True)
    err = np.abs(s_gpu - s_ref).max(axis=-1, keepdims=True)
    worst = float((err / np.maximum(scale, 1e-300)).max())
    assert worst <= SCORE_RTOL, f"row-normwise score error {worst:.3e}"
    return worst


def check_indices(idx_gpu: np.ndarray, idx_ref: np.ndarray, s_ref: np.ndarray, seg_T, seg_K):
    """idx_* [..., Ktot]; s_ref [..., sum T]; returns the number of rows decided in the tie window."""
    assert idx_gpu.shape == idx_ref.shape
    flat_g = idx_gpu.reshape(-1, idx_gpu.shape[-1])
    flat_r = idx_ref.reshape(-1, idx_ref.shape[-1])
    flat_s = s_ref.reshape(-1, s_ref.shape[-1])
    scale = np.abs(flat_s).max(axis=-1)
    exact = np.all(flat_g == flat_r, axis=-1)
    tie_rows = 0
    for row in np.nonzero(~exact)[0]:
        col, kc = 0, 0
        for T, K in zip(seg_T, seg_K):
            g = flat_g[row, kc:kc + K]
            r = flat_r[row, kc:kc + K]
            if not np.array_equal(g, r):
                s = flat_s[row, col:col + T]
                assert np.all(np.diff(g) > 0) and g.min() >= 0 and g.max() < T, "invalid id list"
                kth = np.sort(s)[::-1][K - 1]
                amb = set(np.nonzero(np.abs(s - kth) <= SCORE_RTOL * scale[row])[0].tolist())
                gs, rs = set(g.tolist()), set(r.tolist())
                assert gs - amb == rs - amb, f"row {row}: selection differs outside the tie window"
                tie_rows += 1
            col += T
            kc += K
    return tie_rows


def check_attn(out_gpu: np.ndarray, out_ref: np.ndarray):
    d = np.abs(out_gpu - out_ref)
    mx, mean = float(d.max()), float(d.mean())
    assert mx <= ATTN_MAX_ABS, f"max-abs {mx:.3e}"
    assert mean <= ATTN_MEAN_ABS, f"mean-abs {mean:.3e}"
    return mx, mean


def tile_order_ref(idx: np.ndarray, seg_T, seg_K, cap: int = 16384) -> np.ndarray:
    """The processing order veda_tile_order documents, written out plainly: per (b, h), the
    query tiles sorted by (key, tile id), the key packing the first E entries of the first
    segment block with K_s < T_s (bits = width of T_s - 1, at least 4; E = min(50 // bits, K_s); an entry
    at or after the block's first -1 counts as all ones).  Identity without such a segment
    or beyond `cap` query tiles."""
    B, H, Tq, _ = idx.shape
    seg = next((s for s, (T, K) in enumerate(zip(seg_T, seg_K)) if K < T), None)
    ident = np.broadcast_to(np.arange(Tq, dtype=np.int32), (B, H, Tq)).copy()
    if seg is None or Tq > cap:
        return ident
    T, K = seg_T[seg], seg_K[seg]
    koff = sum(seg_K[:seg])
    bits = max(4, (T - 1).bit_length())
    nent = min(50 // bits, K)
    out = np.empty((B, H, Tq), np.int32)
    for b in range(B):
        for h in range(H):
            keys = []
            for i in range(Tq):
                key, ended = 0, False
                for e in range(nent):
                    t = int(idx[b, h, i, koff + e])
                    ended = ended or t < 0
                    key = (key << bits) | ((1 << bits) - 1 if ended else t)
                keys.append((key, i))
            out[b, h] = [i for _, i in sorted(keys)]
    return out
