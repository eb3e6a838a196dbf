"""Host-side checks of the Python binding and of kernel geometry (no GPU needed).

The binding hands caller-supplied buffers to kernels that read and write them with the
layer's geometry; a smaller or mistyped buffer would be an out-of-bounds device access
that the C ABI cannot detect, so the binding rejects it with ValueError first."""
import numpy as np
import pytest
import torch

from block_sparse_attention_predictor_amd import binding as B


def _layer(H=3, tile=64, p=32):
    return B.make_layer(B=1, H=H, d=128, p=p, tile=tile, n_tokens=1000, query=(0, 640),
                        segments=[(0, 640, 3), (640, 200, 2)], strides=(1000 * H * 128, H * 128, 128))


def test_idx_shape_dtype_contiguity_and_device():
    L = _layer()
    cpu = torch.device("cpu")
    good = torch.empty((1, 3, L.Tq, L.Ktot), dtype=torch.int32)
    B._check_idx(L, good, cpu)
    with pytest.raises(ValueError):
        B._check_idx(L, good.to(torch.int64), cpu)
    with pytest.raises(ValueError):
        B._check_idx(L, torch.empty((1, 3, L.Tq, L.Ktot - 1), dtype=torch.int32), cpu)
    with pytest.raises(ValueError):
        B._check_idx(L, torch.empty((1, 3, L.Tq - 1, L.Ktot), dtype=torch.int32), cpu)
    with pytest.raises(ValueError):   # a transposed view has the right element count, not the layout
        B._check_idx(L, torch.empty((1, 3, L.Ktot, L.Tq), dtype=torch.int32).transpose(2, 3), cpu)
    with pytest.raises(ValueError):
        B._check_idx(L, good, torch.device("meta"))


def test_q_hat_k_hat_shape_dtype_contiguity_and_device():
    L = _layer()
    cpu = torch.device("cpu")
    qh = torch.empty((1, 3, L.Tq, L.p), dtype=torch.float32)
    kh = torch.empty((1, 3, L.Tk, L.p), dtype=torch.float32)
    B._check_hat(L, qh, L.Tq, cpu, "q_hat")
    B._check_hat(L, kh, L.Tk, cpu, "k_hat")
    with pytest.raises(ValueError):
        B._check_hat(L, qh.to(torch.float64), L.Tq, cpu, "q_hat")
    with pytest.raises(ValueError):
        B._check_hat(L, qh, L.Tk, cpu, "k_hat")            # Tq rows where Tk are needed
    with pytest.raises(ValueError):
        B._check_hat(L, torch.empty((1, 3, L.p, L.Tq)).transpose(2, 3), L.Tq, cpu, "q_hat")
    with pytest.raises(ValueError):
        B._check_hat(L, qh, L.Tq, torch.device("meta"), "q_hat")


def test_host_tensors_are_rejected_before_any_call():
    L = _layer()
    qh = torch.empty((1, 3, L.Tq, L.p), dtype=torch.float32)
    kh = torch.empty((1, 3, L.Tk, L.p), dtype=torch.float32)
    with pytest.raises(ValueError):
        B.score_topk(L, qh, kh)
    mass = torch.empty((1, 3, L.Tq, L.Tk), dtype=torch.float32)
    with pytest.raises(ValueError):
        B.block_recall(L, mass, torch.empty((1, 3, L.Tq, L.Ktot), dtype=torch.int32))


@pytest.mark.parametrize("D", [64, 128])
def test_two_group_merge_area_fits_its_buffer(D):
    """The two-group attention kernel parks group 1's accumulators in group 0's K/V
    array (4 stages of 64 keys x D bf16) for the merge: wave w, lane l, accumulator tile
    db < D/32 and quarter e4 < 4 use float4 slot w*(D/32)*4*64 + (db*4 + e4)*64 + l.
    Every slot must be distinct and inside the array at both head dimensions."""
    NW = 4
    sg0_float4 = 4 * 64 * D * 2 // 16
    w, l, db, e4 = np.meshgrid(np.arange(NW), np.arange(64), np.arange(D // 32), np.arange(4), indexing="ij")
    slot = w * (D // 32) * 4 * 64 + (db * 4 + e4) * 64 + l
    assert slot.min() == 0 and slot.max() < sg0_float4
    assert np.unique(slot).size == slot.size


def test_workspace_size_contiguity_and_device():
    cpu = torch.device("cpu")
    ws = B._workspace(None, 1000, cpu)
    assert ws.dtype == torch.uint8 and ws.numel() >= 1000
    good = torch.empty(1000, dtype=torch.uint8)
    assert B._workspace(good, 1000, cpu) is good
    assert B._workspace(torch.empty(250, dtype=torch.float32), 1000, cpu).numel() == 250   # bytes, not elements
    with pytest.raises(ValueError):
        B._workspace(torch.empty(999, dtype=torch.uint8), 1000, cpu)
    with pytest.raises(ValueError):
        B._workspace(torch.empty(2000, dtype=torch.uint8)[::2], 1000, cpu)
    with pytest.raises(ValueError):
        B._workspace(good, 1000, torch.device("meta"))
