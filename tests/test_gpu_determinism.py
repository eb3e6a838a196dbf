"""Bitwise determinism of every kernel family: the same call made twice (the second time on
another stream, after other work has run on the device) must give identical bits.  No kernel
accumulates floating point through atomics or in a launch-dependent order, so any difference
points at a race: an LDS stage read before its DMA landed, a missing barrier, or a selection
whose ties depend on timing.

Layers: a 128-row-tile layer with reference, text and audio ranges (two-group kernel, FP8
kernel, teacher mass) and the 64-row tiny workload (paired kernel); full layers with dense
query rows; the window pattern.
"""
import pytest
import torch

from block_sparse_attention_predictor_amd import binding as Bnd
from block_sparse_attention_predictor_amd import inputs as I
from gpu_util import to_dev_bf16

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    Bnd._load()


def _wl(name):
    if name == "t128":
        return I.custom_workload("det_t128", H=3, d=128, p=32, tile=128, grid=(4, 16, 16), ref=True, text=40,
                                 audio=70, budgets={"video": 3, "ref": 1}, index=73)
    return I.WORKLOADS[name]


def _dev(wl):
    q, k, v = I.make_qkv(wl)
    w = I.make_weights(wl)
    assert not w.fp8
    return tuple(to_dev_bf16(x) for x in (q, k, v, w.wq, w.wk))


def _twice(fn):
    """fn() on the current stream, then again on a side stream after unrelated device work."""
    a = fn()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        junk = torch.randn(1 << 22, device="cuda")
        junk.mul_(3.0).sum()
        b = fn()
    torch.cuda.synchronize()
    return a, b


def _same(a, b):
    if isinstance(a, (tuple, list)):
        assert len(a) == len(b)
        for x, y in zip(a, b):
            _same(x, y)
    elif a is None:
        assert b is None
    else:
        assert a.dtype == b.dtype and a.shape == b.shape
        bits = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[a.element_size()]
        assert torch.equal(a.view(bits), b.view(bits)), "results differ between two identical calls"


@pytest.mark.parametrize("name", ["t128", "tiny"])
def test_select_and_attention_deterministic(name):
    _need_gpu()
    wl = _wl(name)
    q, k, v, wq, wk = _dev(wl)
    L = Bnd.layer_from_workload(wl)
    dense = [(r.start, r.length) for r in wl.dense]

    def run():
        idx, sc = Bnd.select(L, q, k, wq, wk, want_scores=True)
        out, lse = Bnd.sparse_attn(L, q, k, v, idx, dense, want_lse=True)
        return idx, sc, out, lse

    _same(*_twice(run))


def test_fp8_quantiser_and_attention_deterministic():
    _need_gpu()
    wl = _wl("t128")
    q, k, v, wq, wk = _dev(wl)
    L = Bnd.layer_from_workload(wl)
    dense = [(r.start, r.length) for r in wl.dense]
    idx = Bnd.select(L, q, k, wq, wk)

    def run():
        q8, qs = Bnd.quantize_fp8(L, q)
        k8, ks = Bnd.quantize_fp8(L, k)
        out, lse = Bnd.sparse_attn_fp8qk(L, q8, k8, v, qs, ks, idx, dense, want_lse=True)
        return q8, qs, k8, ks, out, lse

    _same(*_twice(run))


def test_teacher_mass_and_recall_deterministic():
    _need_gpu()
    wl = _wl("t128")
    q, k, v, wq, wk = _dev(wl)
    L = Bnd.layer_from_workload(wl)
    dense = [(r.start, r.length) for r in wl.dense]
    idx = Bnd.select(L, q, k, wq, wk)
    full = Bnd.Layer.from_buffer_copy(L)
    for s in range(full.n_seg):
        full.budget[s] = -(-full.seg[s].len // full.tile)

    def run():
        mass, dm, lse = Bnd.block_mass(full, q, k, dense)
        return mass, dm, lse, Bnd.block_recall(L, mass, idx)

    _same(*_twice(run))


@pytest.mark.parametrize("name", ["t128", "tiny"])
def test_full_layer_deterministic(name):
    _need_gpu()
    wl = _wl(name)
    q, k, v, wq, wk = _dev(wl)
    L = Bnd.layer_from_workload(wl)
    dense = [(r.start, r.length) for r in wl.dense]
    dq = [(r.start, r.length) for r in wl.dense]

    def run():
        return Bnd.layer_attn(L, q, k, v, wq, wk, dense, dense_queries=dq)

    _same(*_twice(run))


def test_window_indices_deterministic():
    _need_gpu()
    wl = _wl("tiny")
    L = Bnd.layer_from_workload(wl)
    W = Bnd.make_layer(B=L.B, H=L.H, d=L.d, p=L.p, tile=L.tile, n_tokens=L.n_tokens,
                       query=(L.query.start, L.query.len), segments=[(L.query.start, L.query.len, 1)],
                       strides=(L.stride_b, L.stride_n, L.stride_h))
    ft = wl.query.length // wl.grid[0]

    def run():
        return Bnd.window_indices(W, ft, 1, 1, True)[0]

    _same(*_twice(run))
