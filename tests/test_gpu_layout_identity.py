"""Full-size bit-identity of the attention kernels across storage layouts and timing.

The same layer and index sets run three ways: token-major storage ([B, N, H, d]), the
same values stored head-major ([B, H, N, d]) and passed through the strides, and a
repeat of the first on a side stream after unrelated device work.  No attention kernel's
arithmetic depends on the strides or on the order in which memory requests return, so
all three outputs must agree bit for bit.  A difference is a race: an LDS stage written
by ordinary stores while another wave's LDS DMA into it is in flight, or an operand read
before its DMA landed.  Such races need the skew between waves that full-size memory
traffic brings, which the small determinism layers do not reach, so these run at the
benchmark's sizes: the 90 %-sparsity layer (mid: paired 64-row kernel), the 5.17 s
layer (t2v5s: two-group bf16 kernel and both FP8 kernels) and the R2VA layer (two-group
kernel over two selected segments, the reference one taken whole by every tile), in the
selection's tile order as the benchmark runs them.
"""
import gc

import pytest
import torch

from block_sparse_attention_predictor_amd import binding as Bnd
from block_sparse_attention_predictor_amd import inputs as I

from gpu_util import to_dev_bf16

pytestmark = pytest.mark.gpu


def _bits(x: torch.Tensor) -> torch.Tensor:
    return x.contiguous().view(torch.int16)


def _head_major(x: torch.Tensor) -> torch.Tensor:
    """The same [B, N, H, d] values stored as [B, H, N, d], viewed back as [B, N, H, d]."""
    return x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)


def _side_stream(fn):
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        junk = torch.randn(1 << 24, device="cuda")
        junk.mul_(3.0).sum()
        out = fn()
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", ["mid", "t2v5s", "r2va"])
def test_attention_bits_independent_of_layout_and_timing(name):
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    wl = I.WORKLOADS[name]
    print(f"[{name}] generating inputs", flush=True)
    q, k, v = I.make_qkv(wl)
    w = I.make_weights(wl)
    assert not w.fp8
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    del q, k, v
    L = Bnd.layer_from_workload(wl)
    dense = [(r.start, r.length) for r in wl.dense]
    idx = Bnd.select(L, qd, kd, to_dev_bf16(w.wq), to_dev_bf16(w.wk))
    order = Bnd.tile_order(L, idx)
    qh, kh, vh = _head_major(qd), _head_major(kd), _head_major(vd)
    Lh = Bnd.layer_from_workload(wl, strides=Bnd.strides_of(qh))
    assert Lh.stride_n == wl.d and Lh.stride_h == wl.n_tokens * wl.d

    print(f"[{name}] bf16 attention: token-major, head-major, side stream", flush=True)
    a = Bnd.sparse_attn(L, qd, kd, vd, idx, dense, order=order)
    b = Bnd.sparse_attn(Lh, qh, kh, vh, idx, dense, order=order, out=torch.zeros_like(qh))
    c = _side_stream(lambda: Bnd.sparse_attn(L, qd, kd, vd, idx, dense, order=order))
    torch.cuda.synchronize()
    assert torch.equal(_bits(a), _bits(b)), "bf16 attention: head-major storage changed the output bits"
    assert torch.equal(_bits(a), _bits(c)), "bf16 attention: a repeat on another stream changed the output bits"
    del a, b, c

    if name == "t2v5s":
        print(f"[{name}] FP8 attention paths: token-major, head-major, side stream", flush=True)
        q8, qs = Bnd.quantize_fp8(L, qd)
        k8, ks = Bnd.quantize_fp8(L, kd)
        vt, vs = Bnd.quantize_fp8_vt(L, vd)
        q8h, qsh = Bnd.quantize_fp8(Lh, qh)
        k8h, ksh = Bnd.quantize_fp8(Lh, kh)
        vth, vsh = Bnd.quantize_fp8_vt(Lh, vh)
        torch.cuda.synchronize()
        # the quantisers see the same values in either layout
        assert torch.equal(q8.contiguous(), q8h.contiguous()) and torch.equal(qs, qsh)
        assert torch.equal(k8.contiguous(), k8h.contiguous()) and torch.equal(ks, ksh)
        assert torch.equal(vt, vth) and torch.equal(vs, vsh)

        def fp8qk(lay, q_, k_, v_):
            return Bnd.sparse_attn_fp8qk(lay, q_, k_, v_, qs, ks, idx, dense, order=order)

        a = fp8qk(L, q8, k8, vd)
        b = fp8qk(Lh, q8h, k8h, vh)
        c = _side_stream(lambda: fp8qk(L, q8, k8, vd))
        torch.cuda.synchronize()
        assert torch.equal(_bits(a), _bits(b)), "FP8 Q.K attention: head-major storage changed the output bits"
        assert torch.equal(_bits(a), _bits(c)), "FP8 Q.K attention: a repeat changed the output bits"
        del a, b, c

        def fp8(lay, q_, k_):
            return Bnd.sparse_attn_fp8(lay, q_, k_, vt, qs, ks, vs, idx, dense, order=order)

        a = fp8(L, q8, k8)
        b = fp8(Lh, q8h, k8h)
        c = _side_stream(lambda: fp8(L, q8, k8))
        torch.cuda.synchronize()
        assert torch.equal(_bits(a), _bits(b)), "FP8 attention: head-major storage changed the output bits"
        assert torch.equal(_bits(a), _bits(c)), "FP8 attention: a repeat changed the output bits"
        del a, b, c
    del qd, kd, vd, qh, kh, vh
    gc.collect()
    torch.cuda.empty_cache()
