"""GPU parity of the FP8 Q.K^T path against the oracle (Q1, Q2 and O7 on the decoded
values), through the C ABI:

  * veda_quantize_fp8_e4m3: codes bit-exact and the scale exact, on random tensors with
    planted ties, subnormal-range values and signed zeros, contiguous and head-major
    strides, an all-zero tensor, and the same tensor scaled by a power of two;
  * veda_sparse_attn_fp8qk: the attention bar (max-abs <= 1e-2, mean-abs <= 1e-3, lse
    within 2^-9) against the oracle's attention over the decoded Q and K, on the
    two-group kernel's control-flow cases (0..K blocks per row, -1 padding, partial
    tiles and dense blocks, d = 64 and 128), full-budget rows, and sampled rows of the
    full 1344x768 5.17 s layer in the benchmark's launch configuration.
The FP8 products sum 64 terms at a time with an internal precision of about 2^-12 of
the largest term (measured); at these value ranges that is below 1e-3 in the logits.
"""
import gc
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_predictor_amd import binding as Bnd
from block_sparse_attention_predictor_amd import inputs as I
from oracle import veda_oracle as O
from gpu_util import bf16_to_f64, check_attn, to_dev, to_dev_bf16
from test_gpu_twogroup import _inputs, _padded_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    Bnd._load()


def _codes(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def _layer_for(x_shape, strides, tile=128, segs=None, query=None):
    B, N, H, d = x_shape
    segs = segs or [(0, N, 1)]
    query = query or (0, N)
    return Bnd.make_layer(B=B, H=H, d=d, p=16, tile=tile, n_tokens=N, query=query, segments=segs,
                          strides=strides)


def _planted(seed, shape):
    g = np.random.default_rng(seed)
    x = np.clip(g.standard_normal(shape) * 60.0, -440, 440).astype(np.float32)
    flat = x.reshape(-1)
    flat[0] = 448.0                      # sets the scale to 2^0
    plant = [1.0625, -1.1875, 2.0 ** -10, 1.5 * 2.0 ** -9, 7.5 * 2.0 ** -9, -0.0, 0.0, -2.0 ** -12]
    flat[1:1 + len(plant)] = plant
    flat[100:400] *= 2.0 ** -8          # a stretch in the subnormal range of E4M3
    return I.f32_to_bf16_bits(x)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("head_major", [False, True])
def test_quantize_codes_and_scale(d, head_major):
    _need_gpu()
    B, N, H = 2, 333, 3
    bits = _planted(7 + d, (B, N, H, d))
    if head_major:
        store = np.ascontiguousarray(bits.transpose(0, 2, 1, 3))          # [B, H, N, d] in memory
        dev = to_dev_bf16(store).permute(0, 2, 1, 3)
    else:
        dev = to_dev_bf16(bits)
    strides = tuple(dev.stride()[:3])
    L = _layer_for((B, N, H, d), strides)
    codes_ref, e_ref = O.quantize_fp8(bits)
    assert e_ref == 0
    for shift in (0, -20, 9):
        x = dev
        if shift != 0:   # exact: a power-of-two multiple of every value, same strides
            x = torch.empty_strided(dev.shape, dev.stride(), dtype=torch.bfloat16, device="cuda")
            x.copy_(dev.float() * 2.0 ** shift)
        c8, sc = Bnd.quantize_fp8(L, x)
        torch.cuda.synchronize()
        assert float(sc.cpu()[0]) == 2.0 ** (e_ref + shift)
        assert np.array_equal(_codes(c8), codes_ref), shift        # scaling by 2^s changes no code


@pytest.mark.parametrize("k", [0, 3, -5])
def test_quantize_every_bf16_value_in_range(k):
    """Every finite bf16 value with |x| <= 448 * 2^k, once each (largest first, so the scale
    is 2^k): the codes equal the oracle's nearest-even rounding, ties and the subnormal
    codes included."""
    _need_gpu()
    bits = np.arange(65536, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448.0 * 2.0 ** k)
    b16 = bits[keep].astype(np.uint16)
    b16 = b16[np.argsort(-np.abs(vals[keep]), kind="stable")]
    n = -(-b16.size // 256) * 256
    flat = np.zeros(n, np.uint16)
    flat[:b16.size] = b16
    x = flat.reshape(1, n // 256, 2, 128)
    dev = to_dev_bf16(x)
    L = _layer_for(x.shape, tuple(dev.stride()[:3]))
    c8, sc = Bnd.quantize_fp8(L, dev)
    torch.cuda.synchronize()
    codes_ref, e_ref = O.quantize_fp8(x)
    assert e_ref == k and float(sc.cpu()[0]) == 2.0 ** k
    assert np.array_equal(_codes(c8), codes_ref)


def test_quantize_all_zero_and_signed_zero():
    _need_gpu()
    B, N, H, d = 1, 64, 2, 64
    bits = np.zeros((B, N, H, d), np.uint16)
    bits[0, 3, 1, 5] = 0x8000                                            # -0.0
    dev = to_dev_bf16(bits)
    L = _layer_for((B, N, H, d), tuple(dev.stride()[:3]), tile=64)
    c8, sc = Bnd.quantize_fp8(L, dev)
    torch.cuda.synchronize()
    assert float(sc.cpu()[0]) == 1.0
    ref = np.zeros_like(bits, dtype=np.uint8)
    ref[0, 3, 1, 5] = 0x80
    assert np.array_equal(_codes(c8), ref)


def _fp8_pair(L, qd, kd, q_bits, k_bits):
    """GPU codes and scales, checked against the oracle's; returns them and the exponents."""
    q8, qs = Bnd.quantize_fp8(L, qd)
    k8, ks = Bnd.quantize_fp8(L, kd)
    torch.cuda.synchronize()
    q8r, eq = O.quantize_fp8(q_bits)
    k8r, ek = O.quantize_fp8(k_bits)
    assert float(qs.cpu()[0]) == 2.0 ** eq and float(ks.cpu()[0]) == 2.0 ** ek
    assert np.array_equal(_codes(q8), q8r) and np.array_equal(_codes(k8), k8r)
    return q8, qs, k8, ks, q8r, eq, k8r, ek


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("with_dense", [True, False])
def test_fp8qk_block_counts_padding_and_ragged_tiles(d, with_dense):
    _need_gpu()
    B, H, tile = 1, 2, 128
    segs = [(0, 1000, 3), (1000, 170, 2)]
    dense = [(1170, 70)] if with_dense else []
    N = 1240
    query = (0, 1000)
    Tq = -(-query[1] // tile)
    q, k, v = _inputs(13 + d, B, N, H, d)
    g = np.random.default_rng(6)
    idx = _padded_rows(g, B, H, Tq, segs, tile)
    if not with_dense:
        for h in range(H):
            for i in range(Tq):
                if idx[0, h, i, 0] < 0 and idx[0, h, i, 3] < 0:
                    idx[0, h, i, 0] = i % 8
    L = Bnd.make_layer(B=B, H=H, d=d, p=16, tile=tile, n_tokens=N, query=query, segments=segs,
                       strides=(N * H * d, H * d, d))
    qd, kd, vd = (to_dev_bf16(x) for x in (q, k, v))
    q8, qs, k8, ks, q8r, eq, k8r, ek = _fp8_pair(L, qd, kd, q, k)
    out, lse = Bnd.sparse_attn_fp8qk(L, q8, k8, vd, qs, ks, to_dev(idx), dense, want_lse=True)
    torch.cuda.synchronize()
    o = bf16_to_f64(out)
    lse = lse.cpu().numpy()
    res = O.attend(q8r, k8r, v, idx, tile, query, segs, dense, dq=O.fp8_values(eq), dk=O.fp8_values(ek))
    for (b, h, i), (ref, l_ref) in res.items():
        r0, r1 = i * tile, min((i + 1) * tile, query[1])
        check_attn(o[b, r0:r1, h], ref)
        assert np.abs(lse[b, h, r0:r1] - l_ref).max() <= 2.0 ** -9


def test_fp8qk_full_budget_rows_batches_and_heads():
    """Every tile selected (B = 2, H = 3, d = 128) against dense attention over the decoded
    Q and K computed directly."""
    _need_gpu()
    B, H, d, tile = 2, 3, 128, 128
    segs = [(0, 900, 10 ** 6), (900, 300, 10 ** 6)]
    dense = [(1200, 131)]
    N = 1331
    query = (0, 900)
    q, k, v = _inputs(43, B, N, H, d)
    L = Bnd.make_layer(B=B, H=H, d=d, p=32, tile=tile, n_tokens=N, query=query, segments=segs,
                       strides=(N * H * d, H * d, d))
    qd, kd, vd = (to_dev_bf16(x) for x in (q, k, v))
    q8, qs, k8, ks, q8r, eq, k8r, ek = _fp8_pair(L, qd, kd, q, k)
    out = Bnd.sparse_attn_fp8qk(L, q8, k8, vd, qs, ks, None, dense)
    torch.cuda.synchronize()
    o = bf16_to_f64(out)
    qf, kf = O.dequant_e4m3fn(q8r, eq), O.dequant_e4m3fn(k8r, ek)
    vf = O.bf16_bits_to_f64(v)
    for b in range(B):
        for h in range(H):
            ref, _ = O.attend_rows(qf[b, :900, h], kf[b, :, h], vf[b, :, h], 1 / math.sqrt(d))
            check_attn(o[b, :900, h], ref)


def test_fp8qk_t2v5s_sampled_rows():
    """The 1344x768 5.17 s layer as the benchmark runs it: GPU quantisation of the whole Q
    and K, GPU selection, FP8 attention of every video row in the selection's tile order;
    the oracle checks the scales,
    the codes of the sampled rows and the attention of sampled (head, query tile) pairs."""
    _need_gpu()
    wl = I.WORKLOADS["t2v5s"]
    print("[t2v5s fp8] generating inputs", flush=True)
    q, k, v = I.make_qkv(wl)
    w = I.make_weights(wl)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    L = Bnd.layer_from_workload(wl)
    segs = [(s.start, s.length, s.budget) for s in wl.segments]
    dense = [(r.start, r.length) for r in wl.dense]
    idx = Bnd.select(L, qd, kd, to_dev_bf16(w.wq), to_dev_bf16(w.wk))
    q8, qs, k8, ks = (*Bnd.quantize_fp8(L, qd), *Bnd.quantize_fp8(L, kd))
    out = Bnd.sparse_attn_fp8qk(L, q8, k8, vd, qs, ks, idx, dense, order=Bnd.tile_order(L, idx))
    torch.cuda.synchronize()
    print("[t2v5s fp8] oracle", flush=True)
    # Q2 over the whole tensors: |x| as bf16 magnitude bits orders like the values
    eq = O.fp8_scale_exponent(O.bf16_bits_to_f64(np.array([(q & 0x7FFF).max()], np.uint16))[0])
    ek = O.fp8_scale_exponent(O.bf16_bits_to_f64(np.array([(k & 0x7FFF).max()], np.uint16))[0])
    assert float(qs.cpu()[0]) == 2.0 ** eq and float(ks.cpu()[0]) == 2.0 ** ek
    idx_h = idx.cpu().numpy()
    rng = np.random.default_rng(17)
    Tq = wl.n_query_tiles
    tiles = sorted({0, Tq - 1, (wl.grid[1] * wl.grid[2]) // wl.tile} | set(rng.integers(1, Tq - 1, 2).tolist()))
    heads = sorted(rng.choice(wl.H, 3, replace=False).tolist())
    q8h = q8.cpu().numpy()
    k8h = k8.cpu().numpy()
    o = out[0].float().cpu().numpy()
    for h in heads:
        for i in tiles:
            r0 = wl.query.start + i * wl.tile
            r1 = min(r0 + wl.tile, wl.query.start + wl.query.length)
            toks = O.attended_tokens(idx_h[0, h, i], wl.tile, segs, dense)
            # the codes of exactly the rows this pair reads
            assert np.array_equal(q8h[0, r0:r1, h], O.e4m3fn_round(O.bf16_bits_to_f64(q[0, r0:r1, h]) * 2.0 ** -eq))
            assert np.array_equal(k8h[0, toks, h], O.e4m3fn_round(O.bf16_bits_to_f64(k[0, toks, h]) * 2.0 ** -ek))
            ref, _ = O.attend_rows(O.dequant_e4m3fn(q8h[0, r0:r1, h], eq), O.dequant_e4m3fn(k8h[0, toks, h], ek),
                                   O.bf16_bits_to_f64(v[0, toks, h]), 1 / math.sqrt(wl.d))
            check_attn(o[r0:r1, h].astype(np.float64), ref)
