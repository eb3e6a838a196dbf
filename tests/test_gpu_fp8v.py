"""GPU parity of the FP8-V attention path (veda_sparse_attn_fp8) and its V quantiser
(veda_quantize_fp8_e4m3_vt) against the oracle, through the C ABI.

Quantiser: every code and the scale bit-exact against the oracle's Q1/Q2 codes of V,
read back through the blocked layout the header states (row c of block g keeps tokens
64 g + 16 j .. 64 g + 16 j + 15 in chunk j ^ ((c >> 1) & 3)); tokens past the end are 0.

Attention: the kernel rounds each softmax weight to E4M3FN against a running maximum
that depends on the block order, so its output is no fixed function of the inputs that
the oracle could reproduce.  The oracle computes O7 over the decoded Q, K and V codes
(fp64, exact weights); two bars relate the kernel to it.

  * Exactly representable weights.  With scale = ln 2 and codes whose dot products are
    integers in [-4, 4], every weight is 2^(s - M + 4) for an integer s - M in [-8, 4],
    which E4M3FN holds exactly, so the kernel computes the oracle's result up to its fp32 sums
    (the f8f6f4 products sum 64 terms within 2^-12 of the largest) and the bf16 store:
        |o - o_ref| <= 2^-8 |o_ref| + 2^-11 max_m |v_m|,   |lse - lse_ref| <= 2^-12.
    A misplaced weight or key, a dropped or doubled block, a stale rescale or a wrong
    normaliser all fail it.
  * General logits.  Scaled so that the row's largest exact weight is 1, a rounded
    weight with exact value p_m >= 2^-10 is a normal E4M3 code, off by at most
    e_m = 2^-4 p_m (three mantissa bits); a smaller one is subnormal or 0, off by at
    most u_m = min(p_m, 2^-14), and these errors can all lean one way (values under
    2^-14 all round to 0).  To first order the output moves by
    sum_m dp_m (v_m - o) / sum_m p_m (the normaliser sums the same rounded weights).
    The normal-range roundings act as independent zero-mean errors with variance at
    most e_m^2 / 3 (uniform on [-e_m, e_m] at worst); the subnormal ones are bounded
    outright.  Per output element
        sigma = sqrt(sum_m e_m^2 (v_m - o)^2 / 3) / sum_m p_m,
        b     = sum_m u_m (|v_m| + |o|) / sum_m p_m,
    and with h = 2^-8 |o_ref| + 2^-9 max_m |v_m| (bf16 store, fp32 sums and the FP8
    logits' own error) the bar is |o - o_ref| <= 6 sigma + b + h for every element, a
    root mean square of (o - o_ref) / (sigma + b + h) of at most 1, every output inside
    [min_m v_m, max_m v_m] up to the bf16 store, and
    |lse - lse_ref| <= 6 sigma_l + b_l + 2^-9 with sigma_l = sqrt(sum_m e_m^2 / 3) /
    sum_m p_m and b_l = sum_m u_m / sum_m p_m.
"""
import gc
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_predictor_amd import binding as Bnd
from block_sparse_attention_predictor_amd import inputs as I
from oracle import veda_oracle as O
from gpu_util import bf16_to_f64, to_dev, to_dev_bf16
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


def vt_to_token_major(vt: np.ndarray, n_tokens: int) -> np.ndarray:
    """[B, H, G, d, 64] blocked codes -> [B, n_tokens, H, d] (and asserts the pad is 0)."""
    B, H, G, d, _ = vt.shape
    chunks = vt.reshape(B, H, G, d, 4, 16)
    tok = np.empty_like(chunks)
    for sw in range(4):                       # rows whose chunks are permuted by j -> j ^ sw
        rows = np.nonzero(((np.arange(d) >> 1) & 3) == sw)[0]
        tok[:, :, :, rows] = chunks[:, :, :, rows][:, :, :, :, np.arange(4) ^ sw]
    full = tok.reshape(B, H, G, d, 64).transpose(0, 2, 4, 1, 3).reshape(B, G * 64, H, d)
    assert not full[:, n_tokens:].any(), "codes past the last token"
    return full[:, :n_tokens]


def _quantize_all(L, q, k, v):
    """GPU codes and scales of Q, K (row layout) and V (blocked), each checked bit-exact
    against the oracle; returns the device tensors and the oracle's codes and exponents."""
    qd, kd, vd = (to_dev_bf16(x) for x in (q, k, v))
    q8, qs = Bnd.quantize_fp8(L, qd)
    k8, ks = Bnd.quantize_fp8(L, kd)
    vt, vs = Bnd.quantize_fp8_vt(L, vd)
    torch.cuda.synchronize()
    ref = {}
    for name, bits, dev, sc in (("q", q, q8, qs), ("k", k, k8, ks), ("v", v, None, vs)):
        codes, e = O.quantize_fp8(bits)
        assert float(sc.cpu()[0]) == 2.0 ** e, name
        got = dev.cpu().numpy() if dev is not None else vt_to_token_major(vt.cpu().numpy(), bits.shape[1])
        assert np.array_equal(got, codes), name
        ref[name] = (codes, e)
    return (q8, qs, k8, ks, vt, vs), ref


def _exact_bar(o, ref, vmax):
    err = np.abs(o - ref)
    bar = 2.0 ** -8 * np.abs(ref) + 2.0 ** -11 * vmax
    assert np.all(err <= bar), f"max err {err.max():.3e}, worst excess {(err - bar).max():.3e}"


class StatBar:
    """Accumulates the general-logit bar over rows; `finish` checks the pooled RMS."""

    def __init__(self):
        self.z2 = []
        self.worst = 0.0

    def check(self, o, lse, qf, kf, vf, scale):
        ref, lse_ref = O.attend_rows(qf, kf, vf, scale)
        s = scale * (qf @ kf.T)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        normal = p >= 2.0 ** -10
        e2 = np.where(normal, 2.0 ** -4 * p, 0.0) ** 2
        u = np.where(normal, 0.0, np.minimum(p, 2.0 ** -14))
        psum = p.sum(axis=1)
        # sum_m e_m^2 (v_md - o_d)^2 for every (row, d), expanded in the three sums
        var = e2 @ (vf * vf) - 2 * ref * (e2 @ vf) + ref * ref * e2.sum(axis=1, keepdims=True)
        sigma = np.sqrt(np.maximum(var, 0.0) / 3.0) / psum[:, None]
        b = (u @ np.abs(vf) + np.abs(ref) * u.sum(axis=1, keepdims=True)) / psum[:, None]
        vmax = np.abs(vf).max()
        h = 2.0 ** -8 * np.abs(ref) + 2.0 ** -9 * vmax
        err = np.abs(o - ref)
        z = err / (sigma + b + h)
        assert np.all(err <= 6 * sigma + b + h), f"max err {err.max():.3e}, max z {z.max():.2f}"
        self.z2.append((z ** 2).ravel())
        self.worst = max(self.worst, float(z.max()))
        tol = 2.0 ** -8 * np.abs(o) + 1e-6
        assert np.all(o >= vf.min(axis=0) - tol) and np.all(o <= vf.max(axis=0) + tol), "outside the hull of V"
        if lse is not None:
            sigma_l = np.sqrt(e2.sum(axis=1) / 3.0) / psum
            dl = np.abs(lse - lse_ref)
            bar_l = 6 * sigma_l + u.sum(axis=1) / psum + 2.0 ** -9
            assert np.all(dl <= bar_l), f"lse: max err {dl.max():.3e}, worst excess {(dl - bar_l).max():.3e}"
        return ref

    def finish(self):
        z2 = np.concatenate(self.z2)
        rms = float(np.sqrt(z2.mean()))
        print(f"[fp8v] {z2.size} elements: rms z {rms:.3f}, max z {self.worst:.2f}", flush=True)
        assert rms <= 1.0, rms


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("head_major", [False, True])
def test_quantize_vt_codes_layout_and_pad(d, head_major):
    _need_gpu()
    B, N, H = 2, 333, 3                       # 6 blocks, the last one 13 tokens long
    g = np.random.default_rng(5 + d)
    x = np.clip(g.standard_normal((B, N, H, d)) * 40.0, -440, 440).astype(np.float32)
    x.reshape(-1)[:4] = [448.0, 2.0 ** -10, -0.0, 1.0625]
    bits = I.f32_to_bf16_bits(x)
    if head_major:
        store = np.ascontiguousarray(bits.transpose(0, 2, 1, 3))
        dev = to_dev_bf16(store).permute(0, 2, 1, 3)
    else:
        dev = to_dev_bf16(bits)
    L = Bnd.make_layer(B=B, H=H, d=d, p=16, tile=128, n_tokens=N, query=(0, N), segments=[(0, N, 1)],
                       strides=tuple(dev.stride()[:3]))
    assert Bnd.fp8_vt_bytes(L) == B * H * 6 * d * 64
    vt, vs = Bnd.quantize_fp8_vt(L, dev)
    torch.cuda.synchronize()
    codes, e = O.quantize_fp8(bits)
    assert float(vs.cpu()[0]) == 2.0 ** e
    assert np.array_equal(vt_to_token_major(vt.cpu().numpy(), N), codes)


def _exact_inputs(seed, B, N, H, d):
    """Q rows with four ones, K rows in {-1, 0, 1}: every dot product an integer in [-4, 4]."""
    g = np.random.default_rng(seed)
    q = np.zeros((B, N, H, d), np.float32)
    cols = np.argsort(g.random((B, N, H, d)), axis=-1)[..., :4]
    np.put_along_axis(q, cols, 1.0, axis=-1)
    k = g.integers(-1, 2, (B, N, H, d)).astype(np.float32)
    v = g.standard_normal((B, N, H, d)).astype(np.float32)
    return tuple(I.f32_to_bf16_bits(x) for x in (q, k, v))


@pytest.mark.parametrize("d", [64, 128])
def test_fp8v_exact_weights(d):
    """Power-of-two weights: the kernel must give the oracle's attention to fp32 / bf16."""
    _need_gpu()
    B, H, tile = 1, 2, 128
    segs = [(0, 1000, 3), (1024, 170, 2)]
    dense = [(1216, 70)]
    N = 1286
    query = (0, 1000)
    Tq = -(-query[1] // tile)
    q, k, v = _exact_inputs(31 + d, B, N, H, d)
    idx = _padded_rows(np.random.default_rng(9), B, H, Tq, segs, tile)
    L = Bnd.make_layer(B=B, H=H, d=d, p=16, tile=tile, n_tokens=N, query=query, segments=segs,
                       strides=(N * H * d, H * d, d))
    (q8, qs, k8, ks, vt, vs), ref = _quantize_all(L, q, k, v)
    out, lse = Bnd.sparse_attn_fp8(L, q8, k8, vt, qs, ks, vs, to_dev(idx), dense, scale=math.log(2.0),
                                   want_lse=True)
    torch.cuda.synchronize()
    o = bf16_to_f64(out)
    lse = lse.cpu().numpy()
    (q8r, eq), (k8r, ek), (v8r, ev) = ref["q"], ref["k"], ref["v"]
    res = O.attend(q8r, k8r, v8r, idx, tile, query, segs, dense, scale=math.log(2.0),
                   dq=O.fp8_values(eq), dk=O.fp8_values(ek), dv=O.fp8_values(ev))
    vmax = np.abs(O.dequant_e4m3fn(v8r, ev)).max()
    for (b, h, i), (r, l_ref) in res.items():
        r0, r1 = i * tile, min((i + 1) * tile, query[1])
        _exact_bar(o[b, r0:r1, h], r, vmax)
        assert np.abs(lse[b, h, r0:r1] - l_ref).max() <= 2.0 ** -12


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("with_dense", [True, False])
def test_fp8v_block_counts_padding_and_ragged_tiles(d, with_dense):
    """0..K blocks per row, -1 padding, partial tiles and partial 64-key blocks."""
    _need_gpu()
    B, H, tile = 1, 2, 128
    segs = [(0, 1000, 3), (1024, 170, 2)]
    dense = [(1216, 70)] if with_dense else []
    N = 1286
    query = (0, 1000)
    Tq = -(-query[1] // tile)
    q, k, v = _inputs(13 + d, B, N, H, d)
    idx = _padded_rows(np.random.default_rng(6), B, H, Tq, segs, tile)
    if not with_dense:
        for h in range(H):
            for i in range(Tq):
                if idx[0, h, i, 0] < 0 and idx[0, h, i, 3] < 0:
                    idx[0, h, i, 0] = i % 8
    L = Bnd.make_layer(B=B, H=H, d=d, p=16, tile=tile, n_tokens=N, query=query, segments=segs,
                       strides=(N * H * d, H * d, d))
    (q8, qs, k8, ks, vt, vs), ref = _quantize_all(L, q, k, v)
    out, lse = Bnd.sparse_attn_fp8(L, q8, k8, vt, qs, ks, vs, to_dev(idx), dense, want_lse=True)
    torch.cuda.synchronize()
    o = bf16_to_f64(out)
    lse = lse.cpu().numpy()
    (q8r, eq), (k8r, ek), (v8r, ev) = ref["q"], ref["k"], ref["v"]
    bar = StatBar()
    for h in range(H):
        for i in range(Tq):
            r0, r1 = i * tile, min((i + 1) * tile, query[1])
            toks = O.attended_tokens(idx[0, h, i], tile, segs, dense)
            bar.check(o[0, r0:r1, h], lse[0, h, r0:r1], O.dequant_e4m3fn(q8r[0, r0:r1, h], eq),
                      O.dequant_e4m3fn(k8r[0, toks, h], ek), O.dequant_e4m3fn(v8r[0, toks, h], ev),
                      1 / math.sqrt(d))
    bar.finish()


def test_fp8v_full_budget_rows_batches_and_heads():
    """Every tile selected (B = 2, H = 3, d = 128), no index tensor."""
    _need_gpu()
    B, H, d, tile = 2, 3, 128, 128
    segs = [(0, 896, 10 ** 6), (896, 300, 10 ** 6)]
    dense = [(1216, 131)]
    N = 1347
    query = (0, 896)
    q, k, v = _inputs(43, B, N, H, d)
    L = Bnd.make_layer(B=B, H=H, d=d, p=32, tile=tile, n_tokens=N, query=query, segments=segs,
                       strides=(N * H * d, H * d, d))
    (q8, qs, k8, ks, vt, vs), ref = _quantize_all(L, q, k, v)
    out = Bnd.sparse_attn_fp8(L, q8, k8, vt, qs, ks, vs, None, dense)
    torch.cuda.synchronize()
    o = bf16_to_f64(out)
    (q8r, eq), (k8r, ek), (v8r, ev) = ref["q"], ref["k"], ref["v"]
    toks = np.r_[0:1196, 1216:1347]
    bar = StatBar()
    for b in range(B):
        for h in range(H):
            bar.check(o[b, :896, h], None, O.dequant_e4m3fn(q8r[b, :896, h], eq), O.dequant_e4m3fn(k8r[b, toks, h], ek),
                      O.dequant_e4m3fn(v8r[b, toks, h], ev), 1 / math.sqrt(d))
    bar.finish()


def test_fp8v_rejects_unaligned_starts():
    _need_gpu()
    B, H, d, N = 1, 1, 64, 512
    q, k, v = _inputs(3, B, N, H, d)
    L = Bnd.make_layer(B=B, H=H, d=d, p=16, tile=128, n_tokens=N, query=(0, 256), segments=[(0, 256, 2)],
                       strides=(N * H * d, H * d, d))
    (q8, qs, k8, ks, vt, vs), _ = _quantize_all(L, q, k, v)
    with pytest.raises(Bnd.VedaError):
        Bnd.sparse_attn_fp8(L, q8, k8, vt, qs, ks, vs, None, [(300, 10)])
    L2 = Bnd.make_layer(B=B, H=H, d=d, p=16, tile=128, n_tokens=N, query=(0, 256), segments=[(32, 224, 2)],
                        strides=(N * H * d, H * d, d))
    with pytest.raises(Bnd.VedaError):
        Bnd.sparse_attn_fp8(L2, q8, k8, vt, qs, ks, vs, None)


def test_fp8v_t2v5s_sampled_rows():
    """The 1344x768 5.17 s layer as the benchmark runs it: GPU quantisation of Q, K and V,
    GPU selection, FP8 attention of every video row in the selection's tile order; the
    oracle checks the scales, the
    codes the sampled rows read and the attention of sampled (head, query tile) pairs."""
    _need_gpu()
    wl = I.WORKLOADS["t2v5s"]
    print("[t2v5s fp8v] generating inputs", flush=True)
    q, k, v = I.make_qkv(wl)
    w = I.make_weights(wl)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    L = Bnd.layer_from_workload(wl)
    segs = [(s.start, s.length, s.budget) for s in wl.segments]
    dense = [(r.start, r.length) for r in wl.dense]
    idx = Bnd.select(L, qd, kd, to_dev_bf16(w.wq), to_dev_bf16(w.wk))
    q8, qs = Bnd.quantize_fp8(L, qd)
    k8, ks = Bnd.quantize_fp8(L, kd)
    vt, vs = Bnd.quantize_fp8_vt(L, vd)
    out, lse = Bnd.sparse_attn_fp8(L, q8, k8, vt, qs, ks, vs, idx, dense, want_lse=True,
                                   order=Bnd.tile_order(L, idx))
    torch.cuda.synchronize()
    print("[t2v5s fp8v] oracle", flush=True)
    exps = []
    for bits, sc in ((q, qs), (k, ks), (v, vs)):
        e = O.fp8_scale_exponent(O.bf16_bits_to_f64(np.array([(bits & 0x7FFF).max()], np.uint16))[0])
        assert float(sc.cpu()[0]) == 2.0 ** e
        exps.append(e)
    eq, ek, ev = exps
    idx_h = idx.cpu().numpy()
    rng = np.random.default_rng(19)
    Tq = wl.n_query_tiles
    tiles = sorted({0, Tq - 1, (wl.grid[1] * wl.grid[2]) // wl.tile} | set(rng.integers(1, Tq - 1, 2).tolist()))
    heads = sorted(rng.choice(wl.H, 3, replace=False).tolist())
    q8h, k8h = q8.cpu().numpy(), k8.cpu().numpy()
    v8h = vt_to_token_major(vt[:, heads].cpu().numpy(), v.shape[1])    # the sampled heads only
    o = out[0].float().cpu().numpy().astype(np.float64)
    lse_h = lse.cpu().numpy()
    bar = StatBar()
    for hs, h in enumerate(heads):
        for i in tiles:
            r0 = wl.query.start + i * wl.tile
            r1 = min(r0 + wl.tile, wl.query.start + wl.query.length)
            toks = O.attended_tokens(idx_h[0, h, i], wl.tile, segs, dense)
            assert np.array_equal(q8h[0, r0:r1, h], O.e4m3fn_round(O.bf16_bits_to_f64(q[0, r0:r1, h]) * 2.0 ** -eq))
            assert np.array_equal(k8h[0, toks, h], O.e4m3fn_round(O.bf16_bits_to_f64(k[0, toks, h]) * 2.0 ** -ek))
            assert np.array_equal(v8h[0, toks, hs], O.e4m3fn_round(O.bf16_bits_to_f64(v[0, toks, h]) * 2.0 ** -ev))
            bar.check(o[r0:r1, h], lse_h[0, h, r0 - wl.query.start:r1 - wl.query.start],
                      O.dequant_e4m3fn(q8h[0, r0:r1, h], eq), O.dequant_e4m3fn(k8h[0, toks, h], ek),
                      O.dequant_e4m3fn(v8h[0, toks, hs], ev), 1 / math.sqrt(wl.d))
    bar.finish()
