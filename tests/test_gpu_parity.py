"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, on the
same seeded inputs, at sizes the oracle finishes in seconds (several tiles and
ragged tails), plus edge cases.  Needs an MI355X and the built libveda.so."""
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_predictor_amd import binding as Bnd
from block_sparse_attention_predictor_amd import inputs as I
from oracle import veda_oracle as O

from gpu_util import (bf16_to_f64, check_attn, check_indices, check_scores, to_dev, to_dev_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    Bnd._load()   # fails loudly when the library is missing


# ----------------------------------------------------------------------------- cases

class Case:
    """A layer with inputs; either a named workload or a hand-laid-out edge case."""

    def __init__(self, name, B, H, d, p, tile, n_tokens, query, segments, dense, q, k, v, wq, wk):
        self.name = name
        self.B, self.H, self.d, self.p, self.tile, self.n_tokens = B, H, d, p, tile, n_tokens
        self.query, self.segments, self.dense = query, segments, dense
        self.q, self.k, self.v, self.wq, self.wk = q, k, v, wq, wk

    def layer(self, strides=None):
        if strides is None:
            strides = (self.n_tokens * self.H * self.d, self.H * self.d, self.d)
        return Bnd.make_layer(B=self.B, H=self.H, d=self.d, p=self.p, tile=self.tile,
                              n_tokens=self.n_tokens, query=self.query, segments=self.segments,
                              strides=strides)

    @property
    def seg_T(self):
        return [-(-ln // self.tile) for (_, ln, _) in self.segments]

    @property
    def seg_K(self):
        return [min(b, T) for (_, _, b), T in zip(self.segments, self.seg_T)]


def workload_case(name):
    wl = I.WORKLOADS[name]
    q, k, v = I.make_qkv(wl)
    w = I.make_weights(wl)
    wq = O.dequant_e4m3fn_to_bf16_bits(w.wq, w.pow2_exp) if w.fp8 else w.wq
    wk = O.dequant_e4m3fn_to_bf16_bits(w.wk, w.pow2_exp) if w.fp8 else w.wk
    return Case(name, wl.B, wl.H, wl.d, wl.p, wl.tile, wl.n_tokens,
                (wl.query.start, wl.query.length),
                [(s.start, s.length, s.budget) for s in wl.segments],
                [(r.start, r.length) for r in wl.dense], q, k, v, wq, wk)


def random_case(name, seed, B, H, d, p, tile, layout, query, segments, dense, scale=1.0):
    """layout: total tokens; inputs N(0,1)*scale plus a smooth ramp so scores are not all alike."""
    g = np.random.default_rng(seed)
    N = layout
    base = g.standard_normal((B, N, H, d)).astype(np.float32) * scale
    ramp = np.sin(np.arange(N) / 17.0)[None, :, None, None].astype(np.float32)
    qf = base + 0.5 * ramp * g.standard_normal((1, 1, H, d)).astype(np.float32)
    kf = g.standard_normal((B, N, H, d)).astype(np.float32) * scale + \
        0.5 * ramp * g.standard_normal((1, 1, H, d)).astype(np.float32)
    vf = g.standard_normal((B, N, H, d)).astype(np.float32)
    wq = I.f32_to_bf16_bits(g.standard_normal((H, p, d)).astype(np.float32) / math.sqrt(d))
    wk = I.f32_to_bf16_bits(g.standard_normal((H, p, d)).astype(np.float32) / math.sqrt(d))
    return Case(name, B, H, d, p, tile, N, query, segments, dense,
                I.f32_to_bf16_bits(qf), I.f32_to_bf16_bits(kf), I.f32_to_bf16_bits(vf), wq, wk)


def edge_cases():
    return {
        # ragged everything, d=64, tile=64, two segments, query not at token 0
        "ragged_d64": lambda: random_case(
            "ragged_d64", 1, B=1, H=3, d=64, p=32, tile=64, layout=40 + 300 + 70 + 25,
            query=(40, 300), segments=[(340, 70, 5), (40, 300, 2)], dense=[(0, 40), (410, 25)]),
        # batch 2, d=128, tile=128, p=48 (not a multiple of 32), one budget zero
        "b2_p48_zero_budget": lambda: random_case(
            "b2_p48_zero_budget", 2, B=2, H=2, d=128, p=48, tile=128, layout=700 + 130 + 61,
            query=(0, 700), segments=[(0, 700, 3), (700, 130, 0)], dense=[(830, 61)]),
        # d=64 with tile=128, no dense keys, budget above the tile count
        "d64_t128_nodense": lambda: random_case(
            "d64_t128_nodense", 3, B=1, H=2, d=64, p=16, tile=128, layout=1000,
            query=(0, 1000), segments=[(0, 1000, 99)], dense=[]),
        # d=128 with tile=64, four segments, dense range of one token
        "four_segments": lambda: random_case(
            "four_segments", 4, B=1, H=2, d=128, p=64, tile=64, layout=800,
            query=(100, 500), segments=[(0, 64, 1), (64, 36, 1), (100, 500, 3), (600, 199, 2)],
            dense=[(799, 1)]),
    }


_CACHE = {}


def get_case(name):
    if name not in _CACHE:
        if name in I.WORKLOADS:
            _CACHE[name] = workload_case(name)
        else:
            _CACHE[name] = edge_cases()[name]()
    return _CACHE[name]


def oracle_select(c):
    key = ("sel", c.name)
    if key not in _CACHE:
        _CACHE[key] = O.select(c.q, c.k, c.wq, c.wk, c.tile, c.query, c.segments)
    return _CACHE[key]


def dev_inputs(c):
    key = ("dev", c.name)
    if key not in _CACHE:
        _CACHE[key] = tuple(to_dev_bf16(x) for x in (c.q, c.k, c.v, c.wq, c.wk))
    return _CACHE[key]


SMALL = ["tiny", "mid", "ragged_d64", "b2_p48_zero_budget", "d64_t128_nodense", "four_segments"]


# ----------------------------------------------------------------------------- a0 dequant

@pytest.mark.parametrize("e", [0, -4, 7])
def test_dequant_all_codes(e):
    codes = np.arange(256, dtype=np.uint8)
    got = Bnd.dequant_fp8_e4m3(to_dev(codes), e).view(torch.int16).cpu().numpy().view(np.uint16)
    finite = (codes & 0x7F) != 0x7F
    ref = O.dequant_e4m3fn_to_bf16_bits(codes[finite], e)
    assert np.array_equal(got[finite], ref)
    assert np.array_equal(got[~finite], [0x7FC0, 0xFFC0])


def test_dequant_ragged_length_and_weights():
    w = I.make_weights(I.WORKLOADS["t2v14s"])
    flat = w.wq.reshape(-1)[:12345]            # not a multiple of the 4-byte unit
    got = Bnd.dequant_fp8_e4m3(to_dev(flat), w.pow2_exp).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, O.dequant_e4m3fn_to_bf16_bits(flat, w.pow2_exp))


# ----------------------------------------------------------------------------- a1 + a2

@pytest.mark.parametrize("name", SMALL)
def test_pool_project(name):
    c = get_case(name)
    q, k, v, wq, wk = dev_inputs(c)
    L = c.layer()
    qh, kh = Bnd.project(L, q, k, wq, wk)
    torch.cuda.synchronize()
    _, _, QH, KH = oracle_select(c)
    for got, ref in ((qh.cpu().numpy(), QH), (kh.cpu().numpy(), KH)):
        scale = np.abs(ref).max(axis=(-1, -2), keepdims=True)
        assert np.abs(got - ref).max() <= 2e-6 * scale.max(), name


# ----------------------------------------------------------------------------- a3 + a4

@pytest.mark.parametrize("name", SMALL)
def test_select_scores_and_indices(name):
    c = get_case(name)
    q, k, v, wq, wk = dev_inputs(c)
    L = c.layer()
    idx, sc = Bnd.select(L, q, k, wq, wk, want_scores=True)
    torch.cuda.synchronize()
    idx_ref, S_ref, _, _ = oracle_select(c)
    check_scores(sc.cpu().numpy().astype(np.float64), S_ref)
    check_indices(idx.cpu().numpy(), idx_ref, S_ref, c.seg_T, c.seg_K)


def test_topk_exact_ties_and_signed_zero():
    """Projected vectors with exact, repeated scores: ids must follow the lowest-index rule
    bit for bit (scores are exact small integers, so no tie window is needed)."""
    g = np.random.default_rng(21)
    B, H, p, tile = 1, 2, 32, 64
    Tq, T0, T1 = 5, 37, 300
    segs = [(0, T0 * tile, 7), (T0 * tile, T1 * tile - 10, 40)]
    L = Bnd.make_layer(B=B, H=H, d=64, p=p, tile=tile, n_tokens=(T0 + T1) * tile,
                       query=(0, Tq * tile), segments=segs, strides=((T0 + T1) * tile * H * 64, H * 64, 64))
    qh = np.zeros((B, H, Tq, p), np.float32)
    kh = np.zeros((B, H, T0 + T1, p), np.float32)
    qh[..., 0] = g.integers(-2, 3, (B, H, Tq))
    kh[..., 0] = g.integers(-3, 4, (B, H, T0 + T1))     # many equal scores
    kh[0, 0, 5, 0] = -0.0
    qh[0, 0, 0, 0] = 1.0
    idx, sc = Bnd.score_topk(L, to_dev(qh), to_dev(kh), want_scores=True)
    torch.cuda.synchronize()
    S = qh.astype(np.float64) @ np.swapaxes(kh.astype(np.float64), -1, -2)
    assert np.array_equal(sc.cpu().numpy().astype(np.float64), S)
    ref = np.zeros((B, H, Tq, 47), np.int32)
    for h in range(H):
        for i in range(Tq):
            ref[0, h, i, :7] = O.topk_lowest_index(S[0, h, i, :T0], 7)
            ref[0, h, i, 7:] = O.topk_lowest_index(S[0, h, i, T0:], 40)
    assert np.array_equal(idx.cpu().numpy(), ref)


@pytest.mark.parametrize("K", [1, 7, 137, 256, 257, 2100])
@pytest.mark.parametrize("kind", ["ties", "wide", "equal", "negative"])
def test_topk_long_rows_exact(kind, K):
    """Rows of 2100 key tiles (the length at which the top-k starts its radix below the top
    bit, from the smallest of its group maxima and the largest key), with exact integer
    scores: few values with many ties and signed zeros, values spread over many binades,
    one value everywhere, all negative; budgets on both sides of 256 (the largest budget
    that takes the bound) and the whole segment.  Bit-exact against the lowest-index rule;
    a short second segment checks the rows that do not take the bound."""
    g = np.random.default_rng(31 + K)
    B, H, p, tile = 1, 2, 32, 64
    Tq, T0, T1 = 6, 2100, 40
    segs = [(0, T0 * tile, K), (T0 * tile, T1 * tile, 7)]
    L = Bnd.make_layer(B=B, H=H, d=64, p=p, tile=tile, n_tokens=(T0 + T1) * tile,
                       query=(0, Tq * tile), segments=segs, strides=((T0 + T1) * tile * H * 64, H * 64, 64))
    qh = np.zeros((B, H, Tq, p), np.float32)
    kh = np.zeros((B, H, T0 + T1, p), np.float32)
    if kind == "ties":
        qh[..., 0] = g.integers(-2, 3, (B, H, Tq))
        qh[0, 0, 0, 0] = 1.0
        kh[..., 0] = g.integers(-3, 4, (B, H, T0 + T1))
        kh[0, 0, 5, 0] = -0.0
    elif kind == "wide":      # integers up to 256 are exact in bf16, sums exact in fp32
        qh[..., :2] = g.integers(-100, 101, (B, H, Tq, 2))
        kh[..., :2] = g.integers(-200, 201, (B, H, T0 + T1, 2))
    elif kind == "equal":
        qh[..., 0] = 3.0
        kh[..., 0] = 5.0
    else:
        qh[..., 0] = 1.0
        kh[..., 0] = -g.integers(1, 201, (B, H, T0 + T1))
    idx, sc = Bnd.score_topk(L, to_dev(qh), to_dev(kh), want_scores=True)
    torch.cuda.synchronize()
    S = qh.astype(np.float64) @ np.swapaxes(kh.astype(np.float64), -1, -2)
    assert np.array_equal(sc.cpu().numpy().astype(np.float64), S)
    K0 = min(K, T0)
    ref = np.zeros((B, H, Tq, K0 + 7), np.int32)
    for h in range(H):
        for i in range(Tq):
            ref[0, h, i, :K0] = O.topk_lowest_index(S[0, h, i, :T0], K0)
            ref[0, h, i, K0:] = O.topk_lowest_index(S[0, h, i, T0:], 7)
    assert np.array_equal(idx.cpu().numpy(), ref)


# ----------------------------------------------------------------------------- a5

def _oracle_attn_all(c, idx):
    return O.attend(c.q, c.k, c.v, idx, c.tile, c.query, c.segments, c.dense)


def _gpu_rows(c, out, b, h, i):
    q0 = c.query[0] + i * c.tile
    q1 = c.query[0] + min((i + 1) * c.tile, c.query[1])
    return out[b, q0:q1, h, :]


@pytest.mark.parametrize("name", SMALL)
def test_attention_with_oracle_indices(name):
    c = get_case(name)
    q, k, v, _, _ = dev_inputs(c)
    idx_ref, _, _, _ = oracle_select(c)
    L = c.layer()
    out, lse = Bnd.sparse_attn(L, q, k, v, to_dev(idx_ref), c.dense, want_lse=True)
    torch.cuda.synchronize()
    o = bf16_to_f64(out)
    lse = lse.cpu().numpy()
    res = _oracle_attn_all(c, idx_ref)
    got = np.concatenate([_gpu_rows(c, o, b, h, i) for (b, h, i) in res])
    ref = np.concatenate([r[0] for r in res.values()])
    check_attn(got, ref)
    # the kernel normalises by the sum of the bf16-rounded weights that also multiply V
    # (each within 2^-9 relative of the exact weight), so |lse - lse_ref| <= 2^-9
    # up to fp32 rounding
    for (b, h, i), (_, l_ref) in res.items():
        r0 = i * c.tile
        assert np.abs(lse[b, h, r0:r0 + len(l_ref)] - l_ref).max() <= 2.0 ** -9
    # rows outside the query segment are left untouched (zeros from the caller)
    mask = np.ones(c.n_tokens, bool)
    mask[c.query[0]:c.query[0] + c.query[1]] = False
    assert np.all(o[:, mask] == 0)


@pytest.mark.parametrize("name", ["tiny", "ragged_d64", "b2_p48_zero_budget"])
def test_full_budget_matches_dense_attention(name):
    c = get_case(name)
    q, k, v, _, _ = dev_inputs(c)
    full = [(st, ln, 10 ** 6) for (st, ln, _) in c.segments]
    L = Bnd.make_layer(B=c.B, H=c.H, d=c.d, p=c.p, tile=c.tile, n_tokens=c.n_tokens, query=c.query,
                       segments=full, strides=(c.n_tokens * c.H * c.d, c.H * c.d, c.d))
    Tq = -(-c.query[1] // c.tile)
    idx = np.concatenate([np.broadcast_to(np.arange(T, dtype=np.int32), (c.B, c.H, Tq, T))
                          for T in c.seg_T], axis=-1)
    out = Bnd.sparse_attn(L, q, k, v, to_dev(idx), c.dense)
    torch.cuda.synchronize()
    o = bf16_to_f64(out)
    # dense attention over every segment token and every dense token, computed directly
    keys = np.concatenate([np.arange(st, st + ln) for (st, ln, _) in c.segments] +
                          [np.arange(st, st + ln) for (st, ln) in c.dense])
    qf, kf, vf = (O.bf16_bits_to_f64(x) for x in (c.q, c.k, c.v))
    q0, q1 = c.query[0], c.query[0] + c.query[1]
    for b in range(c.B):
        for h in range(c.H):
            ref, _ = O.attend_rows(qf[b, q0:q1, h], kf[b, keys, h], vf[b, keys, h], 1 / math.sqrt(c.d))
            check_attn(o[b, q0:q1, h], ref)


def test_attention_constant_v_and_scale():
    c = get_case("ragged_d64")
    q, k, _, _, _ = dev_inputs(c)
    idx_ref, _, _, _ = oracle_select(c)
    ones = torch.ones_like(q)
    out = Bnd.sparse_attn(c.layer(), q, k, ones, to_dev(idx_ref), c.dense)
    torch.cuda.synchronize()
    o = bf16_to_f64(out)[:, c.query[0]:c.query[0] + c.query[1]]
    assert np.abs(o - 1.0).max() <= 2 ** -7
    # an explicit scale equals the default 1/sqrt(d)
    a = Bnd.sparse_attn(c.layer(), q, k, dev_inputs(c)[2], to_dev(idx_ref), c.dense)
    b = Bnd.sparse_attn(c.layer(), q, k, dev_inputs(c)[2], to_dev(idx_ref), c.dense,
                        scale=1 / math.sqrt(c.d))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_random_indices_and_strided_layout():
    """Uniformly random index sets; the same layer stored head-major ([B, H, N, d]) through
    strides gives bit-identical results."""
    c = get_case("mid")
    wl = I.WORKLOADS["mid"]
    idx = I.random_indices(wl, seed=3)
    q, k, v, _, _ = dev_inputs(c)
    out = Bnd.sparse_attn(c.layer(), q, k, v, to_dev(idx), c.dense)
    # head-major storage viewed as [B, N, H, d]
    qs, ks, vs = (x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for x in (q, k, v))
    Ls = c.layer(strides=(qs.stride(0), qs.stride(1), qs.stride(2)))
    outs = torch.zeros_like(qs)
    Bnd.sparse_attn(Ls, qs, ks, vs, to_dev(idx), c.dense, out=outs)
    torch.cuda.synchronize()
    assert torch.equal(out, outs.contiguous())
    pairs = [(0, h, i) for h in (0, 7, 23) for i in (0, 1, 100, 251)]
    res = O.attend(c.q, c.k, c.v, idx, c.tile, c.query, c.segments, c.dense, pairs=pairs)
    o = bf16_to_f64(out)
    got = np.concatenate([_gpu_rows(c, o, b, h, i) for (b, h, i) in res])
    check_attn(got, np.concatenate([r[0] for r in res.values()]))


def test_deterministic_across_runs():
    c = get_case("mid")
    q, k, v, wq, wk = dev_inputs(c)
    L = c.layer()
    i1, s1 = Bnd.select(L, q, k, wq, wk, want_scores=True)
    i2, s2 = Bnd.select(L, q, k, wq, wk, want_scores=True)
    o1 = Bnd.sparse_attn(L, q, k, v, i1, c.dense)
    o2 = Bnd.sparse_attn(L, q, k, v, i2, c.dense)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(s1, s2) and torch.equal(o1, o2)


def test_end_to_end_select_then_attend():
    """GPU selection feeding GPU attention, checked against the oracle's attention
    over the very same index sets (after those sets pass the index criterion)."""
    c = get_case("mid")
    q, k, v, wq, wk = dev_inputs(c)
    L = c.layer()
    idx = Bnd.select(L, q, k, wq, wk)
    out = Bnd.sparse_attn(L, q, k, v, idx, c.dense)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    idx_ref, S_ref, _, _ = oracle_select(c)
    check_indices(idx_np, idx_ref, S_ref, c.seg_T, c.seg_K)
    pairs = [(0, h, i) for h in (0, 11, 23) for i in range(0, 252, 25)]
    res = O.attend(c.q, c.k, c.v, idx_np, c.tile, c.query, c.segments, c.dense, pairs=pairs)
    o = bf16_to_f64(out)
    got = np.concatenate([_gpu_rows(c, o, b, h, i) for (b, h, i) in res])
    check_attn(got, np.concatenate([r[0] for r in res.values()]))
