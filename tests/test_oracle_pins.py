"""Pins of the fp64 oracle against things other than itself.

Each expected value here comes from the OCP FP8 spec table (golden file), a
closed form, a library routine (torch float8 conversion, torch SDPA in float64
on the CPU, torch.logsumexp), or brute force on tiny inputs (exhaustive subset
enumeration, exact rational arithmetic with fractions.Fraction).  The last
section plants plausible mistakes in the oracle and checks that some pin fails.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import veda_oracle as O
from block_sparse_attention_predictor_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ============================================================================ O1 FP8 decode

def _golden_e4m3():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3fn_spec_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()
            rows.append((int(code, 16), float(val)))
    return rows


def test_e4m3_spec_table_values():
    for code, val in _golden_e4m3():
        got = O.e4m3fn_value(code)
        if math.isnan(val):
            assert math.isnan(got)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_e4m3_all_codes_match_torch_float8():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([O.e4m3fn_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(mine))
    assert np.array_equal(ref[~nan], mine[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(mine[~nan]))


@pytest.mark.parametrize("e", [0, -4, 3])
def test_e4m3_dequant_exact_in_bf16(e):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    bits = O.dequant_e4m3fn_to_bf16_bits(codes, e)
    back = O.bf16_bits_to_f64(bits)
    assert np.array_equal(back, np.array([O.e4m3fn_value(c) * 2.0 ** e for c in codes]))


def test_e4m3_nan_code_rejected():
    with pytest.raises(ValueError):
        O.dequant_e4m3fn(np.array([0x7F], dtype=np.uint8))


def test_generator_e4m3_quantiser_round_trips_and_matches_torch():
    # every finite code value quantises back to itself
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = np.array([O.e4m3fn_value(c) for c in codes])
    assert np.array_equal(I.f32_to_e4m3fn_bits(vals), codes)
    # random in-range values agree with torch's float8 rounding (nearest even)
    g = np.random.default_rng(3)
    x = (g.standard_normal(20000) * g.choice([1e-3, 0.1, 3.0, 60.0], 20000)).astype(np.float32)
    x = np.clip(x, -440, 440)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(I.f32_to_e4m3fn_bits(x), ref)
    # saturation
    assert I.f32_to_e4m3fn_bits(np.array([1e6, -1e6]))[0] == 0x7E
    assert I.f32_to_e4m3fn_bits(np.array([1e6, -1e6]))[1] == 0xFE


def test_bf16_helpers_match_torch():
    g = np.random.default_rng(4)
    x = (g.standard_normal(50000) * 10.0 ** g.integers(-6, 6, 50000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(I.f32_to_bf16_bits(x), ref)
    back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16_bits_to_f64(ref), back)


# ============================================================================ O2, O3

def test_tile_bounds_ragged_and_offset():
    assert O.tile_bounds(0, 10, 4) == [(0, 4), (4, 8), (8, 10)]
    assert O.tile_bounds(7, 8, 4) == [(7, 11), (11, 15)]
    assert O.tile_bounds(5, 1, 128) == [(5, 6)]
    assert O.tile_bounds(0, 0, 4) == []


def _bits(x):
    return I.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_pool_closed_forms():
    # constant tiles -> that constant; partial tile holding 1..m -> (m+1)/2; 1-token tile
    d = 3
    N = 11
    x = np.zeros((1, N, 1, d), dtype=np.float32)
    x[0, 0:4, 0, :] = 2.5
    x[0, 4:8, 0, :] = -7.0
    x[0, 8:11, 0, :] = np.array([1, 2, 3], dtype=np.float32)[:, None]   # partial tile 1..3
    pooled = O.pool_tiles(_bits(x), 0, 0, 0, N, 4)
    assert np.array_equal(pooled[0], [2.5] * d)
    assert np.array_equal(pooled[1], [-7.0] * d)
    assert np.array_equal(pooled[2], [2.0] * d)                          # (3+1)/2
    one = O.pool_tiles(_bits(x), 0, 0, 9, 1, 4)
    assert np.array_equal(one[0], [2.0] * d)
    # ragged partial tile with m = 5 inside an offset segment
    y = np.zeros((1, 20, 2, 2), dtype=np.float32)
    y[0, 3:8, 1, 0] = np.arange(1, 6)
    pooled = O.pool_tiles(_bits(y), 0, 1, 3, 5, 8)
    assert pooled.shape == (1, 2) and pooled[0, 0] == 3.0 and pooled[0, 1] == 0.0


def test_pool_brute_loop_random():
    g = np.random.default_rng(0)
    x = _bits(g.standard_normal((2, 23, 3, 5)))
    xf = O.bf16_bits_to_f64(x)
    for b in range(2):
        for h in range(3):
            got = O.pool_tiles(x, b, h, 2, 19, 6)
            for i, lo in enumerate(range(2, 21, 6)):
                hi = min(lo + 6, 21)
                for c in range(5):
                    s = Fraction(0)
                    for n in range(lo, hi):
                        s += Fraction(float(xf[b, n, h, c]))
                    assert abs(got[i, c] - float(s / (hi - lo))) <= 1e-15 * max(1.0, abs(float(s)))


# ============================================================================ O4, O5

def test_identity_projection_gives_plain_dot_product():
    g = np.random.default_rng(1)
    qbar = g.standard_normal((5, 6))
    kbar = g.standard_normal((7, 6))
    eye = np.eye(6)
    s = O.tile_scores(O.project(qbar, eye), O.project(kbar, eye))
    for i in range(5):
        for j in range(7):
            assert abs(s[i, j] - float(np.dot(qbar[i], kbar[j]))) < 1e-12


def test_rank_one_scores_closed_form():
    # q_bar_i = a_i u, k_bar_j = b_j v, Wq = e0 u^T, Wk = e0 v^T / |v|^2  =>  s_ij = a_i b_j |u|^2
    u = np.array([1.0, -2.0, 0.5, 3.0])
    v = np.array([0.25, 1.0, -1.0, 2.0])
    a = np.array([1.0, -3.0, 0.5])
    bb = np.array([2.0, 0.0, -1.5, 4.0])
    Wq = np.zeros((2, 4)); Wq[0] = u
    Wk = np.zeros((2, 4)); Wk[0] = v / (v @ v)
    s = O.tile_scores(O.project(np.outer(a, u), Wq), O.project(np.outer(bb, v), Wk))
    expect = np.outer(a, bb) * (u @ u)
    assert np.allclose(s, expect, rtol=0, atol=1e-12)
    # asymmetric shapes: a transposed operand would change the shape
    assert s.shape == (3, 4)


@pytest.mark.parametrize("p", [2, 5])
def test_projection_and_scores_exact_rationals(p):
    g = np.random.default_rng(2 + p)
    qbar = g.integers(-4, 5, (3, 5)).astype(np.float64)
    kbar = g.integers(-4, 5, (4, 5)).astype(np.float64)
    Wq = g.integers(-3, 4, (p, 5)).astype(np.float64)
    Wk = g.integers(-3, 4, (p, 5)).astype(np.float64)
    qh = O.project(qbar, Wq)
    s = O.tile_scores(qh, O.project(kbar, Wk))
    for i in range(3):
        for c in range(p):
            assert qh[i, c] == sum(int(Wq[c, t]) * int(qbar[i, t]) for t in range(5))
        for j in range(4):
            acc = 0
            for c in range(p):
                qv = sum(int(Wq[c, t]) * int(qbar[i, t]) for t in range(5))
                kv = sum(int(Wk[c, t]) * int(kbar[j, t]) for t in range(5))
                acc += qv * kv
            assert s[i, j] == acc


# ============================================================================ O6

def _brute_topk(row, k):
    """Exhaustive: among all k-subsets with the maximal score sum, the lexicographically
    smallest ascending index tuple (equal scores go to the lower index)."""
    T = len(row)
    k = min(k, T)
    best = None
    for comb in itertools.combinations(range(T), k):
        ssum = sum(Fraction(row[j]) for j in comb)
        key = (-ssum, comb)
        if best is None or key < best:
            best = key
    return np.array(best[1], dtype=np.int32)


def test_topk_brute_force_with_exact_ties():
    g = np.random.default_rng(5)
    for trial in range(300):
        T = int(g.integers(1, 11))
        k = int(g.integers(0, T + 2))
        row = g.integers(-3, 4, T).astype(np.float64)   # many exact ties
        if trial % 7 == 0:
            row[g.integers(0, T)] = -0.0
        got = O.topk_lowest_index(row, k)
        assert np.array_equal(got, _brute_topk(row, k)), (row, k, got)


def test_topk_special_cases():
    row = np.array([0.3, -1.0, 2.0, 2.0, 0.3, 5.0])
    assert np.array_equal(O.topk_lowest_index(row, 6), np.arange(6))
    assert np.array_equal(O.topk_lowest_index(row, 99), np.arange(6))      # budget > T clamps
    assert np.array_equal(O.topk_lowest_index(row, 1), [5])
    assert np.array_equal(O.topk_lowest_index(np.array([1.0, 4.0, 4.0]), 1), [1])  # argmax, lowest
    assert np.array_equal(O.topk_lowest_index(np.full(9, 0.5), 4), [0, 1, 2, 3])
    assert np.array_equal(O.topk_lowest_index(np.arange(10.0), 3), [7, 8, 9])
    assert O.topk_lowest_index(row, 0).size == 0
    # -0.0 and +0.0 tie: lower index wins
    assert np.array_equal(O.topk_lowest_index(np.array([-1.0, 0.0, -0.0]), 1), [1])
    assert np.array_equal(O.topk_lowest_index(np.array([-1.0, -0.0, 0.0]), 1), [1])


# ============================================================================ O2..O6 end to end

def _tiny_integer_layer(seed=7):
    """Integer-valued inputs with power-of-two tile counts so every fp64 value is exact."""
    g = np.random.default_rng(seed)
    B, N, H, d, p, tile = 2, 30, 2, 4, 3, 4
    q = _bits(g.integers(-2, 3, (B, N, H, d)))
    k = _bits(g.integers(-2, 3, (B, N, H, d)))
    wq = _bits(g.integers(-1, 2, (H, p, d)))
    wk = _bits(g.integers(-1, 2, (H, p, d)))
    query = (0, 10)                       # tiles 4, 4, 2
    segments = [(10, 6, 1), (0, 10, 2)]   # ragged: tiles 4,2 | 4,4,2
    return q, k, wq, wk, tile, query, segments


def test_select_end_to_end_brute():
    q, k, wq, wk, tile, query, segments = _tiny_integer_layer()
    idx, S, _, _ = O.select(q, k, wq, wk, tile, query, segments)
    qf, kf = O.bf16_bits_to_f64(q), O.bf16_bits_to_f64(k)
    Wq, Wk = O.bf16_bits_to_f64(wq), O.bf16_bits_to_f64(wk)
    B, N, H, d = q.shape
    p = Wq.shape[1]

    def pooled_proj(x, W, b, h, lo, hi):
        mean = [sum(Fraction(float(x[b, n, h, c])) for n in range(lo, hi)) / (hi - lo) for c in range(d)]
        return [sum(Fraction(float(W[h, r, c])) * mean[c] for c in range(d)) for r in range(p)]

    def tiles(st, ln):
        return [(st + i, st + min(i + tile, ln)) for i in range(0, ln, tile)]

    for b in range(B):
        for h in range(H):
            qt = [pooled_proj(qf, Wq, b, h, lo, hi) for lo, hi in tiles(*query)]
            col = 0
            kc = 0
            for (st, ln, bud) in segments:
                kt = [pooled_proj(kf, Wk, b, h, lo, hi) for lo, hi in tiles(st, ln)]
                for i, qv in enumerate(qt):
                    row = [sum(a * c for a, c in zip(qv, kv)) for kv in kt]
                    assert np.array_equal(S[b, h, i, col:col + len(kt)], [float(r) for r in row])
                    K = min(bud, len(kt))
                    assert np.array_equal(idx[b, h, i, kc:kc + K], _brute_topk(row, bud))
                col += len(kt)
                kc += min(bud, len(kt))


def test_select_fp8_weights_path():
    q, k, _, _, tile, query, segments = _tiny_integer_layer()
    g = np.random.default_rng(9)
    codes_q = g.integers(0, 0x7E, (2, 3, 4)).astype(np.uint8)
    codes_k = g.integers(0, 0x7E, (2, 3, 4)).astype(np.uint8)
    i8, S8, _, _ = O.select(q, k, (codes_q, -4), (codes_k, -4), tile, query, segments)
    wq_bits = O.dequant_e4m3fn_to_bf16_bits(codes_q, -4)
    wk_bits = O.dequant_e4m3fn_to_bf16_bits(codes_k, -4)
    ib, Sb, _, _ = O.select(q, k, wq_bits, wk_bits, tile, query, segments)
    assert np.array_equal(i8, ib) and np.array_equal(S8, Sb)


# ============================================================================ O7

def _sdpa_masked(qf, kf, vf, mask, scale):
    """torch SDPA (library) in float64 on the CPU with an explicit boolean mask."""
    qt = torch.from_numpy(qf)[None, None]
    kt = torch.from_numpy(kf)[None, None]
    vt = torch.from_numpy(vf)[None, None]
    m = torch.from_numpy(mask)[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return out[0, 0].numpy()


def _small_attn_layer(seed=11):
    g = np.random.default_rng(seed)
    B, H, d, tile = 1, 2, 8, 4
    query = (0, 14)                               # tiles 4,4,4,2
    segments = [(14, 7, 1), (0, 14, 2)]           # ref-like segment 4,3 ; video 4,4,4,2
    dense = [(21, 3), (26, 2)]                    # dense ranges, not tile aligned
    N = 30
    q = _bits(g.standard_normal((B, N, H, d)))
    k = _bits(g.standard_normal((B, N, H, d)))
    v = _bits(g.standard_normal((B, N, H, d)))
    return q, k, v, tile, query, segments, dense


def _brute_mask(idx_row, tile, segments, dense, N):
    """Boolean [N] mask by scanning every token and asking whether it is attended."""
    mask = np.zeros(N, dtype=bool)
    for n in range(N):
        kc = 0
        for (st, ln, bud) in segments:
            T = -(-ln // tile)
            K = min(bud, T)
            blk = [int(j) for j in idx_row[kc:kc + K]]
            if -1 in blk:                             # padding ends the segment's block
                blk = blk[:blk.index(-1)]
            if st <= n < st + ln and (n - st) // tile in set(blk):
                mask[n] = True
            kc += K
        for (st, ln) in dense:
            if st <= n < st + ln:
                mask[n] = True
    return mask


def test_attention_matches_masked_sdpa():
    q, k, v, tile, query, segments, dense = _small_attn_layer()
    B, N, H, d = q.shape
    Tq = 4
    g = np.random.default_rng(12)
    idx = np.zeros((B, H, Tq, 3), dtype=np.int32)
    for h in range(H):
        for i in range(Tq):
            idx[0, h, i, 0] = g.integers(0, 2)
            idx[0, h, i, 1:] = np.sort(g.choice(4, 2, replace=False))
    res = O.attend(q, k, v, idx, tile, query, segments, dense)
    qf, kf, vf = (O.bf16_bits_to_f64(x) for x in (q, k, v))
    scale = 1 / math.sqrt(d)
    for (b, h, i), (out, lse) in res.items():
        q0, q1 = i * tile, min((i + 1) * tile, query[1])
        mask = _brute_mask(idx[b, h, i], tile, segments, dense, N)
        ref = _sdpa_masked(qf[b, q0:q1, h], kf[b, :, h], vf[b, :, h],
                           np.broadcast_to(mask, (q1 - q0, N)).copy(), scale)
        assert np.allclose(out, ref, rtol=0, atol=1e-13)
        logits = torch.from_numpy(qf[b, q0:q1, h] @ kf[b, :, h].T * scale)
        logits[:, ~torch.from_numpy(mask)] = -math.inf
        assert np.allclose(lse, torch.logsumexp(logits, dim=1).numpy(), rtol=0, atol=1e-12)


def test_full_budget_equals_dense_sdpa():
    q, k, v, tile, query, segments, dense = _small_attn_layer(13)
    full = [(st, ln, 10 ** 6) for (st, ln, _) in segments]
    Ks = [-(-ln // tile) for (_, ln, _) in segments]
    idx = np.concatenate([np.broadcast_to(np.arange(K, dtype=np.int32), (1, 2, 4, K)) for K in Ks], -1)
    res = O.attend(q, k, v, idx, tile, query, full, dense)
    qf, kf, vf = (O.bf16_bits_to_f64(x) for x in (q, k, v))
    keys = np.r_[0:28]      # every segment token and every dense token
    keys = keys[(keys < 24) | (keys >= 26)]
    for (b, h, i), (out, lse) in res.items():
        q0, q1 = i * tile, min((i + 1) * tile, query[1])
        qt = torch.from_numpy(qf[b, q0:q1, h])[None, None]
        kt = torch.from_numpy(kf[b, keys, h])[None, None]
        vt = torch.from_numpy(vf[b, keys, h])[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, 0].numpy()
        assert np.allclose(out, ref, rtol=0, atol=1e-13)


def test_attention_closed_forms():
    q, k, v, tile, query, segments, dense = _small_attn_layer(17)
    B, N, H, d = q.shape
    idx = np.zeros((1, H, 4, 3), dtype=np.int32)
    idx[..., 1] = 1
    idx[..., 2] = 3
    # q = 0  ->  uniform weights  ->  mean of the attended V rows
    qz = np.zeros_like(q)
    vf = O.bf16_bits_to_f64(v)
    res = O.attend(qz, k, v, idx, tile, query, segments, dense)
    for (b, h, i), (out, lse) in res.items():
        sel = list(range(14, 18)) + list(range(4, 8)) + list(range(12, 14)) + [21, 22, 23, 26, 27]
        assert np.allclose(out, vf[b, sel, h].mean(axis=0)[None, :], rtol=0, atol=1e-14)
        assert np.allclose(lse, math.log(len(sel)), atol=1e-14)
    # V = c  ->  c
    vc = _bits(np.full(v.shape, -1.25))
    res = O.attend(q, k, vc, idx, tile, query, segments, dense)
    for out, _ in res.values():
        assert np.allclose(out, -1.25, rtol=0, atol=1e-14)
    # a single attended key  ->  its value row
    one_seg_single = [(13, 1, 1)]                           # a one-token segment
    idx1 = np.zeros((1, H, 4, 1), dtype=np.int32)
    res = O.attend(q, k, v, idx1, tile, query, one_seg_single, [])
    for (b, h, i), (out, lse) in res.items():
        assert np.array_equal(out, np.broadcast_to(vf[b, 13, h], out.shape))


def test_attention_rejects_bad_index_and_empty():
    q, k, v, tile, query, segments, dense = _small_attn_layer()
    bad = np.full((1, 2, 4, 3), 7, dtype=np.int32)
    with pytest.raises(ValueError):
        O.attend(q, k, v, bad, tile, query, segments, dense, pairs=[(0, 0, 0)])
    none = np.zeros((1, 2, 4, 0), dtype=np.int32)
    with pytest.raises(ValueError):
        O.attend(q, k, v, none, tile, query, [(14, 7, 0)], [], pairs=[(0, 0, 0)])


# ============================================================================ planted mistakes

def _pins_fail(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_planted_mistakes_are_caught(monkeypatch):
    """A plausible slip in any oracle step makes at least one pin above fail."""
    planted = {
        # pooling divides by the tile size instead of the number of real tokens
        "pool_tiles": (lambda x, b, h, st, ln, t: np.array(
            [O.bf16_bits_to_f64(x[b, lo:hi, h, :]).sum(0) / t for lo, hi in O.tile_bounds(st, ln, t)]),
            [test_pool_closed_forms]),
        # projection without transposing W
        "project": (lambda pooled, w: pooled @ w,
                    [lambda: test_projection_and_scores_exact_rationals(5)]),
        # scores with a swapped operand order
        "tile_scores": (lambda a, b: -(a @ b.T), [test_rank_one_scores_closed_form]),
        # ties broken toward the higher index
        "topk_lowest_index": (lambda row, k: np.sort(
            (len(row) - 1 - np.argsort(-row[::-1], kind="stable"))[:min(k, len(row))]).astype(np.int32),
            [test_topk_brute_force_with_exact_ties]),
        # the dense key ranges are dropped
        "attended_tokens": (lambda idx_row, tile, segs, dense, _f=O.attended_tokens: _f(idx_row, tile, segs, []),
                            [test_attention_matches_masked_sdpa]),
    }
    for name, (bad, pins) in planted.items():
        with monkeypatch.context() as m:
            m.setattr(O, name, bad)
            assert any(_pins_fail(p) for p in pins), f"planted mistake in {name} not caught"


def test_padding_entries_select_nothing():
    """-1 entries are padding: the same result as leaving the entry out (brute-force mask)."""
    q, k, v, tile, query, segments, dense = _small_attn_layer(19)
    B, N, H, d = q.shape
    idx = np.zeros((1, H, 4, 3), dtype=np.int32)
    idx[..., 0] = 1
    idx[..., 1] = 0
    idx[..., 2] = -1                                  # video segment: one tile + padding
    res = O.attend(q, k, v, idx, tile, query, segments, dense)
    qf, kf, vf = (O.bf16_bits_to_f64(x) for x in (q, k, v))
    for (b, h, i), (out, _) in res.items():
        q0, q1 = i * tile, min((i + 1) * tile, query[1])
        mask = np.zeros(N, bool)
        mask[14 + 4:14 + 7] = True                    # ref segment tile 1 (tokens 18..20)
        mask[0:4] = True                              # video tile 0
        for (st, ln) in dense:
            mask[st:st + ln] = True
        ref = _sdpa_masked(qf[b, q0:q1, h], kf[b, :, h], vf[b, :, h],
                           np.broadcast_to(mask, (q1 - q0, N)).copy(), 1 / math.sqrt(d))
        assert np.allclose(out, ref, rtol=0, atol=1e-13)


def test_padding_ends_the_segment_block():
    """An entry after a -1 in the same segment's block is ignored; the next segment's
    block is read as usual (hand-written masks)."""
    q, k, v, tile, query, segments, dense = _small_attn_layer(21)
    segments = [(0, 14, 3), (14, 7, 2)]               # video first, three entries
    B, N, H, d = q.shape
    idx = np.zeros((1, H, 4, 5), dtype=np.int32)
    idx[..., :3] = [1, -1, 2]                         # video tile 1, then padding; tile 2 unused
    idx[..., 3:] = [-1, 0]                            # reference: padding first, tile 0 unused
    res = O.attend(q, k, v, idx, tile, query, segments, [])
    qf, kf, vf = (O.bf16_bits_to_f64(x) for x in (q, k, v))
    for (b, h, i), (out, _) in res.items():
        q0, q1 = i * tile, min((i + 1) * tile, query[1])
        ref = _sdpa_masked(qf[b, q0:q1, h], kf[b, 4:8, h], vf[b, 4:8, h],
                           np.ones((q1 - q0, 4), bool), 1 / math.sqrt(d))
        assert np.allclose(out, ref, rtol=0, atol=1e-13)


def test_dense_query_rows_match_sdpa():
    q, k, v, tile, query, segments, dense = _small_attn_layer(23)
    qf, kf, vf = (O.bf16_bits_to_f64(x) for x in (q, k, v))
    keys = np.r_[0:28]
    keys = keys[(keys < 24) | (keys >= 26)]          # every segment and dense token
    rows = (21, 3)                                    # e.g. the text tokens as queries
    for h in range(2):
        out, lse = O.attend_all_keys(q, k, v, 0, h, rows, segments, dense)
        qt = torch.from_numpy(qf[0, 21:24, h])[None, None]
        kt = torch.from_numpy(kf[0, keys, h])[None, None]
        vt = torch.from_numpy(vf[0, keys, h])[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, 0].numpy()
        assert np.allclose(out, ref, rtol=0, atol=1e-13)


def test_float16_weights_are_exact():
    """IEEE float16 predictor weights enter the oracle as their exact values."""
    w = np.array([65504.0, -2.0 ** -24, 2.0 ** -14, 1 + 2.0 ** -10, -0.0, 0.333], dtype=np.float16)
    got = O.weights_f64(w)
    assert got.dtype == np.float64
    assert got[:5].tolist() == [65504.0, -2.0 ** -24, 2.0 ** -14, 1 + 2.0 ** -10, 0.0]
    assert math.copysign(1.0, got[4]) == -1.0
    assert got[5] == 0.333 + (float(np.float16(0.333)) - 0.333)     # the float16 value itself
    assert got[5] != 0.333
