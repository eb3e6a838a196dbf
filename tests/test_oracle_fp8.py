"""Pins of the oracle's FP8 Q/K path (Q1 rounding, Q2 scale) against things other than
itself: the E4M3FN code table itself (every finite code is its own nearest value),
midpoints worked out by hand from the format (ties go to the even code), torch's
float8_e4m3fn conversion (a library routine), the closed form of the scale exponent at
powers of two, and a reduction of the FP8 attention to the bf16 attention already pinned
against torch SDPA (every E4M3 value times 2^e is a bf16 value).
"""
import math

import numpy as np
import pytest
import torch

from oracle import veda_oracle as O
from block_sparse_attention_predictor_amd import inputs as I

FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])


def test_every_finite_code_rounds_to_itself():
    vals = np.array([O.e4m3fn_value(int(c)) for c in FINITE])
    assert np.array_equal(O.e4m3fn_round(vals), FINITE.astype(np.uint8))


def test_midpoints_go_to_the_even_code_and_neighbours_to_the_nearest():
    # consecutive non-negative magnitudes: codes c and c + 1 (mantissa 7 -> next binade
    # included); their midpoint rounds to whichever code is even
    for c in range(0, 126):
        lo, hi = O.e4m3fn_value(c), O.e4m3fn_value(c + 1)
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert O.e4m3fn_round(mid) == even, (c, mid)
        assert O.e4m3fn_round(np.nextafter(mid, np.inf)) == c + 1
        assert O.e4m3fn_round(np.nextafter(mid, -np.inf)) == c
        assert O.e4m3fn_round(-mid) == (even | 0x80)
    # hand-worked cases: 1 + 1/16 lies halfway between 1 (0x38) and 1.125 (0x39)
    assert O.e4m3fn_round(1.0625) == 0x38
    assert O.e4m3fn_round(1.1875) == 0x3A          # between 1.125 (0x39) and 1.25 (0x3A)
    assert O.e4m3fn_round(2.0 ** -10) == 0x00      # half the smallest subnormal
    assert O.e4m3fn_round(1.5 * 2.0 ** -9) == 0x02  # between subnormals 1 and 2
    assert O.e4m3fn_round(7.5 * 2.0 ** -9) == 0x08  # between the largest subnormal and 2^-6


def test_saturation_sign_and_nan():
    assert O.e4m3fn_round(448.0) == 0x7E
    assert O.e4m3fn_round(464.0) == 0x7E
    assert O.e4m3fn_round(1e30) == 0x7E
    assert O.e4m3fn_round(-1e30) == 0xFE
    assert O.e4m3fn_round(0.0) == 0x00
    assert O.e4m3fn_round(-0.0) == 0x80
    assert O.e4m3fn_round(-1e-9) == 0x80
    assert O.e4m3fn_round(np.nan) == 0x7F


def test_rounding_matches_torch_float8_in_range():
    g = np.random.default_rng(3)
    # magnitudes over the whole normal and subnormal range, float32-representable
    x = (g.choice([-1.0, 1.0], 200000) * 2.0 ** g.uniform(-12, math.log2(448), 200000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3fn_round(x.astype(np.float64)), ref)


def test_scale_exponent_closed_form():
    assert O.fp8_scale_exponent(0.0) == 0
    for k in range(-140, 121, 7):
        edge = 448.0 * 2.0 ** k
        assert O.fp8_scale_exponent(edge) == k
        assert O.fp8_scale_exponent(np.nextafter(edge, np.inf)) == k + 1
        assert O.fp8_scale_exponent(np.nextafter(edge, -np.inf)) == k
    g = np.random.default_rng(4)
    for a in 2.0 ** g.uniform(-120, 120, 500):
        e = O.fp8_scale_exponent(a)
        assert a <= 448.0 * 2.0 ** e and a > 448.0 * 2.0 ** (e - 1)
        assert e == math.ceil(math.log2(a / 448.0)) or abs(math.log2(a / 448.0) - round(math.log2(a / 448.0))) < 1e-12


def test_quantize_bounds():
    g = np.random.default_rng(5)
    x = (g.standard_normal((2, 50, 3, 64)) * 3.0).astype(np.float32)
    bits = I.f32_to_bf16_bits(x)
    codes, e = O.quantize_fp8(bits)
    xv = O.bf16_bits_to_f64(bits)
    back = O.dequant_e4m3fn(codes, e)
    # the largest element lands in the top binade and no code saturates below it
    amax = np.abs(xv).max()
    assert 224.0 < amax * 2.0 ** -e <= 448.0
    # each value is within half a quantum: 2^-4 relative for normals, 2^-10 * 2^e absolute below
    err = np.abs(back - xv)
    bound = np.maximum(np.abs(xv) * 2.0 ** -4, 2.0 ** (e - 10))
    assert np.all(err <= bound)


def test_fp8_attention_equals_bf16_attention_on_the_decoded_values():
    g = np.random.default_rng(6)
    B, N, H, d, tile = 1, 200, 2, 64, 64
    q, k, v = (I.f32_to_bf16_bits(g.standard_normal((B, N, H, d)).astype(np.float32)) for _ in range(3))
    q8, eq = O.quantize_fp8(q)
    k8, ek = O.quantize_fp8(k)
    # the decoded values are exact in bf16, so the bf16 path (pinned against SDPA) gives
    # the reference for the same logits
    qb = O.f64_to_bf16_bits_rne(O.dequant_e4m3fn(q8, eq))
    kb = O.f64_to_bf16_bits_rne(O.dequant_e4m3fn(k8, ek))
    segs = [(0, 160, 2)]
    dense = [(160, 40)]
    query = (0, 160)
    idx = np.array([[[[0, 2], [1, 2], [0, 1]] for _ in range(H)]], dtype=np.int32)
    a = O.attend(q8, k8, v, idx, tile, query, segs, dense, dq=O.fp8_values(eq), dk=O.fp8_values(ek))
    b = O.attend(qb, kb, v, idx, tile, query, segs, dense)
    for key in a:
        assert np.array_equal(a[key][0], b[key][0]) and np.array_equal(a[key][1], b[key][1])


def test_fp8_v_attention_equals_bf16_attention_on_the_decoded_values():
    """V given as E4M3FN codes (per-tensor scale) through the dv decoder is the bf16
    attention (pinned against SDPA) on the decoded V, which is exact in bf16."""
    g = np.random.default_rng(8)
    B, N, H, d, tile = 1, 200, 2, 64, 64
    q, k, v = (I.f32_to_bf16_bits(3.0 * g.standard_normal((B, N, H, d)).astype(np.float32)) for _ in range(3))
    q8, eq = O.quantize_fp8(q)
    k8, ek = O.quantize_fp8(k)
    v8, ev = O.quantize_fp8(v)
    assert ev != 0 or np.abs(O.bf16_bits_to_f64(v)).max() <= 448
    qb, kb, vb = (O.f64_to_bf16_bits_rne(O.dequant_e4m3fn(c, e)) for c, e in ((q8, eq), (k8, ek), (v8, ev)))
    segs = [(0, 160, 2)]
    dense = [(160, 40)]
    query = (0, 160)
    idx = np.array([[[[0, 2], [1, 2], [0, 1]] for _ in range(H)]], dtype=np.int32)
    a = O.attend(q8, k8, v8, idx, tile, query, segs, dense, dq=O.fp8_values(eq), dk=O.fp8_values(ek),
                 dv=O.fp8_values(ev))
    b = O.attend(qb, kb, vb, idx, tile, query, segs, dense)
    for key in a:
        assert np.array_equal(a[key][0], b[key][0]) and np.array_equal(a[key][1], b[key][1])
    # and the decoded V differs from V by at most E4M3's half step (2^-4 relative, or
    # 2^-10 * 2^e absolute below the normal range)
    vv = O.bf16_bits_to_f64(v)
    dec = O.dequant_e4m3fn(v8, ev)
    assert np.all(np.abs(dec - vv) <= np.maximum(2.0 ** -4 * np.abs(vv), 2.0 ** (-10 + ev)) + 1e-300)
