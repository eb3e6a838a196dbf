"""GPU parity of the online softmax on logit patterns chosen to exercise its running maximum:
the kernels take a block's weights against the running maximum as it stands and redo them
against the block's maximum only when a lane's weights sum above 2^8.  The patterns are
built from exact bf16 values: q = a * e0 and k_n = t_n * e0, so that logit_n = a * t_n /
sqrt(d) exactly.  Every key tile is attended (dense attention over the segment), at
128-row tiles (two-group kernel), 64-row tiles (paired kernel) and through the FP8 Q.K^T
kernel.

  ramp        logits rise steadily across the key blocks (the running maximum falls behind
              again and again, up to the 2^8 limit)
  late_spike  flat logits and one key 60 natural-log units above them in the last block
  flat        all logits equal (q = 0): weights 1 everywhere, no redo after the first block
  deep        all logits near -80 (exp without the maximum would underflow)
  falling     the largest logits in the first block, falling after it
  zigzag      alternating high and low blocks with a rising envelope

Oracle: oracle.veda_oracle.attend_rows (two-pass fp64 softmax).  Bar: max-abs <= 1e-2,
mean-abs <= 1e-3, lse within 2^-9.
"""
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_predictor_amd import binding as Bnd
from block_sparse_attention_predictor_amd import inputs as I
from oracle import veda_oracle as O
from gpu_util import bf16_to_f64, check_attn, to_dev_bf16

pytestmark = pytest.mark.gpu

D = 64
N_KEYS = 1280          # 20 blocks of 64 keys (40 of 32)


def _logit_targets(name, n):
    """Target logits (natural-log units) per key."""
    i = np.arange(n, dtype=np.float64)
    if name == "ramp":
        return -40.0 + 80.0 * i / (n - 1)
    if name == "late_spike":
        t = np.zeros(n)
        t[n - 7] = 60.0
        return t
    if name == "flat":
        return np.zeros(n)
    if name == "deep":
        return -80.0 + 0.01 * (i % 17)
    if name == "falling":
        return 30.0 - 60.0 * i / (n - 1)
    if name == "zigzag":
        blk = (i // 64).astype(int)
        return np.where(blk % 2 == 0, 2.0 * blk, -20.0)
    raise ValueError(name)


def _inputs(name, n_q, seed):
    g = np.random.default_rng(seed)
    scale = 1.0 / math.sqrt(D)
    a = 0.0 if name == "flat" else 8.0
    # k_n[0] = target / (a * scale), rounded to bf16; the other components carry small noise
    # in q = 0 directions, so they add nothing to the logits
    tgt = _logit_targets(name, N_KEYS)
    k = np.zeros((1, n_q + N_KEYS, 1, D), np.float32)
    q = np.zeros((1, n_q + N_KEYS, 1, D), np.float32)
    if a != 0.0:
        k[0, n_q:, 0, 0] = tgt / (a * scale)
    k[0, :, 0, 1:] = g.standard_normal((n_q + N_KEYS, D - 1))
    q[0, :n_q, 0, 0] = a
    v = g.standard_normal((1, n_q + N_KEYS, 1, D)).astype(np.float32)
    return tuple(I.f32_to_bf16_bits(x) for x in (q, k, v))


@pytest.mark.parametrize("tile", [128, 64])
@pytest.mark.parametrize("name", ["ramp", "late_spike", "flat", "deep", "falling", "zigzag"])
def test_softmax_running_maximum_patterns(name, tile):
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    n_q = 2 * tile
    q, k, v = _inputs(name, n_q, 5)
    N = n_q + N_KEYS
    segs = [(n_q, N_KEYS, 10 ** 6)]
    L = Bnd.make_layer(B=1, H=1, d=D, p=16, tile=tile, n_tokens=N, query=(0, n_q), segments=segs,
                       strides=(N * D, D, D))
    qd, kd, vd = (to_dev_bf16(x) for x in (q, k, v))
    out, lse = Bnd.sparse_attn(L, qd, kd, vd, None, [], want_lse=True)
    torch.cuda.synchronize()
    o = bf16_to_f64(out)
    lse = lse.cpu().numpy()
    qf, kf, vf = (O.bf16_bits_to_f64(x) for x in (q, k, v))
    ref, l_ref = O.attend_rows(qf[0, :n_q, 0], kf[0, n_q:, 0], vf[0, n_q:, 0], 1.0 / math.sqrt(D))
    check_attn(o[0, :n_q, 0], ref)
    assert np.abs(lse[0, 0] - l_ref).max() <= 2.0 ** -9


@pytest.mark.parametrize("name", ["ramp", "late_spike", "flat", "deep", "falling", "zigzag"])
def test_softmax_running_maximum_patterns_fp8(name):
    """The same patterns through the FP8 Q.K^T kernel (128-row tiles), against the oracle's
    attention over the decoded Q and K."""
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    tile = 128
    n_q = 2 * tile
    q, k, v = _inputs(name, n_q, 6)
    N = n_q + N_KEYS
    segs = [(n_q, N_KEYS, 10 ** 6)]
    L = Bnd.make_layer(B=1, H=1, d=D, p=16, tile=tile, n_tokens=N, query=(0, n_q), segments=segs,
                       strides=(N * D, D, D))
    qd, kd, vd = (to_dev_bf16(x) for x in (q, k, v))
    q8, qs = Bnd.quantize_fp8(L, qd)
    k8, ks = Bnd.quantize_fp8(L, kd)
    out, lse = Bnd.sparse_attn_fp8qk(L, q8, k8, vd, qs, ks, None, [], want_lse=True)
    torch.cuda.synchronize()
    q8r, eq = O.quantize_fp8(q)
    k8r, ek = O.quantize_fp8(k)
    assert np.array_equal(q8.cpu().numpy(), q8r) and np.array_equal(k8.cpu().numpy(), k8r)
    o = bf16_to_f64(out)
    lse = lse.cpu().numpy()
    qf, kf = O.dequant_e4m3fn(q8r, eq), O.dequant_e4m3fn(k8r, ek)
    vf = O.bf16_bits_to_f64(v)
    ref, l_ref = O.attend_rows(qf[0, :n_q, 0], kf[0, n_q:, 0], vf[0, n_q:, 0], 1.0 / math.sqrt(D))
    check_attn(o[0, :n_q, 0], ref)
    assert np.abs(lse[0, 0] - l_ref).max() <= 2.0 ** -9
