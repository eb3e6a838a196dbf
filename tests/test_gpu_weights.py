"""Selection with predictor weights as the predictor files hold them, through the native
file reader: float16 projections with the competition's predictor width p = 384, bf16 at
p = 384, and an FP8 (E4M3) predictor dequantised on the device, against the oracle."""
import math

import numpy as np
import pytest
import torch
from safetensors.numpy import save_file as save_np
from safetensors.torch import save_file as save_torch

from block_sparse_attention_predictor_amd import binding as Bnd
from block_sparse_attention_predictor_amd import inputs as I
from oracle import veda_oracle as O

from gpu_util import check_indices, check_scores, to_dev_bf16

pytestmark = pytest.mark.gpu


def _layer_inputs(seed, H, d, tile, n_video=900, n_ref=300):
    g = np.random.default_rng(seed)
    N = n_video + n_ref + 40
    field = 0.5 * np.sin(np.arange(N) / 23.0)[None, :, None, None] * g.standard_normal((1, 1, H, d))
    q = I.f32_to_bf16_bits((g.standard_normal((1, N, H, d)) + field).astype(np.float32))
    k = I.f32_to_bf16_bits((g.standard_normal((1, N, H, d)) + field).astype(np.float32))
    segments = [(n_video, n_ref, 3), (0, n_video, 4)]
    return g, N, q, k, segments


def _check(L, q, k, wq_dev, wk_dev, wq_ref, wk_ref, segments, n_video):
    idx, sc = Bnd.select(L, to_dev_bf16(q), to_dev_bf16(k), wq_dev, wk_dev, want_scores=True)
    torch.cuda.synchronize()
    idx_ref, S_ref, _, _ = O.select(q, k, wq_ref, wk_ref, L.tile, (0, n_video), segments)
    check_scores(sc.cpu().numpy().astype(np.float64), S_ref)
    seg_T = [-(-ln // L.tile) for (_, ln, _) in segments]
    seg_K = [min(b, T) for (_, _, b), T in zip(segments, seg_T)]
    check_indices(idx.cpu().numpy(), idx_ref, S_ref, seg_T, seg_K)


@pytest.mark.parametrize("d,tile,p", [(128, 128, 384), (64, 64, 48), (128, 64, 384)])
def test_float16_selector_file(tmp_path, d, tile, p):
    H = 3
    g, N, q, k, segments = _layer_inputs(11 + p, H, d, tile)
    wq = (g.standard_normal((H, p, d)) / math.sqrt(d)).astype(np.float16)
    wk = (g.standard_normal((H, p, d)) / math.sqrt(d)).astype(np.float16)
    path = str(tmp_path / "selector.safetensors")
    save_np({"blocks.0.attn.q": wq, "blocks.0.attn.k": wk}, path, metadata={"hotkey": "5F"})
    Bnd.check_selector_file(path, n_layers=1, shape=(H, p, d))
    with Bnd.SafetensorsFile(path) as f:
        wq_dev, wt = Bnd.predictor_weight(f, "blocks.0.attn.q")
        wk_dev, wt2 = Bnd.predictor_weight(f, "blocks.0.attn.k")
    assert wt == wt2 == 1 and wq_dev.dtype == torch.float16
    L = Bnd.make_layer(B=1, H=H, d=d, p=p, tile=tile, n_tokens=N, query=(0, 900), segments=segments,
                       strides=(N * H * d, H * d, d))
    L.wdtype = 1
    _check(L, q, k, wq_dev, wk_dev, wq, wk, segments, 900)


def test_bf16_p384():
    H, d, tile, p = 2, 128, 128, 384
    g, N, q, k, segments = _layer_inputs(5, H, d, tile)
    wq = I.f32_to_bf16_bits((g.standard_normal((H, p, d)) / math.sqrt(d)).astype(np.float32))
    wk = I.f32_to_bf16_bits((g.standard_normal((H, p, d)) / math.sqrt(d)).astype(np.float32))
    L = Bnd.make_layer(B=1, H=H, d=d, p=p, tile=tile, n_tokens=N, query=(0, 900), segments=segments,
                       strides=(N * H * d, H * d, d))
    _check(L, q, k, to_dev_bf16(wq), to_dev_bf16(wk), wq, wk, segments, 900)


def test_fp8_predictor_file(tmp_path):
    """An E4M3 predictor file: codes read natively, dequantised to bf16 on the device."""
    H, d, tile, p = 3, 128, 128, 64
    g, N, q, k, segments = _layer_inputs(9, H, d, tile)
    w = torch.from_numpy((g.standard_normal((2, H, p, d)) / math.sqrt(d) * 16).astype(np.float32))
    w8 = w.to(torch.float8_e4m3fn)
    path = str(tmp_path / "predictor_fp8.safetensors")
    save_torch({"q": w8[0].contiguous(), "k": w8[1].contiguous()}, path)
    with Bnd.SafetensorsFile(path) as f:
        wq_dev, t1 = Bnd.predictor_weight(f, "q", pow2_exp=-4)
        wk_dev, t2 = Bnd.predictor_weight(f, "k", pow2_exp=-4)
        codes_q, codes_k = f.read("q"), f.read("k")
    assert t1 == t2 == 0 and wq_dev.dtype == torch.bfloat16
    assert np.array_equal(codes_q, w8[0].view(torch.uint8).numpy())
    L = Bnd.make_layer(B=1, H=H, d=d, p=p, tile=tile, n_tokens=N, query=(0, 900), segments=segments,
                       strides=(N * H * d, H * d, d))
    _check(L, q, k, wq_dev, wk_dev, (codes_q, -4), (codes_k, -4), segments, 900)
