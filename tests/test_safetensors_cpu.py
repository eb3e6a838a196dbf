"""The native safetensors reader (host only): round trips of files written by the
safetensors library itself, hand-built malformed files, and the selector-file rules
(Affine launch article, "How the SN120 Competition Works": 100 float16 tensors of shape
(56, 384, 128), at most 560 million bytes)."""
import json
import os
import struct

import numpy as np
import pytest
import torch
from safetensors.numpy import save_file as save_np
from safetensors.torch import save_file as save_torch

from block_sparse_attention_predictor_amd import binding as Bnd

pytestmark = pytest.mark.skipif(not os.path.exists(Bnd.lib_path),
                                reason="libveda.so not built (run __graft_entry__.build())")


def _status(path):
    try:
        Bnd.SafetensorsFile(path).close()
        return 0
    except Bnd.VedaError as e:
        return e.status


def test_round_trip_numpy_dtypes(tmp_path):
    g = np.random.default_rng(1)
    tensors = {
        "f16": g.standard_normal((3, 5)).astype(np.float16),
        "f32": g.standard_normal((2, 2, 2)).astype(np.float32),
        "f64": g.standard_normal((7,)),
        "i8": g.integers(-128, 127, (4, 4), dtype=np.int8),
        "u8": g.integers(0, 255, (9,), dtype=np.uint8),
        "i16": g.integers(-3000, 3000, (5,), dtype=np.int16),
        "u16": g.integers(0, 60000, (5,), dtype=np.uint16),
        "i32": g.integers(-2**31, 2**31 - 1, (3,), dtype=np.int32),
        "u32": g.integers(0, 2**32 - 1, (3,), dtype=np.uint32),
        "i64": g.integers(-2**62, 2**62, (2,), dtype=np.int64),
        "u64": g.integers(0, 2**62, (2,), dtype=np.uint64),
        "bool": g.integers(0, 2, (6,)).astype(bool),
        "scalar": np.array(2.5, dtype=np.float32),
        "empty": np.zeros((0, 4), dtype=np.float16),
        "layer.3.q_proj é\"\\": np.ones((2, 3), dtype=np.float16),
    }
    p = str(tmp_path / "all.safetensors")
    save_np(tensors, p, metadata={"hotkey": "5Gabc", "quote": "a\"b\\cü"})
    with Bnd.SafetensorsFile(p) as f:
        assert sorted(f.names()) == sorted(tensors)
        for name, arr in tensors.items():
            got = f.read(name)
            assert got.dtype == arr.dtype and got.shape == arr.shape
            assert np.array_equal(got, arr)
        assert f.metadata() == {"hotkey": "5Gabc", "quote": "a\"b\\cü"}
        with pytest.raises(KeyError):
            f.read("missing")


def test_round_trip_torch_bf16_and_fp8(tmp_path):
    g = torch.Generator().manual_seed(2)
    w = torch.randn(3, 32, 64, generator=g)
    tensors = {"wq": w.to(torch.bfloat16), "wk8": w.to(torch.float8_e4m3fn),
               "wk5": w.to(torch.float8_e5m2), "h": w.to(torch.float16)}
    p = str(tmp_path / "t.safetensors")
    save_torch(tensors, p)
    with Bnd.SafetensorsFile(p) as f:
        info = {f.info(i)[0]: f.info(i)[1:] for i in range(len(f))}
        assert info["wq"][:2] == ("BF16", (3, 32, 64)) and info["wk8"][:2] == ("F8_E4M3", (3, 32, 64))
        assert info["wk5"][0] == "F8_E5M2" and info["h"][0] == "F16"
        assert np.array_equal(f.read("wq"), tensors["wq"].view(torch.int16).numpy().view(np.uint16))
        assert np.array_equal(f.read("wk8"), tensors["wk8"].view(torch.uint8).numpy())
        assert np.array_equal(f.read("h"), tensors["h"].numpy())


def _write(path, header, data=b"", raw_len=None):
    hdr = header if isinstance(header, bytes) else json.dumps(header).encode()
    n = len(hdr) if raw_len is None else raw_len
    with open(path, "wb") as fh:
        fh.write(struct.pack("<Q", n) + hdr + data)
    return str(path)


def test_hand_built_valid_file(tmp_path):
    hdr = {"a": {"dtype": "U8", "shape": [2], "data_offsets": [0, 2]},
           "__metadata__": {"k": "v"},
           "b": {"shape": [1, 1], "data_offsets": [2, 4], "dtype": "F16"}}
    raw = json.dumps(hdr).encode() + b"   "           # trailing spaces are allowed padding
    p = _write(tmp_path / "ok.safetensors", raw, b"\x01\x02\x00\x3c")
    with Bnd.SafetensorsFile(p) as f:
        assert f.names() == ["a", "b"]                 # file order is kept
        assert f.read("a").tolist() == [1, 2]
        assert f.read("b").tolist() == [[1.0]]
        assert f.metadata() == {"k": "v"}
    assert _status(_write(tmp_path / "empty.safetensors", {})) == 0


def test_malformed_files(tmp_path):
    t = {"dtype": "F32", "shape": [2], "data_offsets": [0, 8]}
    d8 = b"\0" * 8
    cases = {
        "short": None,                                                      # under 8 bytes
        "len_past_end": ({"x": t}, d8, 10 ** 6),
        "bad_json": (b'{"x": {"dtype": "F32", "shape": [2], "data_offsets": [0, 8]}', d8, None),
        "trailing": (b'{"x": {"dtype": "F32", "shape": [2], "data_offsets": [0, 8]}} x', d8, None),
        "leading_zero": (b'{"x": {"dtype": "F32", "shape": [02], "data_offsets": [0, 8]}}', d8, None),
        "negative": (b'{"x": {"dtype": "F32", "shape": [-2], "data_offsets": [0, 8]}}', d8, None),
        "float": (b'{"x": {"dtype": "F32", "shape": [2.0], "data_offsets": [0, 8]}}', d8, None),
        "unknown_dtype": ({"x": {**t, "dtype": "F12"}}, d8, None),
        "unknown_field": ({"x": {**t, "extra": 1}}, d8, None),
        "missing_field": ({"x": {"dtype": "F32", "shape": [2]}}, d8, None),
        "duplicate": (b'{"x": {"dtype": "U8", "shape": [1], "data_offsets": [0, 1]}, '
                      b'"x": {"dtype": "U8", "shape": [1], "data_offsets": [1, 2]}}', b"\0\0", None),
        "count_mismatch": ({"x": {**t, "shape": [3]}}, d8, None),
        "past_data": ({"x": {**t, "data_offsets": [4, 12]}}, d8, None),
        "reversed": ({"x": {**t, "data_offsets": [8, 0]}}, d8, None),
        "hole": ({"x": {"dtype": "U8", "shape": [2], "data_offsets": [0, 2]},
                  "y": {"dtype": "U8", "shape": [2], "data_offsets": [3, 5]}}, b"\0" * 5, None),
        "overlap": ({"x": {"dtype": "U8", "shape": [3], "data_offsets": [0, 3]},
                     "y": {"dtype": "U8", "shape": [2], "data_offsets": [2, 4]}}, b"\0" * 4, None),
        "extra_data": ({"x": t}, d8 + b"\0", None),
        "meta_not_string": ({"__metadata__": {"k": 1}, "x": t}, d8, None),
        "bad_escape": (b'{"x\\q": {"dtype": "F32", "shape": [2], "data_offsets": [0, 8]}}', d8, None),
        "lone_surrogate": (b'{"x\\udc00": {"dtype": "F32", "shape": [2], "data_offsets": [0, 8]}}',
                           d8, None),
        "not_object": (b'["x"]', b"", None),
        # U+0000 cannot come back through a C string
        "nul_in_name": ({"x\u0000y": t}, d8, None),
        "nul_in_metadata": ({"__metadata__": {"k": "a\u0000"}, "x": t}, d8, None),
    }
    for name, spec in cases.items():
        path = tmp_path / f"{name}.safetensors"
        if spec is None:
            path.write_bytes(b"\x01\x02\x03")
            p = str(path)
        else:
            hdr, data, n = spec
            p = _write(path, hdr, data, n)
        assert _status(p) == -8, name
    assert _status(str(tmp_path / "does_not_exist.safetensors")) == -7


def test_selector_rules(tmp_path):
    """Scaled-down selector files (3 layers of (4, 32, 64)); the real rule is 50 layers of
    (56, 384, 128) float16, 100 x 56 x 384 x 128 x 2 = 550 502 400 bytes <= 560 000 000."""
    assert 100 * 56 * 384 * 128 * 2 == 550_502_400 <= 560_000_000
    g = np.random.default_rng(3)
    good = {f"layers.{i}.{w}": g.standard_normal((4, 32, 64)).astype(np.float16)
            for i in range(3) for w in ("q", "k")}
    p = str(tmp_path / "sel.safetensors")
    save_np(good, p, metadata={"hotkey": "5F"})
    names = Bnd.check_selector_file(p, n_layers=3, shape=(4, 32, 64))
    assert sorted(names) == sorted(good)
    with pytest.raises(ValueError):
        Bnd.check_selector_file(p, n_layers=3, shape=(4, 32, 64), max_bytes=os.path.getsize(p) - 1)
    with pytest.raises(ValueError):
        Bnd.check_selector_file(p, n_layers=4, shape=(4, 32, 64))
    with pytest.raises(ValueError):
        Bnd.check_selector_file(p, n_layers=3, shape=(4, 32, 32))
    bad = dict(good)
    bad["layers.0.q"] = good["layers.0.q"].astype(np.float32)
    p2 = str(tmp_path / "sel32.safetensors")
    save_np(bad, p2)
    with pytest.raises(ValueError):
        Bnd.check_selector_file(p2, n_layers=3, shape=(4, 32, 64))
