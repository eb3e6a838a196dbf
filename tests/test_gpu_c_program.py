"""The path driven from plain C: tests/c/run_layer.c (C99, HIP runtime API for device
memory, no PyTorch) runs veda_select and veda_sparse_attn on a layer read from a file; its
indices must pass the selection criterion against the oracle and its output the attention
bar against the oracle's attention over those indices.  Layers: the 64-row tiny workload
(paired kernel) and a 128-row layer with reference, text and audio ranges (two-group
kernel)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from block_sparse_attention_predictor_amd import binding as Bnd
from block_sparse_attention_predictor_amd import inputs as I
from oracle import veda_oracle as O
from gpu_util import check_attn, check_indices

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

pytestmark = pytest.mark.gpu


def _build(tmp_path):
    if shutil.which("gcc") is None:
        pytest.fail("gcc is needed to build the C driver")
    lib_dir = os.path.dirname(Bnd.lib_path)
    exe = str(tmp_path / "run_layer")
    r = subprocess.run(
        ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
         "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(ROCM, "include"),
         os.path.join(ROOT, "tests", "c", "run_layer.c"),
         "-L", lib_dir, "-lveda", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
         f"-Wl,-rpath,{lib_dir}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe],
        capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.parametrize("name", ["tiny", "t128"])
def test_c_program_select_and_attend(tmp_path, name):
    if name == "tiny":
        wl = I.WORKLOADS["tiny"]
    else:
        wl = I.custom_workload("c_t128", H=3, d=128, p=32, tile=128, grid=(4, 16, 16), ref=True, text=40,
                               audio=70, budgets={"video": 3, "ref": 1}, index=71)
    q, k, v = I.make_qkv(wl)
    w = I.make_weights(wl)
    assert not w.fp8
    L = Bnd.layer_from_workload(wl)
    segs = [(s.start, s.length, s.budget) for s in wl.segments]
    dense = [(r.start, r.length) for r in wl.dense]
    src = tmp_path / "in.bin"
    with open(src, "wb") as f:
        f.write(bytes(L))
        f.write(np.array([len(dense)], np.int32).tobytes())
        for st, ln in dense:
            f.write(np.array([st, ln], np.int64).tobytes())
        for x in (q, k, v, w.wq, w.wk):
            f.write(np.ascontiguousarray(x, dtype=np.uint16).tobytes())
    exe = _build(tmp_path)
    dst = tmp_path / "out.bin"
    print(f"[c driver] {name}", flush=True)
    r = subprocess.run([exe, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    raw = np.fromfile(dst, dtype=np.uint8)
    Tq = wl.n_query_tiles
    n_idx = wl.B * wl.H * Tq * wl.k_total
    idx = raw[:4 * n_idx].view(np.int32).reshape(wl.B, wl.H, Tq, wl.k_total)
    out_bits = raw[4 * n_idx:].view(np.uint16).reshape(q.shape)
    idx_ref, S_ref, _, _ = O.select(q, k, w.wq, w.wk, wl.tile, (wl.query.start, wl.query.length), segs)
    seg_T = [wl.seg_tiles(s) for s in wl.segments]
    seg_K = [min(s.budget, t) for s, t in zip(wl.segments, seg_T)]
    check_indices(idx, idx_ref, S_ref, seg_T, seg_K)
    res = O.attend(q, k, v, idx, wl.tile, (wl.query.start, wl.query.length), segs, dense)
    o = O.bf16_bits_to_f64(out_bits)
    for (b, h, i), (ref, _) in res.items():
        r0 = wl.query.start + i * wl.tile
        r1 = min(r0 + wl.tile, wl.query.start + wl.query.length)
        check_attn(o[b, r0:r1, h], ref)
    # rows outside the query segment stay as the program cleared them
    assert np.all(out_bits[:, wl.query.start + wl.query.length:] == 0)
