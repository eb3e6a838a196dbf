"""The C-ABI library without a GPU: it loads, exports every declared symbol, and
its host-side validation returns the documented codes before any device call."""
import ctypes
import os
import re
import subprocess

import pytest

from block_sparse_attention_predictor_amd import binding as Bnd
from block_sparse_attention_predictor_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "veda.h")

pytestmark = pytest.mark.skipif(not os.path.exists(Bnd.lib_path),
                                reason="libveda.so not built (run __graft_entry__.build())")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(veda_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_are_exported():
    names = declared_functions()
    assert len(names) >= 10
    lib = ctypes.CDLL(Bnd.lib_path)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", Bnd.lib_path], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\sT\s(veda_\w+)", out))
    assert set(names) <= exported
    assert set(Bnd.exported_symbols()) == set(names)


def test_version_and_status_strings():
    assert Bnd.abi_version() == 6 == Bnd.ABI_VERSION
    for code in range(-8, 1):
        assert Bnd.status_string(code) and "unknown" not in Bnd.status_string(code)
    assert "unknown" in Bnd.status_string(-99)


def _layer(**kw):
    wl = I.WORKLOADS["r2va"]
    L = Bnd.layer_from_workload(wl)
    for k, v in kw.items():
        setattr(L, k, v)
    return L


def check(L, for_select=True):
    return Bnd._load().veda_layer_check(ctypes.byref(L), 1 if for_select else 0)


def test_valid_layers_pass_and_workspace_size():
    for name in I.WORKLOAD_ORDER:
        wl = I.WORKLOADS[name]
        L = Bnd.layer_from_workload(wl)
        assert check(L) == 0
        assert L.Ktot == wl.k_total and L.Tk == wl.t_total
        assert Bnd._load().veda_k_total(ctypes.byref(L)) == wl.k_total
        ws = Bnd.select_workspace_bytes(L)
        need = 4 * wl.H * wl.p * (wl.n_query_tiles + wl.t_total)
        assert need <= ws <= need + 512


@pytest.mark.parametrize("field,value,code", [
    ("d", 96, -2), ("d", 256, -2), ("tile", 32, -2), ("p", 24, -2), ("p", 0, -2), ("p", 512, -2),
    ("B", 0, -1), ("H", 0, -1), ("n_tokens", 0, -1), ("n_seg", 5, -2), ("n_seg", 0, -1),
    ("stride_n", 0, -1), ("stride_h", 4, -1), ("stride_n", 5124, -1), ("stride_n", 1 << 24, -2),
    ("p", 400, -2), ("p", 384, 0), ("wdtype", 2, -2), ("wdtype", 1, 0), ("reserved", 1, -1),
])
def test_layer_errors(field, value, code):
    assert check(_layer(**{field: value})) == code


def test_range_errors():
    L = _layer()
    L.query.start = L.n_tokens - 10              # query runs past the sequence
    assert check(L) == -4
    L = _layer()
    L.seg[0].start = 129000                      # reference overlaps the video segment
    assert check(L) == -4
    L = _layer()
    L.budget[1] = -1
    assert check(L) == -1
    L = _layer()
    L.seg[1].len = 0
    assert check(L) == -1
    # selection-only limits do not apply to attention
    L = _layer(p=0)
    assert check(L, for_select=False) == 0


def _one_segment(n_q, n_k, tile=64, B=1, H=1):
    n = max(n_q, n_k) + 64
    return Bnd.make_layer(B=B, H=H, d=64, p=16, tile=tile, n_tokens=n, query=(0, n_q),
                          segments=[(0, n_k, 1)], strides=(0, H * 64, 64))


def test_size_limits():
    """Counts the kernels hold in 32 bits and the 2^40 index volume, each at its boundary;
    sizes near INT64_MAX are rejected, not overflowed."""
    big = (1 << 63) - 1
    # query tiles: 2^31 - 1 is accepted, 2^31 is not
    assert check(_one_segment((2**31 - 1) * 64, 64), for_select=False) == 0
    assert check(_one_segment(2**31 * 64, 64), for_select=False) == -2
    # B * H
    assert check(_one_segment(64, 64, B=2**16, H=2**15 - 1), for_select=False) == 0
    assert check(_one_segment(64, 64, B=2**16, H=2**15), for_select=False) == -2
    # B * H * Tq * sum T_s: 2^40 exactly, then one key tile more
    assert check(_one_segment(2**26, 2**26), for_select=False) == 0
    assert check(_one_segment(2**26, 2**26 + 1), for_select=False) == -2
    # lengths near INT64_MAX
    L = Bnd.make_layer(B=1, H=1, d=64, p=16, tile=128, n_tokens=big, query=(0, big),
                       segments=[(0, big, 4)], strides=(0, 64, 64))
    assert check(L) == -2 and check(L, for_select=False) == -2
    assert Bnd.select_workspace_bytes(L) == 0
    lib = Bnd._load()
    assert lib.veda_k_total(ctypes.byref(L)) == 4
    L.seg[0].len = -1
    assert lib.veda_k_total(ctypes.byref(L)) == -1


def test_entry_points_reject_before_device_calls():
    lib = Bnd._load()
    L = _layer()
    fake = ctypes.c_void_p(0x10000)               # never dereferenced: validation fails first
    # null pointers
    assert lib.veda_select(ctypes.byref(L), None, fake, fake, fake, fake, None, fake, 1 << 40, None) == -1
    assert lib.veda_pool_project(ctypes.byref(L), fake, None, fake, fake, fake, fake, None) == -1
    assert lib.veda_score_topk(ctypes.byref(L), fake, fake, None, None, None) == -1
    # misaligned pointer
    odd = ctypes.c_void_p(0x10008)
    assert lib.veda_pool_project(ctypes.byref(L), odd, fake, fake, fake, fake, fake, None) == -1
    # workspace too small
    need = Bnd.select_workspace_bytes(L)
    assert lib.veda_select(ctypes.byref(L), fake, fake, fake, fake, fake, None, fake, need - 1, None) == -3
    # misaligned workspace
    assert lib.veda_select(ctypes.byref(L), fake, fake, fake, fake, fake, None, odd, need, None) == -1
    # attention: dense range overlapping a key segment, dense ranges overlapping each other
    arr, n = Bnd.dense_ranges([(133000, 100)])
    assert lib.veda_sparse_attn(ctypes.byref(L), fake, fake, fake, fake, None, arr, n, 0.0, fake, None, None) == -4
    arr, n = Bnd.dense_ranges([(133100, 100), (133150, 10)])
    assert lib.veda_sparse_attn(ctypes.byref(L), fake, fake, fake, fake, None, arr, n, 0.0, fake, None, None) == -4
    arr, n = Bnd.dense_ranges([(134800, 100)])  # past the end
    assert lib.veda_sparse_attn(ctypes.byref(L), fake, fake, fake, fake, None, arr, n, 0.0, fake, None, None) == -4
    # too many dense ranges
    arr, n = Bnd.dense_ranges([(133056 + i, 1) for i in range(9)])
    assert lib.veda_sparse_attn(ctypes.byref(L), fake, fake, fake, fake, None, arr, n, 0.0, fake, None, None) == -2
    # no keys at all: every budget zero and no dense range
    L0 = _layer()
    L0.budget[0] = 0
    L0.budget[1] = 0
    arr, n = Bnd.dense_ranges([])
    assert lib.veda_sparse_attn(ctypes.byref(L0), fake, fake, fake, None, None, arr, 0, 0.0, fake, None, None) == -5
    # negative or non-finite scale
    arr, n = Bnd.dense_ranges([])
    assert lib.veda_sparse_attn(ctypes.byref(L), fake, fake, fake, fake, None, arr, 0, -1.0, fake, None, None) == -1
    assert lib.veda_sparse_attn(ctypes.byref(L), fake, fake, fake, fake, None, arr, 0, float("nan"), fake, None, None) == -1
    # dequant argument checks
    assert lib.veda_dequant_fp8_e4m3(fake, fake, -1, 0, None) == -1
    assert lib.veda_dequant_fp8_e4m3(None, fake, 8, 0, None) == -1
    assert lib.veda_dequant_fp8_e4m3(fake, ctypes.c_void_p(0x10001), 8, 0, None) == -1
    assert lib.veda_dequant_fp8_e4m3(fake, fake, 8, 30, None) == -2
    assert lib.veda_dequant_fp8_e4m3(fake, fake, 0, 0, None) == 0      # empty: nothing to do


def test_empty_query_segment_is_a_no_op():
    lib = Bnd._load()
    L = _layer()
    L.query.len = 0
    fake = ctypes.c_void_p(0x10000)
    arr, n = Bnd.dense_ranges([])
    assert lib.veda_sparse_attn(ctypes.byref(L), fake, fake, fake, fake, None, arr, 0, 0.0, fake, None, None) == 0
    assert lib.veda_score_topk(ctypes.byref(L), fake, fake, fake, None, None) == 0


def test_layer_attn_and_attention_checks_before_device_calls():
    lib = Bnd._load()
    L = _layer()
    fake = ctypes.c_void_p(0x10000)
    need = Bnd.select_workspace_bytes(L)
    dense, nd = Bnd.dense_ranges([(133056, 512), (133568, 256), (133824, 1024)])
    # a dense query range overlapping the sparse query segment
    dq, nq = Bnd.dense_ranges([(128000, 2000)])
    assert lib.veda_layer_attn(ctypes.byref(L), fake, fake, fake, fake, fake, dense, nd, dq, nq, 0.0,
                               fake, fake, fake, need, None) == -4
    # dense query ranges overlapping each other
    dq, nq = Bnd.dense_ranges([(133056, 512), (133100, 10)])
    assert lib.veda_layer_attn(ctypes.byref(L), fake, fake, fake, fake, fake, dense, nd, dq, nq, 0.0,
                               fake, fake, fake, need, None) == -4
    # too small a workspace, missing V
    dq, nq = Bnd.dense_ranges([(129024, 4032)])
    assert lib.veda_layer_attn(ctypes.byref(L), fake, fake, fake, fake, fake, dense, nd, dq, nq, 0.0,
                               fake, fake, fake, need - 1, None) == -3
    assert lib.veda_layer_attn(ctypes.byref(L), fake, fake, None, fake, fake, dense, nd, dq, nq, 0.0,
                               fake, fake, fake, need, None) == -1
    # attention without an index needs every budget to cover its segment
    assert lib.veda_sparse_attn_check(ctypes.byref(L), fake, fake, fake, None, None, dense, nd, 0.0, fake) == -1
    Lf = _layer()
    Lf.budget[0] = 32
    Lf.budget[1] = 1008
    assert lib.veda_sparse_attn_check(ctypes.byref(Lf), fake, fake, fake, None, None, dense, nd, 0.0, fake) == 0
    assert lib.veda_sparse_attn_check(ctypes.byref(L), fake, fake, fake, fake, None, dense, nd, 0.0, fake) == 0
    # a processing order needs an index and 4-byte alignment
    assert lib.veda_sparse_attn_check(ctypes.byref(Lf), fake, fake, fake, None, fake, dense, nd, 0.0, fake) == -1
    assert lib.veda_sparse_attn_check(ctypes.byref(L), fake, fake, fake, fake, ctypes.c_void_p(0x10002), dense, nd,
                                      0.0, fake) == -1
    assert lib.veda_sparse_attn_check(ctypes.byref(L), fake, fake, fake, fake, fake, dense, nd, 0.0, fake) == 0
    assert lib.veda_sparse_attn(ctypes.byref(Lf), fake, fake, fake, None, fake, dense, nd, 0.0, fake, None,
                                None) == -1
    # veda_tile_order: null or misaligned pointers, an invalid layer; an empty query segment is a no-op
    assert lib.veda_tile_order(ctypes.byref(L), None, fake, None) == -1
    assert lib.veda_tile_order(ctypes.byref(L), fake, None, None) == -1
    assert lib.veda_tile_order(ctypes.byref(L), ctypes.c_void_p(0x10008), fake, None) == -1
    assert lib.veda_tile_order(ctypes.byref(L), fake, ctypes.c_void_p(0x10001), None) == -1
    assert lib.veda_tile_order(None, fake, fake, None) < 0
    Le = _layer()
    Le.query.len = 0
    assert lib.veda_tile_order(ctypes.byref(Le), fake, fake, None) == 0


def _window_layer(L, tile=64, n_seg=1):
    segs = [(0, L, 1)] if n_seg == 1 else [(0, L, 1), (L, 64, 1)]
    return Bnd.make_layer(B=1, H=2, d=64, p=32, tile=tile, n_tokens=L + 64, query=(0, L),
                          segments=segs, strides=((L + 64) * 128, 128, 64))


@pytest.mark.parametrize("L,tile,ft,c,h,anchors", [
    (1000, 64, 70, 3, 1, True), (1000, 64, 70, 3, 1, False), (640, 64, 64, 1, 0, False),
    (640, 128, 64, 5, 1, True), (129024, 128, 4032, 5, 1, False), (350784, 128, 4032, 5, 1, True),
    (350784, 128, 4032, 5, 1, False), (100, 64, 7, 2, 0, True),
])
def test_window_width_matches_oracle(L, tile, ft, c, h, anchors):
    """The host half of the window producer: its longest row equals the oracle's."""
    from oracle import veda_oracle as O
    rows = O.window_tile_rows(L, tile, ft, c, h, anchors)
    assert Bnd.window_width(_window_layer(L, tile), ft, c, h, anchors) == max(len(r) for r in rows)


def test_window_errors_before_device_calls():
    lib = Bnd._load()
    fake = ctypes.c_void_p(0x10000)
    L = _window_layer(1000)
    with pytest.raises(Bnd.VedaError) as e:
        Bnd.window_width(_window_layer(1000, n_seg=2), 70)
    assert e.value.status == -2
    Lq = _window_layer(1000)
    Lq.query.len = 900                          # query differs from the key segment
    assert lib.veda_window_width(ctypes.byref(Lq), 70, 5, 1, 1) == -4
    for args in ((0, 5, 1, 1), (70, 0, 1, 1), (70, 5, -1, 1), (70, 5, 1, 2)):
        assert lib.veda_window_width(ctypes.byref(L), *args) == -1
    w = Bnd.window_width(L, 70, 5, 1, True)
    T = -(-1000 // 64)
    assert lib.veda_window_indices(ctypes.byref(L), 70, 5, 1, 1, fake, w - 1, None) == -1
    assert lib.veda_window_indices(ctypes.byref(L), 70, 5, 1, 1, fake, T + 1, None) == -1
    assert lib.veda_window_indices(ctypes.byref(L), 70, 5, 1, 1, None, w, None) == -1
    assert lib.veda_window_indices(ctypes.byref(L), 70, 5, 1, 1, ctypes.c_void_p(0x10004), w, None) == -1


def test_block_mass_and_recall_checks_before_device_calls():
    lib = Bnd._load()
    L = _layer()
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10004)
    dense, nd = Bnd.dense_ranges([(133056, 512), (133568, 256), (133824, 1024)])
    # budgets are ignored: the teacher attends to every tile (this layer's budgets are small)
    assert lib.veda_block_mass(ctypes.byref(L), None, fake, dense, nd, 0.0, fake, fake, None, None) == -1
    assert lib.veda_block_mass(ctypes.byref(L), fake, fake, dense, nd, 0.0, None, fake, None, None) == -1
    assert lib.veda_block_mass(ctypes.byref(L), fake, fake, dense, nd, 0.0, fake, None, None, None) == -1
    assert lib.veda_block_mass(ctypes.byref(L), fake, fake, dense, nd, 0.0, fake, fake, odd, None) == -1
    assert lib.veda_block_mass(ctypes.byref(L), fake, fake, dense, nd, -2.0, fake, fake, None, None) == -1
    bad, nb = Bnd.dense_ranges([(133000, 100)])      # overlaps the video segment
    assert lib.veda_block_mass(ctypes.byref(L), fake, fake, bad, nb, 0.0, fake, fake, None, None) == -4
    assert lib.veda_block_mass(None, fake, fake, dense, nd, 0.0, fake, fake, None, None) == -1
    Le = _layer()
    Le.query.len = 0                                 # no query rows: nothing to do
    assert lib.veda_block_mass(ctypes.byref(Le), fake, fake, dense, nd, 0.0, fake, fake, None, None) == 0
    assert lib.veda_block_recall(ctypes.byref(L), None, fake, fake, None) == -1
    assert lib.veda_block_recall(ctypes.byref(L), fake, odd, fake, None) == -1
    assert lib.veda_block_recall(ctypes.byref(_layer(d=96)), fake, fake, fake, None) == -2


def test_probe_library_is_separate_and_exports_its_header():
    """The MFMA-only measurement loop lives in libveda_probe.so (include/veda_probe.h), not in
    the method's library or header."""
    from block_sparse_attention_predictor_amd import probe
    names = declared_functions(os.path.join(ROOT, "include", "veda_probe.h"))
    assert names == sorted(probe.exported_symbols())
    out = subprocess.run(["nm", "-D", "--defined-only", probe.lib_path], capture_output=True, text=True).stdout
    assert set(names) <= set(re.findall(r"\sT\s(veda_\w+)", out))
    main = subprocess.run(["nm", "-D", "--defined-only", Bnd.lib_path], capture_output=True, text=True).stdout
    assert not any("probe" in n or "mfma_peak" in n for n in re.findall(r"\sT\s(veda_\w+)", main))
    assert not any("probe" in n or "mfma_peak" in n for n in declared_functions())
    lib = probe._load()
    fake = ctypes.c_void_p(0x10000)
    assert lib.veda_probe_mfma_peak(None, 10, 4, None) == -1
    assert lib.veda_probe_mfma_peak(fake, 0, 4, None) == -1
    assert lib.veda_probe_mfma_peak(fake, 10, 0, None) == -1


def test_package_entry_points_resolve():
    """The package's lazy attributes (build included) resolve without importing in a loop."""
    import block_sparse_attention_predictor_amd as pkg
    import __graft_entry__ as entry
    assert callable(pkg.build) and callable(entry.build) and callable(entry.smoke)
    assert pkg.VedaError is Bnd.VedaError


def test_fp8_entry_points_reject_before_device_calls():
    lib = Bnd._load()
    L = _layer()
    fake = ctypes.c_void_p(0x10000)
    dense, nd = Bnd.dense_ranges([(133056, 512), (133568, 256), (133824, 1024)])
    args = lambda qs, ks: (ctypes.byref(L), fake, fake, fake, qs, ks, fake, None, dense, nd, 0.0, fake, None, None)
    # missing or misaligned scales
    assert lib.veda_sparse_attn_fp8qk(*args(None, fake)) == -1
    assert lib.veda_sparse_attn_fp8qk(*args(fake, ctypes.c_void_p(0x10002))) == -1
    # one-byte rows need strides that are multiples of 16 elements
    L.stride_h = 136
    L.stride_n = 136 * 40
    L.stride_b = L.stride_n * L.n_tokens
    assert lib.veda_sparse_attn_fp8qk(*args(fake, fake)) == -1
    # 64-row tiles and block lists beyond the two-group kernel's table are not supported
    L = _layer(tile=64)
    assert lib.veda_sparse_attn_fp8qk(*args(fake, fake)) == -2
    wl = I.WORKLOADS["t2v14s"]
    Lb = Bnd.layer_from_workload(wl)
    Lb.budget[0] = 4096                          # every tile: 5482 + 40 blocks per query tile
    big, nb = Bnd.dense_ranges([(r.start, r.length) for r in wl.dense])
    assert lib.veda_sparse_attn_fp8qk(ctypes.byref(Lb), fake, fake, fake, fake, fake, fake, None, big, nb, 0.0, fake,
                                      None, None) == -2
    # quantiser: null pointers, misaligned codes or scale
    L = _layer()
    assert lib.veda_quantize_fp8_e4m3(ctypes.byref(L), None, fake, fake, None) == -1
    assert lib.veda_quantize_fp8_e4m3(ctypes.byref(L), fake, ctypes.c_void_p(0x10008), fake, None) == -1
    assert lib.veda_quantize_fp8_e4m3(ctypes.byref(L), fake, fake, ctypes.c_void_p(0x10001), None) == -1
    assert lib.veda_quantize_fp8_e4m3(ctypes.byref(_layer(d=96)), fake, fake, fake, None) == -2


def test_fp8_v_entry_points_reject_before_device_calls():
    """veda_sparse_attn_fp8 / veda_quantize_fp8_e4m3_vt / veda_fp8_vt_bytes: the blocked V size, and
    every rejection the host makes before a launch (scales, strides, tile size, starts off a
    multiple of 64 tokens, sizes the blocked layout cannot index)."""
    lib = Bnd._load()
    L = _layer()
    n_blocks = -(-L.n_tokens // 64)
    assert lib.veda_fp8_vt_bytes(ctypes.byref(L)) == L.B * L.H * n_blocks * L.d * 64
    assert lib.veda_fp8_vt_bytes(ctypes.byref(_layer(d=96))) == 0
    assert lib.veda_fp8_vt_bytes(None) == 0
    fake = ctypes.c_void_p(0x10000)
    dense, nd = Bnd.dense_ranges([(133056, 512), (133568, 256), (133824, 1024)])

    def call(layer, qs=fake, ks=fake, vs=fake, dn=dense, n=nd):
        return lib.veda_sparse_attn_fp8(ctypes.byref(layer), fake, fake, fake, qs, ks, vs, fake, None, dn, n, 0.0, fake,
                                        None, None)
    # missing or misaligned scales
    assert call(L, vs=None) == -1
    assert call(L, ks=ctypes.c_void_p(0x10002)) == -1
    # dense ranges and segments must start on a multiple of 64 tokens (the blocked V layout)
    off, no = Bnd.dense_ranges([(133056 + 32, 480), (133568, 256), (133824, 1024)])
    assert call(L, dn=off, n=no) == -2
    Ls = _layer()
    Ls.seg[1].start += 32
    Ls.seg[1].len -= 32
    assert call(Ls) == -2
    # 64-row tiles are not supported
    assert call(_layer(tile=64)) == -2
    # quantiser: null pointers, misaligned V, codes or scale
    assert lib.veda_quantize_fp8_e4m3_vt(ctypes.byref(L), None, fake, fake, None) == -1
    assert lib.veda_quantize_fp8_e4m3_vt(ctypes.byref(L), ctypes.c_void_p(0x10008), fake, fake, None) == -1
    assert lib.veda_quantize_fp8_e4m3_vt(ctypes.byref(L), fake, ctypes.c_void_p(0x10008), fake, None) == -1
    assert lib.veda_quantize_fp8_e4m3_vt(ctypes.byref(L), fake, fake, ctypes.c_void_p(0x10001), None) == -1
    assert lib.veda_quantize_fp8_e4m3_vt(ctypes.byref(_layer(d=96)), fake, fake, fake, None) == -2
