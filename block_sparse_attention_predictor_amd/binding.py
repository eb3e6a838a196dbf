"""ctypes binding of libveda.so (declared in include/veda.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.  If
the library has not been built, every call raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG, "libveda.so")

MAX_SEGMENTS = 4
MAX_DENSE = 8

STATUS = {0: "VEDA_OK", -1: "VEDA_EINVAL", -2: "VEDA_EUNSUPPORTED", -3: "VEDA_EWORKSPACE",
          -4: "VEDA_ERANGE", -5: "VEDA_ENOKEYS", -6: "VEDA_EHIP", -7: "VEDA_EIO",
          -8: "VEDA_EFORMAT"}


class VedaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


class Range(ctypes.Structure):
    _fields_ = [("start", ctypes.c_int64), ("len", ctypes.c_int64)]


class Layer(ctypes.Structure):
    """Mirror of veda_layer."""
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("d", ctypes.c_int32),
        ("p", ctypes.c_int32), ("tile", ctypes.c_int32), ("n_seg", ctypes.c_int32),
        ("n_tokens", ctypes.c_int64),
        ("stride_b", ctypes.c_int64), ("stride_n", ctypes.c_int64), ("stride_h", ctypes.c_int64),
        ("query", Range),
        ("seg", Range * MAX_SEGMENTS),
        ("budget", ctypes.c_int32 * MAX_SEGMENTS),
        ("wdtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]

    @property
    def Tq(self) -> int:
        return -(-self.query.len // self.tile)

    @property
    def seg_tiles(self):
        return [-(-self.seg[s].len // self.tile) for s in range(self.n_seg)]

    @property
    def Tk(self) -> int:
        return sum(self.seg_tiles)

    @property
    def Ktot(self) -> int:
        return sum(min(self.budget[s], t) for s, t in enumerate(self.seg_tiles))


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise RuntimeError(f"{lib_path} is missing: build it with "
                           "`python -m block_sparse_attention_predictor_amd.build` (needs hipcc)")
    lib = ctypes.CDLL(lib_path)
    P = ctypes.c_void_p
    L = ctypes.POINTER(Layer)
    sig = {
        "veda_abi_version": (ctypes.c_int, []),
        "veda_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "veda_k_total": (ctypes.c_int64, [L]),
        "veda_layer_check": (ctypes.c_int, [L, ctypes.c_int]),
        "veda_select_workspace_bytes": (ctypes.c_size_t, [L]),
        "veda_pool_project": (ctypes.c_int, [L, P, P, P, P, P, P, P]),
        "veda_score_topk": (ctypes.c_int, [L, P, P, P, P, P]),
        "veda_select": (ctypes.c_int, [L, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "veda_select_noalloc": (ctypes.c_int, [L, P, P, P, P, P, P, P]),
        "veda_sparse_attn": (ctypes.c_int, [L, P, P, P, P, P, ctypes.POINTER(Range), ctypes.c_int32,
                                            ctypes.c_float, P, P, P]),
        "veda_dequant_fp8_e4m3": (ctypes.c_int, [P, P, ctypes.c_int64, ctypes.c_int32, P]),
        "veda_sparse_attn_fp8qk": (ctypes.c_int, [L, P, P, P, P, P, P, P, ctypes.POINTER(Range), ctypes.c_int32,
                                                  ctypes.c_float, P, P, P]),
        "veda_quantize_fp8_e4m3": (ctypes.c_int, [L, P, P, P, P]),
        "veda_sparse_attn_fp8": (ctypes.c_int, [L, P, P, P, P, P, P, P, P, ctypes.POINTER(Range), ctypes.c_int32,
                                                ctypes.c_float, P, P, P]),
        "veda_quantize_fp8_e4m3_vt": (ctypes.c_int, [L, P, P, P, P]),
        "veda_fp8_vt_bytes": (ctypes.c_size_t, [L]),
        "veda_tile_order": (ctypes.c_int, [L, P, P, P]),
        "veda_sparse_attn_check": (ctypes.c_int, [L, P, P, P, P, P, ctypes.POINTER(Range), ctypes.c_int32,
                                                  ctypes.c_float, P]),
        "veda_layer_attn": (ctypes.c_int, [L, P, P, P, P, P, ctypes.POINTER(Range), ctypes.c_int32,
                                           ctypes.POINTER(Range), ctypes.c_int32, ctypes.c_float, P, P, P,
                                           ctypes.c_size_t, P]),
        "veda_block_mass": (ctypes.c_int, [L, P, P, ctypes.POINTER(Range), ctypes.c_int32, ctypes.c_float,
                                           P, P, P, P]),
        "veda_block_recall": (ctypes.c_int, [L, P, P, P, P]),
        "veda_st_open": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_void_p)]),
        "veda_st_close": (None, [P]),
        "veda_st_count": (ctypes.c_int64, [P]),
        "veda_st_info": (ctypes.c_int, [P, ctypes.c_int64, ctypes.POINTER(ctypes.c_char_p),
                                        ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                        ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]),
        "veda_st_find": (ctypes.c_int64, [P, ctypes.c_char_p]),
        "veda_st_read": (ctypes.c_int, [P, ctypes.c_int64, P, ctypes.c_int64]),
        "veda_st_metadata_count": (ctypes.c_int64, [P]),
        "veda_st_metadata_at": (ctypes.c_int, [P, ctypes.c_int64, ctypes.POINTER(ctypes.c_char_p),
                                               ctypes.POINTER(ctypes.c_char_p)]),
        "veda_window_width": (ctypes.c_int64, [L, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int32]),
        "veda_window_indices": (ctypes.c_int, [L, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int32, P, ctypes.c_int32, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def exported_symbols():
    return [n for n in ("veda_abi_version", "veda_status_string", "veda_k_total", "veda_layer_check",
                        "veda_select_workspace_bytes", "veda_pool_project", "veda_score_topk",
                        "veda_select", "veda_select_noalloc", "veda_sparse_attn", "veda_dequant_fp8_e4m3",
                        "veda_sparse_attn_check", "veda_layer_attn", "veda_window_width",
                        "veda_window_indices", "veda_block_mass", "veda_block_recall",
                        "veda_st_open", "veda_st_close", "veda_st_count", "veda_st_info",
                        "veda_st_find", "veda_st_read", "veda_st_metadata_count",
                        "veda_st_metadata_at", "veda_sparse_attn_fp8qk",
                        "veda_quantize_fp8_e4m3", "veda_sparse_attn_fp8", "veda_quantize_fp8_e4m3_vt",
                        "veda_fp8_vt_bytes", "veda_tile_order")]


# VEDA_ABI_VERSION of include/veda.h that this binding marshals for
ABI_VERSION = 6


def abi_version() -> int:
    return _load().veda_abi_version()


def status_string(status: int) -> str:
    return _load().veda_status_string(status).decode()


def _check(status: int, where: str):
    if status != 0:
        raise VedaError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ----------------------------------------------------------------------------- layers

def make_layer(*, B: int, H: int, d: int, p: int, tile: int, n_tokens: int,
               query: Tuple[int, int], segments: Sequence[Tuple[int, int, int]],
               strides: Tuple[int, int, int]) -> Layer:
    """segments: [(start, length, budget), ...] in call order; strides in elements (b, n, h)."""
    if len(segments) > MAX_SEGMENTS:
        raise ValueError("too many key segments")
    L = Layer()
    L.B, L.H, L.d, L.p, L.tile = B, H, d, p, tile
    L.n_seg = len(segments)
    L.n_tokens = n_tokens
    L.stride_b, L.stride_n, L.stride_h = strides
    L.query.start, L.query.len = query
    for s, (st, ln, bud) in enumerate(segments):
        L.seg[s].start, L.seg[s].len = st, ln
        L.budget[s] = bud
    return L


def strides_of(x: torch.Tensor) -> Tuple[int, int, int]:
    if x.dim() != 4 or x.stride(3) != 1:
        raise ValueError("expected a [B, N, H, d] tensor with a contiguous last dimension")
    return x.stride(0), x.stride(1), x.stride(2)


def layer_from_workload(wl, strides=None) -> Layer:
    if strides is None:
        strides = (wl.n_tokens * wl.H * wl.d, wl.H * wl.d, wl.d)
    return make_layer(B=wl.B, H=wl.H, d=wl.d, p=wl.p, tile=wl.tile, n_tokens=wl.n_tokens,
                      query=(wl.query.start, wl.query.length),
                      segments=[(s.start, s.length, s.budget) for s in wl.segments],
                      strides=strides)


def dense_ranges(ranges: Sequence[Tuple[int, int]]):
    arr = (Range * max(1, len(ranges)))()
    for i, (st, ln) in enumerate(ranges):
        arr[i].start, arr[i].len = st, ln
    return arr, len(ranges)


# ----------------------------------------------------------------------------- calls

def _check_qkv(layer: Layer, *xs):
    for x in xs:
        if x.dtype != torch.bfloat16 or not x.is_cuda:
            raise ValueError("Q/K/V must be bfloat16 device tensors")
        if strides_of(x) != (layer.stride_b, layer.stride_n, layer.stride_h):
            raise ValueError("tensor strides differ from the layer's strides")
        if x.shape[0] != layer.B or x.shape[1] != layer.n_tokens or x.shape[2] != layer.H \
                or x.shape[3] != layer.d:
            raise ValueError("tensor shape differs from the layer")


def _check_w(layer: Layer, *ws):
    want = torch.float16 if layer.wdtype == 1 else torch.bfloat16
    for w in ws:
        if w.dtype != want or not w.is_cuda or not w.is_contiguous() or \
                tuple(w.shape) != (layer.H, layer.p, layer.d):
            raise ValueError(f"predictor weights must be contiguous {want} [H, p, d] device tensors "
                             "(layer.wdtype selects float16 or bfloat16)")


def _check_idx(layer: Layer, idx, device, ktot=None):
    """idx must be a contiguous int32 [B, H, Tq, Ktot] tensor on `device` (the kernels read
    and write it with the layer's geometry and cannot detect a smaller buffer)."""
    ktot = layer.Ktot if ktot is None else ktot
    if idx.dtype != torch.int32 or not idx.is_contiguous() or \
            tuple(idx.shape) != (layer.B, layer.H, layer.Tq, ktot):
        raise ValueError(f"idx must be contiguous int32 [B, H, Tq, Ktot] = "
                         f"{[layer.B, layer.H, layer.Tq, ktot]}")
    if idx.device != device:
        raise ValueError(f"idx is on {idx.device}, expected {device}")


def _check_hat(layer: Layer, x, rows: int, device, what: str):
    """q_hat / k_hat: contiguous fp32 [B, H, rows, p] on `device`."""
    if x.dtype != torch.float32 or not x.is_contiguous() or \
            tuple(x.shape) != (layer.B, layer.H, rows, layer.p):
        raise ValueError(f"{what} must be contiguous fp32 [B, H, {rows}, p] = "
                         f"{[layer.B, layer.H, rows, layer.p]}")
    if x.device != device:
        raise ValueError(f"{what} is on {x.device}, expected {device}")


def select_workspace_bytes(layer: Layer) -> int:
    return _load().veda_select_workspace_bytes(ctypes.byref(layer))


def _workspace(workspace, nbytes: int, device):
    """The caller's workspace, checked: a contiguous tensor on `device` of at least nbytes
    bytes (the kernels write q_hat and k_hat there and cannot detect a smaller buffer).
    None gives a new one."""
    if workspace is None:
        return torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    if workspace.device != device or not workspace.is_contiguous() or \
            workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace must be a contiguous tensor on {device} of at least {nbytes} bytes")
    return workspace


def project(layer: Layer, q, k, wq, wk, stream=None):
    """Pooled + projected vectors (q_hat [B,H,Tq,p], k_hat [B,H,Tk,p], fp32)."""
    _check_qkv(layer, q, k)
    _check_w(layer, wq, wk)
    dev = q.device
    qh = torch.empty((layer.B, layer.H, layer.Tq, layer.p), dtype=torch.float32, device=dev)
    kh = torch.empty((layer.B, layer.H, layer.Tk, layer.p), dtype=torch.float32, device=dev)
    st = _load().veda_pool_project(ctypes.byref(layer), _ptr(q), _ptr(k), _ptr(wq), _ptr(wk),
                                   _ptr(qh), _ptr(kh), _stream(stream))
    _check(st, "veda_pool_project")
    return qh, kh


def score_topk(layer: Layer, q_hat, k_hat, want_scores: bool = False, stream=None):
    dev = q_hat.device
    if not q_hat.is_cuda:
        raise ValueError("q_hat must be a device tensor")
    _check_hat(layer, q_hat, layer.Tq, dev, "q_hat")
    _check_hat(layer, k_hat, layer.Tk, dev, "k_hat")
    idx = torch.empty((layer.B, layer.H, layer.Tq, layer.Ktot), dtype=torch.int32, device=dev)
    sc = torch.empty((layer.B, layer.H, layer.Tq, layer.Tk), dtype=torch.float32, device=dev) \
        if want_scores else None
    st = _load().veda_score_topk(ctypes.byref(layer), _ptr(q_hat), _ptr(k_hat), _ptr(idx),
                                 _ptr(sc), _stream(stream))
    _check(st, "veda_score_topk")
    return (idx, sc) if want_scores else idx


def select(layer: Layer, q, k, wq, wk, want_scores: bool = False, workspace=None, idx=None,
           stream=None):
    """Tile indices int32 [B, H, Tq, Ktot] (and fp32 scores [B, H, Tq, Tk] if asked)."""
    _check_qkv(layer, q, k)
    _check_w(layer, wq, wk)
    dev = q.device
    if idx is None:
        idx = torch.empty((layer.B, layer.H, layer.Tq, layer.Ktot), dtype=torch.int32, device=dev)
    else:
        _check_idx(layer, idx, dev)
    sc = torch.empty((layer.B, layer.H, layer.Tq, layer.Tk), dtype=torch.float32, device=dev) \
        if want_scores else None
    nbytes = select_workspace_bytes(layer)
    if nbytes == 0:
        _check(_load().veda_layer_check(ctypes.byref(layer), 1), "veda_select")
    workspace = _workspace(workspace, nbytes, dev)
    st = _load().veda_select(ctypes.byref(layer), _ptr(q), _ptr(k), _ptr(wq), _ptr(wk), _ptr(idx),
                             _ptr(sc), _ptr(workspace), nbytes, _stream(stream))
    _check(st, "veda_select")
    return (idx, sc) if want_scores else idx


NOALLOC_SCRATCH_BYTES = 64 << 20   # VEDA_NOALLOC_SCRATCH_BYTES


def select_noalloc(layer: Layer, q, k, wq, wk, idx, scores=None, stream=None):
    """veda_select_noalloc: selection into caller-supplied idx (and optional scores) with the
    workspace in the library's own per-GPU array; nothing is allocated by this call."""
    _check_qkv(layer, q, k)
    _check_w(layer, wq, wk)
    _check_idx(layer, idx, q.device)
    if scores is not None and (scores.dtype != torch.float32 or not scores.is_contiguous() or
                               tuple(scores.shape) != (layer.B, layer.H, layer.Tq, layer.Tk) or
                               scores.device != q.device):
        raise ValueError("scores must be contiguous fp32 [B, H, Tq, Tk] on q's device")
    st = _load().veda_select_noalloc(ctypes.byref(layer), _ptr(q), _ptr(k), _ptr(wq), _ptr(wk), _ptr(idx),
                                     _ptr(scores), _stream(stream))
    _check(st, "veda_select_noalloc")
    return idx


def _check_order(layer: Layer, order, idx, device):
    if order is None:
        return
    if idx is None:
        raise ValueError("an order needs an index")
    if order.dtype != torch.int32 or not order.is_contiguous() or \
            tuple(order.shape) != (layer.B, layer.H, layer.Tq) or order.device != device:
        raise ValueError(f"order must be a contiguous int32 [B, H, Tq] = {[layer.B, layer.H, layer.Tq]} "
                         f"tensor on {device}")


def tile_order(layer: Layer, idx, out=None, stream=None):
    """veda_tile_order: int32 [B, H, Tq], per (b, h) the query tiles sorted by their index rows
    (the processing order for the attention calls' `order` argument)."""
    _check_idx(layer, idx, idx.device)
    if out is None:
        out = torch.empty((layer.B, layer.H, layer.Tq), dtype=torch.int32, device=idx.device)
    _check_order(layer, out, idx, idx.device)
    st = _load().veda_tile_order(ctypes.byref(layer), _ptr(idx), _ptr(out), _stream(stream))
    _check(st, "veda_tile_order")
    return out


def sparse_attn(layer: Layer, q, k, v, idx, dense: Sequence[Tuple[int, int]] = (),
                scale: float = 0.0, out=None, want_lse: bool = False, stream=None, order=None):
    """Block-sparse attention; returns out (bf16, q's shape) [and lse fp32 [B, H, query.len]].
    order: None, or tile_order's output (the query tiles' processing order; results do not
    depend on it)."""
    _check_qkv(layer, q, k, v)
    if out is None:
        out = torch.zeros_like(q)
    else:
        _check_qkv(layer, out)
    lse = torch.empty((layer.B, layer.H, layer.query.len), dtype=torch.float32, device=q.device) \
        if want_lse else None
    if idx is not None:
        _check_idx(layer, idx, q.device)
    _check_order(layer, order, idx, q.device)
    arr, n = dense_ranges(list(dense))
    st = _load().veda_sparse_attn(ctypes.byref(layer), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(order), arr, n,
                                  float(scale), _ptr(out), _ptr(lse), _stream(stream))
    _check(st, "veda_sparse_attn")
    return (out, lse) if want_lse else out


def _check_fp8(layer: Layer, *xs):
    for x in xs:
        if x.dtype != torch.uint8 or not x.is_cuda:
            raise ValueError("FP8 Q/K must be uint8 device tensors of E4M3FN codes")
        if strides_of(x) != (layer.stride_b, layer.stride_n, layer.stride_h):
            raise ValueError("tensor strides differ from the layer's strides")
        if tuple(x.shape) != (layer.B, layer.n_tokens, layer.H, layer.d):
            raise ValueError("tensor shape differs from the layer")


def _check_scale(*xs):
    for x in xs:
        if x.dtype != torch.float32 or not x.is_cuda or x.numel() < 1:
            raise ValueError("FP8 scales must be float32 device tensors (first element used)")


def quantize_fp8(layer: Layer, x, out=None, scale=None, stream=None):
    """bf16 Q or K -> (E4M3FN codes uint8 with x's shape and strides, float32 [1] scale 2^e)."""
    _check_qkv(layer, x)
    if out is None:
        out = torch.empty_strided(tuple(x.shape), tuple(x.stride()), dtype=torch.uint8, device=x.device)
    _check_fp8(layer, out)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    _check_scale(scale)
    st = _load().veda_quantize_fp8_e4m3(ctypes.byref(layer), _ptr(x), _ptr(out), _ptr(scale), _stream(stream))
    _check(st, "veda_quantize_fp8_e4m3")
    return out, scale


def sparse_attn_fp8qk(layer: Layer, q8, k8, v, q_scale, k_scale, idx, dense: Sequence[Tuple[int, int]] = (),
                      scale: float = 0.0, out=None, want_lse: bool = False, stream=None, order=None):
    """veda_sparse_attn with E4M3FN Q and K (codes and per-tensor scales as quantize_fp8 returns
    them); v bf16.  Returns out (bf16, v's shape) [and lse fp32 [B, H, query.len]]."""
    _check_fp8(layer, q8, k8)
    _check_qkv(layer, v)
    _check_scale(q_scale, k_scale)
    if out is None:
        out = torch.zeros_like(v)
    else:
        _check_qkv(layer, out)
    lse = torch.empty((layer.B, layer.H, layer.query.len), dtype=torch.float32, device=v.device) \
        if want_lse else None
    if idx is not None:
        _check_idx(layer, idx, v.device)
    _check_order(layer, order, idx, v.device)
    arr, n = dense_ranges(list(dense))
    st = _load().veda_sparse_attn_fp8qk(ctypes.byref(layer), _ptr(q8), _ptr(k8), _ptr(v), _ptr(q_scale),
                                        _ptr(k_scale), _ptr(idx), _ptr(order), arr, n, float(scale), _ptr(out), _ptr(lse),
                                        _stream(stream))
    _check(st, "veda_sparse_attn_fp8qk")
    return (out, lse) if want_lse else out


def fp8_vt_bytes(layer: Layer) -> int:
    """Bytes of the blocked FP8 V that quantize_fp8_vt writes (0: layer not supported)."""
    return int(_load().veda_fp8_vt_bytes(ctypes.byref(layer)))


def _check_vt(layer: Layer, vt):
    n = fp8_vt_bytes(layer)
    if n == 0:
        raise ValueError("layer not supported by the FP8-V layout")
    if vt.dtype != torch.uint8 or not vt.is_cuda or not vt.is_contiguous() or vt.numel() != n:
        raise ValueError(f"vt must be a contiguous uint8 device tensor of {n} bytes")


def quantize_fp8_vt(layer: Layer, v, out=None, scale=None, stream=None):
    """bf16 V -> (E4M3FN codes in d-major 64-token blocks, uint8 [B, H, ceil(N / 64), d, 64]
    with the chunk permutation of veda_quantize_fp8_e4m3_vt; float32 [1] scale 2^e)."""
    _check_qkv(layer, v)
    if out is None:
        out = torch.empty((layer.B, layer.H, -(-layer.n_tokens // 64), layer.d, 64), dtype=torch.uint8,
                          device=v.device)
    _check_vt(layer, out)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=v.device)
    _check_scale(scale)
    st = _load().veda_quantize_fp8_e4m3_vt(ctypes.byref(layer), _ptr(v), _ptr(out), _ptr(scale), _stream(stream))
    _check(st, "veda_quantize_fp8_e4m3_vt")
    return out, scale


def sparse_attn_fp8(layer: Layer, q8, k8, vt, q_scale, k_scale, v_scale, idx,
                    dense: Sequence[Tuple[int, int]] = (), scale: float = 0.0, out=None, want_lse: bool = False,
                    stream=None, order=None):
    """veda_sparse_attn with E4M3FN Q, K (as quantize_fp8 returns them), V in the blocked layout
    of quantize_fp8_vt, and P rounded to E4M3FN.  Returns out (bf16, q8's shape and strides)
    [and lse fp32 [B, H, query.len]]."""
    _check_fp8(layer, q8, k8)
    _check_vt(layer, vt)
    _check_scale(q_scale, k_scale, v_scale)
    if out is None:
        out = torch.empty_strided(tuple(q8.shape), tuple(q8.stride()), dtype=torch.bfloat16,
                                  device=q8.device).zero_()
    else:
        _check_qkv(layer, out)
    lse = torch.empty((layer.B, layer.H, layer.query.len), dtype=torch.float32, device=q8.device) \
        if want_lse else None
    if idx is not None:
        _check_idx(layer, idx, q8.device)
    _check_order(layer, order, idx, q8.device)
    arr, n = dense_ranges(list(dense))
    st = _load().veda_sparse_attn_fp8(ctypes.byref(layer), _ptr(q8), _ptr(k8), _ptr(vt), _ptr(q_scale),
                                      _ptr(k_scale), _ptr(v_scale), _ptr(idx), _ptr(order), arr, n, float(scale), _ptr(out),
                                      _ptr(lse), _stream(stream))
    _check(st, "veda_sparse_attn_fp8")
    return (out, lse) if want_lse else out


def layer_attn(layer: Layer, q, k, v, wq, wk, dense: Sequence[Tuple[int, int]] = (),
               dense_queries: Sequence[Tuple[int, int]] = (), scale: float = 0.0, out=None,
               idx=None, workspace=None, stream=None):
    """One full layer: selection + sparse attention for the query segment, dense attention
    for every range in dense_queries.  Returns (out, idx)."""
    _check_qkv(layer, q, k, v)
    _check_w(layer, wq, wk)
    dev = q.device
    if out is None:
        out = torch.zeros_like(q)
    else:
        _check_qkv(layer, out)
    if idx is None:
        idx = torch.empty((layer.B, layer.H, layer.Tq, layer.Ktot), dtype=torch.int32, device=dev)
    else:
        _check_idx(layer, idx, dev)
    nbytes = select_workspace_bytes(layer)
    if nbytes == 0:
        _check(_load().veda_layer_check(ctypes.byref(layer), 1), "veda_layer_attn")
    workspace = _workspace(workspace, nbytes, dev)
    darr, nd = dense_ranges(list(dense))
    qarr, nq = dense_ranges(list(dense_queries))
    st = _load().veda_layer_attn(ctypes.byref(layer), _ptr(q), _ptr(k), _ptr(v), _ptr(wq), _ptr(wk),
                                 darr, nd, qarr, nq, float(scale), _ptr(out), _ptr(idx),
                                 _ptr(workspace), nbytes, _stream(stream))
    _check(st, "veda_layer_attn")
    return out, idx


def block_mass(layer: Layer, q, k, dense: Sequence[Tuple[int, int]] = (), scale: float = 0.0,
               want_dense: bool = True, stream=None):
    """Teacher block attention mass fp32 [B, H, Tq, Tk] over every key tile of every segment.
    Returns (mass, dense_mass [B, H, Tq] or None, lse [B, H, query.len])."""
    _check_qkv(layer, q, k)
    dev = q.device
    mass = torch.empty((layer.B, layer.H, layer.Tq, layer.Tk), dtype=torch.float32, device=dev)
    lse = torch.empty((layer.B, layer.H, layer.query.len), dtype=torch.float32, device=dev)
    dm = torch.empty((layer.B, layer.H, layer.Tq), dtype=torch.float32, device=dev) if want_dense else None
    arr, n = dense_ranges(list(dense))
    st = _load().veda_block_mass(ctypes.byref(layer), _ptr(q), _ptr(k), arr, n, float(scale), _ptr(lse),
                                 _ptr(mass), _ptr(dm), _stream(stream))
    _check(st, "veda_block_mass")
    return mass, dm, lse


def block_recall(layer: Layer, mass, idx, stream=None):
    """Recall fp32 [B, H, Tq] of the index set idx [B, H, Tq, Ktot] under the teacher mass."""
    if mass.dtype != torch.float32 or tuple(mass.shape) != (layer.B, layer.H, layer.Tq, layer.Tk) \
            or not mass.is_contiguous() or not mass.is_cuda:
        raise ValueError("mass must be a contiguous fp32 [B, H, Tq, Tk] device tensor")
    _check_idx(layer, idx, mass.device)
    rec = torch.empty((layer.B, layer.H, layer.Tq), dtype=torch.float32, device=mass.device)
    st = _load().veda_block_recall(ctypes.byref(layer), _ptr(mass), _ptr(idx), _ptr(rec), _stream(stream))
    _check(st, "veda_block_recall")
    return rec


def window_width(layer: Layer, frame_tokens: int, chunk_frames: int = 5, halo_chunks: int = 1,
                 anchors: bool = True) -> int:
    """Longest row (key tiles) of the sliding frame-chunk window pattern."""
    w = _load().veda_window_width(ctypes.byref(layer), int(frame_tokens), int(chunk_frames),
                                  int(halo_chunks), 1 if anchors else 0)
    if w < 0:
        raise VedaError(int(w), "veda_window_width")
    return int(w)


def window_indices(layer: Layer, frame_tokens: int, chunk_frames: int = 5, halo_chunks: int = 1,
                   anchors: bool = True, width: Optional[int] = None, device=None, stream=None):
    """Window-pattern tile indices int32 [B, H, Tq, width], rows ascending, -1 padded.
    Returns (idx, attention_layer): the copy of `layer` whose budget[0] is width."""
    if width is None:
        width = window_width(layer, frame_tokens, chunk_frames, halo_chunks, anchors)
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    idx = torch.empty((layer.B, layer.H, layer.Tq, width), dtype=torch.int32, device=dev)
    st = _load().veda_window_indices(ctypes.byref(layer), int(frame_tokens), int(chunk_frames),
                                     int(halo_chunks), 1 if anchors else 0, _ptr(idx), int(width),
                                     _stream(stream))
    _check(st, "veda_window_indices")
    att = Layer.from_buffer_copy(layer)
    att.budget[0] = width
    return idx, att


# ----------------------------------------------------------------------------- predictor files

ST_DTYPES = {1: ("F16", np.float16), 2: ("BF16", np.uint16), 3: ("F32", np.float32),
             4: ("F64", np.float64), 5: ("F8_E4M3", np.uint8), 6: ("F8_E5M2", np.uint8),
             7: ("I8", np.int8), 8: ("U8", np.uint8), 9: ("I16", np.int16), 10: ("U16", np.uint16),
             11: ("I32", np.int32), 12: ("U32", np.uint32), 13: ("I64", np.int64),
             14: ("U64", np.uint64), 15: ("BOOL", np.bool_)}


class SafetensorsFile:
    """A predictor file read through the library's native safetensors reader.  Arrays
    come back as numpy (bf16 as uint16 bits, FP8 as uint8 codes)."""

    def __init__(self, path):
        self._lib = _load()
        h = ctypes.c_void_p()
        _check(self._lib.veda_st_open(os.fsencode(path), ctypes.byref(h)), f"veda_st_open({path})")
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            self._lib.veda_st_close(self._h)
            self._h = None

    __del__ = close

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()

    def __len__(self):
        return int(self._lib.veda_st_count(self._h))

    def info(self, i):
        """(name, dtype name, shape tuple, nbytes) of tensor i (file order)."""
        name = ctypes.c_char_p()
        dt = ctypes.c_int32()
        nd = ctypes.c_int32()
        shape = (ctypes.c_int64 * 8)()
        nb = ctypes.c_int64()
        _check(self._lib.veda_st_info(self._h, i, ctypes.byref(name), ctypes.byref(dt), ctypes.byref(nd),
                                      shape, ctypes.byref(nb)), "veda_st_info")
        return name.value.decode(), ST_DTYPES[dt.value][0], tuple(shape[:nd.value]), nb.value

    def names(self):
        return [self.info(i)[0] for i in range(len(self))]

    def read(self, name) -> np.ndarray:
        i = self._lib.veda_st_find(self._h, name.encode())
        if i < 0:
            raise KeyError(name)
        _, dt, shape, nb = self.info(i)
        np_dt = dict(ST_DTYPES.values())[dt]
        out = np.empty(shape, dtype=np_dt)
        assert out.nbytes == nb
        _check(self._lib.veda_st_read(self._h, i, out.ctypes.data_as(ctypes.c_void_p), nb), "veda_st_read")
        return out

    def metadata(self):
        md = {}
        for i in range(int(self._lib.veda_st_metadata_count(self._h))):
            k, v = ctypes.c_char_p(), ctypes.c_char_p()
            _check(self._lib.veda_st_metadata_at(self._h, i, ctypes.byref(k), ctypes.byref(v)),
                   "veda_st_metadata_at")
            md[k.value.decode()] = v.value.decode()
        return md


def check_selector_file(path, n_layers=50, shape=(56, 384, 128), max_bytes=560_000_000):
    """The selector-file rules the competition publishes: exactly 2 * n_layers float16
    tensors (query and key projection per layer), each of the given shape, and at most
    max_bytes in total.  Returns the tensor names in file order; raises ValueError."""
    size = os.path.getsize(path)
    if size > max_bytes:
        raise ValueError(f"{path}: {size} bytes exceeds {max_bytes}")
    with SafetensorsFile(path) as f:
        infos = [f.info(i) for i in range(len(f))]
    if len(infos) != 2 * n_layers:
        raise ValueError(f"{path}: {len(infos)} tensors, expected {2 * n_layers}")
    for name, dt, shp, _ in infos:
        if dt != "F16" or tuple(shp) != tuple(shape):
            raise ValueError(f"{path}: tensor {name} is {dt}{list(shp)}, expected F16{list(shape)}")
    return [i[0] for i in infos]


def predictor_weight(f: "SafetensorsFile", name: str, device=None, pow2_exp: int = 0):
    """One projection [H, p, d] on the device in a form the selection kernels read, and
    its veda_wdtype: F16 and BF16 as stored; F8_E4M3 codes dequantised to bf16 on the
    device (exact, times 2^pow2_exp)."""
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    arr = f.read(name)
    _, dt, _, _ = f.info(f._lib.veda_st_find(f._h, name.encode()))
    if dt == "F16":
        return torch.from_numpy(arr).to(dev), 1
    if dt == "BF16":
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(dev), 0
    if dt == "F8_E4M3":
        return dequant_fp8_e4m3(torch.from_numpy(arr).to(dev), pow2_exp), 0
    raise ValueError(f"{name}: predictor weights must be F16, BF16 or F8_E4M3, not {dt}")


def dequant_fp8_e4m3(codes: torch.Tensor, pow2_exp: int = 0, stream=None) -> torch.Tensor:
    """E4M3FN bytes (uint8 device tensor) -> bf16 tensor of the same shape, exact."""
    if codes.dtype != torch.uint8 or not codes.is_cuda or not codes.is_contiguous():
        raise ValueError("codes must be a contiguous uint8 device tensor")
    dst = torch.empty(codes.shape, dtype=torch.bfloat16, device=codes.device)
    st = _load().veda_dequant_fp8_e4m3(_ptr(codes), _ptr(dst), codes.numel(), int(pow2_exp),
                                       _stream(stream))
    _check(st, "veda_dequant_fp8_e4m3")
    return dst
