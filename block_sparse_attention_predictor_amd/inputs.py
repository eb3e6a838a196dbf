"""Seeded synthetic workloads for the Veda block-sparse attention path.

This module only *describes* layer shapes and *draws* inputs. It holds none of
the method's arithmetic (no pooling, projection, scoring, selection or
attention), so both the fp64 CPU oracle and the GPU path may import it.

Workloads (token layout: generated video first, ordered frame, row, column;
then an optional reference image; then text, VLM conditioning and audio):

  tiny    B=1 H=2  d=64  p=32 tile=64   video 8x16x16   + 64 text,              k=4
  mid     B=1 H=24 d=128 p=64 tile=64   video 16x24x42  + 256 text,             k=26 (90 %)
  t2v5s   B=1 H=40 d=128 p=64 tile=128  video 32x48x84  + 512 text + 1024 audio, k=50 (95 %)
  r2va    B=1 H=40 d=128 p=64 tile=128  video 32x48x84  + ref 48x84 + 512 text + 256 VLM
                                        + 1024 audio, k = 32 ref + 32 video
  t2v14s  B=1 H=40 d=128 p=64 tile=128  video 87x48x84  + 512 text + 2048 audio, k=137 (95 %),
                                        predictor weights stored as FP8 E4M3FN

The latent geometry matches 1344x768 frames under 16x spatial compression (48x84
latent grid) at 24 fps (Affine launch article, "Inside the MiniMax-H3 Studio");
the R2VA budgets of 32 reference + 32 video tiles per query tile and head, with
text, VLM and audio keys dense, follow the Veda R2VA record (its first paragraph).

Value recipe for video tokens:  x = z + 0.5 * F,  z ~ N(0, 1), with F a
unit-variance smooth field made of M = 16 low-frequency Fourier modes:
    F_{h,c}(f, y, x) = sum_m  alpha_{m,h,c} cos(theta_m) + beta_{m,h,c} sin(theta_m)
    theta_m = 2 pi (ky_m y / GH + kx_m x / GW + kt_m f / NF),   ky, kx in -2..2,
    alpha, beta ~ N(0, 1/M).
The tiny workload redraws alpha, beta per frame with kt = 0 ("per-frame" field);
the others use kt in 0..2 ("spatio-temporal").  Q and K share one field, V has
its own.  The reference image is frame 0's field plus noise.  Text, VLM and audio
tokens are plain N(0, 1).  Everything is rounded to bfloat16 (round to nearest
even) and returned as raw uint16 bit patterns.

Weights Wq, Wk ~ N(0, 1/d), laid out [H, p, d], rounded to bf16; for the FP8
workload they are scaled by 2^4, rounded to OCP E4M3FN (nearest even,
saturating at 448) and stored as bytes with a dequantisation exponent of -4.

Seeds: numpy PCG64 from SeedSequence([0x5EDA, workload index, tensor id, chunk]).
Noise is drawn per chunk of 1024 token rows, so the result does not depend on
the number of threads used to draw it.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

SEED_ROOT = 0x5EDA
N_MODES = 16
FIELD_AMPLITUDE = 0.5
CHUNK_ROWS = 1024

# tensor ids used in the seed sequence
TID_Q, TID_K, TID_V, TID_WQ, TID_WK, TID_FIELD_QK, TID_FIELD_V, TID_MODES = range(8)


@dataclass(frozen=True)
class Segment:
    """A key segment [start, start+length) tiled from its own start, with a top-k budget."""
    name: str
    start: int
    length: int
    budget: int


@dataclass(frozen=True)
class Range:
    name: str
    start: int
    length: int


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    B: int
    H: int
    d: int
    p: int
    tile: int
    grid: Tuple[int, int, int]            # latent frames, rows, columns of the video
    query: Range                          # the sparse query segment (video)
    segments: Tuple[Segment, ...]         # key segments selected by top-k
    dense: Tuple[Range, ...]              # key ranges every query attends to
    n_tokens: int
    per_frame_field: bool = False
    ref_grid: Optional[Tuple[int, int]] = None
    fp8_weights: bool = False
    fp8_pow2_exp: int = 0

    @property
    def n_query_tiles(self) -> int:
        return -(-self.query.length // self.tile)

    def seg_tiles(self, s: Segment) -> int:
        return -(-s.length // self.tile)

    @property
    def k_total(self) -> int:
        return sum(min(s.budget, self.seg_tiles(s)) for s in self.segments)

    @property
    def t_total(self) -> int:
        return sum(self.seg_tiles(s) for s in self.segments)


def _layout(name, index, H, d, p, tile, grid, extra_ref, text, vlm, audio, budgets,
            per_frame=False, fp8=False, pow2=0) -> Workload:
    F, GH, GW = grid
    n_video = F * GH * GW
    pos = 0
    query = Range("video", 0, n_video)
    pos = n_video
    segs = []
    ref_grid = None
    if extra_ref:
        n_ref = GH * GW
        segs.append(Segment("ref", pos, n_ref, budgets["ref"]))
        ref_grid = (GH, GW)
        pos += n_ref
    segs.append(Segment("video", 0, n_video, budgets["video"]))
    # video segment first in call order for T2V; R2VA lists reference then video
    dense = []
    for nm, n in (("text", text), ("vlm", vlm), ("audio", audio)):
        if n:
            dense.append(Range(nm, pos, n))
            pos += n
    return Workload(name=name, index=index, B=1, H=H, d=d, p=p, tile=tile, grid=grid,
                    query=query, segments=tuple(segs), dense=tuple(dense), n_tokens=pos,
                    per_frame_field=per_frame, ref_grid=ref_grid, fp8_weights=fp8,
                    fp8_pow2_exp=pow2)


WORKLOADS = {
    "tiny": _layout("tiny", 0, 2, 64, 32, 64, (8, 16, 16), False, 64, 0, 0,
                    {"video": 4}, per_frame=True),
    "mid": _layout("mid", 1, 24, 128, 64, 64, (16, 24, 42), False, 256, 0, 0,
                   {"video": 26}),
    "t2v5s": _layout("t2v5s", 2, 40, 128, 64, 128, (32, 48, 84), False, 512, 0, 1024,
                     {"video": 50}),
    "r2va": _layout("r2va", 3, 40, 128, 64, 128, (32, 48, 84), True, 512, 256, 1024,
                    {"ref": 32, "video": 32}),
    "t2v14s": _layout("t2v14s", 4, 40, 128, 64, 128, (87, 48, 84), False, 512, 0, 2048,
                      {"video": 137}, fp8=True, pow2=-4),
}
WORKLOAD_ORDER = ["tiny", "mid", "t2v5s", "r2va", "t2v14s"]


def custom_workload(name="custom", *, B=1, H=2, d=64, p=32, tile=64, grid=(2, 8, 8),
                    ref=False, text=0, vlm=0, audio=0, budgets=None, index=99,
                    per_frame=False) -> Workload:
    """A small workload of the same structure, for edge-case tests."""
    budgets = budgets or {"video": 2, "ref": 2}
    wl = _layout(name, index, H, d, p, tile, grid, ref, text, vlm, audio, budgets,
                 per_frame=per_frame)
    if B != 1:
        wl = Workload(**{**wl.__dict__, "B": B})
    return wl


# ----------------------------------------------------------------------------- helpers

def _rng(*ids) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, *ids])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def f32_to_e4m3fn_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to OCP FP8 E4M3FN (nearest, ties to even, saturate to +-448).

    E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent field 0 holds
    subnormals m * 2^-9; no infinities; S.1111.111 is NaN, so 448 = 1.75 * 2^8 is
    the largest finite value.  Inputs must be finite.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = (x < 0) | ((x == 0) & np.signbit(x))
    a = np.minimum(np.abs(x), 448.0)
    out = np.zeros(a.shape, dtype=np.uint8)
    nz = a > 0
    e = np.zeros(a.shape, dtype=np.int64)
    e[nz] = np.floor(np.log2(a[nz])).astype(np.int64)
    e = np.clip(e, -6, 8)                       # below 2^-6 the quantum stays 2^-9
    quantum = np.ldexp(1.0, (e - 3).astype(np.int32))
    q = np.rint(a / quantum)                    # numpy rint: ties to even
    # rounding up may carry into the next binade
    carry = q >= 16
    e = np.where(carry, e + 1, e)
    q = np.where(carry, q / 2, q)
    is_sub = (e == -6) & (q < 8)
    exp_field = np.where(is_sub, 0, e + 7)
    man = np.where(is_sub, q, q - 8)
    over = exp_field > 15
    exp_field = np.where(over, 15, exp_field)
    man = np.where(over, 6, man)
    nan_code = (exp_field == 15) & (man == 7)   # cannot happen after the clamp to 448
    man = np.where(nan_code, 6, man)
    out = ((exp_field.astype(np.uint8) << 3) | man.astype(np.uint8))
    out = np.where(a == 0, 0, out).astype(np.uint8)
    return (out | (sign.astype(np.uint8) << 7)).astype(np.uint8)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _modes(wl: Workload, tid: int, frame: Optional[int] = None):
    """Mode wave numbers and coefficients for one smooth field."""
    g = _rng(wl.index, TID_MODES, tid) if frame is None else _rng(wl.index, TID_MODES, tid, frame)
    ky = g.integers(-2, 3, size=N_MODES)
    kx = g.integers(-2, 3, size=N_MODES)
    if wl.per_frame_field:
        kt = np.zeros(N_MODES, dtype=np.int64)
    else:
        kt = g.integers(0, 3, size=N_MODES)
    gc = _rng(wl.index, tid) if frame is None else _rng(wl.index, tid, frame)
    coeff = gc.standard_normal((2 * N_MODES, wl.H * wl.d), dtype=np.float64) / np.sqrt(N_MODES)
    return ky, kx, kt, coeff.astype(np.float32)


def _field_rows(wl: Workload, modes, f: np.ndarray, y: np.ndarray, x: np.ndarray) -> np.ndarray:
    ky, kx, kt, coeff = modes
    F, GH, GW = wl.grid
    theta = 2.0 * np.pi * (np.outer(y, ky) / GH + np.outer(x, kx) / GW + np.outer(f, kt) / F)
    basis = np.concatenate([np.cos(theta), np.sin(theta)], axis=1).astype(np.float32)
    return basis @ coeff


def make_tensor(wl: Workload, which: str) -> np.ndarray:
    """Draw Q, K or V as uint16 bf16 bits, shape [B, n_tokens, H, d], contiguous."""
    tid = {"q": TID_Q, "k": TID_K, "v": TID_V}[which]
    field_tid = TID_FIELD_V if which == "v" else TID_FIELD_QK
    B, N, H, d = wl.B, wl.n_tokens, wl.H, wl.d
    out = np.empty((B, N, H * d), dtype=np.uint16)
    F, GH, GW = wl.grid
    fpf = GH * GW
    n_video = wl.query.length
    if wl.per_frame_field:
        frame_modes = [_modes(wl, field_tid, fr) for fr in range(F)]
        shared = None
    else:
        frame_modes = None
        shared = _modes(wl, field_tid)
    ref_seg = next((s for s in wl.segments if s.name == "ref"), None)

    def field_for(rows: np.ndarray) -> Optional[np.ndarray]:
        """Field values for token rows (None where the rows carry no field)."""
        res = np.zeros((rows.size, H * d), dtype=np.float32)
        has = np.zeros(rows.size, dtype=bool)
        vid = rows < n_video
        if vid.any():
            r = rows[vid]
            fr, rem = np.divmod(r, fpf)
            yy, xx = np.divmod(rem, GW)
            if frame_modes is None:
                res[vid] = _field_rows(wl, shared, fr, yy, xx)
            else:
                vals = np.empty((r.size, H * d), dtype=np.float32)
                for f_id in np.unique(fr):
                    m = fr == f_id
                    vals[m] = _field_rows(wl, frame_modes[f_id], fr[m], yy[m], xx[m])
                res[vid] = vals
            has[vid] = True
        if ref_seg is not None:
            inref = (rows >= ref_seg.start) & (rows < ref_seg.start + ref_seg.length)
            if inref.any():
                r = rows[inref] - ref_seg.start
                yy, xx = np.divmod(r, GW)
                fr = np.zeros_like(r)
                modes = frame_modes[0] if frame_modes is not None else shared
                res[inref] = _field_rows(wl, modes, fr, yy, xx)
                has[inref] = True
        return res if has.any() else None

    def work(job):
        b, c = job
        r0 = c * CHUNK_ROWS
        r1 = min(N, r0 + CHUNK_ROWS)
        g = _rng(wl.index, tid, b, c)
        z = g.standard_normal((r1 - r0, H * d), dtype=np.float32)
        fld = field_for(np.arange(r0, r1))
        if fld is not None:
            z += np.float32(FIELD_AMPLITUDE) * fld
        out[b, r0:r1] = f32_to_bf16_bits(z)

    jobs = [(b, c) for b in range(B) for c in range(-(-N // CHUNK_ROWS))]
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(work, jobs))
    return out.reshape(B, N, H, d)


def make_qkv(wl: Workload):
    return make_tensor(wl, "q"), make_tensor(wl, "k"), make_tensor(wl, "v")


@dataclass
class Weights:
    """Predictor weights [H, p, d].  Either bf16 bits (uint16) or E4M3FN bytes + exponent."""
    wq: np.ndarray
    wk: np.ndarray
    fp8: bool = False
    pow2_exp: int = 0


def make_weights(wl: Workload) -> Weights:
    shape = (wl.H, wl.p, wl.d)
    wq = _rng(wl.index, TID_WQ).standard_normal(shape, dtype=np.float64) / np.sqrt(wl.d)
    wk = _rng(wl.index, TID_WK).standard_normal(shape, dtype=np.float64) / np.sqrt(wl.d)
    if wl.fp8_weights:
        s = 2.0 ** (-wl.fp8_pow2_exp)
        return Weights(f32_to_e4m3fn_bits(wq * s), f32_to_e4m3fn_bits(wk * s), True, wl.fp8_pow2_exp)
    return Weights(f32_to_bf16_bits(wq.astype(np.float32)), f32_to_bf16_bits(wk.astype(np.float32)))


def random_indices(wl: Workload, seed: int = 0) -> np.ndarray:
    """Uniformly random valid index sets [B, H, Tq, Ktot] (ascending within each segment)."""
    g = _rng(wl.index, 1000 + seed)
    out = np.empty((wl.B, wl.H, wl.n_query_tiles, wl.k_total), dtype=np.int32)
    col = 0
    for s in wl.segments:
        T = wl.seg_tiles(s)
        k = min(s.budget, T)
        keys = g.random((wl.B, wl.H, wl.n_query_tiles, T))
        pick = np.sort(np.argsort(keys, axis=-1)[..., :k], axis=-1)
        out[..., col:col + k] = pick
        col += k
    return out


def full_indices(wl: Workload) -> np.ndarray:
    """Every tile of every segment: the dense case expressed as an index set."""
    parts = []
    for s in wl.segments:
        T = wl.seg_tiles(s)
        parts.append(np.broadcast_to(np.arange(T, dtype=np.int32),
                                     (wl.B, wl.H, wl.n_query_tiles, T)))
    return np.ascontiguousarray(np.concatenate(parts, axis=-1))


def with_full_budget(wl: Workload) -> Workload:
    segs = tuple(Segment(s.name, s.start, s.length, wl.seg_tiles(s)) for s in wl.segments)
    return Workload(**{**wl.__dict__, "segments": segs})


def with_budget(wl: Workload, budget: int) -> Workload:
    """The same layer with one top-k budget for every key segment (budget sweeps)."""
    segs = tuple(Segment(s.name, s.start, s.length, budget) for s in wl.segments)
    return Workload(**{**wl.__dict__, "segments": segs})
