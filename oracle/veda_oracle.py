"""fp64 CPU oracle for Veda-style learned block-sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run
this module: only the test suite, the smoke check and the benchmark's CPU
baseline do.  It shares no code with the HIP kernels or their host library.

What it computes, step by step, in the order the method runs (one attention
layer of a video diffusion transformer):

  O1  dequantise FP8 predictor weights to exact values          (Veda R2VA record:
      the predictor is stored in FP8 and dequantised to BF16 at load)
  O2  cut the query segment and every key segment into token tiles
  O3  mean-pool Q and K over each tile (real tokens only)       (Affine launch article,
      "Training the Selector": a lightweight predictor distilled from a full-attention
      teacher selects blocks; pooling per tile is this implementation's reading)
  O4  project the pooled vectors through the per-layer query / key projections
      Wq[h], Wk[h] of shape [p, d]                              (same article: miners train
      the selector's query and key projections; "How the SN120 Competition Works"
      gives their per-layer tensor shape)
  O5  score every (query tile, key tile) pair per head: <q_hat, k_hat>, unscaled
  O6  keep a fixed top-k budget of key tiles per (query tile, head) and per key
      segment, ties to the lower tile index, listed ascending    (Veda R2VA record:
      reference and current-video tiles chosen independently with fixed budgets)
  O7  attend each query row to the tokens of the selected tiles plus every dense
      key range (text / VLM / audio stay dense, same record), with a two-pass
      softmax at scale 1/sqrt(d)

the teacher quantity the predictor is distilled from, and how much of it a
selection keeps:

  T1  teacher block attention mass                          (Affine launch article,
      "Training the Selector, Not the Generator": the predictor is distilled from a
      full-attention teacher's attention patterns; at block granularity this is read
      as the dense softmax mass that a query tile's rows put on each key tile,
      averaged over the rows)
  T2  recall of an index set: the selected tiles' share of the segment tiles' mass

the FP8 form of O7's first product (the pages store weights in FP8, R2VA record
first paragraph; this extension quantises the logits' operands too):

  Q1  nearest OCP E4M3FN code of a value, ties to the even code, beyond 448 saturating
  Q2  per-tensor power-of-two scale: 2^e with e the smallest integer such that
      max|x| <= 448 * 2^e; Q and K are coded as Q1(x / 2^e) and O7 then runs on the
      decoded values (code value times 2^e)

and, as a fixed index producer beside the learned one:

  P1  the sliding frame-chunk window with boundary anchors   (VDN article, "The
      mechanism: solving instead of stepping": chunks of consecutive latent frames
      attend to themselves and their neighbouring chunks; every frame also attends
      to the first and last frames, which attend to every frame), carried to tile
      granularity: a query tile takes a key tile when some query token of it may
      attend some key token of the other

All arithmetic is float64 from the exact bf16 (or E4M3) input values.  Library
primitives used as single steps: numpy mean over a slice, matmul, stable argsort,
exp and log.  There is no blocking, fusion or reordering beyond the definitions.
Parity pins: every function here is pinned by tests that do not call it to
produce their expected values (brute force, closed forms, library special
cases); quality of the selection versus full attention with trained weights is
*parity unpinned* (it needs the real model, weights and videos).
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np


# ----------------------------------------------------------------------------- O1

def e4m3fn_value(byte: int) -> float:
    """Value of one OCP FP8 E4M3FN code (OCP 8-bit floating point spec v1.0).

    Layout S.EEEE.MMM, exponent bias 7.  Exponent field 0 encodes subnormals
    (M/8) * 2^-6; otherwise (1 + M/8) * 2^(E-7).  There are no infinities; the
    codes S.1111.111 are NaN.
    """
    byte = int(byte)
    s = (byte >> 7) & 1
    e = (byte >> 3) & 0xF
    m = byte & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        mag = (m / 8.0) * 2.0 ** -6
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


_E4M3_TABLE = np.array([e4m3fn_value(b) for b in range(256)], dtype=np.float64)


def dequant_e4m3fn(codes: np.ndarray, pow2_exp: int = 0) -> np.ndarray:
    """O1: E4M3FN bytes times 2^pow2_exp, as float64 (exact)."""
    codes = np.asarray(codes, dtype=np.uint8)
    vals = _E4M3_TABLE[codes] * (2.0 ** pow2_exp)
    if np.isnan(vals).any():
        raise ValueError("NaN code in FP8 predictor weights")
    return vals


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """A bfloat16 value is the float32 whose upper 16 bits are the stored bits."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest bfloat16 (ties to even); used only to assert that
    dequantised FP8 values are exactly representable in bf16."""
    x = np.asarray(x, dtype=np.float64)
    f32 = x.astype(np.float32)
    if not np.array_equal(f32.astype(np.float64), x):
        raise ValueError("value not representable in float32")
    u = f32.view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def dequant_e4m3fn_to_bf16_bits(codes: np.ndarray, pow2_exp: int = 0) -> np.ndarray:
    """O1 as the path stores it: exact bf16 bit patterns of the dequantised weights."""
    vals = dequant_e4m3fn(codes, pow2_exp)
    bits = f64_to_bf16_bits_rne(vals)
    if not np.array_equal(bf16_bits_to_f64(bits), vals):
        raise AssertionError("dequantised FP8 value not exact in bf16")
    return bits


# ----------------------------------------------------------------------------- O2

def tile_bounds(start: int, length: int, tile: int) -> List[Tuple[int, int]]:
    """O2: tile i covers tokens [start + i*tile, min(start + (i+1)*tile, start + length))."""
    return [(start + i, start + min(i + tile, length)) for i in range(0, length, tile)]


# ----------------------------------------------------------------------------- O3

def pool_tiles(x_bits: np.ndarray, b: int, h: int, start: int, length: int,
               tile: int) -> np.ndarray:
    """O3: mean of the rows of x[b, n, h, :] over each tile's real tokens.

    x_bits: uint16 bf16 bits [B, N, H, d].  Returns float64 [T, d].
    """
    bounds = tile_bounds(start, length, tile)
    d = x_bits.shape[3]
    out = np.empty((len(bounds), d), dtype=np.float64)
    rows = bf16_bits_to_f64(x_bits[b, start:start + length, h, :])
    for i, (lo, hi) in enumerate(bounds):
        out[i] = rows[lo - start:hi - start].mean(axis=0)
    return out


# ----------------------------------------------------------------------------- O4, O5

def project(pooled: np.ndarray, w: np.ndarray) -> np.ndarray:
    """O4: x_hat = W x_bar for each pooled vector; W is [p, d] (out x in), no bias."""
    return pooled @ w.T


def tile_scores(q_hat: np.ndarray, k_hat: np.ndarray) -> np.ndarray:
    """O5: s[i, j] = sum_c q_hat[i, c] * k_hat[j, c]  (no scale, no temperature)."""
    return q_hat @ k_hat.T


# ----------------------------------------------------------------------------- O6

def topk_lowest_index(row: np.ndarray, k: int) -> np.ndarray:
    """O6 for one row of one segment: the min(k, T) largest scores, equal scores
    ordered by lower tile index first, returned in ascending tile order.

    Stable sort of the negated scores keeps equal keys in index order; -0.0 and
    +0.0 compare equal, so they tie.
    """
    T = row.shape[0]
    k = min(k, T)
    order = np.argsort(-row, kind="stable")
    return np.sort(order[:k]).astype(np.int32)


# ----------------------------------------------------------------------------- selection

def weights_f64(w) -> np.ndarray:
    """Predictor weights as float64 [H, p, d]: bf16 bits (uint16), IEEE float16 values
    (numpy float16, converted exactly), or FP8 bytes as (codes, pow2_exp)."""
    if isinstance(w, tuple):  # (codes, pow2_exp)
        codes, e = w
        return dequant_e4m3fn(codes, e)
    if w.dtype == np.float16:
        return w.astype(np.float64)
    return bf16_bits_to_f64(w)


def select(q_bits, k_bits, wq, wk, tile: int, query: Tuple[int, int],
           segments: Sequence[Tuple[int, int, int]], heads: Optional[Iterable[int]] = None):
    """O2..O6 for a whole layer.

    query = (start, length); segments = [(start, length, budget), ...] in call order.
    wq / wk: uint16 bf16 bits [H, p, d] or (E4M3 codes, pow2_exp).
    Returns (idx int32 [B, H, Tq, Ktot], scores float64 [B, H, Tq, sum T_s],
             q_hat [B, H, Tq, p], k_hat [B, H, sum T_s, p]).
    """
    B, N, H, d = q_bits.shape
    Wq = weights_f64(wq)
    Wk = weights_f64(wk)
    p = Wq.shape[1]
    Tq = -(-query[1] // tile)
    Ts = [-(-ln // tile) for (_, ln, _) in segments]
    Ks = [min(bud, T) for (_, _, bud), T in zip(segments, Ts)]
    Tk = sum(Ts)
    heads = list(range(H)) if heads is None else list(heads)
    idx = np.zeros((B, H, Tq, sum(Ks)), dtype=np.int32)
    S = np.zeros((B, H, Tq, Tk), dtype=np.float64)
    QH = np.zeros((B, H, Tq, p), dtype=np.float64)
    KH = np.zeros((B, H, Tk, p), dtype=np.float64)
    for b in range(B):
        for h in heads:
            idx[b, h], S[b, h], QH[b, h], KH[b, h] = select_head(q_bits, k_bits, Wq[h], Wk[h], b, h, tile,
                                                                query, segments)
    return idx, S, QH, KH


def select_head(q_bits, k_bits, wq_h: np.ndarray, wk_h: np.ndarray, b: int, h: int, tile: int,
                query: Tuple[int, int], segments: Sequence[Tuple[int, int, int]]):
    """O3..O6 for one (batch, head); wq_h / wk_h are that head's float64 [p, d] weights.
    Returns (idx int32 [Tq, Ktot], scores float64 [Tq, sum T_s], q_hat [Tq, p],
    k_hat [sum T_s, p])."""
    Tq = -(-query[1] // tile)
    Ts = [-(-ln // tile) for (_, ln, _) in segments]
    Ks = [min(bud, T) for (_, _, bud), T in zip(segments, Ts)]
    q_hat = project(pool_tiles(q_bits, b, h, query[0], query[1], tile), wq_h)
    k_hat = np.concatenate(
        [project(pool_tiles(k_bits, b, h, st, ln, tile), wk_h) for (st, ln, _) in segments], axis=0)
    s = tile_scores(q_hat, k_hat)
    idx = np.zeros((Tq, sum(Ks)), dtype=np.int32)
    col = 0
    kc = 0
    for (st, ln, bud), T, K in zip(segments, Ts, Ks):
        for i in range(Tq):
            idx[i, kc:kc + K] = topk_lowest_index(s[i, col:col + T], bud)
        col += T
        kc += K
    return idx, s, q_hat, k_hat


# ----------------------------------------------------------------------------- O7

def attended_tokens(idx_row: np.ndarray, tile: int, segments: Sequence[Tuple[int, int, int]],
                    dense: Sequence[Tuple[int, int]]) -> np.ndarray:
    """Token positions one query tile attends to: selected tiles of each segment,
    then every dense range.  Within a segment's block of entries, -1 marks padding:
    it and every later entry of that block select nothing (a library convention so
    that rows of different lengths share one width; the pages define no padding)."""
    toks = []
    kc = 0
    for (st, ln, bud) in segments:
        T = -(-ln // tile)
        K = min(bud, T)
        for j in idx_row[kc:kc + K]:
            j = int(j)
            if j == -1:          # padding: the rest of this segment's block is unused
                break
            if not (0 <= j < T):
                raise ValueError("tile index out of range")
            toks.append(np.arange(st + j * tile, st + min((j + 1) * tile, ln)))
        kc += K
    for (st, ln) in dense:
        toks.append(np.arange(st, st + ln))
    return np.concatenate(toks) if toks else np.zeros(0, dtype=np.int64)


def attend_rows(q_rows: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray,
                scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """O7 on explicit float64 rows: two-pass softmax(scale * q k^T) v and its log-sum-exp."""
    logits = scale * (q_rows @ k_rows.T)
    mu = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - mu)
    Z = w.sum(axis=1, keepdims=True)
    out = (w @ v_rows) / Z
    # self-check: normalised weights sum to one
    if not np.all(np.abs((w / Z).sum(axis=1) - 1.0) <= 1e-12):
        raise AssertionError("softmax rows do not sum to one")
    return out, (mu + np.log(Z))[:, 0]


def attend_tile(q_bits, k_bits, v_bits, b: int, h: int, qtile: int, idx_row: np.ndarray,
                tile: int, query: Tuple[int, int], segments, dense,
                scale: Optional[float] = None, dq=bf16_bits_to_f64, dk=bf16_bits_to_f64,
                dv=bf16_bits_to_f64):
    """O7 for one (batch, head, query tile): returns (out [t, d], lse [t]) in float64.
    dq / dk / dv turn stored Q / K / V elements into values (bf16 bits by default;
    fp8_values for E4M3FN codes)."""
    d = q_bits.shape[3]
    if scale is None or scale == 0.0:
        scale = 1.0 / math.sqrt(d)
    q0 = query[0] + qtile * tile
    q1 = query[0] + min((qtile + 1) * tile, query[1])
    toks = attended_tokens(idx_row, tile, segments, dense)
    if toks.size == 0:
        raise ValueError("query tile attends to no keys")
    qr = dq(q_bits[b, q0:q1, h, :])
    kr = dk(k_bits[b, toks, h, :])
    vr = dv(v_bits[b, toks, h, :])
    return attend_rows(qr, kr, vr, scale)


def attend_all_keys(q_bits, k_bits, v_bits, b: int, h: int, rows: Tuple[int, int], segments,
                    dense, scale: Optional[float] = None):
    """Dense attention of the query rows [start, start + len) over every token of every
    key segment and every dense range (the text / VLM / audio / reference query rows
    of a layer, whose attention stays dense).  Returns (out [len, d], lse [len])."""
    d = q_bits.shape[3]
    if scale is None or scale == 0.0:
        scale = 1.0 / math.sqrt(d)
    toks = np.concatenate([np.arange(st, st + ln) for (st, ln, _) in segments] +
                          [np.arange(st, st + ln) for (st, ln) in dense])
    qr = bf16_bits_to_f64(q_bits[b, rows[0]:rows[0] + rows[1], h, :])
    kr = bf16_bits_to_f64(k_bits[b, toks, h, :])
    vr = bf16_bits_to_f64(v_bits[b, toks, h, :])
    return attend_rows(qr, kr, vr, scale)


def attend(q_bits, k_bits, v_bits, idx: np.ndarray, tile: int, query: Tuple[int, int],
           segments, dense, scale: Optional[float] = None,
           pairs: Optional[Iterable[Tuple[int, int, int]]] = None,
           dq=bf16_bits_to_f64, dk=bf16_bits_to_f64, dv=bf16_bits_to_f64):
    """O7 over a layer, or over the (b, h, query tile) triples in `pairs` (dq / dk / dv as
    in attend_tile).

    Returns dict {(b, h, qtile): (out [t, d], lse [t])}.
    """
    B, N, H, d = q_bits.shape
    Tq = -(-query[1] // tile)
    if pairs is None:
        pairs = [(b, h, i) for b in range(B) for h in range(H) for i in range(Tq)]
    res = {}
    for (b, h, i) in pairs:
        res[(b, h, i)] = attend_tile(q_bits, k_bits, v_bits, b, h, i, idx[b, h, i], tile,
                                     query, segments, dense, scale, dq, dk, dv)
    return res


# ----------------------------------------------------------------------------- Q1, Q2

# codes 0x00 .. 0x7E: every non-negative finite E4M3FN value, in ascending order
_E4M3_MAGS = _E4M3_TABLE[:127]


def e4m3fn_round(x) -> np.ndarray:
    """Q1: the E4M3FN code nearest to each float64 value (by definition: the closest of
    the finite magnitudes; an exact tie goes to the even code, i.e. mantissa bit 0;
    magnitudes at or beyond 448 give 448).  The sign bit is x's, so -0.0 and negative
    values that round to zero give 0x80; NaN gives 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    hi = np.clip(np.searchsorted(_E4M3_MAGS, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = a - _E4M3_MAGS[lo]
    d_hi = _E4M3_MAGS[hi] - a
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    code = np.where(a >= 448.0, 126, code)
    code = code | np.where(np.signbit(x), 0x80, 0)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def fp8_scale_exponent(amax: float) -> int:
    """Q2: the smallest integer e with amax <= 448 * 2^e (0 for amax == 0)."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    e = math.frexp(amax)[1] - 10
    while 448.0 * 2.0 ** e < amax:
        e += 1
    return e


def quantize_fp8(x_bits: np.ndarray) -> Tuple[np.ndarray, int]:
    """Q2 on a bf16 tensor (all of it): (E4M3FN codes of x / 2^e, e)."""
    x = bf16_bits_to_f64(x_bits)
    e = fp8_scale_exponent(np.abs(x).max() if x.size else 0.0)
    return e4m3fn_round(x * 2.0 ** -e), e


def fp8_values(e: int):
    """Decoder for attend / attend_tile: E4M3FN codes times 2^e, as float64."""
    return lambda codes: dequant_e4m3fn(codes, e)


# ----------------------------------------------------------------------------- T1, T2

def block_mass(q_bits, k_bits, b: int, h: int, tile: int, query: Tuple[int, int], segments,
               dense, scale: Optional[float] = None, qtiles: Optional[Sequence[int]] = None):
    """T1 for one (batch, head): every key of every segment and dense range is attended.

    For query tile i with rows n and P_n = softmax over all keys of scale * q_n . k:
        mass[i, j]    = (1 / rows_i) * sum_n sum_{m in key tile j} P_n(m)
        dense_mass[i] = (1 / rows_i) * sum_n sum_{m in dense ranges} P_n(m)
    Key tile columns run over the segments in order (segment s from sum_{t<s} T_t).
    Returns (mass [len(qtiles), Tk], dense_mass [len(qtiles)], lse {qtile: [rows]}).
    """
    d = q_bits.shape[3]
    if scale is None or scale == 0.0:
        scale = 1.0 / math.sqrt(d)
    toks, cols = [], []
    toff = 0
    for (st, ln, _bud) in segments:
        t = np.arange(st, st + ln)
        toks.append(t)
        cols.append(toff + (t - st) // tile)
        toff += -(-ln // tile)
    Tk = toff
    for (st, ln) in dense:
        toks.append(np.arange(st, st + ln))
        cols.append(np.full(ln, -1))
    toks = np.concatenate(toks)
    cols = np.concatenate(cols)
    seg_keys = cols >= 0
    kr = bf16_bits_to_f64(k_bits[b, toks, h, :])
    Tq = -(-query[1] // tile)
    qtiles = list(range(Tq)) if qtiles is None else list(qtiles)
    mass = np.zeros((len(qtiles), Tk))
    dmass = np.zeros(len(qtiles))
    lses = {}
    for r, i in enumerate(qtiles):
        q0 = query[0] + i * tile
        q1 = query[0] + min((i + 1) * tile, query[1])
        qr = bf16_bits_to_f64(q_bits[b, q0:q1, h, :])
        logits = scale * (qr @ kr.T)
        mx = logits.max(axis=1, keepdims=True)
        lse = mx[:, 0] + np.log(np.exp(logits - mx).sum(axis=1))
        p = np.exp(logits - lse[:, None])
        per_key = p.sum(axis=0) / (q1 - q0)
        mass[r] = np.bincount(cols[seg_keys], weights=per_key[seg_keys], minlength=Tk)
        dmass[r] = per_key[~seg_keys].sum()
        lses[i] = lse
    return mass, dmass, lses


def block_recall(mass_row: np.ndarray, idx_row: np.ndarray, tile: int, segments) -> float:
    """T2: mass of the tiles idx_row selects (segment blocks in order, a -1 ends its
    block) over the mass of every segment tile; 1 when that total is 0."""
    sel = 0.0
    kc = toff = 0
    for (st, ln, bud) in segments:
        T = -(-ln // tile)
        K = min(bud, T)
        for j in idx_row[kc:kc + K]:
            j = int(j)
            if j == -1:
                break
            sel += mass_row[toff + j]
        kc += K
        toff += T
    tot = float(mass_row.sum())
    return sel / tot if tot > 0 else 1.0


# ----------------------------------------------------------------------------- P1

def window_frame_mask(n_frames: int, chunk_frames: int, halo_chunks: int,
                      anchors: bool) -> np.ndarray:
    """P1 at frame level: bool [F, F], entry (i, j) true when query frame i attends
    key frame j.  Frames fall in chunks of chunk_frames consecutive frames; a chunk
    attends itself and halo_chunks chunks on each side.  With anchors, every frame
    also attends the first and the last frame, and those two attend every frame."""
    if n_frames < 1 or chunk_frames < 1 or halo_chunks < 0:
        raise ValueError("bad window pattern")
    chunk = np.arange(n_frames) // chunk_frames
    m = np.abs(chunk[:, None] - chunk[None, :]) <= halo_chunks
    if anchors:
        m[:, 0] = m[:, -1] = True
        m[0, :] = m[-1, :] = True
    return m


def window_tile_rows(seg_len: int, tile: int, frame_tokens: int, chunk_frames: int,
                     halo_chunks: int, anchors: bool) -> List[np.ndarray]:
    """P1 at tile granularity over one segment that is both the queries and the keys:
    for each query tile, the ascending key tiles it takes.  A tile overlaps the
    frames its tokens belong to; query tile a takes key tile b when a frame of a
    attends a frame of b (integer matrix product of the overlap relations)."""
    F = -(-seg_len // frame_tokens)
    T = -(-seg_len // tile)
    over = np.zeros((T, F), dtype=np.int64)           # tile t overlaps frame f
    for t, (lo, hi) in enumerate(tile_bounds(0, seg_len, tile)):
        over[t, lo // frame_tokens:(hi - 1) // frame_tokens + 1] = 1
    m = window_frame_mask(F, chunk_frames, halo_chunks, anchors).astype(np.int64)
    take = (over @ m @ over.T) > 0
    return [np.flatnonzero(take[t]).astype(np.int32) for t in range(T)]


def window_indices(rows: Sequence[np.ndarray], width: Optional[int] = None) -> np.ndarray:
    """Rows of P1 as one int32 [Tq, width] array, each row ascending then -1."""
    width = max(len(r) for r in rows) if width is None else width
    out = np.full((len(rows), width), -1, dtype=np.int32)
    for t, r in enumerate(rows):
        if len(r) > width:
            raise ValueError("row longer than width")
        out[t, :len(r)] = r
    return out
