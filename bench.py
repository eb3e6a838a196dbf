"""Benchmark of one Veda block-sparse attention layer on one MI355X.

A step is the whole hot path for one layer: veda_select (tile pooling +
projection, pooled scores + per-segment top-k) followed by veda_sparse_attn
(block-sparse attention over the selected tiles and the dense key ranges).
Inputs are seeded synthetic tensors already resident in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload t2v5s]

Prints one JSON line.  `value` is the dense-equivalent attention TFLOP/s of the
whole step (4*B*H*Nq*Nk_all*d / (selector + attention time)).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dense-equiv attention TFLOP/s + selector+attn ms/layer at 90/95% sparsity"
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="t2v5s")
    ap.add_argument("--also", default="mid", help="second workload reported beside (or 'none')")
    ap.add_argument("--dense-reps", type=int, default=0,
                    help="reps of the dense baselines (0: 10, or 5 for layers above 200k tokens)")
    ap.add_argument("--kernel-reps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip timing selection + attention on every workload (field 'sweep')")
    ap.add_argument("--no-patterns", action="store_true",
                    help="skip the budget 16/32/64 and VDN window timings (field 'patterns')")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the FP8 paths' timing (fields 'fp8qk' and 'fp8')")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 1 GiB device copy first (byte-counter calibration)")
    ap.add_argument("--seed", type=int, default=None,
                    help="input seed for every workload (default: each workload's own index)")
    ap.add_argument("--record", default=None, metavar="FILE",
                    help="also append the JSON line, with a UTC time stamp, to FILE (JSON Lines, one record "
                         "per run; existing records are never rewritten)")
    return ap.parse_args(argv)


SEED = None   # --seed: replaces every workload's input seed


def workload(name):
    """The named workload, with its input seed replaced when --seed is given."""
    import dataclasses
    from block_sparse_attention_predictor_amd import inputs as I
    wl = I.WORKLOADS[name]
    return wl if SEED is None else dataclasses.replace(wl, index=SEED)


def append_record(path: str, line: dict) -> None:
    """Append one run's record to a JSON Lines file, as a single write of one line."""
    rec = dict(line)
    rec["recorded_at"] = time.strftime("%Y-%m-%dT%H:%M:%SZ", time.gmtime())
    data = (json.dumps(rec) + "\n").encode()
    fd = os.open(path, os.O_WRONLY | os.O_APPEND | os.O_CREAT, 0o644)
    try:
        os.write(fd, data)
    finally:
        os.close(fd)


def attended_tokens_per_tile(wl, idx: np.ndarray, widths=None) -> np.ndarray:
    """Real key tokens each (b, h, query tile) attends to, from the index sets used
    (a -1 entry ends its segment's block).  widths: index columns per segment."""
    total = np.zeros(idx.shape[:-1], dtype=np.int64)
    col = 0
    for si, s in enumerate(wl.segments):
        T = wl.seg_tiles(s)
        tl = np.full(T, wl.tile, dtype=np.int64)
        tl[-1] = s.length - (T - 1) * wl.tile
        K = widths[si] if widths is not None else min(s.budget, T)
        blk = idx[..., col:col + K]
        live = np.cumprod(blk >= 0, axis=-1).astype(bool)
        total += np.where(live, tl[np.where(live, blk, 0)], 0).sum(-1)
        col += K
    return total + sum(r.length for r in wl.dense)


def query_rows_per_tile(wl) -> np.ndarray:
    rows = np.full(wl.n_query_tiles, wl.tile, dtype=np.int64)
    rows[-1] = wl.query.length - (wl.n_query_tiles - 1) * wl.tile
    return rows


class Layer:
    """Device-resident inputs of one workload plus the calls of one step."""

    def __init__(self, name):
        import torch
        from block_sparse_attention_predictor_amd import binding as B
        from block_sparse_attention_predictor_amd import inputs as I
        self.B = B
        self.I = I
        self.wl = wl = workload(name)
        self.q, self.k, self.v = I.make_qkv(wl)
        self.w = I.make_weights(wl)
        dev = torch.device("cuda:0")

        def up(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

        self.qd, self.kd, self.vd = up(self.q), up(self.k), up(self.v)
        if self.w.fp8:
            # load-time step: FP8 predictor -> bf16 on the GPU
            self.wq = B.dequant_fp8_e4m3(torch.from_numpy(self.w.wq).to(dev), self.w.pow2_exp)
            self.wk = B.dequant_fp8_e4m3(torch.from_numpy(self.w.wk).to(dev), self.w.pow2_exp)
        else:
            self.wq, self.wk = up(self.w.wq), up(self.w.wk)
        self.L = B.layer_from_workload(wl)
        self.dense = [(r.start, r.length) for r in wl.dense]
        self.idx = torch.empty((wl.B, wl.H, wl.n_query_tiles, wl.k_total), dtype=torch.int32, device=dev)
        self.order = torch.empty((wl.B, wl.H, wl.n_query_tiles), dtype=torch.int32, device=dev)
        self.ws = torch.empty(B.select_workspace_bytes(self.L) + 256, dtype=torch.uint8, device=dev)
        self.out = torch.zeros_like(self.qd)
        torch.cuda.synchronize()

    def select(self):
        """The selection and the processing order of its query tiles (veda_tile_order)."""
        self.B.select(self.L, self.qd, self.kd, self.wq, self.wk, workspace=self.ws, idx=self.idx)
        self.B.tile_order(self.L, self.idx, out=self.order)

    def attn(self, idx=None, L=None, order=None):
        """Attention over the selection in its processing order, or over other index sets (in
        the order given, else the natural one)."""
        self.B.sparse_attn(L or self.L, self.qd, self.kd, self.vd, self.idx if idx is None else idx,
                           self.dense, out=self.out, order=self.order if idx is None else order)

    def step(self):
        self.select()
        self.attn()

    def dense_queries(self):
        """Every non-video query row (reference image, text, VLM, audio) attends densely."""
        wl = self.wl
        return ([(s.start, s.length) for s in wl.segments if s.name != "video"] +
                [(r.start, r.length) for r in wl.dense])

    def full_layer(self):
        self.B.layer_attn(self.L, self.qd, self.kd, self.vd, self.wq, self.wk, self.dense,
                          self.dense_queries(), out=self.out, idx=self.idx, workspace=self.ws)

    def dense_query_flops(self):
        wl = self.wl
        nk_all = sum(s.length for s in wl.segments) + sum(r.length for r in wl.dense)
        return 4.0 * wl.B * wl.H * sum(n for _, n in self.dense_queries()) * nk_all * wl.d

    def dense_flops(self):
        wl = self.wl
        nk_all = sum(s.length for s in wl.segments) + sum(r.length for r in wl.dense)
        return 4.0 * wl.B * wl.H * wl.query.length * nk_all * wl.d

    def actual_flops(self, idx_np, widths=None):
        per_tile = attended_tokens_per_tile(self.wl, idx_np, widths)  # [B, H, Tq]
        rows = query_rows_per_tile(self.wl)
        return 4.0 * self.wl.d * float((per_tile * rows[None, None, :]).sum())

    def full_budget_layer(self):
        full = self.I.with_full_budget(self.wl)
        return self.B.layer_from_workload(full), full


def time_events(fn, reps):
    import torch
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(reps):
        s.record()
        fn()
        e.record()
        e.synchronize()
        times.append(s.elapsed_time(e))
    return float(np.mean(times)), float(np.min(times)), float(np.median(times))


def index_stats(wl, idx_np):
    """Selection statistics per head (video segment): mean Jaccard overlap of neighbouring
    query tiles' index sets, and the number of distinct key tiles a head selects."""
    col = 0
    for s in wl.segments:
        K = min(s.budget, wl.seg_tiles(s))
        if s.name == "video":
            break
        col += K
    sel = idx_np[0, :, :, col:col + K]                     # [H, Tq, K]
    H, Tq, _ = sel.shape
    T = wl.seg_tiles([s for s in wl.segments if s.name == "video"][0])
    onehot = np.zeros((H, Tq, T), dtype=bool)
    np.put_along_axis(onehot, sel.astype(np.int64), True, axis=-1)
    inter = (onehot[:, 1:] & onehot[:, :-1]).sum(-1)
    union = (onehot[:, 1:] | onehot[:, :-1]).sum(-1)
    jac = (inter / np.maximum(union, 1)).mean(axis=1)     # [H]
    distinct = onehot.any(axis=1).sum(-1)                  # [H]
    return {"jaccard_neighbour_mean": round(float(jac.mean()), 4),
            "jaccard_neighbour_min_head": round(float(jac.min()), 4),
            "distinct_tiles_per_head_mean": round(float(distinct.mean()), 1), "tiles": int(T)}


def device_peaks(log):
    """What this device reaches on an MFMA-only loop and on a plain 1 GiB copy."""
    import torch
    from block_sparse_attention_predictor_amd import probe
    probe.mfma_peak(50, 2048)
    torch.cuda.synchronize()
    ms, _, _ = time_events(lambda: probe.mfma_peak(2000, 2048), 3)
    _, flops = probe.mfma_peak(1, 1)
    flops *= 2000 * 2048
    n = 1 << 29
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    cms, _, _ = time_events(lambda: dst.copy_(src), 5)
    del src, dst
    out = {"mfma_bf16_tflops": round(flops / (ms * 1e-3) / 1e12, 1),
           "copy_gbs": round(2.0 * n * 2 / (cms * 1e-3) / 1e9, 1)}
    log(f"device peaks: {out}")
    return out


def environment():
    """Device and software versions.  No other program is started from this process once it
    has used the GPU; the clock under load comes from the hardware counters in profiles/."""
    import platform
    import torch
    p = torch.cuda.get_device_properties(0)
    env = {"device": p.name, "arch": getattr(p, "gcnArchName", ""), "cus": p.multi_processor_count,
           "hip": torch.version.hip, "torch": torch.__version__, "host": platform.node(),
           "host_cpus": len(os.sched_getaffinity(0))}
    try:
        env["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        env["rocm"] = None
    return env


def copy_calibration():
    """A plain device copy of known size (1 GiB read + 1 GiB written), run once so that
    hardware byte counters can be scaled against it in a profiled run."""
    import torch
    n = 1 << 29                                   # bf16 elements = 1 GiB
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


FLUSH_BYTES = 512 << 20   # written before every cold step: more than the Infinity Cache and every L2


def timed_steps(lay, steps, flush=None):
    """K steps, each bracketed by events on the launch stream: e0 | select | e1 | attention | e2.
    With `flush`, a 512 MiB device write runs before every step, outside the events, so each
    step starts with cold caches.  Returns (step_ms, select_ms, attn_ms, wall_s) lists."""
    import torch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if flush is not None:
            flush.fill_(1.0)
        ev[i][0].record()
        lay.select()
        ev[i][1].record()
        lay.attn()
        ev[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sel = [a.elapsed_time(b) for a, b, _ in ev]
    att = [b.elapsed_time(c) for _, b, c in ev]
    return [x + y for x, y in zip(sel, att)], sel, att, wall


def measure(name, steps, warmup, kernel_reps, dense_reps, with_dense, log):
    """One workload.  The headline figures are cold: every step starts after a 512 MiB write
    that evicts the Infinity Cache and the L2s, as a layer of a model does after the layers
    before it; the same K steps run back to back (warm) are reported beside them."""
    import torch
    lay = Layer(name)
    wl = lay.wl
    for _ in range(warmup):
        lay.step()
    torch.cuda.synchronize()
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=lay.qd.device)
    log(f"[{name}] timing {steps} cold steps")
    step_ms, sel_ms, att_ms, wall = timed_steps(lay, steps, flush)
    del flush
    log(f"[{name}] timing {steps} warm steps")
    w_step, w_sel, w_att, w_wall = timed_steps(lay, steps)
    ms_step = float(np.mean(step_ms))
    sel_mean, sel_min = float(np.mean(sel_ms)), float(np.min(sel_ms))
    att_mean, att_min = float(np.mean(att_ms)), float(np.min(att_ms))
    idx_np = lay.idx.cpu().numpy()
    flops_actual = lay.actual_flops(idx_np)
    flops_dense = lay.dense_flops()
    res = {
        "workload": name, "ms_per_step": ms_step, "wall_s": wall,
        "selector_ms": sel_mean, "attn_ms": att_mean, "selector_ms_min": sel_min, "attn_ms_min": att_min,
        "dense_equiv_tflops_step": flops_dense / (ms_step * 1e-3) / 1e12,
        "dense_equiv_tflops_attn": flops_dense / (att_mean * 1e-3) / 1e12,
        "actual_tflops_attn": flops_actual / (att_mean * 1e-3) / 1e12,
        "actual_attn_tflop": flops_actual / 1e12, "dense_equiv_tflop": flops_dense / 1e12,
        "sparsity_actual": 1.0 - flops_actual / flops_dense,
        "selector_ms_median": float(np.median(sel_ms)), "attn_ms_median": float(np.median(att_ms)),
        "ms_per_step_median": float(np.median(step_ms)),
        "warm": {"ms_per_step": float(np.mean(w_step)), "ms_per_step_median": float(np.median(w_step)),
                 "selector_ms": float(np.mean(w_sel)), "attn_ms": float(np.mean(w_att)),
                 "attn_ms_median": float(np.median(w_att)), "attn_ms_min": float(np.min(w_att)),
                 "actual_tflops_attn": flops_actual / (float(np.mean(w_att)) * 1e-3) / 1e12,
                 "dense_equiv_tflops_step": flops_dense / (float(np.mean(w_step)) * 1e-3) / 1e12,
                 "wall_s": w_wall},
    }
    # one full layer as the model runs it: also the dense (non-video) query rows
    lay.full_layer()
    torch.cuda.synchronize()
    fl_mean, fl_min, _ = time_events(lay.full_layer, max(3, kernel_reps // 2))
    res["full_layer_ms"] = fl_mean
    res["dense_query_rows"] = sum(n for _, n in lay.dense_queries())
    res["dense_query_tflop"] = lay.dense_query_flops() / 1e12
    # pooling bandwidth: Q rows of the query segment + K rows of every key segment, once
    pool_bytes = 2.0 * wl.B * wl.H * wl.d * (wl.query.length + sum(sg.length for sg in wl.segments))
    res["pool_bytes"] = pool_bytes
    # the pooling pass alone (pool + project kernel), median of kernel_reps for both figures
    _, _, pool_med = time_events(lambda: lay.B.project(lay.L, lay.qd, lay.kd, lay.wq, lay.wk), kernel_reps)
    res["pool_ms"] = pool_med
    res["pool_gbs"] = pool_bytes / (pool_med * 1e-3) / 1e9
    # the processing-order kernel alone (part of selector_ms), median of kernel_reps
    _, _, order_med = time_events(lambda: lay.B.tile_order(lay.L, lay.idx, out=lay.order), kernel_reps)
    res["order_ms"] = order_med
    res["index_stats"] = index_stats(wl, idx_np)
    if with_dense:
        Lf, wlf = lay.full_budget_layer()
        idx_full = torch.from_numpy(lay.I.full_indices(wl)).to(lay.qd.device)
        lay.attn(idx_full, Lf)
        torch.cuda.synchronize()
        reps = dense_reps if dense_reps > 0 else (5 if wl.n_tokens > 200_000 else 10)
        log(f"[{name}] dense baseline (every tile selected), {reps} reps")
        d_mean, d_min, _ = time_events(lambda: lay.attn(idx_full, Lf), reps)
        res["dense_reps"] = reps
        res["dense_ms"] = d_mean
        res["dense_tflops"] = flops_dense / (d_mean * 1e-3) / 1e12
        res["speedup_vs_dense"] = d_mean / ms_step
        del idx_full
        res["sdpa_dense"] = sdpa_dense(lay, reps, log)
        if "ms_median" in res["sdpa_dense"]:
            # the speedup is claimed against the faster of the two dense baselines
            res["speedup_vs_fastest_dense"] = min(d_mean, res["sdpa_dense"]["ms_median"]) / ms_step
    return lay, res


def measure_patterns(lay, kernel_reps, log):
    """Other index producers through the same attention kernel: the learned selector at
    top-k budgets 16 / 32 / 64 per key segment, and the fixed VDN window pattern
    (chunks of five latent frames, one neighbour chunk each side, boundary anchors);
    each with its recall of the teacher block attention mass (random predictor
    weights: the recall figures measure the pipeline, not a trained selector)."""
    import torch
    wl, B, I = lay.wl, lay.B, lay.I
    dev = lay.qd.device
    flops_dense = lay.dense_flops()
    out = {}
    # teacher block attention mass (dense lse pass + per-tile mass pass over all keys)
    mass, _, _ = B.block_mass(lay.L, lay.qd, lay.kd, lay.dense)
    torch.cuda.synchronize()
    log(f"[{wl.name}] teacher block mass")
    t_ms, _, _ = time_events(lambda: B.block_mass(lay.L, lay.qd, lay.kd, lay.dense), max(2, kernel_reps // 4))
    teacher_flops = 2 * 2.0 * wl.B * wl.H * wl.query.length * wl.d * \
        (sum(sg.length for sg in wl.segments) + sum(r.length for r in wl.dense))
    rec = B.block_recall(lay.L, mass, lay.idx)
    r_ms, _, _ = time_events(lambda: B.block_recall(lay.L, mass, lay.idx), kernel_reps)
    out["teacher"] = {"mass_ms": round(t_ms, 3), "tflops": round(teacher_flops / (t_ms * 1e-3) / 1e12, 1),
                      "recall_ms": round(r_ms, 4), "recall_selector": round(float(rec.mean()), 4)}

    def recall_of(L, idx):
        return round(float(B.block_recall(L, mass, idx).mean()), 4)

    for k in (16, 32, 64):
        wk = I.with_budget(wl, k)
        Lk = B.layer_from_workload(wk)
        idx = torch.empty((wl.B, wl.H, wl.n_query_tiles, wk.k_total), dtype=torch.int32, device=dev)
        ws = torch.empty(B.select_workspace_bytes(Lk) + 256, dtype=torch.uint8, device=dev)

        def sel(Lk=Lk, idx=idx, ws=ws):
            B.select(Lk, lay.qd, lay.kd, lay.wq, lay.wk, workspace=ws, idx=idx)

        sel()
        order = B.tile_order(Lk, idx)           # the step's configuration: the selection's tile order
        torch.cuda.synchronize()
        log(f"[{wl.name}] budget {k}")
        s_ms, _, _ = time_events(sel, kernel_reps)
        a_ms, _, _ = time_events(lambda: lay.attn(idx, Lk, order), kernel_reps)
        fl = lay.actual_flops(idx.cpu().numpy(), [min(k, wl.seg_tiles(sg)) for sg in wl.segments])
        out[f"budget_{k}"] = {"selector_ms": round(s_ms, 4), "attn_ms": round(a_ms, 4),
                              "density": round(fl / flops_dense, 4),
                              "actual_tflops_attn": round(fl / (a_ms * 1e-3) / 1e12, 1),
                              "recall": recall_of(Lk, idx)}
        del idx, ws, order
    video = [s for s in wl.segments if s.name == "video"]
    if len(wl.segments) == 1 and video and video[0].start == wl.query.start \
            and video[0].length == wl.query.length:
        ft = wl.grid[1] * wl.grid[2]

        def win():
            return B.window_indices(lay.L, ft, 5, 1, True)

        idx, Lw = win()
        torch.cuda.synchronize()
        log(f"[{wl.name}] VDN window pattern, width {Lw.budget[0]}")
        p_ms, _, _ = time_events(win, kernel_reps)
        reps = max(2, kernel_reps // 4)
        a_ms, _, _ = time_events(lambda: lay.attn(idx, Lw), reps)
        fl = lay.actual_flops(idx.cpu().numpy(), [int(Lw.budget[0])])
        out["vdn_window"] = {"chunk_frames": 5, "halo_chunks": 1, "anchors": True,
                             "width": int(Lw.budget[0]), "indices_ms": round(p_ms, 4),
                             "attn_ms": round(a_ms, 4), "density": round(fl / flops_dense, 4),
                             "actual_tflops_attn": round(fl / (a_ms * 1e-3) / 1e12, 1),
                             "recall": recall_of(Lw, idx)}
        del idx
    del mass
    torch.cuda.synchronize()
    return out


def random_pattern(lay, kernel_reps, log):
    """Uniformly random index sets of the same budgets, in the natural tile order: the worst
    case for K/V reuse."""
    import torch
    wl = lay.wl
    idx = torch.from_numpy(lay.I.random_indices(wl)).to(lay.qd.device)
    lay.attn(idx)
    torch.cuda.synchronize()
    ms, _, med = time_events(lambda: lay.attn(idx), kernel_reps)
    fl = lay.actual_flops(idx.cpu().numpy())
    log(f"[{wl.name}] random index sets: {med:.3f} ms")
    return {"attn_ms": round(ms, 4), "attn_ms_median": round(med, 4),
            "actual_tflops_attn": round(fl / (med * 1e-3) / 1e12, 1)}


def measure_fp8(lay, kernel_reps, log):
    """The two FP8 paths on the same layer and index sets, Q and K quantised on the GPU
    (E4M3FN, per-tensor power-of-two scale):
      * fp8qk: veda_sparse_attn_fp8qk, FP8 first product, bf16 P.V.  Its peak is the
        harmonic mean of the FP8 and bf16 rates (equal flops in each product);
      * fp8: veda_sparse_attn_fp8, V quantised to the blocked FP8 layout and P rounded to
        E4M3FN, both products at the FP8 rate."""
    import torch
    B, wl = lay.B, lay.wl
    q8, qs = B.quantize_fp8(lay.L, lay.qd)
    k8, ks = B.quantize_fp8(lay.L, lay.kd)
    vt, vs = B.quantize_fp8_vt(lay.L, lay.vd)
    out8 = torch.zeros_like(lay.qd)
    out8v = torch.zeros_like(lay.qd)

    def quant():
        B.quantize_fp8(lay.L, lay.qd, out=q8, scale=qs)
        B.quantize_fp8(lay.L, lay.kd, out=k8, scale=ks)

    def quant_v():
        B.quantize_fp8_vt(lay.L, lay.vd, out=vt, scale=vs)

    def attn8():
        B.sparse_attn_fp8qk(lay.L, q8, k8, lay.vd, qs, ks, lay.idx, lay.dense, out=out8, order=lay.order)

    def attn8v():
        B.sparse_attn_fp8(lay.L, q8, k8, vt, qs, ks, vs, lay.idx, lay.dense, out=out8v, order=lay.order)

    lay.select()
    lay.attn()
    quant()
    quant_v()
    attn8()
    attn8v()
    torch.cuda.synchronize()
    q_ms, _, q_med = time_events(quant, kernel_reps)
    qv_ms, _, qv_med = time_events(quant_v, kernel_reps)
    a_ms, a_min, a_med = time_events(attn8, kernel_reps)
    v_ms, v_min, v_med = time_events(attn8v, kernel_reps)
    fl = lay.actual_flops(lay.idx.cpu().numpy())
    q0, q1 = wl.query.start, wl.query.start + wl.query.length
    diff = (out8[:, q0:q1].float() - lay.out[:, q0:q1].float()).abs()
    diffv = (out8v[:, q0:q1].float() - lay.out[:, q0:q1].float()).abs()
    mixed_peak = 2.0 / (1.0 / PEAK_FP8_TFLOPS + 1.0 / PEAK_BF16_TFLOPS)
    tf = fl / (a_med * 1e-3) / 1e12
    tfv = fl / (v_med * 1e-3) / 1e12
    log(f"[{wl.name}] fp8 Q.K^T attention: {a_med:.3f} ms ({tf:.0f} TFLOP/s), quantising Q and K {q_med:.3f} ms")
    log(f"[{wl.name}] fp8 Q.K^T + P.V attention: {v_med:.3f} ms ({tfv:.0f} TFLOP/s), quantising V {qv_med:.3f} ms")
    res = {"attn_ms": round(a_ms, 4), "attn_ms_median": round(a_med, 4), "attn_ms_min": round(a_min, 4),
           "quantize_qk_ms": round(q_med, 4), "actual_tflops_attn": round(tf, 1),
           "mixed_peak_tflops": round(mixed_peak, 1), "frac_mixed_peak": round(tf / mixed_peak, 4),
           "speedup_vs_bf16_attn": None,
           "max_abs_vs_bf16_out": round(float(diff.max()), 5), "mean_abs_vs_bf16_out": round(float(diff.mean()), 6),
           "kernel": f"sparse_attn_fp8qk_pingpong_kernel<{wl.d}>"}
    resv = {"attn_ms": round(v_ms, 4), "attn_ms_median": round(v_med, 4), "attn_ms_min": round(v_min, 4),
            "quantize_qk_ms": round(q_med, 4), "quantize_v_ms": round(qv_med, 4),
            "actual_tflops_attn": round(tfv, 1), "peak_tflops": PEAK_FP8_TFLOPS,
            "frac_fp8_peak": round(tfv / PEAK_FP8_TFLOPS, 4), "speedup_vs_bf16_attn": None,
            "speedup_vs_fp8qk_attn": round(a_med / v_med, 3),
            "max_abs_vs_bf16_out": round(float(diffv.max()), 5),
            "mean_abs_vs_bf16_out": round(float(diffv.mean()), 6),
            "kernel": f"sparse_attn_fp8_pingpong_kernel<{wl.d}>"}
    del out8, out8v

    def attn8_with(idx, order=None):
        """Both FP8 paths of this layer with the given index sets (for the parity leg)."""
        return {"fp8qk": B.sparse_attn_fp8qk(lay.L, q8, k8, lay.vd, qs, ks, idx, lay.dense, order=order),
                "fp8": B.sparse_attn_fp8(lay.L, q8, k8, vt, qs, ks, vs, idx, lay.dense, order=order)}

    return res, resv, attn8_with


def sdpa_dense(lay, reps, log):
    """torch's scaled_dot_product_attention (flash / memory-efficient backends only) at the
    dense shape of the layer, every token a key: context for the dense baseline."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel
    wl = lay.wl
    q0, nq = wl.query.start, wl.query.length
    try:
        qh = lay.qd[:, q0:q0 + nq].transpose(1, 2).contiguous()
        kh = lay.kd.transpose(1, 2).contiguous()
        vh = lay.vd.transpose(1, 2).contiguous()
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
            torch.nn.functional.scaled_dot_product_attention(qh, kh, vh)
            torch.cuda.synchronize()
            ms, _, med = time_events(lambda: torch.nn.functional.scaled_dot_product_attention(qh, kh, vh), reps)
        del qh, kh, vh
        flops = 4.0 * wl.B * wl.H * nq * wl.n_tokens * wl.d
        log(f"[{wl.name}] torch SDPA dense: {med:.1f} ms")
        return {"ms": round(ms, 3), "ms_median": round(med, 3), "tflops": round(flops / (med * 1e-3) / 1e12, 1)}
    except Exception as e:   # a backend missing on this build is reported, not fatal
        return {"error": f"{type(e).__name__}: {str(e)[:200]}"}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


SCORE_RTOL = 1e-4                 # row-normwise pooled-score bar; also the tie window
ATTN_MAX_ABS, ATTN_MEAN_ABS = 1e-2, 1e-3


def selection_parity(idx_gpu, sc_gpu, idx_ref, S_ref, seg_T, seg_K):
    """Compare one head's GPU selection [Tq, Ktot] / scores [Tq, Tk] with the oracle's.
    Returns (worst row-normwise score error, rows differing, rows differing outside the
    tie window: a tile whose oracle score lies within SCORE_RTOL * max|s| of the k-th
    score of its segment may go either way; every GPU row must also be a valid list)."""
    scale = np.maximum(np.abs(S_ref).max(axis=-1), 1e-300)
    err = float((np.abs(sc_gpu.astype(np.float64) - S_ref).max(axis=-1) / scale).max())
    differ = np.nonzero(~np.all(idx_gpu == idx_ref, axis=-1))[0]
    outside = 0
    for r in differ:
        col, kc, bad = 0, 0, False
        for T, K in zip(seg_T, seg_K):
            g, o = idx_gpu[r, kc:kc + K], idx_ref[r, kc:kc + K]
            if not np.array_equal(g, o):
                s = S_ref[r, col:col + T]
                kth = np.sort(s)[::-1][K - 1]
                amb = set(np.nonzero(np.abs(s - kth) <= SCORE_RTOL * scale[r])[0].tolist())
                valid = np.all(np.diff(g) > 0) and g.min() >= 0 and g.max() < T
                bad |= (not valid) or (set(g.tolist()) - amb != set(o.tolist()) - amb)
            col += T
            kc += K
        outside += int(bad)
    return err, int(differ.size), outside


def cpu_baseline(lay, log, budget_s=20.0, attn8_with=None):
    """The fp64 oracle on the same layer, timed on the host cores: selection of every head
    (every row), then attention on random (head, query tile) pairs for about 2/3 of
    budget_s, extrapolated to the whole layer.  Its results are compared with the GPU's
    in the same run: the GPU's scores and index sets of every head, and the GPU's attention
    fed the oracle's index sets on the sampled pairs."""
    import torch
    from oracle import veda_oracle as O
    wl = lay.wl
    segs = [(s.start, s.length, s.budget) for s in wl.segments]
    query = (wl.query.start, wl.query.length)
    dense = [(r.start, r.length) for r in wl.dense]
    seg_T = [wl.seg_tiles(s) for s in wl.segments]
    seg_K = [min(s.budget, T) for s, T in zip(wl.segments, seg_T)]
    if lay.w.fp8:
        wq = (lay.w.wq, lay.w.pow2_exp)
        wk = (lay.w.wk, lay.w.pow2_exp)
    else:
        wq, wk = lay.w.wq, lay.w.wk
    Wq, Wk = O.weights_f64(wq), O.weights_f64(wk)
    # GPU selection with scores, outside every timed region
    idx_gpu, sc_gpu = lay.B.select(lay.L, lay.qd, lay.kd, lay.wq, lay.wk, want_scores=True)
    idx_gpu = idx_gpu.cpu().numpy()
    sc_gpu = sc_gpu.cpu().numpy()
    torch.cuda.synchronize()
    # oracle selection, every head
    idx_ref = np.zeros_like(idx_gpu)
    t_sel, score_err, rows_differ, rows_outside = 0.0, 0.0, 0, 0
    log(f"[cpu] oracle selection of {wl.B * wl.H} heads")
    for b in range(wl.B):
        for h in range(wl.H):
            t0 = time.perf_counter()
            r, S, _, _ = O.select_head(lay.q, lay.k, Wq[h], Wk[h], b, h, wl.tile, query, segs)
            t_sel += time.perf_counter() - t0
            idx_ref[b, h] = r
            e, dif, out_ = selection_parity(idx_gpu[b, h], sc_gpu[b, h], r, S, seg_T, seg_K)
            score_err = max(score_err, e)
            rows_differ += dif
            rows_outside += out_
    del sc_gpu
    # GPU attention fed the oracle's index sets (and the FP8 Q.K^T path, if given, likewise)
    # (in their processing order, as the timed step runs)
    idx_ref_dev = torch.from_numpy(idx_ref).to(lay.qd.device)
    order_ref = lay.B.tile_order(lay.L, idx_ref_dev)
    out_gpu = lay.B.sparse_attn(lay.L, lay.qd, lay.kd, lay.vd, idx_ref_dev, lay.dense, order=order_ref)
    out8 = attn8_with(idx_ref_dev, order_ref) if attn8_with is not None else {}
    del idx_ref_dev, order_ref
    torch.cuda.synchronize()
    # oracle attention on random (head, tile) pairs until the budget is used
    rng = np.random.default_rng(0)
    pairs, t_att = [], 0.0
    diffs, diffs8 = [], {name: [] for name in out8}
    Tq = wl.n_query_tiles
    while t_att < budget_s * 2 / 3 and len(pairs) < wl.B * wl.H * Tq:
        pr = (int(rng.integers(0, wl.B)), int(rng.integers(0, wl.H)), int(rng.integers(0, Tq)))
        t0 = time.perf_counter()
        res = O.attend(lay.q, lay.k, lay.v, idx_ref, wl.tile, query, segs, dense, pairs=[pr])
        t_att += time.perf_counter() - t0
        pairs.append(pr)
        ref = res[pr][0]
        r0 = wl.query.start + pr[2] * wl.tile
        got = out_gpu[pr[0], r0:r0 + ref.shape[0], pr[1]].to(torch.float64).cpu().numpy()
        diffs.append(np.abs(got - ref).ravel())
        for name, o8 in out8.items():
            got8 = o8[pr[0], r0:r0 + ref.shape[0], pr[1]].to(torch.float64).cpu().numpy()
            diffs8[name].append(np.abs(got8 - ref).ravel())
    del out_gpu, out8
    d = np.concatenate(diffs)
    log(f"[cpu] oracle attention on {len(pairs)} (head, tile) pairs")
    layer_s = t_sel + t_att * (wl.B * wl.H * Tq) / len(pairs)
    threads = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            threads = min(threads, max(blas))
    except Exception:  # pragma: no cover
        pass
    parity = {
        "score_err": score_err, "score_bar": SCORE_RTOL,
        "idx_rows": int(wl.B * wl.H * Tq), "idx_rows_differing": rows_differ,
        "idx_mismatch_outside_window": rows_outside,
        "attn_max_abs": float(d.max()), "attn_mean_abs": float(d.mean()),
        "attn_bars": [ATTN_MAX_ABS, ATTN_MEAN_ABS], "attn_pairs": len(pairs), "attn_rows": int(d.size // wl.d),
        "ok": bool(score_err <= SCORE_RTOL and rows_outside == 0 and d.max() <= ATTN_MAX_ABS
                   and d.mean() <= ATTN_MEAN_ABS),
        "what": ("GPU selection of every head and row against the oracle's (scores, index sets); GPU attention "
                 "fed the oracle's index sets against the oracle on the sampled (head, query tile) pairs"),
    }
    what8 = {"fp8qk": ("FP8 Q.K^T attention (Q, K quantised to E4M3FN) against the fp64 oracle of the bf16 "
                       "inputs on the same pairs: the error of FP8 logits, outside the bf16 attention bar"),
             "fp8": ("FP8 attention (Q, K, V quantised to E4M3FN, P rounded to E4M3FN) against the fp64 "
                     "oracle of the bf16 inputs on the same pairs: the error of the FP8 formats, outside "
                     "the bf16 attention bar")}
    for name, ds in diffs8.items():
        d8 = np.concatenate(ds)
        parity[f"{name}_vs_oracle"] = {"max_abs": float(d8.max()), "mean_abs": float(d8.mean()),
                                       "pairs": len(pairs), "what": what8[name]}
    log(f"[cpu] parity: {parity}")
    return {
        "value": lay.dense_flops() / layer_s / 1e12, "unit": "TFLOP/s (dense-equivalent)",
        "cores": threads, "kind": "oracle",
        "sample": (f"selection on all {wl.B * wl.H} heads (all {Tq} query tiles) in {t_sel:.1f} s; attention on "
                   f"{len(pairs)} random (head, query tile) pairs in {t_att:.1f} s; extrapolated to the whole "
                   f"layer: {layer_s:.0f} s per layer"),
        "layer_s_extrapolated": layer_s,
        "cpu": _cpu_model() or platform.processor() or platform.machine(),
    }, parity


def attention_kernel_name(wl):
    """The attention kernel the library launches for this layer: the two-group kernel for
    128-row tiles whose 64-key block list fits its 3072-entry LDS table, its paired form
    for 64-row tiles whose 32-key block list fits 1536 entries, else the single-pipeline one."""
    kbk = 64 if wl.tile == 128 else 32
    blocks = sum(min(s.budget, -(-s.length // wl.tile)) for s in wl.segments) * (wl.tile // kbk)
    blocks += sum(-(-r.length // kbk) for r in wl.dense)
    if wl.tile == 128 and blocks <= 3072:
        return f"sparse_attn_pingpong_kernel<{wl.d}>"
    if wl.tile == 64 and blocks <= 1536:
        return f"sparse_attn_pingpong_pair_kernel<{wl.d}>"
    return f"sparse_attn_kernel<{wl.d}, {wl.tile // 32}, {32 if wl.tile == 64 else 64}>"


def recorded_traffic(workload):
    """HBM-side bytes per attention launch from the committed rocprofv3 byte-counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by a plain 1 GiB copy), or None when no summary
    exists for this workload or the kernel source changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_sparse_attn_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    with open(os.path.join(ROOT, t["source"]), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != t["source_sha256"]:
            return None
    return (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]) * 1024.0


def main():
    global SEED
    args = parse()
    SEED = args.seed
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the path is built and "
                                   "measured on one GPU's share of a layer and is not sharded across GPUs"}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU"}))
        sys.exit(1)

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    if args.calib_copy:
        copy_calibration()
    lay, res = measure(args.workload, args.steps, args.warmup, args.kernel_reps, args.dense_reps,
                       not args.no_dense, log)
    wl = lay.wl
    patterns = None if args.no_patterns else measure_patterns(lay, args.kernel_reps, log)
    if patterns is not None:
        patterns["random_indices"] = random_pattern(lay, args.kernel_reps, log)
    fp8qk, fp8, attn8_with = None, None, None
    if not args.no_fp8 and lay.wl.tile == 128:
        fp8qk, fp8, attn8_with = measure_fp8(lay, args.kernel_reps, log)
        fp8qk["speedup_vs_bf16_attn"] = round(res["attn_ms_median"] / fp8qk["attn_ms_median"], 3)
        fp8["speedup_vs_bf16_attn"] = round(res["attn_ms_median"] / fp8["attn_ms_median"], 3)
    peaks = device_peaks(log)
    also = None
    if args.also and args.also != "none" and args.also != args.workload:
        lay2, res2 = measure(args.also, args.steps, args.warmup, args.kernel_reps, args.dense_reps,
                             not args.no_dense, log)
        also = res2
        del lay2
    sweep = None
    if not args.no_sweep:
        sweep = {}
        for name in ("tiny", "mid", "t2v5s", "r2va", "t2v14s"):
            if name == args.workload:
                r = res
            else:
                lay_s, r = measure(name, max(3, args.steps // 2), 1, args.kernel_reps, args.dense_reps,
                                   False, log)
                del lay_s
            sweep[name] = {k: round(r[k], 4) for k in ("ms_per_step", "selector_ms", "attn_ms", "full_layer_ms",
                                                       "actual_tflops_attn", "dense_equiv_tflops_step",
                                                       "sparsity_actual")}
            import torch
            torch.cuda.empty_cache()
    cpu, parity = None, None
    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline(lay, log, attn8_with=attn8_with)
        if fp8qk is not None and "fp8qk_vs_oracle" in parity:
            fp8qk["vs_oracle_bf16_inputs"] = parity.pop("fp8qk_vs_oracle")
        if fp8 is not None and "fp8_vs_oracle" in parity:
            fp8["vs_oracle_bf16_inputs"] = parity.pop("fp8_vs_oracle")
    attn8_with = None
    torch.cuda.empty_cache()
    achieved = res["actual_tflops_attn"]
    traffic = recorded_traffic(args.workload)
    attn_kernel = attention_kernel_name(wl)
    line = {
        "metric": METRIC,
        "value": round(res["dense_equiv_tflops_step"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": wl.B, "H": wl.H, "d": wl.d, "p": wl.p,
                   "tile": wl.tile, "n_tokens": wl.n_tokens, "query_tokens": wl.query.length,
                   "budgets": {s.name: s.budget for s in wl.segments},
                   "dense_tokens": sum(r.length for r in wl.dense), "seed": wl.index},
        "selector_ms": round(res["selector_ms"], 4),
        "order_ms": round(res["order_ms"], 4),
        "full_layer_ms": round(res["full_layer_ms"], 4),
        "attn_ms": round(res["attn_ms"], 4),
        "dense_equiv_tflops_attn": round(res["dense_equiv_tflops_attn"], 2),
        "actual_tflops_attn": round(achieved, 2),
        "mfma_util": round(achieved / PEAK_BF16_TFLOPS, 4),
        "dense_ms": round(res.get("dense_ms", float("nan")), 3) if "dense_ms" in res else None,
        "speedup_vs_dense": round(res["speedup_vs_dense"], 2) if "speedup_vs_dense" in res else None,
        "mfma_util_vs_measured_peak": round(achieved / peaks["mfma_bf16_tflops"], 4),
        "selector_ms_median": round(res["selector_ms_median"], 4),
        "attn_ms_median": round(res["attn_ms_median"], 4),
        "ms_per_step_median": round(res["ms_per_step_median"], 4),
        "warm": {k: round(v, 4) for k, v in res["warm"].items()},
        "protocol": {"headline": "cold: a 512 MiB device write before every step, outside the step's events",
                     "warm": "the same steps back to back", "statistic": "mean over the timed steps",
                     "dense_reps": res.get("dense_reps")},
        "pool": {"ms": round(res["pool_ms"], 4), "gbs": round(res["pool_gbs"], 1),
                 "frac_hbm_peak": round(res["pool_gbs"] / PEAK_HBM_GBS, 4),
                 "frac_copy": round(res["pool_gbs"] / peaks["copy_gbs"], 4),
                 "bytes": res["pool_bytes"]},
        "index_stats": res["index_stats"],
        "sdpa_dense": res.get("sdpa_dense"),
        "speedup_vs_fastest_dense": round(res["speedup_vs_fastest_dense"], 2)
        if "speedup_vs_fastest_dense" in res else None,
        "device_peaks": peaks,
        "env": environment(),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": (round(traffic / 1e9, 2) if traffic else None),
                     "traffic_unit": "GB per launch (FETCH_SIZE+WRITE_SIZE, copy-calibrated)",
                     "kernel": attn_kernel, "algorithmic": f"{res['actual_attn_tflop']:.3f} TFLOP per launch"},
        "cpu_baseline": cpu,
        "parity": parity,
        "patterns": patterns,
        "fp8qk": fp8qk,
        "fp8": fp8,
        "also": also,
        "sweep": sweep,
        "detail": res,
    }
    print(json.dumps(line))
    if args.record:
        append_record(args.record, line)


if __name__ == "__main__":
    main()
