"""bench.py on the host: the one-GPU contract and the kernel it names for each layer."""
import importlib.util
import json
import os
import subprocess
import sys

from block_sparse_attention_predictor_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_attention_kernel_name_follows_the_launcher_rule():
    """128-row tiles whose block list fits 3072 table entries take the two-group kernel."""
    b = _bench()
    names = {n: b.attention_kernel_name(wl) for n, wl in I.WORKLOADS.items()}
    assert names["t2v5s"] == names["r2va"] == names["t2v14s"] == "sparse_attn_pingpong_kernel<128>"
    assert names["mid"] == "sparse_attn_pingpong_pair_kernel<128>"
    assert names["tiny"] == "sparse_attn_pingpong_pair_kernel<64>"


def test_record_appends_one_json_line_per_run(tmp_path):
    b = _bench()
    p = str(tmp_path / "runs.jsonl")
    assert b.parse(["--record", p]).record == p and b.parse([]).record is None
    b.append_record(p, {"metric": "m", "value": 1.0})
    first = open(p).read()
    b.append_record(p, {"metric": "m", "value": 2.0})
    text = open(p).read()
    assert text.startswith(first)                      # earlier records are left as they were
    recs = [json.loads(x) for x in text.splitlines()]
    assert [r["value"] for r in recs] == [1.0, 2.0]
    assert all(r["recorded_at"].endswith("Z") for r in recs)


def test_seed_replaces_every_workloads_input_seed():
    import numpy as np
    b = _bench()
    assert b.parse(["--seed", "7"]).seed == 7 and b.parse([]).seed is None
    base = b.workload("tiny")
    b.SEED = 7
    try:
        w7 = b.workload("tiny")
    finally:
        b.SEED = None
    assert w7.index == 7 != base.index
    assert (w7.n_tokens, w7.segments, w7.dense) == (base.n_tokens, base.segments, base.dense)
    q0, q7 = I.make_qkv(base)[0], I.make_qkv(w7)[0]
    assert q0.shape == q7.shape and not np.array_equal(q0, q7)


def test_selection_parity_counts_only_mismatches_outside_the_tie_window():
    import numpy as np
    bench = _bench()
    # one segment of 6 tiles, k = 2; row 0: tiles 1 and 4 tie exactly for the 2nd place
    S = np.array([[0.0, 5.0, 1.0, 2.0, 5.0, 9.0],
                  [9.0, 8.0, 1.0, 0.5, 0.25, 0.0]])
    ref = np.array([[1, 5], [0, 1]], dtype=np.int32)
    sc = S.astype(np.float32)
    # identical
    assert bench.selection_parity(ref.copy(), sc, ref, S, [6], [2]) == (0.0, 0, 0)
    # the tie goes the other way: differs, but inside the window
    g = np.array([[4, 5], [0, 1]], dtype=np.int32)
    err, differ, outside = bench.selection_parity(g, sc, ref, S, [6], [2])
    assert (differ, outside) == (1, 0)
    # a clear mismatch in row 1
    g = np.array([[1, 5], [0, 2]], dtype=np.int32)
    assert bench.selection_parity(g, sc, ref, S, [6], [2])[1:] == (1, 1)
    # an invalid (not ascending) row counts as outside
    g = np.array([[5, 4], [0, 1]], dtype=np.int32)
    assert bench.selection_parity(g, sc, ref, S, [6], [2])[1:] == (1, 1)
    # score error is row-normwise
    sc2 = sc.copy()
    sc2[1, 3] += 9.0 * 2e-4
    assert abs(bench.selection_parity(ref, sc2, ref, S, [6], [2])[0] - 2e-4) < 1e-6
