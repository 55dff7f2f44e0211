"""Host logic of bench.py that needs no GPU: the sweep log that lets an
interrupted sweep resume."""
import json

import bench
from speculative_decode_verify_gate_amd import synth


def test_sweep_log_round_trip_and_cut_line(tmp_path):
    path = tmp_path / "points.jsonl"
    log = bench.SweepLog(str(path))
    a = {"leg": "sweep", "workload": "v2lite", "rho": 0.85, "n": 3, "passes": 50}
    b = {"leg": "rho", "workload": "v2stack", "rho": 0.5, "n": 7, "passes": 32, "layers": 26}
    log.put(a, {"n": 3, "x": 1.5})
    log.put(b, {"u_bar": 0.25, "stack_us": {"route": 1.0}})
    with open(path, "a") as f:
        f.write('{"key": {"leg": "sweep", "n": 9}, "rec')  # cut by an interruption
    again = bench.SweepLog(str(path))
    # keys match whatever the order of their fields
    assert again.get(dict(reversed(list(a.items())))) == {"n": 3, "x": 1.5}
    assert again.get(b) == {"u_bar": 0.25, "stack_us": {"route": 1.0}}
    assert again.get({**a, "n": 4}) is None and again.get({**a, "passes": 200}) is None
    assert len(again.done) == 2
    # appending after a cut line still gives whole lines from then on
    again.put({**a, "n": 5}, {"n": 5})
    lines = path.read_text().splitlines()
    assert json.loads(lines[-1]) == {"key": {**a, "n": 5}, "record": {"n": 5}}
    assert bench.SweepLog(str(path)).get({**a, "n": 5}) == {"n": 5}


def test_a_logged_sweep_is_taken_whole_from_the_log(tmp_path):
    # every n is in the log, so run_sweep measures nothing (no GPU here)
    cfg = synth.CONFIGS["v2lite"]
    log = bench.SweepLog(str(tmp_path / "points.jsonl"))
    for n in (1, 2, 3):
        key = {"leg": "sweep", "workload": cfg.name, "rho": cfg.rho, "n": n, "passes": 50}
        log.put(key, {"n": n, "from": "log"})
    out = bench.run_sweep(cfg, None, [None], {}, [1, 2, 3], 50, points=log)
    assert out == [{"n": n, "from": "log"} for n in (1, 2, 3)]


def test_no_log_file_without_a_path(tmp_path):
    log = bench.SweepLog(None)
    log.put({"n": 1}, {"x": 1})
    assert list(tmp_path.iterdir()) == []


def test_share_document_bounds_the_allreduce_per_link():
    whole = synth.CONFIGS["v3"]
    share = synth.share_config(whole, 8)
    sweep = [{"n": 16, "tokens": 64, "perslot": {"us": 700.0}, "dedup": {"us": 500.0}}]
    doc = bench.shard_doc(whole, share, 8, sweep, 2)
    rec = doc["by_n"][0]
    # 64 tokens x 7168 fp32 = 1,835,008 bytes; a ring moves 2 (G - 1) / G of
    # them over each link: 3,211,264 bytes at 153 GB/s = 20.99 us
    assert rec["allreduce_MB"] == round(64 * 7168 * 4 / 1e6, 4)
    assert rec["allreduce_ring_us_bound"] == 20.99
    assert rec["G_gpu_pass_us_lower_bound"] == {"perslot": 720.99, "dedup": 520.99}
    assert doc["share_d_ff"] == 256 and doc["G"] == 8
    json.dumps(doc)
