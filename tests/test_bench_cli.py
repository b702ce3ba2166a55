"""bench.py's contract parts that need no GPU: asking for more than one GPU
ends at once with a message on one JSON line; the bucket-size overrides;
the code digest that ties the committed counter summary to the kernel
sources, and the traffic entry it gates."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_bucket_size_overrides_make_one_bucket_per_phase():
    """Limits larger than the model put every parameter in one gather bucket
    and one gradient bucket; the algorithmic bytes do not change."""
    sys.path.insert(0, ROOT)
    import bench
    import oracle
    from synth import get_config
    cfg = get_config("c2")
    one = bench.with_bucket_sizes(cfg, 1e12, 1e12)
    assert bench.with_bucket_sizes(cfg) is cfg
    assert (one.prefetch_bucket_size, one.reduce_bucket_size) == (10 ** 12, 10 ** 12)
    L = oracle.make_layout(cfg.world_size, cfg.threshold, cfg.ds_ids, cfg.numels)
    assert len(oracle.gather_buckets(L, one.prefetch_bucket_size)) == 1
    assert len(oracle.reduce_buckets(L, one.reduce_bucket_size)) == 1
    assert len(oracle.gather_buckets(L, cfg.prefetch_bucket_size)) == 3
    only_reduce = bench.with_bucket_sizes(cfg, None, 7)
    assert only_reduce.prefetch_bucket_size == cfg.prefetch_bucket_size and only_reduce.reduce_bucket_size == 7


def test_code_digest_ignores_comments_and_layout_only():
    """The digest that ties profiles/ to the kernel sources changes with the
    code and not with comments or whitespace."""
    sys.path.insert(0, ROOT)
    import bench
    code = "int f(int x) {\n  return x + 1; // one\n}\n/* block\n comment */\n"
    same = "int f(int x) { return x + 1; }   // other words\n"
    other = "int f(int x) { return x + 2; }\n"
    assert bench._code_only(code) == bench._code_only(same)
    assert bench._code_only(code) != bench._code_only(other)


def test_committed_traffic_summary_matches_the_current_kernels(monkeypatch):
    """profiles/gather_traffic_c4.json was taken on the current kernel
    sources, so the bench line carries its HBM bytes per launch; with any
    other digest the entry is withheld (None)."""
    sys.path.insert(0, ROOT)
    import bench
    with open(os.path.join(ROOT, "profiles", "gather_traffic_c4.json")) as fh:
        t = json.load(fh)
    assert t["source_digest"] == bench.source_digest()
    hbm = bench.traffic_entry("c4")
    assert abs(hbm - (t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"])) <= 1    # each rounded down
    # fetched plus written bytes sit just below the algorithmic count: the own part is read once
    assert 0.9 * t["algorithmic_bytes_per_launch"] < hbm <= t["algorithmic_bytes_per_launch"]
    monkeypatch.setattr(bench, "source_digest", lambda: "0" * 16)
    assert bench.traffic_entry("c4") is None
    assert bench.traffic_entry("no_such_workload") is None


def test_auto_launch_granularity():
    """--single-launch auto: one launch for a phase whose pass moves less
    than 4 GB (the small workloads), per-bucket launches for the large ones;
    never a single gather launch under the coordinator's schedule, nor a
    single reduce launch on the non-contiguous gradient path."""
    sys.path.insert(0, ROOT)
    import bench
    from synth import get_config
    pick = {c: bench.auto_single_launch(get_config(c), get_config(c).bench_rank) for c in ("c1", "c2", "c3", "c4", "c5")}
    assert pick == {"c1": "both", "c2": "both", "c3": "both", "c4": "none", "c5": "none"}
    c2 = get_config("c2")
    assert bench.auto_single_launch(c2, 0, reduce_path="coalesced") == "gather"
    assert bench.auto_single_launch(c2, 0, schedule="trace") == "reduce"
