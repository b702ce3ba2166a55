"""bench.py's command-line contract that needs no GPU: asking for more than
one GPU ends at once with a message on one JSON line; the bucket-size
overrides (CPU only)."""

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
