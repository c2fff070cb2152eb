"""Host-side pieces of bench.py (no GPU): the stored traffic counters are
keyed to the forward kernel's code, so a comment or blank-space edit keeps
the key and any code edit changes it (bench.py then reports no traffic);
the stored counters are well formed; --gpus other than 1 is refused with a
message."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def hash_of(text, tmp_path):
    p = tmp_path / "k.hip"
    p.write_text(text)
    old = bench.FWD_KERNEL_SOURCE
    bench.FWD_KERNEL_SOURCE = str(p)
    try:
        return bench.source_hash()
    finally:
        bench.FWD_KERNEL_SOURCE = old


def test_hash_ignores_comments_and_blank_space(tmp_path):
    src = "// header\nint f(int x) {  /* twice */\n  return 2 * x;  // doubled\n}\n"
    h = hash_of(src, tmp_path)
    assert hash_of("int f(int x) {\n\n   return 2 * x;\n}", tmp_path) == h
    assert hash_of(src.replace("2 * x", "3 * x"), tmp_path) != h


def test_stored_counters_are_well_formed():
    with open(bench.TRAFFIC_FILE) as f:
        tr = json.load(f)
    assert len(tr["kernel_source_sha256_16"]) == 16
    assert tr["bytes_per_launch"] > tr["algorithmic_record_bytes_per_launch"] > 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0 and "one GPU" in r.stderr


def test_input_hash_is_stable_and_sees_every_input():
    from head_latent_attention_sparse_amd import workloads

    w = workloads.tiny()
    h = bench.input_hash(w)
    assert h == bench.input_hash(workloads.tiny()) and len(h) == 64
    w.indices[5] = -1
    assert bench.input_hash(w) != h
    w = workloads.tiny()
    w.setup_inserts[0].kv_c[3, 7] = 2.0
    assert bench.input_hash(w) != h
    w = workloads.tiny()
    w.softmax_scale *= 2
    assert bench.input_hash(w) != h


def test_cpu_oracle_pool_runs_every_row():
    """The baseline's worker pool (forked, numpy only) covers every row once and
    reports the worker count as its cores."""
    from head_latent_attention_sparse_amd import workloads

    w = workloads.tiny()
    cpu = bench.CpuOracle(w, workers=2)
    try:
        r = cpu.run()
    finally:
        cpu.close()
    assert r["cores"] == 2 and r["kind"] == "oracle" and r["value"] > 0
    assert f"all {w.num_tokens} rows" in r["sample"]
