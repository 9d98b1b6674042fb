"""Host-side checks of the benchmark: its unmasked-entry count (the FLOP denominator) equals the
oracle's for every workload, and more than one GPU is refused."""

import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle
from workloads import configs


@pytest.mark.parametrize("key", sorted(configs.WORKLOADS))
def test_unmasked_count_matches_oracle(key):
    w = configs.WORKLOADS[key]
    v = configs.global_mask(w)
    if key == "c5":
        v = oracle.localize(*v, configs.C5_CHUNK_START, configs.C5_CHUNK_LEN, 131072)[:4]
    assert bench.unmasked_entries(v, w.nq) == oracle.unmasked_count(*v, w.nq)


def test_random_vectors_count():
    r = np.random.default_rng(5)
    for _ in range(20):
        nq, nk = int(r.integers(1, 50)), int(r.integers(1, 50))
        v = [r.integers(-10, nq + 10, size=nk) for _ in range(4)]
        assert bench.unmasked_entries(v, nq) == oracle.unmasked_count(*v, nq)


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_source_hash_ignores_comments_only():
    """The counter records are tied to the kernels' code, not to their comments."""
    src = "int f(int x) {  // add one\n  /* block\n comment */\n  return x + 1;\n}\n"
    same = "// header\nint f(int x) {\n\n  return x + 1;   // other words\n}\n"
    other = "int f(int x) {\n  return x + 2;\n}\n"
    assert bench.code_text(src) == bench.code_text(same)
    assert bench.code_text(src) != bench.code_text(other)


def test_workloads_table_renders_the_committed_lines():
    """The per-workload table in the profiles is made from the committed bench lines."""
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    path = os.path.join(root, "profiles", "bench_workloads.jsonl")
    r = subprocess.run([sys.executable, "-m", "mask_aware_flashattention_amd.rocprof_summary",
                        "workloads", path], capture_output=True, text=True, cwd=root)
    assert r.returncode == 0, r.stderr
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("| ") and "---" not in ln]
    with open(path) as fh:
        n = sum(1 for ln in fh if ln.strip())
    assert len(lines) == n + 1  # header + one row per bench line
    assert any("one global call" in ln for ln in lines)
