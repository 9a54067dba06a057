"""Host-side checks of bench.py: the algorithmic byte and flop counts it
divides by, the causal element count, the source hash that gates committed
counter records, and the one-GPU guard.  No GPU needed."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from row_wise_online_amd import workloads as wl  # noqa: E402


def test_resident_bytes_of_the_headline_workload():
    # x read once, y written once, m and d: 2 * 4096 * 4096 * 4 + 2 * 4 * 4096
    w = wl.WORKLOADS["c2"]
    assert bench.algorithmic_bytes(w, "resident", 2) == 134_250_496


def test_bf16_resident_bytes():
    w = wl.WORKLOADS["c3"]
    assert bench.algorithmic_bytes(w, "resident", 0) == 2 * 32768 * 1024 * 2


def test_two_read_paths_count_the_second_read():
    w = wl.WORKLOADS["c4"]
    xy = w.M * w.N * 4
    assert bench.algorithmic_bytes(w, "stream", 0) == 3 * xy
    assert bench.algorithmic_bytes(w, "resident", 0) == 2 * xy


def test_split_bytes_include_the_state_tables():
    import row_wise_online_amd as rw
    w = wl.WORKLOADS["c5"]
    xy = w.M * w.N * 4
    ws = rw.softmax_plan(w.M, w.N, "f32", 256, "split")["workspace_bytes"]
    assert ws > 0
    assert bench.algorithmic_bytes(w, "split", 3, cus=256) == \
        3 * xy + 4 * w.M * 3 + 2 * ws


def test_cross_entropy_and_stats_read_once():
    w = wl.WORKLOADS["c2"]
    xy = w.M * w.N * 4
    assert bench.algorithmic_bytes(w, "resident", 0, "cross_entropy") == xy + 12 * w.M + 4
    assert bench.algorithmic_bytes(w, "resident", 3, "stats") == xy + 12 * w.M


def test_normalize_reads_x_and_the_state_once():
    # pass 2 alone: x read, y written, 8 B of row state read, on any path
    for name in ("c2", "c5"):
        w = wl.WORKLOADS[name]
        xy = w.M * w.N * w.esize
        for path in ("resident", "split", "normalize"):
            assert bench.algorithmic_bytes(w, path, 0, "normalize") == 2 * xy + 8 * w.M


def test_causal_elements_closed_form():
    # square rows with offset 0 keep the lower triangle: M (M + 1) / 2
    w = wl.WORKLOADS["c2"]
    assert bench.valid_elements(w, 0) == 4096 * 4097 // 2
    assert bench.valid_elements(w, None) == 4096 * 4096
    # an offset past the last column keeps every element
    assert bench.valid_elements(w, 5000) == 4096 * 4096
    # causal: the masked part of x is not read, y is written whole
    assert bench.algorithmic_bytes(w, "resident", 0, causal=0) == \
        (4096 * 4097 // 2 + 4096 * 4096) * 4


def test_attention_flops():
    a2 = wl.ATTN_WORKLOADS["a2"]
    assert a2.flops() == 4 * 131072 * 131072 * 128
    a3 = wl.ATTN_WORKLOADS["a3"]
    assert a3.flops() == 4 * (131072 * 131073 // 2) * 128


def test_source_hash_ignores_compiler_temporaries(tmp_path, monkeypatch):
    src = tmp_path / "row_wise_online_amd" / "csrc"
    src.mkdir(parents=True)
    (src / "api.hip").write_text("a")
    (src / "common.hpp").write_text("b")
    (src / "attention.hip").write_text("c")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    soft, att = bench.kernel_source_hash("softmax"), bench.kernel_source_hash("attention")
    (src / "attention.hip-hip-amdgcn-amd-amdhsa.hipfb").write_text("junk")
    (src / "api.o").write_text("junk")
    assert bench.kernel_source_hash("softmax") == soft
    assert bench.kernel_source_hash("attention") == att
    # each family sees its own sources
    (src / "attention.hip").write_text("c2")
    assert bench.kernel_source_hash("softmax") == soft
    assert bench.kernel_source_hash("attention") != att
    (src / "common.hpp").write_text("b2")
    assert bench.kernel_source_hash("softmax") != soft


@pytest.mark.parametrize("args", [["--gpus", "2"], ["--gpus", "8"]])
def test_more_than_one_gpu_is_refused(args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
