"""Host-side logic of bench.py (no GPU): the refusal of several GPUs, the
algorithmic byte model against the hand-computed table for the 128K
workload, the traffic-counter ingestion and its source-hash guard."""
import json
import os
import subprocess
import sys

import pytest

import bench
from sparse_kv_cache_step_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_of_the_128k_workload():
    """Per layer-step at b 8, s 131072, c 8, k 256, o 48, w 32, r 160, d 128,
    bf16: landmarks 268.4 MB, gathered A rows 41.9 MB, B 2.6 MB, outlier K+V
    12.6 MB, local K+V 1.0 MB, selected V 33.6 MB: 360.2 MB, 360.3 MB with the
    queries and outputs."""
    ab = bench.algorithmic_bytes(synth.LLAMA_128K)
    mb = {k: v / 1e6 for k, v in ab.items()}
    assert round(mb["landmarks"], 1) == 268.4
    assert round(mb["a_rows"], 1) == 41.9
    assert round(mb["b_factor"], 1) == 2.6
    assert round(mb["outlier_kv"], 1) == 12.6
    assert round(mb["local_kv"], 1) == 1.0
    assert round(mb["selected_v"], 1) == 33.6
    assert round(sum(v for k, v in mb.items() if k not in ("q", "out")), 1) == 360.2
    assert round(sum(mb.values()), 1) == 360.3


def _csv(path, rows):
    with open(path, "w") as fh:
        fh.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for d, name, counter, value in rows:
            fh.write(f'{d},"{name}",{counter},{value}\n')


def test_counter_ingestion_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    """FETCH_SIZE reading half of the copy's bytes gives scale 2; the kernel's
    mean over its launches is scaled by it; per-XCD rows of one dispatch add."""
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    copy_kib = bench.COPY_BYTES / 1024
    score = "void skv::score_mfma_kernel<128, 0>(...)"
    attn = "void skv::attn_mfma_kernel<128, 4, 5, false>(...)"
    fetch = tmp_path / "f.csv"
    write = tmp_path / "w.csv"
    _csv(fetch, [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", copy_kib / 2),
                 (2, score, "FETCH_SIZE", 600.0), (2, score, "FETCH_SIZE", 400.0),
                 (3, score, "FETCH_SIZE", 1000.0), (4, attn, "FETCH_SIZE", 50.0)])
    _csv(write, [(1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", copy_kib),
                 (2, score, "WRITE_SIZE", 10.0), (3, score, "WRITE_SIZE", 30.0), (4, attn, "WRITE_SIZE", 4.0)])
    # the hashes are of the real sources, which the patched ROOT does not hold
    monkeypatch.setattr(bench, "kernel_source_hash", lambda which="score": "h-" + which)
    assert bench.ingest_counters(str(fetch), str(write), "w", "cmd") == 0
    rec = json.load(open(tmp_path / "profiles" / "traffic_score_w.json"))
    assert rec["fetch_bytes_per_launch"] == int(1000.0 * 1024 * 2)
    assert rec["write_bytes_per_launch"] == int(20.0 * 1024)
    assert rec["source_hash"] == "h-score"
    rec = json.load(open(tmp_path / "profiles" / "traffic_attn_w.json"))
    assert rec["bytes_per_launch"] == int(50.0 * 1024 * 2 + 4.0 * 1024)
    # reported only while the sources match
    assert bench.measured_traffic("w", "score") == int(1000.0 * 1024 * 2 + 20.0 * 1024)
    monkeypatch.setattr(bench, "kernel_source_hash", lambda which="score": "changed")
    assert bench.measured_traffic("w", "score") is None


@pytest.mark.parametrize("which", list(bench.TRAFFIC_KERNELS))
def test_kernel_source_hash_finds_the_kernel_text(which):
    h = bench.kernel_source_hash(which)
    assert len(h) == 16 and h == bench.kernel_source_hash(which)


def test_missing_kernel_text_gives_no_traffic_record(monkeypatch):
    monkeypatch.setitem(bench.TRAFFIC_KERNELS, "score", ("x", "select.hip", ("void no_such_kernel(",)))
    assert bench.kernel_source_hash("score") is None
    assert bench.measured_traffic("llama3-8b-128k-b8", "score") is None


def test_cpu_model_is_named():
    """The oracle's timing names the host CPU it ran on."""
    name = bench.cpu_model()
    assert isinstance(name, str) and name.strip()
