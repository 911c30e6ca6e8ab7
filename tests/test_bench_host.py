"""Host logic of bench.py (no GPU): the JSON contract's refusal of several
GPUs, the key that ties committed traffic counters to the kernels' code, and
the CPU baseline's sample."""
import json
import os
import subprocess
import sys

import numpy as np

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_text_ignores_comments_and_blank_space():
    a = "int x = 1; // one\n/* block\n comment */ float y;\n"
    b = "int  x = 1;\n\n float y;   // another remark\n"
    assert bench._code_text(a) == bench._code_text(b) == "int x = 1; float y;"
    assert bench._code_text("int x = 2;") != bench._code_text(a)


def test_fc_source_sha_is_stable():
    assert bench.fc_source_sha() == bench.fc_source_sha()
    assert len(bench.fc_source_sha()) == 64


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_cpu_baseline_sample_reaches_sixteen_kept_routes():
    cfg = synth.WORKLOADS["ep_share_T4096"]
    rng = np.random.default_rng(0)
    rid = rng.integers(0, 896, (cfg.T, cfg.K)).astype(np.int32)
    n = bench._sample_tokens(cfg, rid, 16)
    kept = (rid[:n] < cfg.E_local).sum()
    assert kept >= 16 and (rid[:n - 1] < cfg.E_local).sum() < 16
    full = synth.WORKLOADS["decode_T8"]
    assert bench._sample_tokens(full, rng.integers(0, 896, (8, 16)).astype(np.int32), 16) == 1


def test_host_record_names_the_cores():
    hr = bench.host_record()
    assert hr["host_cores"] == os.cpu_count()
