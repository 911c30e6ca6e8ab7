"""Host logic of bench.py (no GPU): the JSON contract's refusal of several
GPUs and the key that ties committed traffic counters to the kernels' code."""
import json
import os
import subprocess
import sys

import bench

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
