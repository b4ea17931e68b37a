"""bench.py's command-line contract, on the host (no GPU is touched)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
    assert not r.stdout.lstrip().startswith("{")      # no result line


def test_defaults_time_a_settled_state(monkeypatch):
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert a.gpus == 1 and a.steps == 100 and a.warmup == 100
    assert a.min_untimed_steps >= 100     # the clocks settle over the first ~100 steps


def test_kernel_source_hash_ignores_comments_not_code():
    import bench
    a = "int f(int x) {\n  return x + 1;   // add one\n}\n/* block\n comment */\n"
    b = "int f(int x) {   // renamed nothing\n  return x + 1;\n}\n"
    c = "int f(int x) {\n  return x + 2;\n}\n"
    assert bench.code_tokens(a) == bench.code_tokens(b)
    assert bench.code_tokens(a) != bench.code_tokens(c)
    h = bench.kernel_sources_sha256()
    assert isinstance(h, str) and len(h) == 64 and h == bench.kernel_sources_sha256()
