"""The benchmark's command-line contract, checked without a GPU: more than
one GPU is refused with a message (this build measures one GPU), and an
unknown extra configuration is refused before any work starts."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def run(*args):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_unknown_extra_configuration_is_refused_first():
    r = run("--extras", "decode_0p5b_s128,no_such_config")
    assert r.returncode == 1
    assert "unknown --extras no_such_config" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_extra_configurations():
    r = run("--help")
    assert r.returncode == 0
    for name in ("decode_0p5b_s128", "batched_qwen3_4b", "q4_decode_s16384", "prefill_0p5b_chunk256_at3841"):
        assert name in r.stdout
