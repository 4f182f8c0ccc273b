"""Host checks of bench.py's command line (no GPU): the benchmark runs on one GPU and
refuses more with a message and exit status 2, before it touches torch or a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    p = _bench("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def test_help_lists_the_contract_flags():
    p = _bench("--help")
    assert p.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--config"):
        assert flag in p.stdout
