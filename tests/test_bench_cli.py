"""bench.py's command line on the CPU: the workload names it offers, and the
refusal of more than one GPU (the library has no multi-GPU path)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], stdout=subprocess.PIPE,
                          stderr=subprocess.STDOUT, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stdout


def test_help_lists_every_workload():
    r = _bench("--help")
    assert r.returncode == 0
    for name in ("decode_8k_b1", "mtp_verify_128k_b64", "swa_decode_32k_b64", "decode_1m_b4",
                 "prefill_chunk_16k_at_112k"):
        assert name in r.stdout
