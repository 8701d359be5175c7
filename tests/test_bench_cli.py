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


def test_parity_check_of_timed_buffers():
    """The bench's check of its timed buffers: the oracle's own results (rounded
    to bf16 as the output buffer holds them) pass; a selection that differs in
    one id, or an output off by 0.05 in one element, fails."""
    import numpy as np
    import torch

    sys.path.insert(0, ROOT)
    try:
        import bench
    finally:
        sys.path.pop(0)
    rng = np.random.default_rng(1)
    n = 3
    refs = []
    for t in range(n):
        sel = np.sort(rng.choice(1000, size=512, replace=False))
        refs.append((t, sel, rng.standard_normal((64, 192)) * 0.3, rng.standard_normal(64)))
    sel_host = np.stack([r[1] for r in refs]).astype(np.int32)
    out = torch.tensor(np.stack([r[2] for r in refs]), dtype=torch.float32).to(torch.bfloat16)
    lse = torch.tensor(np.stack([r[3] for r in refs]), dtype=torch.float32)
    ok = bench.parity_check(refs, sel_host, out, lse)
    assert ok["pass"] and ok["selection"] == "bit-exact" and ok["tokens"] == n
    bad_sel = sel_host.copy()
    bad_sel[1, 7] += 1
    assert not bench.parity_check(refs, bad_sel, out, lse)["pass"]
    bad_out = out.clone()
    bad_out[2, 5, 9] += 0.05
    assert not bench.parity_check(refs, sel_host, bad_out, lse)["pass"]
    window_refs = [(t, None, o, l) for t, _, o, l in refs]
    assert bench.parity_check(window_refs, None, out, lse)["selection"] is None
