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


def test_cpu_baseline_leg_on_a_small_workload():
    """The bench's oracle leg on a small CPU workload: it reports the host's core
    counts, its BLAS threads and the per-token time of its two parts, and the
    results it returns for the parity check pass that check against the oracle's
    own selections and outputs (as the timed buffers would hold them)."""
    import numpy as np
    import torch

    sys.path.insert(0, ROOT)
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    try:
        import bench
        from gpu_helpers import OracleView
    finally:
        sys.path.pop(0)
        sys.path.pop(0)
    from sparse_block_indexed_amd import inputs as I
    wl = I.make_workload(I.WorkloadSpec("tiny", batch=2, seq_lens=[5000, 700], q_per_seq=2), seed=3, device="cpu")
    ov = OracleView(wl)
    sel_host = np.stack([ov.selection(t) for t in range(wl.n_tok)]).astype(np.int32)
    base, refs = bench.cpu_baseline(wl, sel_host, budget_s=30.0, max_tokens=4)
    assert base["kind"] == "oracle" and base["value"] > 0 and len(refs) == wl.n_tok
    assert base["host"]["os_cpu_count"] == os.cpu_count() and base["host"]["blas_threads"] >= 1
    assert base["seconds_per_token"]["indexer_topk"] > 0 and base["seconds_per_token"]["attention"] > 0
    for t, sel, _, _ in refs:
        assert sel.tolist() == sel_host[t].tolist()
    out = torch.zeros((wl.n_tok, 64, 192), dtype=torch.bfloat16)
    lse = torch.zeros((wl.n_tok, 64), dtype=torch.float32)
    for t, _, o, l in refs:
        out[t] = torch.tensor(o, dtype=torch.float32).to(torch.bfloat16)
        lse[t] = torch.tensor(l, dtype=torch.float32)
    assert bench.parity_check(refs, sel_host, out, lse)["pass"]


def test_counter_records_follow_code_not_comments(tmp_path):
    """A counter record's source hash ignores comments and spacing, and changes
    with the code."""
    sys.path.insert(0, ROOT)
    try:
        import bench
    finally:
        sys.path.pop(0)
    saved = bench.CSRC
    bench.CSRC = str(tmp_path)
    try:
        def h(text):
            (tmp_path / "k.hip").write_text(text)
            return bench.source_hash("k.hip")
        base = h("int f(int x) {\n  return x + 1;   // add one\n}\n")
        assert h("/* header */\nint f(int x) {\n    return x + 1;\n}\n") == base
        assert h("int f(int x) {\n  return x + 2;   // add one\n}\n") != base
    finally:
        bench.CSRC = saved
