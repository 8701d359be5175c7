"""Benchmark of the sparse layer's decode/verify step on one MI355X.

One step = indexer score + top-512 block select (sa_indexer_topk) followed by
block-sparse GQA attention over the selected + current blocks (sa_sparse_decode,
which merges partitions itself when it splits), for one batch of the 128K-context
MTP verify workload: 64 sequences with lengths uniform in [98304, 131072], the
last 4 positions of each as query tokens (256 tokens), bf16 paged KV with
randomly permuted 64-token pages, integer index inputs in [-4, 4], Q/K/V ~ N(0,1).
Inputs are resident in HBM before timing starts.

`--workload NAME` runs one of the other workloads instead (decode_8k_b1:
decode at 8K, batch 1; swa_decode_32k_b64: sliding-window decode at
16K-32K, batch 64; decode_1m_b4: decode at 1M, batch 4;
prefill_chunk_16k_at_112k: a 16,384-token prefill chunk after 112K tokens);
the default is the headline mtp_verify_128k_b64.

The step is captured as HIP graphs and replayed, 10 steps per replay as a
served forward replays its layers (`--eager` issues every call from Python
instead); each step runs every kernel of the step on the same resident inputs.

Prints one JSON line. `value` is query tokens per second of the whole step
(wall clock over back-to-back steps). The roofline object covers the dominant
kernel (the attention kernel): its algorithmic bytes (distinct K/V blocks read
+ Q + O + selection + lse) divided by its mean duration, measured with HIP
events on the launch stream around graph replays of 5 back-to-back calls.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-attn decode query-tokens/s at 128K ctx, batch 64; achieved HBM GB/s"
PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
GRAPH_STEPS = 10          # steps per graph replay in the timed loop
SCALE = 1.0 / math.sqrt(192.0)
CSRC = os.path.join(ROOT, "sparse_block_indexed_amd", "csrc")
# the kernels of each timed phase, and the sources they are built from
PHASE_KERNELS = {"indexer_topk": ("score_kernel", "score_gemm_kernel", "score_mfma_kernel", "select_kernel",
                                  "finalize_kernel"),
                 "sparse_decode": ("attention_kernel", "merge_kernel"),
                 "swa_decode": ("attention_kernel", "merge_kernel")}
PHASE_SOURCES = {"indexer_topk": ("sa_indexer.hip",), "sparse_decode": ("sa_attention.hip", "sa_merge.hip"),
                 "swa_decode": ("sa_attention.hip", "sa_merge.hip")}


def pmc_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"pmc_{workload}.json")


def source_hash(name: str) -> str:
    """Hash of a kernel source's code: comments and white space are left out,
    so that a counter record stays valid across edits that change no code."""
    import re
    with open(os.path.join(CSRC, name), encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"\s+", " ", text).strip()
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def counter_traffic(workload: str, phase: str):
    """HBM bytes per call of a phase from the committed rocprofv3 counter runs
    of the workload, or None if there are none or they were taken on other
    kernel sources."""
    try:
        with open(pmc_file(workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if any(rec.get("source_sha256_16", {}).get(n) != source_hash(n) for n in PHASE_SOURCES[phase]):
        return None
    return rec.get("phases", {}).get(phase, {}).get("bytes_per_call")


def counter_mean(workload: str, phase: str, kernel: str, counter: str):
    """Mean per dispatch of a further counter of one kernel from the committed
    counter runs of the workload, or None (no such run, or other sources)."""
    try:
        with open(pmc_file(workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if any(rec.get("source_sha256_16", {}).get(n) != source_hash(n) for n in PHASE_SOURCES[phase]):
        return None
    e = rec.get("phases", {}).get(phase, {}).get("kernels", {}).get(kernel, {}).get(counter)
    return None if e is None else e["mean"]


def _pmc_rows(directory: str, counter: str):
    """(kernel name, value) per dispatch from a rocprofv3 --pmc CSV directory."""
    import csv
    import glob
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    per = {}
    with open(files[0], newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return [(name, v) for (_, name), v in per.items()]


def write_pmc_record(args):
    """profiles/pmc_<workload>.json from rocprofv3 --pmc runs of this benchmark
    (FETCH_SIZE and WRITE_SIZE of the workload, the same two counters of the
    1 GiB copy, and optional further counters): per phase, the counters of
    each of its kernels averaged over their dispatches; HBM bytes per call =
    FETCH_SIZE x the copy's read scale + WRITE_SIZE x its write scale, summed
    over the phase's kernels (each call launches each of them once)."""
    dirs = dict(x.split("=", 1) for x in args.pmc_dir)
    copy = dict(x.split("=", 1) for x in args.pmc_copy)
    one_gib_kib = float(1 << 20)
    # the copies only (the run also fills the source buffer once)
    cfs = [v for n, v in _pmc_rows(copy["FETCH_SIZE"], "FETCH_SIZE") if "copyBuffer" in n or "copy_kernel" in n]
    cws = [v for n, v in _pmc_rows(copy["WRITE_SIZE"], "WRITE_SIZE") if "copyBuffer" in n or "copy_kernel" in n]
    launches = 5   # bench.py --copy-calibration copies 1 GiB five times
    if len(cfs) != launches or len(cws) != launches:
        raise SystemExit(f"expected {launches} copy dispatches, found {len(cfs)} / {len(cws)}")
    cf, cw = sum(cfs), sum(cws)
    cal = {"bytes_read_per_copy": 1 << 30, "bytes_written_per_copy": 1 << 30, "copies": launches,
           "fetch_size_kib_per_copy": cf / launches, "write_size_kib_per_copy": cw / launches,
           "fetch_scale": one_gib_kib / (cf / launches), "write_scale": one_gib_kib / (cw / launches)}
    phases = {}
    for phase, kernels in PHASE_KERNELS.items():
        ph = {}
        for counter, d in dirs.items():
            for name, v in _pmc_rows(d, counter):
                short = next((k for k in kernels if f"::{k}" in name), None)
                if short is None:
                    continue
                e = ph.setdefault(short, {}).setdefault(counter, [])
                e.append(v)
        if not ph:
            continue
        if phase == "swa_decode" and not args.workload.startswith("swa"):
            continue
        if phase == "sparse_decode" and args.workload.startswith("swa"):
            continue
        kern = {}
        total = 0.0
        for short, cs in ph.items():
            kern[short] = {c: {"dispatches": len(v), "mean": sum(v) / len(v)} for c, v in cs.items()}
            b = 0.0
            if "FETCH_SIZE" in cs:
                b += kern[short]["FETCH_SIZE"]["mean"] * 1024 * cal["fetch_scale"]
            if "WRITE_SIZE" in cs:
                b += kern[short]["WRITE_SIZE"]["mean"] * 1024 * cal["write_scale"]
            kern[short]["hbm_bytes_per_launch"] = b
            total += b
        phases[phase] = {"kernels": kern, "bytes_per_call": int(round(total))}
    rec = {"workload": args.workload,
           "commands": {c: f"rocprofv3 --pmc {c} -d pmc/{args.workload}_{c} -o bench --output-format csv "
                           f"-- python3 bench.py --workload {args.workload} --eager --steps 3 --warmup 1 "
                           f"--cold-steps 0 --no-cpu-baseline" for c in dirs},
           "copy_calibration_command": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) -d pmc/copy_<counter> "
                                       "-o copy --output-format csv -- python3 bench.py --copy-calibration",
           "copy_calibration": cal, "phases": phases,
           "source_sha256_16": {n: source_hash(n) for n in ("sa_indexer.hip", "sa_attention.hip", "sa_merge.hip")}}
    with open(pmc_file(args.workload), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps({k: v["bytes_per_call"] for k, v in phases.items()}))


def cpu_baseline(wl, sel_host, window=None, budget_s: float = 20.0, max_tokens: int = 64, kv_fp8=None,
                 q_groups=None, kidx_fp8=None):
    """The fp64 oracle timed on this host over a bounded sample of the same
    workload: whole sequences' query tokens (evenly spaced ones when a sequence
    has more than max_tokens), until the budget is spent.
    kv_fp8 = (k_codes, v_codes, k_scale, v_scale) times the one-byte KV form,
    kidx_fp8 (E4M3 codes) the one-byte index keys, q_groups ([n_tok][4][256]
    index queries) per-KV-group selection.

    Returns (baseline, refs): refs holds (token, selection or None, O, lse) of
    every token the oracle ran, for the parity check of the timed buffers."""
    import torch
    from oracle import sa_oracle as O
    from sparse_block_indexed_amd import inputs as I
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(x.get("num_threads", 1)) for x in threadpool_info()] + [1])
    except Exception:
        threads = 1
    done, t_cpu = 0, 0.0
    t_sel, t_att = 0.0, 0.0   # the two parts of the oracle's per-token work
    seqs_done = 0
    refs = []
    dev = wl.k_cache.device
    for b in range(wl.batch):
        toks = [t for t in range(wl.n_tok) if int(wl.q_seq[t]) == b]
        if not toks:
            continue
        if len(toks) > max_tokens:
            toks = toks[::-(-len(toks) // max_tokens)]
        row = wl.page_table[b]
        # host copies of what the oracle reads (not timed): the sequence's index
        # keys and the pages of every attended block
        max_cb = max(int(wl.q_pos[t]) // 8 for t in toks)
        npg = (max_cb + 7) // 8
        kidx = None
        if window is None:
            prow = torch.as_tensor(row[:npg].astype(np.int64), device=dev)
            kidx = (I.bf16_bits(wl.k_idx_cache.index_select(0, prow)) if kidx_fp8 is None
                    else kidx_fp8.index_select(0, prow).cpu().numpy())
        pages = set()
        for t in toks:
            p = int(wl.q_pos[t])
            if window is None:
                pages |= {int(x) // 8 for x in np.asarray(sel_host[t]).reshape(-1) if x >= 0} | {p // 64}
            else:
                pages |= set(range(max(0, p - window + 1) // 64, p // 64 + 1))
        logical = np.array(sorted(pages), dtype=np.int64)
        idx = torch.as_tensor(row[logical].astype(np.int64), device=dev)
        if kv_fp8 is None:
            kc, vc = I.bf16_bits(wl.k_cache.index_select(0, idx)), I.bf16_bits(wl.v_cache.index_select(0, idx))
            fp8_scales = None
        else:
            kc, vc = (kv_fp8[0].index_select(0, idx).cpu().numpy(), kv_fp8[1].index_select(0, idx).cpu().numpy())
            fp8_scales = (kv_fp8[2], kv_fp8[3])
        compact = np.full(row.shape[0], -1, dtype=np.int64)
        compact[logical] = np.arange(len(logical))
        qb = [I.bf16_bits(wl.q[t]) for t in toks]
        qib = [I.bf16_bits(wl.q_idx[t] if q_groups is None else q_groups[t]) for t in toks]
        t0 = time.perf_counter()
        for j, t in enumerate(toks):
            p = int(wl.q_pos[t])
            ta = time.perf_counter()
            if window is not None:
                sel = None
                tb = time.perf_counter()
                o, l = O.attend_positions(O.bf16_to_f64(qb[j]), kc, vc, compact, O.window_positions(p, window),
                                          SCALE, fp8_scales=fp8_scales)
            elif q_groups is None:
                keys = O.index_keys(kidx, np.arange(npg), p // 8, fp8=kidx_fp8 is not None)
                sel = O.indexer_topk_token(O.bf16_to_f64(qib[j]), keys, 512)
                tb = time.perf_counter()
                o, l = O.attend_positions(O.bf16_to_f64(qb[j]), kc, vc, compact, O.sparse_token_positions(sel, p),
                                          SCALE, fp8_scales=fp8_scales)
            else:
                keys = O.index_keys(kidx, np.arange(npg), p // 8, fp8=kidx_fp8 is not None)
                sel = np.stack([O.indexer_topk_token(O.bf16_to_f64(qib[j][g]), keys, 512) for g in range(4)])
                tb = time.perf_counter()
                o, l = O.sparse_attention_token_grouped(qb[j], kc, vc, compact, sel, p, SCALE,
                                                        fp8_scales=fp8_scales)
            t_sel += tb - ta
            t_att += time.perf_counter() - tb
            refs.append((t, sel, o, l))
            done += 1
            if time.perf_counter() - t0 + t_cpu >= budget_s:
                break
        t_cpu += time.perf_counter() - t0
        seqs_done += 1
        if t_cpu >= budget_s or done >= max_tokens:
            break
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return ({"value": done / t_cpu, "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
             "sample": f"{done} query tokens ({seqs_done} sequences) of the {wl.spec.name} workload, fp64 numpy "
                       f"oracle, {t_cpu:.1f} s of CPU time, host copies excluded",
             "host": {"os_cpu_count": os.cpu_count(), "affinity_cores": affinity, "blas_threads": threads},
             "seconds_per_token": {"indexer_topk": t_sel / max(done, 1), "attention": t_att / max(done, 1)}},
            refs)


MAX_ABS, REL_RMS, LSE_ABS = 2e-2, 5e-3, 1e-3


def parity_check(refs, sel_host, out, lse):
    """The timed step's own buffers against the oracle's results for the same
    tokens: selections bit for bit, outputs within max-abs 2e-2 and relative RMS
    5e-3 over the compared tokens, lse within 1e-3."""
    from oracle import sa_oracle as O
    from sparse_block_indexed_amd import inputs as I
    if not refs:
        return {"tokens": 0, "pass": False}
    toks = [r[0] for r in refs]
    bad_sel = [t for t, sel, _, _ in refs if sel is not None and not np.array_equal(np.asarray(sel_host[t]), sel)]
    got = O.bf16_to_f64(I.bf16_bits(out[toks]))
    ref = np.stack([r[2] for r in refs])
    err = np.abs(got - ref)
    rel = float(np.sqrt((err ** 2).sum()) / max(np.sqrt((ref ** 2).sum()), 1e-300))
    dl = float(np.abs(lse[toks].cpu().numpy().astype(np.float64) - np.stack([r[3] for r in refs])).max())
    ok = (not bad_sel) and np.isfinite(got).all() and err.max() <= MAX_ABS and rel <= REL_RMS and dl <= LSE_ABS
    return {"tokens": len(toks),
            "selection": None if refs[0][1] is None else ("bit-exact" if not bad_sel else
                                                          f"{len(bad_sel)} tokens differ"),
            "max_abs": float(err.max()), "rel_rms": rel, "lse_max_abs": dl,
            "tolerance": f"max-abs {MAX_ABS}, rel-RMS {REL_RMS}, lse {LSE_ABS}", "pass": bool(ok)}


def capture(fn, reps: int = 1):
    """A HIP graph of `reps` back-to-back calls of fn (warmed up on a side stream first)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    torch.cuda.synchronize()
    return g


def time_steps(run_step, steps: int, eager: bool) -> float:
    """Wall-clock ms per step over exactly `steps` back-to-back steps: eager calls,
    or graph replays of GRAPH_STEPS steps (plus single-step replays for the rest)."""
    import torch
    if not eager:
        g_one, g_many = capture(run_step), capture(run_step, GRAPH_STEPS)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if eager:
        for _ in range(steps):
            run_step()
    else:
        for _ in range(steps // GRAPH_STEPS):
            g_many.replay()
        for _ in range(steps % GRAPH_STEPS):
            g_one.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def time_phase(fn, steps: int, eager: bool, stream, reps: int = 5) -> float:
    """Mean ms per call of one phase: HIP events on the launch stream around
    `reps` back-to-back calls (one graph replay, or eager calls)."""
    import torch
    runner = (lambda: [fn() for _ in range(reps)]) if eager else capture(fn, reps).replay
    runner()
    torch.cuda.synchronize()
    times = []
    for _ in range(max(2, steps // reps)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        runner()
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) / reps)
    return float(np.mean(times))


WORKLOAD_NAMES = ("decode_8k_b1", "mtp_verify_128k_b64", "swa_decode_32k_b64", "decode_1m_b4",
                  "prefill_chunk_16k_at_112k")
HEADLINE = "mtp_verify_128k_b64"
WINDOW_WORKLOAD = "swa_decode_32k_b64"        # the sliding-window layer
LONG_CONTEXT_WORKLOAD = "decode_1m_b4"        # the index-key scan dominates its bytes
PREFILL_WORKLOAD = "prefill_chunk_16k_at_112k"  # reported against the MFMA peak


def layer_group(args, wl, dev):
    """One hybrid layer group per step (SGLang blog, "Hybrid Attention": three
    sliding-window layers per sparse layer): three window-512 layers, then the
    sparse layer (indexer + top-512 + attention). Each layer has its own seeded
    Q and caches over the same sequences, as the layers of a model do. The
    layers' calls run back to back from one captured graph; in a model the
    other ops of each layer sit between them, which is why the group is a
    schedule of four calls and not one fused kernel."""
    import torch
    from sparse_block_indexed_amd import bytes_model as B
    from sparse_block_indexed_amd import inputs as I
    from sparse_block_indexed_amd import ops
    name = args.workload
    if args.fp8_kv or args.per_group_selection or args.fp8_index_keys:
        raise SystemExit("--layer-group runs the bf16 layers only")
    n_tok, topk, window = wl.n_tok, 512, 512
    pt, sl, qs, qp = wl.device_ints(dev)
    layers = [I.layer_inputs(wl, seed=7000 + 10 * I.WORKLOADS[name][1] + i) for i in range(3)] + [wl]
    Sw = ops.resolve_num_splits(n_tok, window // 8 + 2, args.num_splits)
    Ss = ops.resolve_num_splits(n_tok, topk + 1, args.num_splits)
    f32 = dict(dtype=torch.float32, device=dev)
    outs = [torch.empty((n_tok, 64, 192), dtype=torch.bfloat16, device=dev) for _ in layers]
    lses = [torch.empty((n_tok, 64), **f32) for _ in layers]
    pw = (torch.empty((n_tok, Sw, 64, 192), **f32), torch.empty((n_tok, Sw, 64), **f32)) if Sw > 1 else (None, None)
    ps = (torch.empty((n_tok, Ss, 64, 192), **f32), torch.empty((n_tok, Ss, 64), **f32)) if Ss > 1 else (None, None)
    ctr = ops.merge_counters(n_tok, dev) if max(Sw, Ss) > 1 and args.fused_merge else None
    sel = torch.empty((n_tok, topk), dtype=torch.int32, device=dev)
    ws = torch.empty(ops.indexer_workspace_size(n_tok, wl.max_pages_per_seq, topk), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def swa(i):
        L = layers[i]
        ops.swa_decode(L.q, L.k_cache, L.v_cache, pt, sl, qs, qp, window, SCALE, num_splits=Sw, out=outs[i],
                       out_lse=lses[i], part_o=pw[0], part_lse=pw[1], merge_counters=ctr)

    def indexer():
        ops.indexer_topk(wl.q_idx, wl.k_idx_cache, pt, sl, qs, qp, topk, sel_idx=sel, workspace=ws)

    def sparse():
        ops.sparse_decode(wl.q, wl.k_cache, wl.v_cache, pt, sl, qs, qp, sel, SCALE, num_splits=Ss, out=outs[3],
                          out_lse=lses[3], part_o=ps[0], part_lse=ps[1], merge_counters=ctr)

    def run_group():
        for i in range(3):
            swa(i)
        indexer()
        sparse()

    for _ in range(args.warmup):
        run_group()
    torch.cuda.synchronize()
    ms = time_steps(run_group, args.steps, args.eager)
    ms_eager = time_steps(run_group, args.steps, True) if not args.eager else ms
    phase_ms = {"swa_decode": time_phase(lambda: swa(0), args.steps, args.eager, stream),
                "indexer_topk": time_phase(indexer, args.steps, args.eager, stream),
                "sparse_decode": time_phase(sparse, args.steps, args.eager, stream)}
    run_group()
    torch.cuda.synchronize()
    sel_host = sel.cpu().numpy()
    nbytes = {"swa_decode": B.swa_attention_bytes(wl.q_seq, wl.q_pos, window),
              "indexer_topk": B.indexer_topk_bytes(wl.q_seq, wl.q_pos, topk),
              "sparse_decode": B.sparse_attention_bytes(wl.q_seq, wl.q_pos, sel_host)}
    count = {"swa_decode": 3, "indexer_topk": 1, "sparse_decode": 1}
    dominant = max(phase_ms, key=lambda k: count[k] * phase_ms[k])
    achieved = nbytes[dominant] / (phase_ms[dominant] * 1e-3) / 1e9
    sep = ctr is None
    kname = {"swa_decode": "attention_kernel<true, bf16>%s (sa_swa_decode)" % (" + merge_kernel" if Sw > 1 and sep else ""),
             "indexer_topk": "sa_indexer_topk (score_kernel + select)",
             "sparse_decode": "attention_kernel<false, bf16>%s (sa_sparse_decode)"
                              % (" + merge_kernel" if Ss > 1 and sep else "")}
    group_bytes = sum(count[k] * nbytes[k] for k in nbytes)
    # parity of the timed buffers: the first window layer and the sparse layer, a few tokens each
    _, w_refs = cpu_baseline(layers[0], None, window, budget_s=2.0, max_tokens=4)
    _, s_refs = cpu_baseline(wl, sel_host, None, budget_s=2.0, max_tokens=4)
    parity = {"window_layer_0": parity_check(w_refs, None, outs[0], lses[0]),
              "sparse_layer": parity_check(s_refs, sel_host, outs[3], lses[3])}
    parity["pass"] = all(v["pass"] for v in parity.values())
    return {
        "metric": f"{name} hybrid layer group (3 window + 1 sparse layer) query-tokens/s; achieved HBM GB/s",
        "value": n_tok / (ms * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name + "_layer_group", "layers": "3 x window 512 + 1 x sparse top-512",
                   "batch": wl.batch, "query_tokens": n_tok, "num_splits_window": Sw, "num_splits_sparse": Ss,
                   "kv_cache": "bf16", "launch": "eager" if args.eager else "hip_graph"},
        "eager_ms_per_step": ms_eager,
        "achieved_hbm_gbps": group_bytes / (ms * 1e-3) / 1e9,
        "step_breakdown_ms": {"swa_decode x3": 3 * phase_ms["swa_decode"],
                              "indexer_topk": phase_ms["indexer_topk"],
                              "sparse_decode": phase_ms["sparse_decode"]},
        "per_call_ms": phase_ms,
        "algorithmic_bytes": {k: count[k] * nbytes[k] for k in nbytes},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": None, "kernel": kname[dominant]},
        "parity": parity,
    }


def read_ceiling_gbps(dev, reps: int = 20) -> float:
    """The rate a plain streaming read reaches on this GPU: a 4 GiB float tensor
    summed in rows of 1,024 by torch (HIP events, median of reps)."""
    import torch
    z = torch.ones(1 << 30, dtype=torch.float32, device=dev)
    z.view(-1, 1024).sum(dim=1)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        z.view(-1, 1024).sum(dim=1)
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    del z
    torch.cuda.empty_cache()
    return (4 << 30) / float(np.median(ts)) / 1e9


def ceilings(dev):
    """Practical ceilings of this device, measured with torch's own kernels
    (HIP events, medians): copy and read bandwidth (a 4 GiB float tensor summed
    in rows of 1,024), and the time per step of a
    HIP graph whose steps are chains of n dependent one-element kernels (GRAPH_STEPS
    steps per replay, as the timed loop replays them)."""
    import torch

    def med(fn, reps=20):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    res = {}
    x = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    t = med(lambda: y.copy_(x))
    res["copy_1gib"] = {"us": t * 1e6, "read_plus_write_gbps": 2 * (1 << 30) / t / 1e9}
    del x, y
    # row sums (4 MiB written): torch's full reduction reads at ~4 TB/s only
    res["read_4gib_row_sums"] = {"read_gbps": read_ceiling_gbps(dev)}
    one = torch.zeros(1, dtype=torch.float32, device=dev)
    floor = {}
    for n in (1, 2, 3, 4, 8):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(GRAPH_STEPS * n):
                one.add_(1.0)
        t = med(g.replay)
        g1 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g1):
            for _ in range(n):
                one.add_(1.0)
        t1 = med(g1.replay)
        floor[str(n)] = {"us_per_step": t / GRAPH_STEPS * 1e6, "us_per_replay_of_one_step": t1 * 1e6}
    res["graph_chain_floor"] = floor
    res["how"] = ("medians of 20 timed calls; graph_chain_floor[n]: a graph of %d steps of n dependent "
                  "one-element kernels (per step), and a graph of one such step (per replay)" % GRAPH_STEPS)
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="BLAS threads for the oracle baseline (0: the process default)")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="extra steps, each after a 1 GiB write that evicts L2/MALL (reported separately)")
    ap.add_argument("--workload", default=HEADLINE, choices=WORKLOAD_NAMES,
                    help="the workload (default: the headline %s)" % HEADLINE)
    ap.add_argument("--num-splits", type=int, default=-1,
                    help="partitions per (token, group) for the attention call: a count, 0 (each token's own "
                         "length decides) or -1 (fill the GPU: the count follows the call's size)")
    ap.add_argument("--fp8-index-keys", action="store_true",
                    help="score one-byte (OCP E4M3) index keys: the same integer values, half the bytes")
    ap.add_argument("--fp8-kv", action="store_true",
                    help="attend one-byte (OCP E4M3) K/V caches quantised from the bf16 ones "
                         "(k_scale 1/32, v_scale 1/16)")
    ap.add_argument("--per-group-selection", action="store_true",
                    help="one index query and one top-512 set per (token, KV group) instead of per token")
    ap.add_argument("--layer-group", action="store_true",
                    help="one step = a hybrid layer group: 3 sliding-window layers + 1 sparse layer, each with its "
                         "own Q and caches over the workload's sequences")
    ap.add_argument("--fused-merge", action="store_true",
                    help="split calls merge in the attention launch (the last partition of each token and group "
                         "merges; counters zeroed once) instead of in a second launch")
    ap.add_argument("--eager", action="store_true",
                    help="issue every call from Python instead of replaying captured HIP graphs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling the HBM byte counters)")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure the device's practical ceilings: a 1 GiB device copy, a 4 GiB read "
                         "(torch row sums), and graphs of chains of 1 .. 8 one-element kernels (the launch floor of "
                         "a step of that many dependent kernels)")
    ap.add_argument("--pmc-record", action="store_true",
                    help="host only: write profiles/pmc_<workload>.json from rocprofv3 --pmc output directories")
    ap.add_argument("--pmc-dir", action="append", default=[], metavar="COUNTER=DIR",
                    help="a --pmc run of this workload (FETCH_SIZE, WRITE_SIZE, further counters)")
    ap.add_argument("--pmc-copy", action="append", default=[], metavar="COUNTER=DIR",
                    help="a --pmc run of --copy-calibration (FETCH_SIZE and WRITE_SIZE)")
    args = ap.parse_args()
    if args.pmc_record:
        write_pmc_record(args)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        x = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 1 << 30, "copy_bytes_written": 1 << 30, "launches": 5}))
        return

    if args.ceilings:
        print(json.dumps(ceilings(dev)), flush=True)
        return

    from sparse_block_indexed_amd import bytes_model as B
    from sparse_block_indexed_amd import inputs as I
    from sparse_block_indexed_amd import ops

    ops.load_library()
    assert set(WORKLOAD_NAMES) == set(I.WORKLOADS)
    name = args.workload
    wl = I.named_workload(name, device=dev)
    if args.layer_group:
        res = layer_group(args, wl, dev)
        print(json.dumps(res), flush=True)
        if not res["parity"]["pass"]:
            print("parity check of the timed buffers FAILED", file=sys.stderr)
            sys.exit(3)
        return
    pt, sl, qs, qp = wl.device_ints(dev)
    kidx = I.fp8_e4m3_codes(wl.k_idx_cache) if args.fp8_index_keys else wl.k_idx_cache
    per_group = args.per_group_selection
    qidx = I.grouped_index_queries(wl.n_tok, seed=1000 + I.WORKLOADS[name][1], device=dev) if per_group else wl.q_idx
    if args.fp8_kv:
        k_scale, v_scale = 1.0 / 32, 1.0 / 16
        kc, vc = I.quantize_kv_fp8(wl.k_cache, wl.v_cache, k_scale, v_scale)
        kv_kw = dict(k_scale=k_scale, v_scale=v_scale)
    else:
        kc, vc, kv_kw = wl.k_cache, wl.v_cache, {}
    topk = 512
    window = 512 if name == WINDOW_WORKLOAD else None
    n_tok = wl.n_tok
    max_blocks = (window // 8 + 2) if window else topk + 1
    S = ops.resolve_num_splits(n_tok, max_blocks, args.num_splits)
    sel = torch.empty((n_tok, 4, topk) if per_group else (n_tok, topk), dtype=torch.int32, device=dev)
    ws = None if window else torch.empty(ops.indexer_workspace_size(n_tok, wl.max_pages_per_seq, topk, per_group),
                                         dtype=torch.uint8, device=dev)
    out = torch.empty((n_tok, 64, 192), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((n_tok, 64), dtype=torch.float32, device=dev)
    part_o = torch.empty((n_tok, S, 64, 192), dtype=torch.float32, device=dev) if S > 1 else None
    part_lse = torch.empty((n_tok, S, 64), dtype=torch.float32, device=dev) if S > 1 else None
    # split calls merge in the same launch: arrival counters, zeroed once
    ctr = ops.merge_counters(n_tok, dev) if S > 1 and args.fused_merge else None
    stream = torch.cuda.current_stream()

    def run_indexer():
        ops.indexer_topk(qidx, kidx, pt, sl, qs, qp, topk, sel_idx=sel, workspace=ws)

    def run_attention():
        if window is None:
            ops.sparse_decode(wl.q, kc, vc, pt, sl, qs, qp, sel, SCALE, num_splits=S, out=out,
                              out_lse=lse, part_o=part_o, part_lse=part_lse, merge_counters=ctr, **kv_kw)
        else:
            ops.swa_decode(wl.q, kc, vc, pt, sl, qs, qp, window, SCALE, num_splits=S, out=out,
                           out_lse=lse, part_o=part_o, part_lse=part_lse, merge_counters=ctr, **kv_kw)

    def run_step():
        if window is None:
            run_indexer()
        run_attention()

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    # The step is captured as HIP graphs and replayed (GRAPH_STEPS steps per
    # replay, as a served decode forward replays its layers from one graph):
    # every replay runs all kernels of the step on the same inputs; only the
    # host's per-call argument handling is gone. --eager issues every call.
    launch_step = run_step if args.eager else capture(run_step).replay
    ms_per_step = time_steps(run_step, args.steps, args.eager)
    idx_ms = time_phase(run_indexer, args.steps, args.eager, stream) if window is None else 0.0
    attn_ms = time_phase(run_attention, args.steps, args.eager, stream)
    # leave the step's own results in sel / out for the byte counts below
    run_step()
    torch.cuda.synchronize()

    # cold-cache steps: a 1 GiB write between steps evicts L2 and the 256 MB MALL
    cold_ms = None
    if args.cold_steps > 0:
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        cold = []
        for _ in range(args.cold_steps):
            flush.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch_step()
            e1.record(stream)
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        cold_ms = float(np.mean(cold))
        del flush

    sel_host = sel.cpu().numpy() if window is None else None
    kvb = 1 if args.fp8_kv else 2
    if window is None and per_group:
        attn_bytes = B.sparse_attention_bytes_grouped(wl.q_seq, wl.q_pos, sel_host, kv_bytes=kvb)
        idx_bytes = B.indexer_topk_bytes(wl.q_seq, wl.q_pos, topk, key_bytes=1 if args.fp8_index_keys else 2,
                                         queries_per_token=4)
        attn_flops = sum(B.sparse_attention_flops(wl.q_pos, sel_host[:, g], num_heads=16) for g in range(4))
        idx_flops = 4 * B.indexer_flops(wl.q_pos)
    elif window is None:
        attn_bytes = B.sparse_attention_bytes(wl.q_seq, wl.q_pos, sel_host, kv_bytes=kvb)
        idx_bytes = B.indexer_topk_bytes(wl.q_seq, wl.q_pos, topk, key_bytes=1 if args.fp8_index_keys else 2)
        attn_flops = B.sparse_attention_flops(wl.q_pos, sel_host)
        idx_flops = B.indexer_flops(wl.q_pos)
    else:
        attn_bytes = B.swa_attention_bytes(wl.q_seq, wl.q_pos, window, kv_bytes=kvb)
        idx_bytes, idx_flops = 0, 0
        attn_flops = B.swa_attention_flops(wl.q_pos, window)
    config = {"workload": name, "batch": wl.batch, "query_tokens": n_tok,
              "context": (f"uniform [{wl.spec.seq_len_range[0]}, {wl.spec.seq_len_range[1]}]"
                          if wl.spec.seq_len_range else str(sorted(set(int(x) for x in wl.seq_lens)))),
              "block_tokens": 8, "page_tokens": 64, "heads": "64q/4kv", "head_dim": 192, "num_splits": S}
    config["kv_cache"] = "fp8_e4m3" if args.fp8_kv else "bf16"
    config["launch"] = "eager" if args.eager else "hip_graph"
    config["merge"] = None if S == 1 else ("in the attention launch" if args.fused_merge else "second launch")
    config["num_splits_request"] = {-1: "fill_gpu", 0: "by_length"}.get(args.num_splits, args.num_splits)
    # value: steps back to back with inputs resident in HBM and L2/MALL not flushed between steps
    config["cache"] = "warm"
    if window is None:
        config["topk_blocks"] = topk
        config["index_keys"] = "fp8_e4m3" if args.fp8_index_keys else "bf16"
        config["selection"] = "per_kv_group" if per_group else "per_token"
    else:
        config["window"] = window
    tags = [t for t, on in (("fp8 index keys", args.fp8_index_keys), ("fp8 KV", args.fp8_kv),
                            ("per-KV-group selection", per_group)) if on]
    metric = METRIC if (name == HEADLINE and not tags) else \
        f"{name}{' (' + ', '.join(tags) + ')' if tags else ''} query-tokens/s; achieved HBM GB/s"
    result = {
        "metric": metric,
        "value": n_tok / (ms_per_step * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": config,
        "achieved_hbm_gbps": (attn_bytes + idx_bytes) / (ms_per_step * 1e-3) / 1e9,
        "step_breakdown_ms": ({} if window else {"indexer_topk": idx_ms}) |
                             {("swa_decode" if window else "sparse_decode"): attn_ms},
        "algorithmic_bytes": {"indexer_topk": idx_bytes, ("swa_decode" if window else "sparse_decode"): attn_bytes},
        "algorithmic_flops": {"indexer_topk": idx_flops, ("swa_decode" if window else "sparse_decode"): attn_flops},
    }
    kname = "attention_kernel<%s, %s>%s (%s%s)" % ("true" if window else "false", "fp8" if args.fp8_kv else "bf16",
                                                   " + merge_kernel" if S > 1 and not args.fused_merge else "",
                                                   "sa_swa_decode" if window else "sa_sparse_decode",
                                                   "_fp8kv" if args.fp8_kv else "")
    if name == PREFILL_WORKLOAD:
        # the prefill chunk is a dense-contraction workload on paper: report MFMA utilisation
        tf = (attn_flops + idx_flops) / (ms_per_step * 1e-3) / 1e12
        result["mfma_utilisation"] = tf / (PEAK_BF16_TFLOPS)
        attn_tf = attn_flops / (attn_ms * 1e-3) / 1e12
        traffic = None if tags else counter_traffic(name, "sparse_decode")
        result["roofline"] = {"bound": "mfma", "achieved": attn_tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                              "frac": attn_tf / PEAK_BF16_TFLOPS, "traffic": traffic, "kernel": kname}
        if not tags:
            # the MFMA counters of the same kernel (rocprofv3 --pmc MfmaUtil, MfmaFlopsBF16), and the rate of
            # its counted HBM traffic: the gathered K/V, not the matrix cores, bound this kernel
            util = counter_mean(name, "sparse_decode", "attention_kernel", "MfmaUtil")
            flops = counter_mean(name, "sparse_decode", "attention_kernel", "MfmaFlopsBF16")
            result["roofline"]["counters"] = {
                "mfma_util_pct": util, "mfma_flops_bf16_per_launch": flops,
                "hbm_traffic_gbps": None if traffic is None else traffic / (attn_ms * 1e-3) / 1e9}
    elif name == LONG_CONTEXT_WORKLOAD:
        # at 1M context the index-key scan is the dominant read
        achieved = idx_bytes / (idx_ms * 1e-3) / 1e9
        result["roofline"] = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                              "frac": achieved / PEAK_HBM_GBPS,
                              "traffic": None if tags else counter_traffic(name, "indexer_topk"),
                              "kernel": "sa_indexer_topk (score_kernel + select_kernel)"}
    else:
        achieved = attn_bytes / (attn_ms * 1e-3) / 1e9
        result["roofline"] = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                              "frac": achieved / PEAK_HBM_GBPS,
                              "traffic": None if tags else counter_traffic(name, "swa_decode" if window
                                                                           else "sparse_decode"),
                              "kernel": kname}
    # the same kernel against what a plain streaming read reaches on this GPU
    # (measured here, after the timed loop); for the prefill chunk its counted
    # HBM traffic rate is compared
    ceiling = read_ceiling_gbps(dev)
    rl = result["roofline"]
    rate = rl["achieved"] if rl["unit"] == "GB/s" else rl.get("counters", {}).get("hbm_traffic_gbps")
    rl["read_ceiling_gbps"] = ceiling
    rl["frac_of_read_ceiling"] = None if rate is None else rate / ceiling
    if cold_ms is not None:
        result["cold_cache"] = {"ms_per_step": cold_ms, "query_tokens_per_s": n_tok / (cold_ms * 1e-3),
                                "how": "one-step graph replays timed with HIP events, each after a 1 GiB write "
                                       "that evicts L2 and the 256 MB MALL"}
    # The oracle leg: timed on the host as the CPU baseline, and its results
    # compared with the buffers of the step just timed (outside the timed loop).
    # With --no-cpu-baseline the oracle still runs a few tokens for the check.
    import contextlib
    limit = contextlib.nullcontext()
    if args.cpu_threads > 0:   # cap the oracle's BLAS threads (e.g. 1 for a one-core figure)
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=args.cpu_threads)
    with limit:
        baseline, refs = cpu_baseline(wl, sel_host, window,
                                      budget_s=2.0 if args.no_cpu_baseline else 20.0,
                                      max_tokens=4 if args.no_cpu_baseline else 64,
                                      kv_fp8=(kc, vc, kv_kw["k_scale"], kv_kw["v_scale"]) if args.fp8_kv else None,
                                      q_groups=qidx if per_group else None,
                                      kidx_fp8=kidx if args.fp8_index_keys else None)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = baseline
    result["parity"] = parity_check(refs, sel_host, out, lse)
    print(json.dumps(result), flush=True)
    if not result["parity"]["pass"]:
        print("parity check of the timed buffers FAILED", file=sys.stderr)
        sys.exit(3)


if __name__ == "__main__":
    main()
