#!/usr/bin/env python3
"""Benchmark one Orthrus dual-view decode step on one MI355X.

A step is the whole hot path for one batch: for every one of 36 layers the
diffusion-view block attention, then for every layer the AR verify block
attention (each layer streams its own shared KV cache; the diffusion pass of
all layers runs before the verify pass, as in the decode cycle of the Orthrus
paper notes §4.1), then one greedy consensus over the [K, 151936] verify
logits.  Default workload: Qwen3-8B attention shapes (32 q heads, 8 KV heads,
head_dim 128), cached prefix L = 32768, block K = 32, batch 1, synthetic
N(0, 1) bf16 inputs resident in HBM.

Prints ONE JSON line (rank 0, N = 1).  `value` is the achieved HBM throughput
of the whole step in TB/s: the algorithmic bytes of the step (each layer-view
reads its cache, q and block K/V and writes its output; the consensus reads
the logits) divided by the step time.
"""
from __future__ import annotations

import argparse
import contextlib
import ctypes
import json
import os
import statistics
import sys
import time

METRIC = "dual-view step µs and achieved HBM TB/s at Qwen3-8B shape, L=32K, K=32"
HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "attn_stream_traffic.json")
ATTN_SOURCE = os.path.join(ROOT, "dual_view_block_amd", "csrc", "attention.hip")
STREAM_KERNEL = "attn_stream_kernel"
COPY_KERNEL = "copyBuffer"  # the runtime's device-to-device copy kernel


class _Markers:
    """roctx ranges around the bench phases, so that a trace taken with
    `rocprofv3 --marker-trace` shows where each phase's kernels fall.  The
    marker library of the ROCm profiler SDK is loaded if present; without it
    every range is a no-op."""

    def __init__(self):
        self.lib = None
        for name in ("librocprofiler-sdk-roctx.so.1", "librocprofiler-sdk-roctx.so"):
            for path in (name, os.path.join("/opt/rocm/lib", name)):
                try:
                    lib = ctypes.CDLL(path)
                except OSError:
                    continue
                lib.roctxRangePushA.argtypes, lib.roctxRangePushA.restype = [ctypes.c_char_p], ctypes.c_int
                lib.roctxRangePop.argtypes, lib.roctxRangePop.restype = [], ctypes.c_int
                self.lib = lib
                return

    @contextlib.contextmanager
    def range(self, name: str):
        if self.lib is not None:
            self.lib.roctxRangePushA(("bench:" + name).encode())
        try:
            yield
        finally:
            if self.lib is not None:
                self.lib.roctxRangePop()


MARKERS = _Markers()


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_8b_32k")
    ap.add_argument("--cache-len", type=int, default=None)
    ap.add_argument("--block-k", type=int, default=None)
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--k-sweep", default="1,4,8,16,32,64,128",
                    help="block sizes timed for the latency-vs-K line ('' to skip)")
    ap.add_argument("--graph", action="store_true", help="replay the step as one HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cycles", type=int, default=64,
                    help="synthetic decode cycles timed after the step (0 to skip): per cycle both "
                         "views of every layer, greedy consensus and the cache commit, replayed "
                         "from a HIP graph")
    ap.add_argument("--cycle-sets", type=int, default=32,
                    help="distinct input sets the cycles rotate through (one graph round); their "
                         "first-mismatch indices are the quantiles of the acceptance law")
    ap.add_argument("--t0-cycles", type=int, default=64,
                    help="synthetic T>0 decode cycles timed (0 to skip): as --cycles, with the rejection-"
                         "sampling consensus over target and draft probabilities and given uniforms")
    ap.add_argument("--t0-sets", type=int, default=8, help="input sets the T>0 cycles rotate through")
    ap.add_argument("--t0-noise", type=float, default=0.2,
                    help="draft logits = target logits + N(0, noise) for the T>0 cycles (0.2 gives a "
                         "per-candidate acceptance of about 0.92 at sigma 3, V 151936)")
    ap.add_argument("--tree-cycles", type=int, default=32,
                    help="synthetic tree-verification cycles timed (0 to skip): per cycle the diffusion "
                         "attention of every layer, top-m marginals, a best-first draft tree, its masks, the "
                         "tree-masked verify attention of every layer, tree consensus and the path commit")
    ap.add_argument("--kl-rows", type=int, default=8192,
                    help="rows of the forward-KL measurement (256 blocks x K = 32 diffusion positions "
                         "of one packed training sequence; 0 to skip)")
    ap.add_argument("--train-attn", type=int, default=1,
                    help="time the training dual-pass attention (forward and diffusion-row backward) of "
                         "one packed 2048-token sequence at the workload's heads (0 to skip)")
    ap.add_argument("--configs", type=int, default=1,
                    help="also time the other configuration points (C2, C3, C4 at L=131072, C5); 0 skips")
    ap.add_argument("--dyn-k", type=int, default=1,
                    help="time dynamic block sizes: the step at live block lengths 1..K and adaptive-length "
                         "decode cycles against fixed-K cycles (0 to skip)")
    ap.add_argument("--dyn-k-min", type=int, default=4, help="floor of the adaptive block length")
    ap.add_argument("--dyn-low-rate", type=float, default=0.5,
                    help="the low per-candidate match rate the adaptive cycles are also timed at")
    ap.add_argument("--accept-rate", type=float, default=0.912,
                    help="per-candidate match probability of the synthetic acceptance law "
                         "(0.912: 10.8 tokens per cycle at K = 32)")
    ap.add_argument("--traffic", default=TRAFFIC_JSON,
                    help="JSON record of rocprofv3-derived HBM bytes per streaming-kernel launch "
                         "(ignored if the code of attention.hip changed since it was taken)")
    ap.add_argument("--profile-target", choices=["attn-stream", "copy", "forward-kl", "train-attn", "consensus"],
                    default=None,
                    help="run only the streaming kernel over every layer-view (or a plain copy "
                         "kernel of --copy-mib MiB, or the forward KL with its gradient at "
                         "--kl-rows x vocab) --steps times, for rocprofv3 counter runs")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--summarize-trace", metavar="RESULTS_DB",
                    help="print per-kernel durations (markdown) from a rocprofv3 --kernel-trace "
                         "results database and exit")
    ap.add_argument("--trace-phases", default=None,
                    help="with --summarize-trace: streaming-kernel dispatch ranges to summarise separately "
                         "(label=a:b,...; bench.py prints them for its own run)")
    ap.add_argument("--make-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                        "COPY_WRITE_CSV"),
                    help="turn four rocprofv3 --pmc counter_collection.csv files into the traffic "
                         "record (written to --traffic) and exit")
    return ap.parse_args()


def attn_bytes(w) -> int:
    """Algorithmic bytes of one layer-view: cache K+V rows [0, L), q, k/v block, out."""
    return stream_bytes(w) + w.batch * w.n_q_heads * w.block_k * w.head_dim * 2  # out has q's shape


def stream_bytes(w) -> int:
    """Algorithmic bytes the streaming kernel reads: cache K+V rows [0, L), q, k/v block."""
    bf = 2
    cache = 2 * w.batch * w.n_kv_heads * w.cache_len * w.head_dim * bf
    q = w.batch * w.n_q_heads * w.block_k * w.head_dim * bf
    blk = 2 * w.batch * w.n_kv_heads * w.block_k * w.head_dim * bf
    return cache + q + blk


def _code_sha256(path: str) -> str:
    """SHA-256 of a C++/HIP source with comments and whitespace removed: it
    changes whenever the code does, not when only its comments do."""
    import hashlib
    import re

    with open(path) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = re.sub(r"\s+", " ", src).strip()
    return hashlib.sha256(src.encode()).hexdigest()


def _counter_kib(csv_path: str, kernel: str, counter: str) -> float:
    """Mean per-dispatch value of `counter` over the dispatches of `kernel`."""
    import csv

    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not vals:
        raise SystemExit(f"no {counter} rows for {kernel} in {csv_path}")
    return sum(vals) / len(vals)


def make_traffic(paths, out_path: str, copy_mib: int) -> None:
    """HBM bytes per streaming launch: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) each scaled by what the same counter reads for a plain copy
    kernel of known size (copy_mib MiB read, copy_mib MiB written)."""
    f_csv, w_csv, cf_csv, cw_csv = paths
    fetch = _counter_kib(f_csv, STREAM_KERNEL, "FETCH_SIZE")
    write = _counter_kib(w_csv, STREAM_KERNEL, "WRITE_SIZE")
    cfetch = _counter_kib(cf_csv, COPY_KERNEL, "FETCH_SIZE")
    cwrite = _counter_kib(cw_csv, COPY_KERNEL, "WRITE_SIZE")
    nbytes = copy_mib * 2**20
    rf, rw = nbytes / cfetch, nbytes / cwrite  # true bytes per counted KiB
    rec = {"kernel": STREAM_KERNEL, "code_sha256": _code_sha256(ATTN_SOURCE),
           "fetch_kib_per_launch": fetch, "write_kib_per_launch": write,
           "copy_bytes_each_way": nbytes, "copy_fetch_kib": cfetch, "copy_write_kib": cwrite,
           "fetch_bytes_per_kib": rf, "write_bytes_per_kib": rw,
           "read_bytes_per_launch": round(fetch * rf), "write_bytes_per_launch": round(write * rw),
           "bytes_per_launch": round(fetch * rf + write * rw)}
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def load_traffic(path: str):
    """bytes_per_launch of the traffic record, or None if absent or stale."""
    if not path or not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("code_sha256") != _code_sha256(ATTN_SOURCE):
        print("[bench] traffic record predates the current attention.hip: reporting null",
              file=sys.stderr, flush=True)
        return None
    return rec.get("bytes_per_launch")


def summarize_trace(db_path: str, phases: str = None) -> None:
    """Per-kernel duration statistics of a rocprofv3 kernel-trace database
    (every dispatch of the library's kernels it holds), as a markdown table,
    plus the median idle gap between consecutive dispatches.  `phases`
    ("label=a:b,label=a:b", as bench.py prints them) adds the statistics of
    the streaming kernel's dispatches a..b-1 (in launch order) of each phase."""
    import re
    import sqlite3

    con = sqlite3.connect(db_path)
    rows = list(con.execute("select name, start, end, grid_x, grid_y, grid_z, workgroup_x from kernels "
                            "order by start"))
    rows = [r for r in rows if "orthrus::" in r[0]]   # the library's kernels only
    groups = {}
    for name, t0, t1, gx, gy, gz, wg in rows:
        nm = re.sub(r"\(.*", "", name.replace("(anonymous namespace)::", "").replace("void ", ""))
        groups.setdefault((nm, gx, gy, gz, wg), []).append((t1 - t0) / 1e3)
    print("| kernel | grid (threads) | wg | dispatches | mean µs | median µs | min µs | p90 µs |")
    print("|---|---|---|---|---|---|---|---|")
    for (nm, gx, gy, gz, wg), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        v = sorted(v)
        print(f"| {nm} | {gx} × {gy} × {gz} | {wg} | {len(v)} | {statistics.mean(v):.2f} | "
              f"{statistics.median(v):.2f} | {v[0]:.2f} | {v[int(0.9 * (len(v) - 1))]:.2f} |")
    if phases:
        # the streaming kernel's most frequent (grid, work-group) launch shape
        key = max((k for k in groups if "attn_stream_kernel" in k[0]), key=lambda k: len(groups[k]))
        durs = groups[key]  # in launch order (rows are sorted by start)
        print()
        print(f"Phases of {key[0]} ({key[1]} × {key[2]} × {key[3]}), dispatch index ranges in launch order:")
        print()
        print("| phase | dispatches | mean µs | median µs | min µs |")
        print("|---|---|---|---|---|")
        for item in phases.split(","):
            label, rng = item.split("=")
            a, b = (int(x) for x in rng.split(":"))
            v = durs[a:b]
            if not v:
                continue
            sv = sorted(v)
            print(f"| {label} | {len(v)} | {statistics.mean(v):.2f} | {statistics.median(v):.2f} | {sv[0]:.2f} |")
    gaps = {}
    for a, b in zip(rows, rows[1:]):
        key = tuple(re.sub(r"[<(].*", "", x[0].replace("(anonymous namespace)::", "")).split("::")[-1]
                    for x in (a, b))
        gaps.setdefault(key, []).append((b[1] - a[2]) / 1e3)
    print()
    for (na, nb), v in sorted(gaps.items()):
        if len(v) > 3:
            print(f"- gap {na} -> {nb}: {len(v)} pairs, median {statistics.median(v):.2f} µs")


def greedy_bytes(w) -> int:
    return w.batch * w.block_k * (w.vocab * 4 + 4) + w.batch * (4 + 4) + w.batch * w.block_k * 4


def attn_flops(w, causal: bool) -> int:
    """2 matmuls (QK^T, PV) over the visible keys of every query row."""
    L, K = w.cache_len, w.block_k
    vis = K * (L + (K + 1) / 2.0) if causal else K * (L + K)
    return int(4 * w.batch * w.n_q_heads * w.head_dim * vis)


class Step:
    """Every call of one decode step, prepared once (pointers resolved).  With
    ``blk_len`` (int32 [B] on the device) every call runs over each sequence's
    first blk_len[b] block positions (dynamic block sizes)."""

    def __init__(self, w, caches, device, blk_len=None):
        import torch

        import dual_view_block_amd as dvb
        from synth import cache_lengths, greedy_inputs, view_inputs

        self.w = w
        self.cache_len = cache_lengths(w, device)
        self.calls = {"diff": [], "verify": []}
        self.keep = []
        desc_q = torch.empty((w.batch, w.n_q_heads, w.block_k, w.head_dim), dtype=torch.bfloat16,
                             device=device)
        ws_bytes = dvb.orthrus_attn_workspace_size(dvb.attn_desc(desc_q, caches[0][0]))
        self.splits = dvb.orthrus_attn_num_splits(dvb.attn_desc(desc_q, caches[0][0]))
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
        for view, mode in (("diff", dvb.ORTHRUS_MASK_DIFF_BIDIR), ("verify", dvb.ORTHRUS_MASK_VERIFY_CAUSAL)):
            for layer, (kc, vc) in enumerate(caches):
                q, kb, vb = view_inputs(w, layer, view, device)
                out = torch.empty_like(q)
                lse = torch.empty(q.shape[:3], dtype=torch.float32, device=device)
                self.calls[view].append(dvb.PreparedAttention(mode, q, kb, vb, kc, vc, self.cache_len, out,
                                                              lse, ws, blk_len=blk_len))
        logits, cand, _ = greedy_inputs(w, device=device)
        B, K = w.batch, w.block_k
        self.acc = torch.empty(B, dtype=torch.int32, device=device)
        self.am = torch.empty((B, K), dtype=torch.int32, device=device)
        self.corr = torch.empty(B, dtype=torch.int32, device=device)
        cws = torch.empty(dvb.orthrus_consensus_workspace_size(B, K, w.vocab), dtype=torch.uint8, device=device)
        self.greedy = dvb.PreparedGreedy(logits, cand, self.acc, self.am, self.corr, cws, blk_len=blk_len)
        self.keep += [logits, cand, ws, cws]

    def run(self, stream_ptr: int) -> None:
        for c in self.calls["diff"]:
            c(stream_ptr)
        for c in self.calls["verify"]:
            c(stream_ptr)
        self.greedy(stream_ptr)


def time_steps(step, steps: int, warmup: int, graph: bool):
    import torch

    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    g = None
    if graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step.run(side.cuda_stream)  # warm the side stream before capture
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step.run(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
    run = (lambda: g.replay()) if g is not None else (lambda: step.run(sp))
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(steps):
        run()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    return t0.elapsed_time(t1) / steps, wall / steps * 1e3


KERNEL_WARM_RUNS, KERNEL_TIMED_RUNS = 1, 5


def time_kernels(step, reps: int = KERNEL_TIMED_RUNS, warm: int = KERNEL_WARM_RUNS):
    """Average device duration per launch, from HIP events on the launch stream
    around a run of back-to-back launches over every layer of both views: the
    streaming kernel alone (orthrus_block_attn_partial), the merge kernel alone
    (orthrus_block_attn_merge) and the whole call (orthrus_block_attn_*).  After
    `warm` untimed runs, the median over `reps` timed runs is reported (the
    first run after the steps measured up to 10 % slower than the rest)."""
    import torch

    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    calls = step.calls["diff"] + step.calls["verify"]
    out = {}
    for what in ("stream", "merge", "call"):
        per = []
        fns = [c.partial if what == "stream" else (c.merge if what == "merge" else c.__call__) for c in calls]
        for _ in range(warm):
            for fn in fns:
                fn(sp)
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for fn in fns:
                fn(sp)
            e1.record(stream)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) * 1e3 / len(fns))
        out[f"attn_{what}_us"] = statistics.median(per)
    out["launches_per_run"] = len(calls)
    return out


def commit_bytes(w, rows: float) -> float:
    """Algorithmic bytes of one all-layer commit of `rows` rows per sequence:
    the block rows read and the cache rows written (K and V), plus the small
    per-sequence state (length, accept count, correction, candidates in; length,
    anchor, tokens, token count out)."""
    kv = 2 * w.layers * w.batch * w.n_kv_heads * rows * w.head_dim * 2
    state = w.batch * (4 * 4 + 2 * 4 * w.block_k + 4 * 3)
    return 2 * kv + state


def cycle_sets(w, n_sets: int, accept_rate: float, device):
    """Input sets of synthetic decode cycles: first mismatches at the quantiles
    of the truncated geometric law with per-candidate match rate
    `accept_rate`."""
    from synth import cycle_inputs

    sets = cycle_inputs(w, n_sets, accept_rate=accept_rate, device=device, stratified=True)
    for s in sets:
        s["logits"], s["cand"] = s["logits"].to(device), s["cand"].to(device)
    return sets


def sample_cycle_sets(w, n_sets: int, noise: float, device):
    """Input sets of synthetic T>0 decode cycles: target and draft
    probabilities (draft logits = target logits + N(0, noise)), candidates
    drawn from the draft and the uniforms of the accept tests."""
    from synth import sample_cycle_inputs

    return sample_cycle_inputs(w, n_sets, draft_noise=noise, device=device)


def time_cycles(w, kc_all, vc_all, device, n_cycles: int, n_sets: int, accept_rate: float, sets=None,
                k_min: int = 0):
    """Synthetic decode cycles (both views of every layer, greedy consensus --
    or T>0 consensus when the input sets carry probabilities -- and the
    commit) issued through dual_view_block_amd.cycle.DecodeCycles: one round of
    `n_sets` cycles is captured into a HIP graph and replayed; lengths advance
    on the device.  With k_min > 0 the block length is adaptive: every
    sequence starts at K and the commit's rule sets each next length (floor
    k_min).  Returns a dict of the measured figures."""
    import torch

    from dual_view_block_amd.cycle import DecodeCycles
    from synth import cache_lengths

    lens = cache_lengths(w, device)
    if sets is None:
        sets = cycle_sets(w, n_sets, accept_rate, device)
    blk = None
    if k_min > 0:
        blk = torch.full((w.batch,), w.block_k, dtype=torch.int32, device=device)
    drv = DecodeCycles(kc_all, vc_all, lens, sets, blk_len=blk, k_min=max(k_min, 1))
    drv.run(n_sets)                      # eager warm-up round
    torch.cuda.synchronize()
    drv.capture()
    torch.cuda.synchronize()
    rounds = max(1, n_cycles // n_sets)
    stream = torch.cuda.current_stream()
    l0 = lens.clone()
    k_seen = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record(stream)
    drv.replay(rounds)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    tokens = int((lens - l0).sum().item())
    if blk is not None:  # block lengths the timed cycles ended with, then one more eager round to sample them
        k_end = blk.cpu().tolist()
        for c in range(n_sets):
            k_seen.append(int(blk[0].item()))
            drv.issue(c)
        torch.cuda.synchronize()
    cycles = rounds * n_sets
    us = e0.elapsed_time(e1) * 1e3 / cycles
    n_tok = [int(x) for s in range(n_sets) for x in drv.n_tokens[s].cpu().tolist()]

    # the commit alone: back-to-back all-layer commits of one input set on the same stream
    commit = drv._calls[0][-1]
    reps = 16
    sp = stream.cuda_stream
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(reps):
        commit(sp)
    c1.record(stream)
    torch.cuda.synchronize()
    commit_us = c0.elapsed_time(c1) * 1e3 / reps
    rows = float(drv.n_tokens[0].float().mean().item())
    del drv
    extra = {}
    if blk is not None:
        extra = {"block_len": "adaptive", "k_min": k_min, "block_len_after_timed_cycles": k_end,
                 "block_len_per_cycle_one_round": k_seen,
                 "mean_block_len": round(sum(k_seen) / len(k_seen), 2)}
    return {**extra, "cycles": cycles, "input_sets": n_sets, "launch": "hip_graph",
            "us_per_cycle": round(us, 2), "cycles_per_s": round(1e6 / us, 2),
            "host_wall_us_per_cycle": round(wall / cycles * 1e6, 2),
            "tokens_per_cycle": round(tokens / (cycles * w.batch), 3),
            "tokens_per_s": round(tokens / (us * 1e-6 * cycles), 1),
            "accept_rate": accept_rate, "n_tokens_per_set": n_tok,
            "cache_len_after": lens.cpu().tolist(),
            "commit_us": round(commit_us, 3), "commit_rows": rows,
            "commit_achieved_gbs": round(commit_bytes(w, rows) / (commit_us * 1e-6) / 1e9, 1)}


def time_dynamic_k(w, caches, kc_all, vc_all, device, args, fixed_cycles):
    """Dynamic block sizes.  (1) The step with every sequence's block length
    set to k (capacity K): both views of every layer and the greedy consensus
    over the first k positions.  (2) Decode cycles whose block length adapts
    (start K, floor k_min) against fixed-K cycles on the same input sets, at the
    default match rate and at a low one."""
    import torch

    blk = torch.full((w.batch,), w.block_k, dtype=torch.int32, device=device)
    st = Step(w, caches, device, blk_len=blk)
    by_k = {}
    for k in (1, 4, 8, 16, w.block_k):
        if k > w.block_k:
            continue
        blk.fill_(k)
        mk, _ = time_steps(st, args.steps, args.warmup, False)
        by_k[k] = round(mk * 1e3, 2)
        print(f"[bench] live block length {k} of {w.block_k}: step {mk * 1e3:.1f} us", file=sys.stderr, flush=True)
    del st
    out = {"step_us_vs_live_block_len": by_k, "k_min": args.dyn_k_min, "cycles": {}}
    for rate in (args.accept_rate, args.dyn_low_rate):
        sets = cycle_sets(w, args.cycle_sets, rate, device)
        fixed = fixed_cycles if (rate == args.accept_rate and fixed_cycles is not None) else \
            time_cycles(w, kc_all, vc_all, device, args.cycles, args.cycle_sets, rate, sets=sets)
        adapt = time_cycles(w, kc_all, vc_all, device, args.cycles, args.cycle_sets, rate, sets=sets,
                            k_min=args.dyn_k_min)
        keep = ("us_per_cycle", "tokens_per_cycle", "tokens_per_s")
        out["cycles"][str(rate)] = {
            "fixed_k": {k: fixed[k] for k in keep},
            "adaptive": {k: adapt[k] for k in keep + ("mean_block_len", "block_len_per_cycle_one_round")},
            "adaptive_over_fixed_tokens_per_s": round(adapt["tokens_per_s"] / fixed["tokens_per_s"], 3)}
        print(f"[bench] match rate {rate}: fixed K={w.block_k} {fixed['tokens_per_s']:.0f} tokens/s "
              f"({fixed['us_per_cycle']:.0f} us/cycle), adaptive {adapt['tokens_per_s']:.0f} tokens/s "
              f"({adapt['us_per_cycle']:.0f} us/cycle, mean block {adapt['mean_block_len']})",
              file=sys.stderr, flush=True)
        del sets
    # a larger capacity: K = 128 buffers whose live block is 32, and adaptive
    # cycles at that capacity against fixed K = 128 cycles (8 input sets)
    if w.block_k < 128:
        w128 = w.replace(block_k=128)
        blk128 = torch.full((w.batch,), 128, dtype=torch.int32, device=device)
        st = Step(w128, caches, device, blk_len=blk128)
        cap = {}
        for k in (32, 128):
            blk128.fill_(k)
            mk, _ = time_steps(st, args.steps, args.warmup, False)
            cap[k] = round(mk * 1e3, 2)
        del st
        sets = cycle_sets(w128, 8, args.accept_rate, device)
        fixed = time_cycles(w128, kc_all, vc_all, device, 16, 8, args.accept_rate, sets=sets)
        adapt = time_cycles(w128, kc_all, vc_all, device, 16, 8, args.accept_rate, sets=sets, k_min=args.dyn_k_min)
        keep = ("us_per_cycle", "tokens_per_cycle", "tokens_per_s")
        out["capacity_128"] = {
            "step_us_vs_live_block_len": cap,
            "cycles_at_match_rate": args.accept_rate,
            "fixed_k128": {k: fixed[k] for k in keep},
            "adaptive": {k: adapt[k] for k in keep + ("mean_block_len",)},
            "adaptive_over_fixed_tokens_per_s": round(adapt["tokens_per_s"] / fixed["tokens_per_s"], 3)}
        print(f"[bench] capacity 128: step {cap[32]:.0f} us at live 32, {cap[128]:.0f} us at 128; cycles at rate "
              f"{args.accept_rate}: fixed K=128 {fixed['tokens_per_s']:.0f} tokens/s, adaptive "
              f"{adapt['tokens_per_s']:.0f} tokens/s (mean block {adapt['mean_block_len']})", file=sys.stderr, flush=True)
        del sets
    return out


def time_forward_kl(device, rows: int, vocab: int, reps: int = 10):
    """Fused forward KL(P_AR || P_Diff) over the vocabulary (the distillation
    loss) on bf16 logits [rows, vocab]: the loss alone and the loss with its
    draft-logit gradient, each timed with HIP events around `reps` back-to-back
    calls on the launch stream.  Algorithmic bytes: both logit arrays read once
    (+ the bf16 gradient written once, + the fp32 losses)."""
    import torch

    import dual_view_block_amd as dvb
    from synth import kl_inputs

    a, b = kl_inputs(rows, vocab, 3.0, torch.bfloat16, seed=5, device=device)
    kl = torch.empty(rows, dtype=torch.float32, device=device)
    grad = torch.empty_like(a)
    ws = torch.empty(dvb.orthrus_kl_workspace_size(rows, vocab, torch.bfloat16), dtype=torch.uint8, device=device)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    out = {"rows": rows, "vocab": vocab, "dtype": "bf16"}
    for name, g in (("loss", None), ("loss_and_grad", grad)):
        call = dvb.PreparedForwardKL(a, b, kl, g, ws, grad_scale=1.0 / rows)
        call(sp)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call(sp)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        nbytes = 2 * rows * vocab * 2 + rows * 4 + (rows * vocab * 2 if g is not None else 0)
        gbs = nbytes / (us * 1e-6) / 1e9
        out[name] = {"us": round(us, 2), "algorithmic_bytes": nbytes, "achieved_gbs": round(gbs, 1),
                     "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    out["mean_kl"] = round(float(kl.mean().item()), 4)
    del a, b, grad
    return out


def _time_calls(fn, reps: int, stream) -> float:
    """Average µs of `fn()` over `reps` back-to-back calls (HIP events on `stream`)."""
    import torch

    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


# The other configuration points, timed as whole steps on their own caches:
# (label, workload, overrides).  C4 at L = 131072 is timed over its K sweep.
CONFIG_POINTS = (
    ("C2", "qwen3_1p7b_layer", {}),
    ("C3", "qwen3_8b_8k", {}),
    ("C4", "qwen3_8b_128k", {}),
    ("C4", "qwen3_8b_128k", {"block_k": 1}),
    ("C4", "qwen3_8b_128k", {"block_k": 4}),
    ("C4", "qwen3_8b_128k", {"block_k": 8}),
    ("C4", "qwen3_8b_128k", {"block_k": 16}),
    ("C5", "ragged_b16", {}),
)


def step_bytes_lens(w, len_sum: int) -> int:
    """Algorithmic bytes of one step when the sequences' cached lengths sum to
    `len_sum`: every layer-view reads its cache rows, q and the block K/V and
    writes its output; the greedy consensus reads the logits."""
    bf = 2
    cache = 2 * w.n_kv_heads * len_sum * w.head_dim * bf
    q = w.batch * w.n_q_heads * w.block_k * w.head_dim * bf
    blk = 2 * w.batch * w.n_kv_heads * w.block_k * w.head_dim * bf
    return 2 * w.layers * (cache + 2 * q + blk) + greedy_bytes(w)


class _SampleStep:
    """A step whose consensus is the T>0 rejection sampler instead of greedy."""

    def __init__(self, step, sample_call):
        self.step, self.sample_call = step, sample_call

    def run(self, stream_ptr: int) -> None:
        for c in self.step.calls["diff"] + self.step.calls["verify"]:
            c(stream_ptr)
        self.sample_call(stream_ptr)


def time_configs(device, steps: int, warmup: int):
    """Step time of every other configuration point (eager launches, HIP events
    on the launch stream, as for the headline step).  The ragged batch is also
    timed with the T>0 sampler as its consensus, and the sampler alone."""
    import torch

    import dual_view_block_amd as dvb
    from synth import WORKLOADS, model_cache, sample_inputs

    out = {}
    for label, name, kw in CONFIG_POINTS:
        w = WORKLOADS[name].replace(**kw)
        kc, vc = model_cache(w, device)
        caches = [(kc[layer], vc[layer]) for layer in range(w.layers)]
        st = Step(w, caches, device)
        ms, _ = time_steps(st, steps, warmup, False)
        len_sum = int(st.cache_len.sum().item())
        nbytes = step_bytes_lens(w, len_sum)
        rec = {"config": label, "workload": w.name, "layers": w.layers, "batch": w.batch,
               "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
               "cache_len": (f"U{{{w.ragged_min}..{w.cache_len}}}" if w.ragged_min else w.cache_len),
               "cache_len_sum": len_sum, "block_k": w.block_k, "consensus": "greedy",
               "step_us": round(ms * 1e3, 2), "algorithmic_bytes_per_step": nbytes,
               "achieved_tbs": round(nbytes / (ms * 1e-3) / 1e12, 4),
               "frac_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               "tokens_verified_per_s": round(w.batch * w.block_k / (ms * 1e-3), 1)}
        if label == "C5":
            p, q, cand, u = sample_inputs(w, device=device)
            B, K, V = p.shape
            acc = torch.empty(B, dtype=torch.int32, device=device)
            corr = torch.empty(B, dtype=torch.int32, device=device)
            sws = torch.empty(dvb.orthrus_consensus_workspace_size(B, K, V), dtype=torch.uint8, device=device)

            def sample(sp, p=p, q=q, cand=cand, u=u, acc=acc, corr=corr, sws=sws):
                dvb.orthrus_consensus_sample(p, q, cand, u, acc, corr, sws, stream=sp)

            stream = torch.cuda.current_stream()
            rec["sample_consensus_us"] = round(_time_calls(lambda: sample(stream.cuda_stream), 20, stream), 2)
            ms_s, _ = time_steps(_SampleStep(st, sample), steps, warmup, False)
            rec["step_with_sample_consensus_us"] = round(ms_s * 1e3, 2)
            rec["sample_accept_len"] = acc.cpu().tolist()
            del p, q, cand, u, sws
        out[f"{label}_{w.name}_k{w.block_k}"] = rec
        print(f"[bench] {label} {w.name} K={w.block_k}: step {ms * 1e3:.1f} us "
              f"({rec['achieved_tbs']:.2f} TB/s)"
              + (f", sampler {rec['sample_consensus_us']:.1f} us" if label == "C5" else ""),
              file=sys.stderr, flush=True)
        del st, caches, kc, vc
        torch.cuda.empty_cache()
    return out


def time_tree_cycles(w, kc_all, vc_all, device, n_cycles: int, n_sets: int = 4, m: int = 4):
    """Tree-verification cycles through dual_view_block_amd.cycle.TreeDecodeCycles
    (one round of `n_sets` cycles captured in a HIP graph and replayed), plus
    the time of each tree-specific call.  Synthetic inputs: random N(0, 3)
    diffusion and verify logits (the tokens accepted per cycle depend on the
    model and are not reported as a figure of merit)."""
    import torch

    import dual_view_block_amd as dvb
    from dual_view_block_amd.cycle import TreeDecodeCycles
    from synth import cache_lengths, view_inputs

    K, V = w.block_k, w.vocab
    g = torch.Generator(device=device)
    g.manual_seed(17)
    sets = []
    for si in range(n_sets):
        ws = w.replace(seed=w.seed * 97 + si)
        sets.append({"diff": [view_inputs(ws, l, "diff", device) for l in range(w.layers)],
                     "verify": [view_inputs(ws, l, "verify", device) for l in range(w.layers)],
                     "diff_logits": torch.randn((w.batch * (K - 1), V), generator=g, device=device) * 3,
                     "verify_logits": torch.randn((w.batch, K, V), generator=g, device=device) * 3})
    lens = cache_lengths(w, device)
    anchor = torch.zeros(w.batch, dtype=torch.int32, device=device)
    drv = TreeDecodeCycles(kc_all, vc_all, lens, anchor, sets, m=m)
    drv.run(n_sets)
    torch.cuda.synchronize()
    drv.capture()
    torch.cuda.synchronize()
    rounds = max(1, n_cycles // n_sets)
    stream = torch.cuda.current_stream()
    l0 = lens.clone()
    us = _time_calls(lambda: drv.replay(1), rounds, stream) / n_sets
    tokens = int((lens - l0).sum().item())
    # the tree-specific calls alone, back to back on the first set's data
    s0 = sets[0]
    sp = stream.cuda_stream
    part = {
        "topk_us": _time_calls(lambda: dvb.orthrus_topk_logprobs(s0["diff_logits"], m, logp=drv.logp, idx=drv.idx,
                                                                 workspace=drv.topk_ws, stream=sp), 16, stream),
        "tree_build_us": _time_calls(lambda: dvb.orthrus_tree_build(
            drv.logp.view(w.batch, K - 1, m), drv.idx.view(w.batch, K - 1, m), drv.anchor, K, parent=drv.parent,
            tokens=drv.tokens, depth=drv.depth, stream=sp), 16, stream),
        "tree_masks_us": _time_calls(lambda: dvb.orthrus_tree_masks(drv.parent, mask=drv.mask, stream=sp), 16,
                                     stream),
        "tree_consensus_us": _time_calls(lambda: dvb.orthrus_consensus_tree_greedy(
            s0["verify_logits"], drv.tokens, drv.parent, accept_len=drv.accept_len, path=drv.path,
            correction=drv.correction, workspace=drv.cons_ws, stream=sp), 16, stream),
    }
    ver = drv._sets[0]["verify"]
    part["masked_verify_call_us"] = _time_calls(lambda: [c(sp) for c in ver], 3, stream) / len(ver)
    del drv
    return {"cycles": rounds * n_sets, "input_sets": n_sets, "n_nodes": K, "top_m": m, "launch": "hip_graph",
            "us_per_cycle": round(us, 2), "cycles_per_s": round(1e6 / us, 2),
            "tokens_per_cycle_synthetic": round(tokens / (rounds * n_sets * w.batch), 3),
            **{k: round(v, 2) for k, v in part.items()}}


MFMA_BF16_PEAK_TFLOPS = 2500.0


def train_attn_flops(seq_len: int, anchors, block_k: int, n_q_heads: int, head_dim: int):
    """Matrix flops of the training attention.  Forward: QK^T and PV over the
    allowed keys of every row (AR row i: i+1 keys; diffusion row of block n:
    a_n + K keys).  Backward (diffusion rows): QK^T, dO V^T and dS K over all
    their keys, plus dS^T Q and P^T dO over the block's own keys."""
    diff_keys = sum(int(a) + block_k for a in anchors) * block_k  # sum over diffusion rows
    ar_keys = seq_len * (seq_len + 1) // 2
    fwd = 4 * n_q_heads * head_dim * (ar_keys + diff_keys)
    n_rows = len(anchors) * block_k
    bwd = 2 * n_q_heads * head_dim * (3 * diff_keys + 2 * n_rows * block_k)
    return fwd, bwd


def time_train_attn(w, device, reps: int = 10):
    """Training dual-pass attention of one packed sequence (L 2048, 256
    anchor blocks of K 32, the workload's heads): forward (AR + diffusion
    rows) and the diffusion-row backward, HIP events around `reps`
    back-to-back calls each."""
    import torch

    import dual_view_block_amd as dvb
    from synth import train_attn_inputs

    L, N, K = 2048, 256, 32
    x = train_attn_inputs(w.n_q_heads, w.n_kv_heads, L, N, K, w.head_dim, seed=5, device=device)
    stream = torch.cuda.current_stream()
    fwd = lambda: dvb.orthrus_train_attn_fwd(x["q_ar"], x["k_ar"], x["v_ar"], x["q_diff"], x["k_diff"],
                                             x["v_diff"], x["anchors"], K, out_ar=out_ar, lse_ar=lse_ar,
                                             out_diff=out_d, lse_diff=lse_d)
    out_ar, lse_ar, out_d, lse_d = dvb.orthrus_train_attn_fwd(x["q_ar"], x["k_ar"], x["v_ar"], x["q_diff"],
                                                              x["k_diff"], x["v_diff"], x["anchors"], K)
    g = torch.Generator(device=device)
    g.manual_seed(7)
    d_out = torch.randn(x["q_diff"].shape, generator=g, device=device).to(torch.bfloat16)
    dq, dk, dv = (torch.empty_like(x["q_diff"]), torch.empty_like(x["k_diff"]), torch.empty_like(x["v_diff"]))
    bwd = lambda: dvb.orthrus_train_attn_bwd(x["k_ar"], x["v_ar"], x["q_diff"], x["k_diff"], x["v_diff"],
                                             x["anchors"], K, out_d, lse_d, d_out, dq=dq, dk=dk, dv=dv)
    f_fwd, f_bwd = train_attn_flops(L, x["anchors"].cpu().tolist(), K, w.n_q_heads, w.head_dim)
    out = {"seq_len": L, "n_blocks": N, "block_k": K, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
           "head_dim": w.head_dim, "dtype": "bf16"}
    for name, fn, flops in (("forward", fwd, f_fwd), ("backward", bwd, f_bwd)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        tf = flops / (us * 1e-6) / 1e12
        out[name] = {"us": round(us, 2), "flops": flops, "tflops": round(tf, 1),
                     "frac_mfma_bf16_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
    return out


def profile_target(args, w, caches, device) -> None:
    """Only the kernel under study, for rocprofv3 counter runs (no timing)."""
    import torch

    if args.profile_target == "copy":
        src = torch.ones(args.copy_mib * 2**20, dtype=torch.uint8, device=device)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)  # device-to-device: one copy kernel, reads and writes copy_mib MiB
    elif args.profile_target == "train-attn":
        for _ in range(args.steps):
            time_train_attn(w, device, reps=1)
    elif args.profile_target == "consensus":
        import dual_view_block_amd as dvb
        from synth import WORKLOADS, greedy_inputs, sample_inputs

        logits, cand, _ = greedy_inputs(w, device=device)  # [1, 32, 151936]
        wr = WORKLOADS["ragged_b16"]
        p, q, sc, u = sample_inputs(wr, device=device)     # [16, 32, 151936], drafts independent of targets
        pc, qc, scc, uc = sample_inputs(wr, device=device, draft_noise=0.5)  # drafts close to their targets
        for _ in range(args.steps):
            dvb.orthrus_consensus_greedy(logits, cand)
            dvb.orthrus_consensus_sample(p, q, sc, u)
            dvb.orthrus_consensus_sample(pc, qc, scc, uc)
    elif args.profile_target == "forward-kl":
        import dual_view_block_amd as dvb
        from synth import kl_inputs

        a, b = kl_inputs(args.kl_rows, w.vocab, 3.0, torch.bfloat16, seed=5, device=device)
        for _ in range(args.steps):
            dvb.orthrus_forward_kl(a, b, want_grad=True, grad_scale=1.0 / args.kl_rows)
    else:
        step = Step(w, caches, device)
        sp = torch.cuda.current_stream().cuda_stream
        for _ in range(args.steps):
            for view in ("diff", "verify"):
                for c in step.calls[view]:
                    c.partial(sp)
    torch.cuda.synchronize()
    print(f"[bench] profile target {args.profile_target} done", file=sys.stderr, flush=True)


def _cpu_model() -> str:
    """The host CPU's model name (the `lscpu` "Model name" field)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, caches, device, budget_s: float = 10.0):
    """The oracle, untuned, on the host cores, over a bounded sample of the same
    workload, reported in TB/s of the same algorithmic bytes.

    Inputs (the layer's cache, the block inputs, the logits) are generated and
    copied to the host outside the timed intervals; only the oracle calls are
    timed.  With the BLAS pool at its default size: whole layers of the step
    (diffusion + verify view, all heads) until about `budget_s` seconds of
    oracle time, plus one greedy consensus.  Then again with one thread: the
    diffusion view of layer 0 and the greedy consensus."""
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    from synth import cache_lengths, greedy_inputs, view_inputs

    lens = cache_lengths(w, "cpu")
    logits, cand, _ = greedy_inputs(w)

    def layer_inputs(layer):
        kc, vc = caches[layer]
        views = []
        for view, mode in (("diff", oracle.MASK_DIFF_BIDIR), ("verify", oracle.MASK_VERIFY_CAUSAL)):
            views.append((mode, [t.cpu() for t in view_inputs(w, layer, view, device)]))
        return kc.cpu(), vc.cpu(), views

    t = time.perf_counter()
    oracle.greedy_consensus(logits, cand)
    dt = time.perf_counter() - t
    nbytes = greedy_bytes(w)
    layers = 0
    first = None
    for layer in range(w.layers):
        kc_h, vc_h, views = layer_inputs(layer)
        if first is None:
            first = (kc_h, vc_h, views[0])
        for mode, (q, kb, vb) in views:
            t = time.perf_counter()
            oracle.block_attention(q, kb, vb, kc_h, vc_h, lens, mode)
            dt += time.perf_counter() - t
            nbytes += attn_bytes(w)
        layers += 1
        if dt >= budget_s:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])

    # one thread: one layer-view and the consensus
    kc_h, vc_h, (mode, (q, kb, vb)) = first
    with threadpool_limits(limits=1):
        t = time.perf_counter()
        oracle.greedy_consensus(logits, cand)
        oracle.block_attention(q, kb, vb, kc_h, vc_h, lens, mode)
        dt1 = time.perf_counter() - t
    nbytes1 = greedy_bytes(w) + attn_bytes(w)
    step_bytes = 2 * w.layers * attn_bytes(w) + greedy_bytes(w)
    return {"value": nbytes / dt / 1e12, "unit": "TB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{layers} of {w.layers} layers (diffusion + verify view, all heads) + one greedy "
                      f"consensus, L={w.cache_len}, K={w.block_k}: {dt:.2f} s of oracle calls with "
                      f"{threads} BLAS threads ({len(os.sched_getaffinity(0))} host CPUs usable); inputs "
                      "generated and copied to the host outside the timed calls",
            "cpu_model": _cpu_model(),
            "seconds": round(dt, 3),
            "step_seconds_extrapolated": round(dt / nbytes * step_bytes, 2),
            "one_thread": {"value": nbytes1 / dt1 / 1e12, "unit": "TB/s", "cores": 1,
                           "sample": "layer 0 diffusion view + one greedy consensus",
                           "seconds": round(dt1, 3),
                           "step_seconds_extrapolated": round(dt1 / nbytes1 * step_bytes, 2)}}


def main():
    args = _parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.trace_phases)
        return
    if args.make_traffic:
        make_traffic(args.make_traffic, args.traffic, args.copy_mib)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this decode step is "
              "not sharded across GPUs -- run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    from synth import WORKLOADS, model_cache

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU (no HIP device visible)", file=sys.stderr)
        sys.exit(1)
    device = torch.device("cuda:0")
    w = WORKLOADS[args.workload]
    if args.cache_len:
        w = w.replace(cache_len=args.cache_len, max_len=None)
    if args.block_k:
        w = w.replace(block_k=args.block_k)
    if args.layers:
        w = w.replace(layers=args.layers)
    print(f"[bench] workload {w}", file=sys.stderr, flush=True)
    if args.profile_target in ("copy", "forward-kl", "train-attn", "consensus"):
        profile_target(args, w, None, device)
        return
    # one layer-major cache for all layers, with room past L for the rows the
    # synthetic decode cycles commit (the step itself reads rows [0, L) only)
    w = w.replace(max_len=max(w.capacity, w.cache_len + (args.cycles + 2 * args.cycle_sets) * w.block_k,
                              w.cache_len + (args.t0_cycles + args.t0_sets) * w.block_k,
                              w.cache_len + (args.tree_cycles + 8) * w.block_k))
    kc_all, vc_all = model_cache(w, device)
    caches = [(kc_all[layer], vc_all[layer]) for layer in range(w.layers)]
    torch.cuda.synchronize()
    print(f"[bench] caches ready: {w.layers} layers x {2 * caches[0][0].numel() * 2 / 2**20:.0f} MiB "
          f"(capacity {w.capacity})", file=sys.stderr, flush=True)

    if args.profile_target:
        profile_target(args, w, caches, device)
        return
    step = Step(w, caches, device)
    splits = step.splits
    with MARKERS.range("steps"):
        ms, wall_ms = time_steps(step, args.steps, args.warmup, args.graph)
    with MARKERS.range("kernel_timing"):
        kern = time_kernels(step)
    # where this run's streaming-kernel dispatches fall, in launch order, for
    # reading a kernel trace of the same command (bench.py --summarize-trace)
    n_l = len(step.calls["diff"]) + len(step.calls["verify"])
    pre = (1 if args.graph else 0) + args.warmup
    t0 = (pre + args.steps) * n_l
    b0 = t0 + KERNEL_WARM_RUNS * n_l
    phases = {"timed_steps": (pre * n_l, t0), "back_to_back": (b0, b0 + KERNEL_TIMED_RUNS * n_l)}
    phase_arg = ",".join(f"{k}={a}:{b}" for k, (a, b) in phases.items())
    print(f"[bench] streaming-kernel dispatch phases: {phase_arg}", file=sys.stderr, flush=True)
    print(f"[bench] step {ms * 1e3:.1f} us (host wall {wall_ms * 1e3:.1f} us), streaming kernel "
          f"{kern['attn_stream_us']:.2f} us, merge {kern['attn_merge_us']:.2f} us, call "
          f"{kern['attn_call_us']:.2f} us", file=sys.stderr, flush=True)
    acc = step.acc.cpu().tolist()

    sweep = {}
    ks = [int(k) for k in args.k_sweep.split(",") if k.strip()] if args.k_sweep else []
    for K in ks:
        if K == w.block_k:
            sweep[K] = ms * 1e3
            continue
        wk = w.replace(block_k=K)
        sk = Step(wk, caches, device)
        with MARKERS.range(f"k_sweep_K{K}"):
            mk, _ = time_steps(sk, args.steps, args.warmup, args.graph)
        sweep[K] = mk * 1e3
        del sk
        print(f"[bench] K={K}: step {mk * 1e3:.1f} us", file=sys.stderr, flush=True)

    cyc = None
    if args.cycles > 0:
        with MARKERS.range("decode_cycles"):
            cyc = time_cycles(w, kc_all, vc_all, device, args.cycles, args.cycle_sets, args.accept_rate)
        print(f"[bench] cycles: {cyc['us_per_cycle']:.1f} us/cycle, {cyc['tokens_per_cycle']:.2f} tokens/cycle, "
              f"commit {cyc['commit_us']:.2f} us", file=sys.stderr, flush=True)

    t0c = None
    if args.t0_cycles > 0:
        t0_sets = sample_cycle_sets(w, args.t0_sets, args.t0_noise, device)
        with MARKERS.range("decode_cycles_t0"):
            t0c = time_cycles(w, kc_all, vc_all, device, args.t0_cycles, args.t0_sets, None, sets=t0_sets)
        t0c.pop("accept_rate", None)
        t0c.update(consensus="sample", draft_noise=args.t0_noise)
        del t0_sets
        print(f"[bench] T>0 cycles: {t0c['us_per_cycle']:.1f} us/cycle, {t0c['tokens_per_cycle']:.2f} tokens/cycle, "
              f"{t0c['tokens_per_s']:.0f} tokens/s", file=sys.stderr, flush=True)

    dyn = None
    if args.dyn_k:
        with MARKERS.range("dynamic_k"):
            dyn = time_dynamic_k(w, caches, kc_all, vc_all, device, args, cyc)

    tcy = None
    if args.tree_cycles > 0:
        with MARKERS.range("tree_cycles"):
            tcy = time_tree_cycles(w, kc_all, vc_all, device, args.tree_cycles)
        print(f"[bench] tree cycles: {tcy['us_per_cycle']:.1f} us/cycle; masked verify call "
              f"{tcy['masked_verify_call_us']:.1f} us, topk {tcy['topk_us']:.1f} us, build {tcy['tree_build_us']:.1f} "
              f"us, tree consensus {tcy['tree_consensus_us']:.1f} us", file=sys.stderr, flush=True)

    tra = None
    if args.train_attn:
        with MARKERS.range("train_attention"):
            tra = time_train_attn(w, device)
        print(f"[bench] training attention L2048 x 256 blocks: forward {tra['forward']['us']:.1f} us "
              f"({tra['forward']['tflops']:.0f} TFLOP/s), backward {tra['backward']['us']:.1f} us "
              f"({tra['backward']['tflops']:.0f} TFLOP/s)", file=sys.stderr, flush=True)

    fkl = None
    if args.kl_rows > 0:
        with MARKERS.range("forward_kl"):
            fkl = time_forward_kl(device, args.kl_rows, w.vocab)
        print(f"[bench] forward KL {fkl['rows']}x{fkl['vocab']} bf16: loss {fkl['loss']['us']:.1f} us "
              f"({fkl['loss']['achieved_gbs']:.0f} GB/s), loss+grad {fkl['loss_and_grad']['us']:.1f} us "
              f"({fkl['loss_and_grad']['achieved_gbs']:.0f} GB/s)", file=sys.stderr, flush=True)

    cfg = None
    if args.configs:
        del step
        torch.cuda.empty_cache()
        with MARKERS.range("other_configs"):
            cfg = time_configs(device, args.steps, args.warmup)

    step_bytes = 2 * w.layers * attn_bytes(w) + greedy_bytes(w)
    value = step_bytes / (ms * 1e-3) / 1e12
    pbytes = stream_bytes(w)
    achieved = pbytes / (kern["attn_stream_us"] * 1e-6) / 1e9
    traffic = load_traffic(args.traffic)
    flops = w.layers * (attn_flops(w, False) + attn_flops(w, True))
    # the timed launches cover both views equally: their mean per launch
    sflops = (attn_flops(w, False) + attn_flops(w, True)) // 2
    line = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.layers, "batch": w.batch, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "cache_len": w.cache_len,
                   "block_k": w.block_k, "vocab": w.vocab, "consensus": "greedy",
                   "launch": "hip_graph" if args.graph else "eager", "splits": splits},
        "step_us": round(ms * 1e3, 2),
        "tokens_verified_per_s": round(w.batch * w.block_k / (ms * 1e-3), 1),
        "algorithmic_bytes_per_step": step_bytes,
        "frac_hbm_peak_step": round(value * 1e3 / HBM_PEAK_GBS, 4),
        "mfma_tflops_step": round(flops / (ms * 1e-3) / 1e12, 2),
        "frac_mfma_bf16_peak_step": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "stream_kernel_mfma": {"flops_per_launch": sflops,
                               "tflops": round(sflops / (kern["attn_stream_us"] * 1e-6) / 1e12, 1),
                               "frac_bf16_peak": round(sflops / (kern["attn_stream_us"] * 1e-6) / 1e12
                                                       / MFMA_BF16_PEAK_TFLOPS, 4)},
        "step_us_vs_block_k": {str(k): round(v, 2) for k, v in sweep.items()},
        "k32_over_k1": round(sweep[32] / sweep[1], 4) if 32 in sweep and 1 in sweep else None,
        "kernel_us": {k: round(v, 3) for k, v in kern.items()},
        "accept_len": acc,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "attn_stream_kernel<128,4> (one launch per orthrus_block_attn_* call)",
                     "algorithmic_bytes_per_launch": pbytes,
                     "duration_us": round(kern["attn_stream_us"], 3),
                     "duration_from": f"HIP events around {KERNEL_TIMED_RUNS} runs of back-to-back streaming "
                                      f"launches after {KERNEL_WARM_RUNS} untimed, median",
                     "trace_phases": phase_arg,
                     "call_achieved_gbs": round(attn_bytes(w) / (kern["attn_call_us"] * 1e-6) / 1e9, 1)},
    }
    if cyc is not None:
        line["decode_cycles"] = cyc
    if t0c is not None:
        line["decode_cycles_t0"] = t0c
    if dyn is not None:
        line["dynamic_k"] = dyn
    if fkl is not None:
        line["forward_kl"] = fkl
    if tra is not None:
        line["train_attention"] = tra
    if tcy is not None:
        line["tree_cycles"] = tcy
    if cfg is not None:
        line["other_configs"] = cfg
    if not args.no_cpu_baseline:
        with MARKERS.range("cpu_baseline"):
            line["cpu_baseline"] = cpu_baseline(w, caches, device)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
