"""Benchmark of the CSA indexer hot path (score + top-512) on one MI355X.

By default one run measures all five scoring workloads and prints ONE JSON
line whose headline is chunked prefill (4096 query rows of one request over a
65,536-token prefix plus the chunk itself: 69.2 M scored pairs, the largest of
the five by scored pairs and FLOP).  The line's `workloads` object holds every
workload's own step time, pairs/s, queries/s and step-level fraction of its
roofline (HBM for the decode shapes, bf16 MFMA for prefill) next to the
target fraction, so one run's clock covers all five:

  tiny-decode      B = 1, 2048 contiguous entries
  decode-batch     B = 32, L_b ~ U[32k, 128k] tokens, N_b = L_b // 4, paged
  long-decode      B = 8 x 262,144 entries (1M tokens), paged
  resident-subset  B = 40 x 384 resident 64-entry chunks of 4096, chunk lists
  chunked-prefill  4096 rows, causal bounds (65537 + i) // 4, 272 blocks

One step = one idx_score_topk call.  Inputs are resident in HBM before timing;
the pool and q are replicated so consecutive steps read different copies (more
bytes than the 256 MB MALL), and the K timed steps run as replays of a
captured HIP graph so host launch cost stays out of the GPU timeline.
`value` is scored (query, entry) pairs per second of the whole path;
`roofline` covers the score kernel (the dominant kernel), timed live with HIP
events that each launch's dispatch stamps with the kernel's start and end on
the stream it runs on.  Algorithmic bytes: one 132-byte key row per scored
pair on the decode shapes (the request's rows once for prefill, whose rows
share them), q, w, bounds, tables and chunk lists once, the output indices
once; logits and candidate lists are overhead, not counted.

`--workload NAME` measures one workload alone (its own line).
`--workload index-fill` measures the index-plane writer: one step is one
idx_write_keys call that quantises the 262,144 compressed keys of one
1M-token request into a shuffled paged pool; `value` is keys written per
second and `roofline` covers the writer kernel.

`--q8` measures the quantised-query variant on a scoring workload: each step
is one idx_score_topk_fp8q (the score kernel quantises q per head by the
writer's rule, then scores on fp8 MFMA); the prefill roofline is then priced
at the fp8 MFMA peak.  `--mxfp4` measures the MXFP4 variant the same way (one
idx_score_topk_mxfp4 per step: query and keys rounded to MXFP4 blocks inside
the score kernel, e2m1 MFMA; the prefill roofline priced at the fp4 peak).

`--block-size 16` re-lays a scoring workload's pool into 16-row blocks, each
placed on its own (the block table grows fourfold, chunk lists are cut into
small blocks), and measures the same step over that layout.

`--workload memory-indexer` measures the Level-1 resident-set selection: one
step is one idx_select_resident call over 8 requests at 1M tokens (262,144
entries each) scored at 3 layers, KMAX 384 pages; `value` is scored pairs per
second over all layers.  The layers' queries and weights are stacked, so the
step is one score launch over every (layer, row) writing selection bits, a
page pass and the page top-k, and `roofline` covers that score launch;
`--separate-layers` gives each layer its own tensors (one score launch per
layer writing scores; `roofline` then covers the last layer's launch).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, TFLOP/s
MFMA_FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, TFLOP/s
MFMA_FP4_PEAK_TFLOPS = 10100.0   # MI355X dense fp4 MFMA, TFLOP/s
PROFILE_DIR = os.path.join(ROOT, "profiles")
SCORE_SOURCES = ["sparse_attention_kv_paged_amd/csrc/idx_score.hip",
                 "sparse_attention_kv_paged_amd/csrc/idx_device.h",
                 "sparse_attention_kv_paged_amd/csrc/idx_internal.h"]
WRITE_SOURCES = ["sparse_attention_kv_paged_amd/csrc/idx_write.hip",
                 "sparse_attention_kv_paged_amd/csrc/idx_write.h",
                 "sparse_attention_kv_paged_amd/csrc/idx_internal.h"]
WORKLOADS = {"tiny-decode": 0, "decode-batch": 1, "long-decode": 2,
             "chunked-prefill": 3, "resident-subset": 4}
WRITE_WORKLOAD = "index-fill"
RESIDENT_WORKLOAD = "memory-indexer"
WRITE_BYTES_PER_KEY = 128 * 2 + 8 + 132      # bf16 key in, int64 slot, pool row out


def kernel_of(workload: str):
    """(kernel name, its sources, profile file prefix) measured for a workload."""
    if workload == "index-fill":
        return "write_keys_kernel", WRITE_SOURCES, "write_keys"
    return "score_kernel", SCORE_SOURCES, "score_kernel"


def score_source_hash(sources=SCORE_SOURCES) -> str:
    h = hashlib.sha256()
    for p in sources:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


SUITE = ["tiny-decode", "decode-batch", "long-decode", "resident-subset", "chunked-prefill"]
HEADLINE = "chunked-prefill"
# target fractions of the roofline for the whole score + top-k step
TARGET_HBM_FRAC = 0.70            # decode shapes
TARGET_MFMA_FRAC = 0.50           # prefill


def shares_request_keys(wl) -> bool:
    """Every query row reads the same request's blocks (prefill): the keys
    are counted once, not once per row."""
    return wl.q_req is not None and wl.block_table is not None and wl.block_table.shape[0] == 1


def algorithmic_bytes(wl, pairs: int, q8: bool = False) -> int:
    """Bytes the whole path must move at minimum: one 132-byte key row per
    scored (query, entry) pair on the decode shapes (rows shared by every
    query of a prefill request are counted once), q (bf16, or 132-byte
    quantised rows per head), w, bounds, tables and chunk lists once, and the
    selected indices written once.  Logits and candidate lists are overhead
    of a particular kernel design and are not counted."""
    if shares_request_keys(wl):
        keys = int((wl.block_table >= 0).sum()) * wl.block_size * 132
    else:
        keys = pairs * 132
    q_bytes = wl.B * wl.H * (wl.D + 4) if q8 else wl.q.nbytes
    extra = q_bytes + wl.w.nbytes + wl.limits.nbytes + wl.B * wl.k * 4
    for a in (wl.block_table, wl.q_req, wl.chunk_ids, wl.n_chunks):
        if a is not None:
            extra += a.nbytes
    return keys + extra


def score_kernel_bytes(wl, pairs: int, q8: bool = False, logits_written: bool = True) -> int:
    """Algorithmic bytes of one score-kernel launch taken alone (the roofline
    of that kernel): the path's bytes without the indices, plus a 4-byte
    logit per pair when the launch stores logits for a separate selection."""
    return algorithmic_bytes(wl, pairs, q8) - wl.B * wl.k * 4 + (pairs * 4 if logits_written else 0)


def _read_kv(path):
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            key, _, val = line.partition("=")
            kv[key.strip()] = val.strip()
    return kv


def read_traffic(workload: str):
    """HBM bytes per score-kernel launch from the committed rocprofv3 counter
    summary, or None if absent or taken on a different kernel source."""
    _, sources, prefix = kernel_of(workload)
    path = os.path.join(PROFILE_DIR, f"{prefix}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    kv = _read_kv(path)
    if kv.get("source_hash", kv.get("score_source_hash")) != score_source_hash(sources):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_mfma(name: str):
    """(MFMA busy fraction, clock GHz) of the score kernel from the committed
    counter summary, or (None, None) if absent or taken on other sources."""
    path = os.path.join(PROFILE_DIR, f"score_kernel_{name}_mfma.txt")
    if not os.path.exists(path):
        return None, None
    kv = _read_kv(path)
    if kv.get("source_hash") != score_source_hash(SCORE_SOURCES):
        return None, None
    try:
        return float(kv["mfma_busy_frac"]), float(kv["clock_ghz"])
    except (KeyError, ValueError):
        return None, None


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(dirpath, suffix):
    for root, _, files in os.walk(dirpath):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError(f"no *{suffix} under {dirpath}")


def summarize_trace(trace_dir, workload, command, out):
    """Kernel-time summary of a `rocprofv3 --kernel-trace --stats
    --output-format csv` run, as text for profiles/."""
    rows = _csv_rows(_find(trace_dir, "kernel_stats.csv"))
    _, sources, _ = kernel_of(workload)
    lines = [f"# rocprofv3 kernel statistics, workload {workload}",
             f"# command: {command}",
             f"source_hash = {score_source_hash(sources)}",
             f"{'kernel':72s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'share':>6s}"]
    for r in rows:
        lines.append(f"{r['Name'][:72]:72s} {int(r['Calls']):6d} {float(r['AverageNs'])/1e3:10.3f} "
                     f"{float(r['MinNs'])/1e3:10.3f} {float(r['MaxNs'])/1e3:10.3f} {float(r['Percentage']):6.2f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_pmc(fetch_dir, write_dir, workload, command, out):
    """HBM traffic per launch of the workload's measured kernel from two
    counter runs (FETCH_SIZE, WRITE_SIZE, KiB per dispatch), each scaled by
    what the same counter reads for the 1 GiB device copy that
    `--copy-calibration` runs (1 GiB read and 1 GiB written per dispatch)."""
    kname, sources, _ = kernel_of(workload)

    def per_kernel(dirpath, counter):
        vals = {}
        for r in _csv_rows(_find(dirpath, "counter_collection.csv")):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Kernel_Name"], r["Dispatch_Id"])
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        score = [v for (n, _), v in vals.items() if kname in n]
        copy = [v for (n, _), v in vals.items() if "copy" in n.lower() and v > 5e5]
        return score, copy
    import statistics
    fs, fc = per_kernel(fetch_dir, "FETCH_SIZE")
    ws, wc = per_kernel(write_dir, "WRITE_SIZE")
    gib_kib = float(1 << 20)
    fetch_scale = gib_kib / statistics.median(fc)
    write_scale = gib_kib / statistics.median(wc)
    fetch_b = statistics.median(fs) * 1024 * fetch_scale
    write_b = statistics.median(ws) * 1024 * write_scale
    lines = [f"# rocprofv3 HBM counters for {kname}, workload {workload}",
             f"# command: {command}",
             f"# FETCH_SIZE and WRITE_SIZE are KiB per dispatch; each is scaled by the same",
             f"# counter's reading for a 1 GiB device copy (1 GiB read, 1 GiB written).",
             f"source_hash = {score_source_hash(sources)}",
             f"dispatches = {len(fs)}",
             f"fetch_kib_per_launch_raw = {statistics.median(fs):.1f}",
             f"write_kib_per_launch_raw = {statistics.median(ws):.1f}",
             f"copy_fetch_kib_raw = {statistics.median(fc):.1f}",
             f"copy_write_kib_raw = {statistics.median(wc):.1f}",
             f"fetch_scale = {fetch_scale:.4f}",
             f"write_scale = {write_scale:.4f}",
             f"fetch_bytes_per_launch = {fetch_b:.0f}",
             f"write_bytes_per_launch = {write_b:.0f}",
             f"hbm_bytes_per_launch = {fetch_b + write_b:.0f}"]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


MFMA_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU",
                 "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"]
SIMDS = 256 * 4


def summarize_mfma(pmc_dir, workload, command, out):
    """MFMA utilisation of the score kernel from one counter run of
    MFMA_COUNTERS.  The profiler's CSV holds each counter summed over its
    instances, so GRBM_GUI_ACTIVE is the sum over the 8 XCDs: busy =
    SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs) / (GRBM_GUI_ACTIVE / 8 x
    1024 SIMDs), the profiler's MfmaUtil ratio; the clock the kernel ran at
    is GRBM_GUI_ACTIVE / 8 over the dispatch's duration.  Plus the
    instruction mix."""
    import statistics
    kname, sources, _ = kernel_of(workload.replace("-q8", ""))
    per = {}
    for r in _csv_rows(_find(pmc_dir, "counter_collection.csv")):
        if kname not in r["Kernel_Name"]:
            continue
        d = per.setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        d["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    rows = [d for d in per.values() if all(c in d for c in MFMA_COUNTERS)]
    med = {c: statistics.median(d[c] for d in rows) for c in MFMA_COUNTERS + ["ns"]}
    active = med["GRBM_GUI_ACTIVE"] / 8
    busy = med["SQ_VALU_MFMA_BUSY_CYCLES"] / (active * SIMDS)
    lines = [f"# rocprofv3 MFMA counters for {kname}, workload {workload}",
             f"# command: {command}",
             f"# medians over dispatches; busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x {SIMDS} SIMDs)",
             f"source_hash = {score_source_hash(sources)}",
             f"dispatches = {len(rows)}"]
    lines += [f"{c.lower()} = {med[c]:.0f}" for c in MFMA_COUNTERS]
    lines += [f"dispatch_ns = {med['ns']:.0f}",
              f"clock_ghz = {active / med['ns']:.3f}",
              f"mfma_busy_frac = {busy:.4f}",
              f"coexec_frac_of_mfma_busy = {med['SQ_VALU_MFMA_COEXEC_CYCLES'] / med['SQ_VALU_MFMA_BUSY_CYCLES']:.4f}",
              f"valu_insts_per_mfma_inst = {med['SQ_INSTS_VALU'] / med['SQ_INSTS_MFMA']:.2f}"]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_counters(pmc_dir, kname, workload, command, out, items=None):
    """Medians per dispatch of every counter in one `rocprofv3 --pmc` run for
    the kernels whose name contains `kname`, one section per kernel (template
    instantiation) and, given `items` (work items per dispatch), the VALU
    instructions per item (SQ_INSTS_VALU counts wave64 instructions)."""
    import statistics
    per = {}
    for r in _csv_rows(_find(pmc_dir, "counter_collection.csv")):
        if kname not in r["Kernel_Name"]:
            continue
        d = per.setdefault((r["Kernel_Name"], r["Dispatch_Id"]), {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        d["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    lines = [f"# rocprofv3 counters for {kname}, workload {workload}",
             f"# command: {command}",
             f"# medians over dispatches, per kernel"]
    for name in sorted({n for n, _ in per}):
        ds = [d for (n, _), d in per.items() if n == name]
        names = sorted({c for d in ds for c in d if c != "ns"})
        med = {c: statistics.median(d[c] for d in ds if c in d) for c in names + ["ns"]}
        lines += ["", f"[{name}]", f"dispatches = {len(ds)}"]
        lines += [f"{c.lower()} = {med[c]:.0f}" for c in names]
        lines.append(f"dispatch_ns = {med['ns']:.0f}")
        if items and "SQ_INSTS_VALU" in med:
            lines.append(f"items_per_dispatch = {items}")
            lines.append(f"valu_insts_per_item = {med['SQ_INSTS_VALU'] * 64 / items:.2f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_baseline(wl, pairs: int, min_seconds: float, max_sample_pairs: int = 4_000_000, mxfp4: bool = False):
    """The oracle as it stands on the host cores, timed on a bounded sample:
    full passes of the workload until `min_seconds` of wall time, or, when one
    pass holds more than `max_sample_pairs` pairs, passes over evenly spaced
    rows (score + top-k of those rows) scaled by the pairs they score.  With
    mxfp4, the oracle's MXFP4 scoring (the quantised-query variant's oracle
    consumes quantised rows, so --q8 times the plain definition)."""
    import numpy as np
    from oracle import oracle
    threads = oracle.max_threads()
    rows, sample_pairs, what = None, pairs, f"full pass(es) of the {wl.name} workload"
    if pairs > max_sample_pairs:
        stride = int(np.ceil(pairs / max_sample_pairs))
        rows = np.arange(0, wl.B, stride)
        per_row = np.asarray(wl.pairs_per_row(), dtype=np.int64)
        sample_pairs = int(per_row[rows].sum())
        what = f"pass(es) over 1 row in {stride} ({len(rows)} of {wl.B} rows) of the {wl.name} workload"
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.score_topk(wl, rows=rows, mxfp4=mxfp4)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return {"value": sample_pairs * reps / el, "unit": "pairs/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} {what} ({sample_pairs} pairs, score + top-{wl.k}) in {el:.1f} s"}


def run_steps(step, K, R, use_graph):
    """K timed steps (replays of captured graphs of up to R steps, or eager
    launches), bracketed by synchronisations; returns ms per step."""
    import torch
    graphs = []
    if use_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        per = min(R, K)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(per):
                step(i)
        graphs = [g] * (K // per)
        if K % per:
            g2 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g2):
                for i in range(K % per):
                    step(i)
            graphs.append(g2)
        for g_ in set(graphs):
            g_.replay()
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    if graphs:
        for g_ in graphs:
            g_.replay()
    else:
        for i in range(K):
            step(i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = max(wall * 1e3, gpu_ms) / K
    print(f"[bench] {K} steps: {ms_per_step * 1e3:.2f} us/step (wall {wall * 1e3:.3f} ms, "
          f"events {gpu_ms:.3f} ms)", file=sys.stderr, flush=True)
    return ms_per_step


def kernel_ms_live(step, n):
    """Average duration of the measured kernel over n eager steps: each
    launch's dispatch stamps a pair of events with the kernel's start and end
    on its own stream; the steps queue behind a busy wait so the queue never
    drains while the host enqueues."""
    import numpy as np
    import torch
    from sparse_attention_kv_paged_amd import lib
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:            # create the hipEvents; the library re-records them
        a.record()
        b.record()
    torch.cuda.synchronize()
    torch.cuda._sleep(int(5e7))
    for i in range(n):
        lib.idx_profile_events(*evs[i])
        step(i)
    lib.idx_profile_events(None, None)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def spread(ms):
    """Mean (what `achieved` divides by) and p10 / p50 / p90 of per-launch
    kernel times, in ms."""
    import numpy as np
    p10, p50, p90 = np.percentile(ms, [10, 50, 90])
    return float(np.mean(ms)), {"kernel_ms_p10": float(p10), "kernel_ms_p50": float(p50),
                                "kernel_ms_p90": float(p90), "launches": len(ms)}


def copy_calibration(n):
    """n plain device copies of 1 GiB (the reference reading for HBM counters)."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(n):
        dst.copy_(src)
    torch.cuda.synchronize()


GEMM_CAL_SIZE = 8192


def gemm_calibration(n, size=GEMM_CAL_SIZE):
    """n plain bf16 GEMMs C = A B (size x size x size, torch.matmul, which
    dispatches to the vendor GEMM library): the dense bf16 MFMA rate a
    library kernel sustains on this chip, for context next to the spec peak.
    Prints one JSON line."""
    import torch
    torch.cuda.set_device(0)
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(size, size, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(size, size, device="cuda", dtype=torch.bfloat16, generator=g)
    c = torch.empty(size, size, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(n):
        torch.matmul(a, b, out=c)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / n
    tflops = 2.0 * size ** 3 / (ms * 1e-3) / 1e12
    print(json.dumps({"calibration": "bf16 GEMM, torch.matmul", "m": size, "n": size, "k": size,
                      "gemms": n, "ms_per_gemm": ms, "tflops": tflops,
                      "frac_of_spec_peak": tflops / MFMA_BF16_PEAK_TFLOPS}), flush=True)


def summarize_gemm_mfma(pmc_dir, command, out, size=GEMM_CAL_SIZE):
    """MFMA utilisation and clock of the library GEMM kernel of a
    `--gemm-calibration` run under the MFMA_COUNTERS (the most frequent
    kernel that issues MFMAs), computed as for the score kernel, plus the
    TFLOP/s of a dispatch from its duration."""
    import statistics
    per, names = {}, {}
    for r in _csv_rows(_find(pmc_dir, "counter_collection.csv")):
        d = per.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"]})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        d["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    rows = [d for d in per.values() if all(c in d for c in MFMA_COUNTERS) and d["SQ_INSTS_MFMA"] > 0]
    for d in rows:
        names[d["name"]] = names.get(d["name"], 0) + 1
    kname = max(names, key=names.get)
    rows = [d for d in rows if d["name"] == kname]
    med = {c: statistics.median(d[c] for d in rows) for c in MFMA_COUNTERS + ["ns"]}
    active = med["GRBM_GUI_ACTIVE"] / 8
    busy = med["SQ_VALU_MFMA_BUSY_CYCLES"] / (active * SIMDS)
    tflops = 2.0 * size ** 3 / med["ns"] / 1e3
    lines = [f"# rocprofv3 MFMA counters for the library bf16 GEMM ({size} x {size} x {size}, torch.matmul)",
             f"# command: {command}",
             f"# medians over dispatches; busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x {SIMDS} SIMDs)",
             f"kernel = {kname[:100]}",
             f"dispatches = {len(rows)}"]
    lines += [f"{c.lower()} = {med[c]:.0f}" for c in MFMA_COUNTERS]
    lines += [f"dispatch_ns = {med['ns']:.0f}",
              f"tflops = {tflops:.1f}",
              f"frac_of_spec_peak = {tflops / MFMA_BF16_PEAK_TFLOPS:.4f}",
              f"clock_ghz = {active / med['ns']:.3f}",
              f"mfma_busy_frac = {busy:.4f}"]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def bench_writer(args):
    """One step = one idx_write_keys of the index-fill workload (262,144 keys
    of one 1M-token request into a shuffled paged pool)."""
    import numpy as np
    import torch
    from oracle import oracle
    from sparse_attention_kv_paged_amd import lib, workloads

    torch.cuda.set_device(0)
    wr = workloads.index_fill()
    n = wr.n
    print(f"[bench] workload {wr.name}: {wr.description}", file=sys.stderr, flush=True)
    k = torch.from_numpy(wr.k.view(np.int16)).cuda()
    slots = torch.from_numpy(wr.slots).cuda()
    pool = torch.from_numpy(wr.pool).cuda()
    per_copy = k.numel() * 2 + pool.numel()
    R = args.replicas or max(4, min(64, math.ceil(1.0e9 / per_copy)))
    ks = [k] + [k.clone() for _ in range(R - 1)]
    pools = [pool] + [pool.clone() for _ in range(R - 1)]

    def step(i):
        lib.idx_write_keys(ks[i % R], slots, pools[i % R])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_per_step = run_steps(step, args.steps, R, not args.no_graph)
    kern_ms, kern_spread = spread(kernel_ms_live(step, args.steps))
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)

    algo = n * WRITE_BYTES_PER_KEY
    roofline = {"kernel": "write_keys_kernel", "bound": "hbm",
                "achieved": algo / (kern_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "traffic": read_traffic(WRITE_WORKLOAD), "algorithmic_bytes": algo, "kernel_ms": kern_ms,
                **kern_spread}
    roofline["frac"] = roofline["achieved"] / roofline["peak"]
    out = {
        "metric": "index-plane writer keys quantised and stored/s; % of HBM peak, 1 MI355X",
        "value": n / (ms_per_step * 1e-3),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wr.name, "keys": n, "head_dim": 128, "block": 64,
                   "description": wr.description, "replicas": R, "graph": not args.no_graph},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        # the oracle writer (one thread) on leading slices of the keys
        sample = min(n, 4096)
        out_pool = wr.pool.copy()
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.write_keys(wr.k[:sample], wr.slots[:sample], out_pool)
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        out["cpu_baseline"] = {"value": sample * reps / el, "unit": "keys/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{reps} passes over the first {sample} keys of {wr.name} in {el:.1f} s"}
    print(json.dumps(out), flush=True)


def bench_resident(args):
    """One step = one idx_select_resident of the memory-indexer workload."""
    import numpy as np
    import torch
    from oracle import oracle
    from sparse_attention_kv_paged_amd import lib, workloads

    torch.cuda.set_device(0)
    rl = workloads.memory_indexer()
    print(f"[bench] workload {rl.name}: {rl.description}", file=sys.stderr, flush=True)
    dls = [lib.to_device(wl) for wl in rl.layers]
    if args.separate_layers:
        # each layer's q and w its own tensor: one score launch per layer
        qs, wts = [d.q for d in dls], [d.w for d in dls]
    else:
        # the layers' q and w stacked: one score launch over every (layer, row)
        q_all = torch.stack([d.q for d in dls])
        w_all = torch.stack([d.w for d in dls])
        qs, wts = [q_all[l] for l in range(len(dls))], [w_all[l] for l in range(len(dls))]
    pairs_layer = [wl.pairs() for wl in rl.layers]
    pairs = int(sum(pairs_layer))
    out_pages = torch.empty((rl.B, rl.kmax), dtype=torch.int32, device="cuda")
    out_count = torch.empty(rl.B, dtype=torch.int32, device="cuda")
    ws = lib.new_workspace(lib.resident_workspace_bytes(len(dls), rl.B, rl.n_cols, rl.kmax), "cuda")

    def step(i):
        lib.idx_select_resident(qs, wts, [d.keys for d in dls], rl.n_cols,
                                rl.kmax, ensemble=rl.ensemble, threshold=rl.threshold, n_sink=rl.n_sink,
                                n_recent=rl.n_recent, out_pages=out_pages, out_count=out_count, workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # the three layers' pools (830 MB) exceed the 256 MB MALL: no replicas needed
    ms_per_step = run_steps(step, args.steps, 1, not args.no_graph)
    # the hook stamps every score launch of a step; the events keep the last
    # launch: the one over every layer (stacked), or the last layer's
    kern_ms, kern_spread = spread(kernel_ms_live(step, args.steps))
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
    if args.separate_layers:
        algo = score_kernel_bytes(rl.layers[-1], pairs_layer[-1])      # one layer's launch, its scores stored
    else:
        # every layer's keys, q, w and tables, and the selection bits written
        words = -(-rl.n_cols // 64) * 2
        algo = sum(score_kernel_bytes(w_, p_, logits_written=False) for w_, p_ in zip(rl.layers, pairs_layer))
        algo += len(rl.layers) * rl.B * words * 4
    roofline = {"kernel": "score_kernel", "bound": "hbm", "achieved": algo / (kern_ms * 1e-3) / 1e9,
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                # the counters were taken on the one launch over every layer
                "traffic": None if args.separate_layers else read_traffic(RESIDENT_WORKLOAD),
                "algorithmic_bytes": algo, "kernel_ms": kern_ms, **kern_spread}
    roofline["frac"] = roofline["achieved"] / roofline["peak"]
    # the step: every layer's keys, q, w and tables once, the pages written
    step_bytes = sum(score_kernel_bytes(w_, p_, logits_written=False) for w_, p_ in zip(rl.layers, pairs_layer))
    step_bytes += rl.B * rl.kmax * 4
    out = {
        "metric": "Level-1 resident-set selection: scored pairs/s over all layers; % of HBM peak, 1 MI355X",
        "value": pairs / (ms_per_step * 1e-3),
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": rl.name, "queries": rl.B, "layers": len(rl.layers), "n_cols": rl.n_cols,
                   "kmax": rl.kmax, "threshold": rl.threshold, "n_sink": rl.n_sink, "n_recent": rl.n_recent,
                   "ensemble": "max" if rl.ensemble == 0 else "mean", "pairs": pairs,
                   "layers_stacked": not args.separate_layers,
                   "description": rl.description, "graph": not args.no_graph},
        "requests_per_s": rl.B / (ms_per_step * 1e-3),
        "path_hbm_frac": step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        # the oracle on one request: three layers' double scores, then the selection
        reps, t0 = 0, time.perf_counter()
        while True:
            sc = oracle.level1_scores(rl.layers, rows=[reps % rl.B])
            oracle.level1_select(sc, rl.limits[[reps % rl.B]], rl.ensemble, rl.threshold, rl.n_sink,
                                 rl.n_recent, rl.kmax)
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        per_row = pairs / rl.B
        out["cpu_baseline"] = {"value": per_row * reps / el, "unit": "pairs/s", "cores": oracle.max_threads(),
                               "kind": "oracle",
                               "sample": f"{reps} requests of {rl.name} (3 layers x {rl.n_cols} entries, "
                                         f"score + selection) in {el:.1f} s"}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=96)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="suite",
                    choices=["suite"] + sorted(WORKLOADS) + [WRITE_WORKLOAD, RESIDENT_WORKLOAD],
                    help="suite (default): all five scoring workloads in one run, headline chunked-prefill")
    ap.add_argument("--replicas", type=int, default=0, help="pool copies (0 = enough for >= 1 GB)")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a graph")
    ap.add_argument("--q8", action="store_true",
                    help="quantised-query variant: idx_score_topk_fp8q (q quantised per head inside the score "
                         "kernel, fp8 MFMA)")
    ap.add_argument("--mxfp4", action="store_true",
                    help="MXFP4 variant: idx_score_topk_mxfp4 (q and keys rounded to MXFP4 blocks of 32 inside the "
                         "score kernel, e2m1 MFMA)")
    ap.add_argument("--separate-layers", action="store_true",
                    help="memory-indexer: each layer's q and w in a tensor of its own (one score launch per layer)")
    ap.add_argument("--block-size", type=int, default=64, choices=(64, 16),
                    help="pool block rows of the scoring workloads (16: the same keys re-laid in 16-row blocks)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="also run N plain device copies of 1 GiB (for HBM counter scaling)")
    ap.add_argument("--summarize-trace", metavar="DIR", help="write profiles/ summary of a kernel-trace run")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/ summary of FETCH_SIZE / WRITE_SIZE runs")
    ap.add_argument("--summarize-mfma", metavar="DIR", help="write profiles/ summary of an MFMA counter run")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("KERNEL", "DIR"),
                    help="write profiles/ summary of any --pmc run for kernels whose name contains KERNEL")
    ap.add_argument("--gemm-calibration", type=int, default=0, metavar="N",
                    help="only time N plain bf16 GEMMs of 8192^3 (torch.matmul): the library's sustained MFMA rate")
    ap.add_argument("--summarize-gemm", metavar="DIR",
                    help="write profiles/ summary of an MFMA counter run of --gemm-calibration")
    ap.add_argument("--command", default="", help="the profiled command, recorded in the summary")
    args = ap.parse_args()

    trace_prefix = {WRITE_WORKLOAD: "write_keys", RESIDENT_WORKLOAD: "select_resident"}.get(args.workload,
                                                                                          "score_topk")
    prof_name = (args.workload + ("-b16" if args.block_size == 16 else "") + ("-q8" if args.q8 else "")
                 + ("-mxfp4" if args.mxfp4 else ""))
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, prof_name, args.command,
                        os.path.join(PROFILE_DIR, f"{trace_prefix}_{prof_name}_trace.txt"))
        return
    if args.summarize_counters:
        kname, pdir = args.summarize_counters
        items = None
        if args.workload in WORKLOADS and "topk" in kname:
            from sparse_attention_kv_paged_amd import workloads
            items = int(scoring_workload(args.workload, args, workloads).pairs())   # scored pairs
        summarize_counters(pdir, kname, prof_name, args.command,
                           os.path.join(PROFILE_DIR, f"{kname}_{prof_name}_counters.txt"), items)
        return
    if args.summarize_gemm:
        summarize_gemm_mfma(args.summarize_gemm, args.command,
                            os.path.join(PROFILE_DIR, "gemm_bf16_calibration_mfma.txt"))
        return
    if args.gemm_calibration:
        gemm_calibration(args.gemm_calibration)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma, prof_name, args.command,
                       os.path.join(PROFILE_DIR, f"score_kernel_{prof_name}_mfma.txt"))
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], prof_name, args.command,
                      os.path.join(PROFILE_DIR, f"{kernel_of(args.workload)[2]}_{prof_name}_pmc.txt"))
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              f"the library runs on one GPU and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    if (args.q8 or args.mxfp4 or args.block_size != 64) and args.workload in (WRITE_WORKLOAD, RESIDENT_WORKLOAD):
        print(f"--q8, --mxfp4 and --block-size apply to the scoring workloads, not {args.workload}",
              file=sys.stderr)
        sys.exit(2)
    if args.q8 and args.mxfp4:
        print("--q8 and --mxfp4 are two different variants; pick one", file=sys.stderr)
        sys.exit(2)
    if args.workload == WRITE_WORKLOAD:
        bench_writer(args)
        return
    if args.workload == RESIDENT_WORKLOAD:
        bench_resident(args)
        return

    import torch
    torch.cuda.set_device(0)
    names = SUITE if args.workload == "suite" else [args.workload]
    results = {}
    for name in names:
        results[name] = measure_scoring(name, args)
    head = HEADLINE if args.workload == "suite" else args.workload
    out = results[head].pop("_line")
    for r in results.values():
        r.pop("_line", None)
    if args.workload == "suite":
        out["workloads"] = results
    if not args.no_cpu_baseline:
        from sparse_attention_kv_paged_amd import workloads
        wl = scoring_workload(head, args, workloads)
        out["cpu_baseline"] = cpu_baseline(wl, out["config"]["pairs"], args.cpu_seconds, mxfp4=args.mxfp4)
    print(json.dumps(out), flush=True)


def scoring_workload(name, args, workloads):
    cfg = WORKLOADS[name]
    wl = workloads.config(cfg)
    if args.block_size != 64:
        wl = workloads.reblock(wl, seed=50 + cfg, block_size=args.block_size, name=f"{wl.name}-b{args.block_size}")
    return wl


def measure_scoring(name, args):
    """K steps of idx_score_topk (or the quantised-query step) over one
    scoring workload.  Returns the workload's summary; its "_line" entry is
    the full JSON line for that workload alone."""
    import torch
    from sparse_attention_kv_paged_amd import lib, workloads

    wl = scoring_workload(name, args, workloads)
    pairs = wl.pairs()
    prof_name = wl.name + ("-q8" if args.q8 else "") + ("-mxfp4" if args.mxfp4 else "")
    print(f"[bench] workload {wl.name}: {wl.description}; pairs {pairs}", file=sys.stderr, flush=True)
    d = lib.to_device(wl)
    pool_bytes = d.keys.pool.numel()
    R = args.replicas or max(4, min(64, math.ceil(1.0e9 / max(pool_bytes, 1))))
    pools = [d.keys.pool] + [d.keys.pool.clone() for _ in range(R - 1)]
    qs = [d.q] + [d.q.clone() for _ in range(R - 1)]
    keys = [lib.Keys(pool=p, limits=d.keys.limits, block_table=d.keys.block_table,
                     q_req=d.keys.q_req, chunk_ids=d.keys.chunk_ids, n_chunks=d.keys.n_chunks,
                     block_size=wl.block_size)
            for p in pools]
    k = wl.k
    out_idx = torch.empty((wl.B, k), dtype=torch.int32, device="cuda")
    out_val = torch.empty((wl.B, k), dtype=torch.float32, device="cuda")
    ws = lib.new_workspace(lib.workspace_bytes(lib.IDX_OP_SCORE_TOPK, wl.B, wl.n_cols, k), "cuda")

    if args.q8:
        # the query quantised inside the score kernel (one launch before the
        # top-k, as the bf16 path)
        def step(i):
            lib.idx_score_topk_fp8q(qs[i % R], d.w, keys[i % R], wl.n_cols, k,
                                    out_idx=out_idx, out_val=out_val, workspace=ws)
    elif args.mxfp4:
        def step(i):
            lib.idx_score_topk_mxfp4(qs[i % R], d.w, keys[i % R], wl.n_cols, k,
                                     out_idx=out_idx, out_val=out_val, workspace=ws)
    else:
        def step(i):
            lib.idx_score_topk(qs[i % R], d.w, keys[i % R], wl.n_cols, k,
                               out_idx=out_idx, out_val=out_val, workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    # ---- timed region: K steps (graph replays), then the score kernel's own
    # duration from dispatch-stamped events over K eager steps
    ms_per_step = run_steps(step, K, R, not args.no_graph)
    kern_ms, kern_spread = spread(kernel_ms_live(step, K))
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)

    # the quantised-query step reads q as bf16 too (the kernel quantises it)
    algo = algorithmic_bytes(wl, pairs)
    kern_bytes = score_kernel_bytes(wl, pairs, logits_written=False)
    flop = 2.0 * wl.H * wl.D * pairs
    mfma_peak = (MFMA_FP8_PEAK_TFLOPS if args.q8 else MFMA_FP4_PEAK_TFLOPS if args.mxfp4
                 else MFMA_BF16_PEAK_TFLOPS)
    traffic = read_traffic(prof_name)
    prefill = shares_request_keys(wl)
    if prefill:
        # one request's keys are shared by every query: the contraction bounds it
        roofline = {"kernel": "score_kernel", "bound": "mfma",
                    "achieved": flop / (kern_ms * 1e-3) / 1e12, "peak": mfma_peak,
                    "unit": "TFLOP/s", "traffic": traffic, "algorithmic_flop": flop,
                    "algorithmic_bytes": kern_bytes, "kernel_ms": kern_ms, **kern_spread}
        # counters: the MFMA pipe's busy fraction and the clock the chip held
        busy, clock = read_mfma(prof_name)
        roofline["mfma_busy_frac"] = busy
        roofline["clock_ghz"] = clock
        path = {"bound": "mfma", "frac": flop / (ms_per_step * 1e-3) / 1e12 / mfma_peak,
                "target_frac": TARGET_MFMA_FRAC,
                "target_ms": flop / (TARGET_MFMA_FRAC * mfma_peak * 1e12) * 1e3}
    else:
        roofline = {"kernel": "score_kernel", "bound": "hbm",
                    "achieved": kern_bytes / (kern_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "traffic": traffic, "algorithmic_bytes": kern_bytes, "kernel_ms": kern_ms,
                    **kern_spread}
        path = {"bound": "hbm", "frac": algo / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "target_frac": TARGET_HBM_FRAC if wl.name != "tiny-decode" else None,
                "target_ms": algo / (TARGET_HBM_FRAC * HBM_PEAK_GBS * 1e9) * 1e3}
    roofline["frac"] = roofline["achieved"] / roofline["peak"]
    summary = {
        "ms_per_step": ms_per_step,
        "pairs": pairs,
        "queries": wl.B,
        "pairs_per_s": pairs / (ms_per_step * 1e-3),
        "queries_per_s": wl.B / (ms_per_step * 1e-3),
        "algorithmic_bytes": algo,
        "algorithmic_flop": flop,
        "path": path,
        "score_kernel_ms": kern_ms,
        "score_kernel_ms_p50": kern_spread["kernel_ms_p50"],
        "description": wl.description,
    }
    summary["_line"] = {
        "metric": "indexer scored pairs/s + top-512 queries/s; % of HBM/MFMA peak, 1 MI355X",
        "value": pairs / (ms_per_step * 1e-3),
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if args.q8 else "fp4" if args.mxfp4 else "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "queries": wl.B, "heads": wl.H, "head_dim": wl.D,
                   "query": ("e4m3, quantised per head in the score kernel" if args.q8 else
                             "MXFP4 (blocks of 32, keys too), rounded in the score kernel" if args.mxfp4 else "bf16"),
                   "block": wl.block_size, "k": k, "n_cols": wl.n_cols, "pairs": pairs,
                   "description": wl.description, "replicas": R, "graph": not args.no_graph},
        "queries_per_s": wl.B / (ms_per_step * 1e-3),
        "path": path,
        "roofline": roofline,
    }
    del pools, qs, keys, d, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return summary


if __name__ == "__main__":
    main()
