"""Benchmark of the lightning-indexer hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 1] [--kv mxfp4|fp8] [--warm]

One step is one pass of the whole hot path over one batch: the K-cache store of the
step's new rows (decode: the newest token of every sequence; prefill: every token),
the paged MQA scorer, and the per-row top-k.  Inputs are seeded synthetic data with
the shapes of the pages' isolated-scorer workloads, resident in HBM before timing.

By default the pool is rotated over enough replicas that every step reads its K cache
from HBM rather than from the 256 MB last-level cache ("cold"); --warm uses one pool.
Prints one JSON line.  Times come from HIP events recorded on the stream the kernels
run on.  While the host enqueues a timed region a spin kernel holds the GPU, so the
region runs back to back and its events measure GPU time, not host launch gaps.  Each
kernel's duration is the mean over K back-to-back launches of that kernel alone (one
event pair around them).  `value` is the GPU time per step of the step replayed as a
HIP graph; the eager step and the graph's host wall time are reported beside it.

    python bench.py --summarize DIR...   # tables from rocprofv3 csv output
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
FP4_PEAK_TFLOPS = 10100.0        # dense MXFP4 MFMA
FP8_PEAK_TFLOPS = 5000.0         # dense FP8 MFMA
LLC_BYTES = 256 << 20            # last-level (Infinity) cache


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1, choices=[0, 1, 2, 3, 4])
    ap.add_argument("--kv", default="mxfp4", choices=["mxfp4", "fp8"])
    ap.add_argument("--warm", action="store_true", help="one pool replica (cache-resident)")
    ap.add_argument("--heads", type=int, default=0, help="override the workload's head count (decode workloads)")
    ap.add_argument("--eager", action="store_true",
                    help="report the eager step time as the value (default: HIP-graph replay of the step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", action="store_true", help="the one workload named by --config/--kv, not the whole set")
    ap.add_argument("--separate", action="store_true",
                    help="time the step as three calls even where the fused decode step applies")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before timing, copy a buffer of this many MiB three times (a plain copy of "
                         "known size that scales the memory-traffic counters)")
    ap.add_argument("--summarize", nargs="+", metavar="DIR",
                    help="print per-kernel tables from rocprofv3 csv output directories and exit")
    ap.add_argument("--traffic-key", help="with --summarize: record the scorer's copy-scaled "
                                          "FETCH_SIZE + WRITE_SIZE per launch under this key in profiles/traffic.json")
    ap.add_argument("--calib-mib", type=int, default=0, help="with --traffic-key: the size of the calibration copy")
    return ap.parse_args()


def algorithmic_bytes(W, fmt, n_step_rows):
    """Bytes the method must move, per launch (valid cells only; masked cells,
    unused pool pages and the avoided K gather are excluded)."""
    bpt = 68 if fmt == 0 else 132
    valid = np.array([W.valid_len(r) for r in range(W.rows)], np.int64)
    n_valid = int(valid.sum())
    tokens = int(np.minimum(W.ctx, W.max_ctx).sum())  # K rows read once per sequence
    q_b = W.rows * W.H * (68 if fmt == 0 else 128)
    pages = int(sum((int(c) + W.page_size - 1) // W.page_size for c in W.ctx))
    scorer = tokens * bpt + q_b + W.rows * W.H * 4 + pages * 4 + W.B * 4 + n_valid * 4
    topk = n_valid * 4 + W.rows * W.topk * 4 + W.B * 4
    kstore = n_step_rows * (256 + bpt + 4 + 8) + 128 * 4 + n_step_rows * 256
    flops = n_valid * W.H * 2 * 128
    return {"scorer": scorer, "topk": topk, "kstore": kstore, "flops": flops, "valid_cells": n_valid}


def decode_form(W):
    """The scorer keeps every query row of a sequence in registers when
    n_q * ceil(H/16) <= 16 (HBM-bound decode form); otherwise it runs its prefill form."""
    return W.n_q * ((W.H + 15) // 16) <= 16


def step_rows(W):
    """K rows one step appends: the last n_q tokens of every sequence (all tokens for
    a prefill chunk, one per sequence for plain decode)."""
    rows = []
    for o, c in zip(W.seq_row_offsets()[:-1], W.ctx):
        n = min(W.n_q, int(c))
        rows.append(np.arange(int(o) + int(c) - n, int(o) + int(c), dtype=np.int64))
    return np.concatenate(rows)


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_key, src_hash):
    """HBM bytes per launch from the committed counter summary, if it was taken on
    the current kernel source (else None)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        e = d.get(kernel_key)
        if e and e.get("source_hash") == src_hash:
            return e.get("hbm_bytes_per_launch")
    except (ValueError, OSError):
        return None
    return None


SCORER_SOURCES = ("logits.hip", "logits_stream.hip", "scorer.hpp", "device_common.hpp", "launch.hpp")


def scorer_source_hash():
    return source_hash([os.path.join(ROOT, "sparse_attention_indexer_idx_amd", "csrc", f) for f in SCORER_SOURCES])


FUSED_SOURCES = SCORER_SOURCES + ("decode_step.hip", "topk_row.hpp", "kstore_row.hpp")


def fused_source_hash():
    return source_hash([os.path.join(ROOT, "sparse_attention_indexer_idx_amd", "csrc", f) for f in FUSED_SOURCES])


TOPK_SOURCES = ("topk.hip", "topk_row.hpp", "device_common.hpp", "launch.hpp")


def topk_source_hash():
    return source_hash([os.path.join(ROOT, "sparse_attention_indexer_idx_amd", "csrc", f) for f in TOPK_SOURCES])


def _short_kernel(name):
    import re
    m = re.search(r"((?:\w+::)*\w+(?:<[^()]*>)?)\(", name.replace("(anonymous namespace)::", ""))
    return (m.group(1) if m else name).split("::")[-1]


def summarize(dirs, traffic_key=None, calib_mib=0):
    """Markdown tables from rocprofv3 csv output: kernel-trace statistics and, for
    counter runs, the mean of each counter per (kernel, grid size).  With a traffic key,
    the scorer's FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what the same
    counters read for the calibration copy of calib_mib MiB, and stored per launch."""
    import csv
    import glob
    import collections
    counters = collections.defaultdict(list)
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "*kernel_stats.csv"))):
            print(f"\nkernel trace ({f}):\n")
            print("| kernel | calls | avg µs | min µs | max µs | % of GPU time |\n|---|---|---|---|---|---|")
            for r in csv.DictReader(open(f)):
                print(f"| `{_short_kernel(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                      f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
        for f in sorted(glob.glob(os.path.join(d, "*kernel_trace.csv"))):
            # bench.py times each kernel alone over K back-to-back launches; the longest
            # run of consecutive dispatches of one kernel is that loop
            rows = sorted(csv.DictReader(open(f)), key=lambda r: int(r["Start_Timestamp"]))
            best = {}
            i = 0
            while i < len(rows):
                j = i
                while j + 1 < len(rows) and rows[j + 1]["Kernel_Name"] == rows[i]["Kernel_Name"]:
                    j += 1
                name = _short_kernel(rows[i]["Kernel_Name"])
                if j - i + 1 > best.get(name, (0,))[0]:
                    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows[i:j + 1]]
                    best[name] = (j - i + 1, float(np.mean(dur)), float(np.median(dur)))
                i = j + 1
            print(f"\nlongest back-to-back run per kernel ({f}):\n")
            print("| kernel | launches in the run | mean µs | median µs |\n|---|---|---|---|")
            for name, (cnt, mean, med) in sorted(best.items(), key=lambda t: -t[1][0]):
                if cnt >= 10:
                    print(f"| `{name}` | {cnt} | {mean:.2f} | {med:.2f} |")
        for f in sorted(glob.glob(os.path.join(d, "*counter_collection.csv"))):
            for r in csv.DictReader(open(f)):
                key = (_short_kernel(r["Kernel_Name"]), int(r["Grid_Size"]), r["Counter_Name"])
                counters[key].append(float(r["Counter_Value"]))
    if counters:
        print("\n| kernel (grid threads) | counter | dispatches | mean per dispatch |\n|---|---|---|---|")
        for (k, g, c), v in sorted(counters.items()):
            print(f"| `{k}` ({g}) | {c} | {len(v)} | {np.mean(v):.6g} |")
    if not traffic_key:
        return
    def pick(pred, counter, reduce):
        vals = [(g, np.mean(v), max(v)) for (k, g, c), v in counters.items() if pred(k) and c == counter]
        if not vals:
            raise SystemExit(f"no {counter} rows for the requested kernel")
        return reduce(vals)
    scorer = lambda k: k.startswith("logits_") and not k.startswith("logits_cand")
    copy = lambda k: "copyBuffer" in k
    big = lambda vals: max(vals, key=lambda t: t[2])  # the largest grid = the timed launches
    known_kib = calib_mib * 1024.0
    f_fetch = known_kib / pick(copy, "FETCH_SIZE", lambda v: max(t[2] for t in v))
    f_write = known_kib / pick(copy, "WRITE_SIZE", lambda v: max(t[2] for t in v))
    p = os.path.join(ROOT, "profiles", "traffic.json")
    d = json.load(open(p)) if os.path.exists(p) else {}
    fused = lambda k: k.startswith("decode_step_kernel")
    topk = lambda k: k.startswith("topk_kernel")
    for key, pred, shash in ((traffic_key, scorer, scorer_source_hash()),
                             (traffic_key + "_fused", fused, fused_source_hash()),
                             (traffic_key + "_topk", topk, topk_source_hash())):
        if not any(pred(k) and c == "FETCH_SIZE" for (k, g, c) in counters):
            continue
        _, fetch, _ = pick(pred, "FETCH_SIZE", big)
        _, write, _ = pick(pred, "WRITE_SIZE", big)
        entry = {"fetch_kib_per_launch": fetch, "write_kib_per_launch": write,
                 "copy_scale_fetch": round(f_fetch, 4), "copy_scale_write": round(f_write, 4),
                 "hbm_bytes_per_launch": int(round((fetch * f_fetch + write * f_write) * 1024)),
                 "source_hash": shash}
        d[key] = entry
        print(f"\n{key}: {json.dumps(entry)}")
    with open(p, "w") as fh:
        json.dump(d, fh, indent=1, sort_keys=True)
        fh.write("\n")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(W, fmt, budget_s, max_rows=4096):
    """The oracle, as it stands, on the host cores: one step (K store of the new rows,
    logits and top-k of the rows) over every row when there are at most max_rows, else
    over a seeded sample of rows (256, or max_rows if fewer), scaled to the whole step."""
    import oracle
    pt = W.page_table
    pids = np.unique(pt[pt >= 0]).astype(np.int64)
    remap = np.full(W.num_pages, -1, np.int64)
    remap[pids] = np.arange(pids.size)
    page_bytes = (68 if fmt == 0 else 132) * W.page_size
    pool = np.zeros(pids.size * page_bytes, np.uint8)
    cpt = np.where(pt >= 0, remap[np.maximum(pt, 0)], -1).astype(np.int32)
    slots = remap[W.slots // W.page_size] * W.page_size + W.slots % W.page_size
    oracle.k_store(pool, 0, page_bytes, pids.size, W.page_size, fmt, W.k_rows, W.gamma, W.eps, W.positions,
                   W.cos_sin, slots)  # cache fill: not timed
    if fmt == 0:
        q, qs = oracle.q_quant_mxfp4(W.q_rows)
        w = W.w
    else:
        q, w = oracle.q_quant_fp8(W.q_rows, W.w)
        qs = None
    rows_all = np.arange(W.rows, dtype=np.int64)
    if W.rows <= max_rows:
        sample_rows = rows_all
    else:
        rng = np.random.default_rng(7)
        sample_rows = np.sort(rng.choice(W.rows, min(256, max_rows), replace=False)).astype(np.int64)
    new = step_rows(W)
    times = []
    t_end = time.perf_counter() + budget_s
    while True:
        t0 = time.perf_counter()
        oracle.k_store(pool, 0, page_bytes, pids.size, W.page_size, fmt, W.k_rows[new], W.gamma, W.eps,
                       W.positions[new], W.cos_sin, slots[new])
        lg = oracle.logits_paged(pool, 0, page_bytes, pids.size, W.page_size, fmt, q, qs, w, cpt, W.ctx, W.B, W.n_q,
                                 W.H, W.max_ctx, sample_rows)
        oracle.topk(lg, W.ctx, W.n_q, W.topk, sample_rows)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() > t_end or len(times) >= 5:
            break
    per_step = float(np.median(times)) * (W.rows / sample_rows.size)
    sample = (f"{len(times)} oracle step(s): K store of {len(new)} rows + logits and top-k of "
              f"{sample_rows.size}/{W.rows} rows" + ("" if sample_rows.size == W.rows else ", scaled to all rows"))
    return {"value": round(per_step * 1e6, 1), "unit": "us/call", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": sample, "cpu": cpu_model(), "nproc": os.cpu_count()}


def scorer_kernel(W):
    """The scorer form idx_logits_paged takes for this shape (mirrors its routing)."""
    ht = (W.H + 15) // 16
    stream_ok = W.n_q <= 4 and W.B <= 1024 and W.max_ctx <= (1 << 30) and W.B * ((W.max_ctx + 63) // 64) < (1 << 31)
    if stream_ok and W.n_q > 1 and W.n_q * ht > 4:
        return "logits_stream_kernel"
    if stream_ok and W.n_q == 1 and W.B * W.max_ctx >= (1 << 21):
        return "logits_stream_kernel"
    if W.n_q * ht <= 16:
        return "logits_decode_rows_kernel" if (W.n_q > 1 and W.n_q * ht > 4) else "logits_decode_kernel"
    return "logits_prefill_kernel"


def make_held(torch):
    def held(fn, n, host_s):
        """GPU time of n back-to-back calls fn(0..n-1): a spin kernel holds the GPU while
        the host enqueues them, and one event pair brackets the whole run, so neither
        host launch gaps nor per-call event overhead enter the average.  Returns the mean
        per call and the means of groups of 10 calls (µs)."""
        torch.cuda.synchronize()
        groups = max(1, n // 10)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(groups + 1)]
        torch.cuda._sleep(int((2.0 * host_s * n + 2e-3) * 2.4e9))
        ev[0].record()
        for gi in range(groups):
            for i in range(gi * n // groups, (gi + 1) * n // groups):
                fn(i)
            ev[gi + 1].record()
        torch.cuda.synchronize()
        per = [ev[gi].elapsed_time(ev[gi + 1]) * 1e3 / ((gi + 1) * n // groups - gi * n // groups)
               for gi in range(groups)]
        return ev[0].elapsed_time(ev[-1]) * 1e3 / n, np.array(per)
    return held


def time_graph(torch, step_fn, L, steps):
    """GPU time per step of `steps` steps replayed from HIP graphs: graph A holds L
    consecutive steps (L a multiple of the replica count, at least 8, so a replay's fixed
    launch cost is shared as it is across the layers of a captured model), graph B the
    steps mod L remaining ones, so the timed region is exactly `steps` steps; and the host
    wall time of the same steps enqueued as the host goes (ms per step, both)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(L):
            step_fn(i)  # warm the captured configuration eagerly on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                step_fn(i)
        return g
    graph_a = capture(L)
    rem = steps % L
    graph_b = capture(rem) if rem else None

    def replay_k():
        for _ in range(steps // L):
            graph_a.replay()
        if graph_b is not None:
            graph_b.replay()
    replay_k()  # warm-up replays (untimed)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    replay_k()
    host_s = (time.perf_counter() - h0) / steps
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int((2.0 * host_s * steps + 2e-3) * 2.4e9))
    g0.record()
    replay_k()
    g1.record()
    torch.cuda.synchronize()
    gpu_ms = g0.elapsed_time(g1) / steps
    t0 = time.perf_counter()
    replay_k()
    torch.cuda.synchronize()
    return gpu_ms, (time.perf_counter() - t0) * 1e3 / steps


class Run:
    """Device inputs of one workload, resident in HBM: pool replicas holding the whole
    context (rotated so that each step reads K from HBM rather than the last-level cache),
    packed Q and weights, page table, lengths, output buffers and the step's new rows."""

    def __init__(self, torch, bd, wl, config, kv, warm=False, heads=0, calib_copy_mib=0):
        self.torch, self.bd = torch, bd
        self.config, self.kv = config, kv
        fmt = self.fmt = 0 if kv == "mxfp4" else 1
        W = self.W = wl.make_workload(config, kv_format=fmt, scale={"H": heads} if heads else None)
        dev = self.dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
        P = W.page_size
        page_bytes = (68 if fmt == 0 else 132) * P
        stride = max(W.page_stride_bytes, page_bytes)
        pool_bytes = W.offset_bytes + W.num_pages * stride
        used_bytes = int(np.minimum(W.ctx, W.max_ctx).sum()) * (68 if fmt == 0 else 132)
        # Prefill re-reads its small K from L2 by design and writes far more logits than
        # the last-level cache holds, so only decode rotates pool replicas.
        self.prefill = not decode_form(W)
        replicas = 1 if (warm or self.prefill) else max(2, int(np.ceil(2 * LLC_BYTES / max(used_bytes, 1))) + 1)
        self.replicas = min(replicas, 64, max(1, int((64 << 30) // pool_bytes)))
        self.cache = "warm" if warm else f"cold ({self.replicas} pool replicas rotated)"
        k_all = dev(W.k_rows.view(np.int16)).view(torch.bfloat16)
        self.gamma, self.cos_sin = dev(W.gamma), dev(W.cos_sin)
        positions, slots = dev(W.positions), dev(W.slots)
        self.pools = []
        for _ in range(self.replicas):
            t = torch.empty((pool_bytes + 256,), dtype=torch.uint8, device="cuda")
            shift = (-t.data_ptr()) % 256
            self.pools.append((t, bd.make_pool(t[shift:], W.offset_bytes, stride, W.num_pages, P, fmt)))
        self.store = bd.idx_k_store_mxfp4 if fmt == 0 else bd.idx_k_store_fp8
        for _, pv in self.pools:  # fill every replica's cache with the whole context (setup)
            self.store(pv, k_all, self.gamma, W.eps, positions, self.cos_sin, slots)
        self.q_bf16 = dev(W.q_rows.reshape(-1, 128).view(np.int16)).view(torch.bfloat16)
        nvec = self.q_bf16.shape[0]
        if fmt == 0:
            self.q = torch.empty((nvec, 64), dtype=torch.uint8, device="cuda")
            self.qs = torch.empty((nvec, 4), dtype=torch.uint8, device="cuda")
            bd.idx_q_quant_mxfp4(self.q_bf16, self.q, self.qs)
            self.w = dev(W.w.reshape(-1))
        else:
            self.q = torch.empty((nvec, 128), dtype=torch.uint8, device="cuda")
            self.qs = None
            self.w = torch.empty((nvec,), dtype=torch.float32, device="cuda")
            bd.idx_q_quant_fp8(self.q_bf16, dev(W.w.reshape(-1)), self.q, self.w)
        self.pt, self.ctx = dev(W.page_table), dev(W.ctx)
        self.logits = torch.empty((W.rows, W.max_ctx), dtype=torch.float32, device="cuda")
        self.out = torch.empty((W.rows, W.topk), dtype=torch.int32, device="cuda")
        self.new = step_rows(W)
        nd = dev(self.new)
        self.k_new, self.pos_new, self.slot_new = k_all[nd], positions[nd], slots[nd]
        del k_all, positions, slots
        self.ws = torch.zeros((max(bd.idx_workspace_bytes(W.B, W.n_q, W.H, W.max_ctx, W.topk), 256) // 4,),
                              dtype=torch.int32, device="cuda")
        if calib_copy_mib:  # a plain device copy of known size, outside the timed region
            src = torch.ones((calib_copy_mib << 20,), dtype=torch.uint8, device="cuda")
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            del src, dst
        torch.cuda.synchronize()

    def pool(self, i):
        return self.pools[i % self.replicas][1]

    def k_store(self, i):
        W = self.W
        self.store(self.pool(i), self.k_new, self.gamma, W.eps, self.pos_new, self.cos_sin, self.slot_new)

    def score(self, i):
        W = self.W
        self.bd.idx_logits_paged(self.pool(i), self.q, self.qs, self.w, self.pt, self.ctx, W.B, W.n_q, W.H,
                                 W.max_ctx, self.logits)

    def topk(self, i):
        W = self.W
        self.bd.idx_topk(self.logits, self.ctx, W.B, W.n_q, W.topk, self.out)

    def step(self, i):
        self.k_store(i)
        self.score(i)
        self.topk(i)

    def fused_step(self, i):
        W = self.W
        self.bd.idx_decode_step(self.pool(i), self.k_new, self.gamma, W.eps, self.pos_new, self.cos_sin,
                                self.slot_new, self.q, self.qs, self.w, self.pt, self.ctx, W.B, W.n_q, W.H, W.max_ctx,
                                self.logits, W.topk, self.out, self.ws)

    def fuses(self):
        """Whether idx_decode_step runs this step as its one fused kernel."""
        W = self.W
        if len(self.new) != W.B * W.n_q:
            return False
        try:
            return self.bd.idx_decode_step_fused(W.B, W.n_q, W.H, W.max_ctx) == 1
        except self.bd.IdxError as e:
            if e.status != self.bd.IDX_EUNSUPPORTED:
                raise
            return False


def scorer_roof(R, ab, s_mean):
    """Roofline of the scorer: algorithmic bytes (decode forms, against HBM) or FP4 / FP8
    flops (prefill form, against the MFMA peak of its format) over its mean duration."""
    W, fmt = R.W, R.fmt
    shash = scorer_source_hash()
    if R.prefill:
        achieved = ab["flops"] / (s_mean * 1e-6) / 1e12
        peak = FP4_PEAK_TFLOPS if fmt == 0 else FP8_PEAK_TFLOPS
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "algorithmic_flops": ab["flops"]}
    else:
        achieved = ab["scorer"] / (s_mean * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["kernel"] = scorer_kernel(W)
    roof["traffic"] = traffic_from_profiles(f"cfg{R.config}_{R.kv}", shash)
    roof["algorithmic_bytes"] = ab["scorer"]
    roof["source_hash"] = shash
    return roof


def topk_roof(R, ab, t_mean):
    """Roofline of the top-k: logits read (valid cells) and indices written over its mean
    duration, against HBM."""
    gbs = ab["topk"] / (t_mean * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": ab["topk"], "kernel": "topk_kernel",
            "traffic": traffic_from_profiles(f"cfg{R.config}_{R.kv}_topk", topk_source_hash()),
            "source_hash": topk_source_hash()}


def summary(R, held, steps, cpu_budget_s, with_cpu):
    """One workload measured the short way: each kernel alone back to back, the step
    replayed from HIP graphs, the scorer's and the top-k's rooflines, and the oracle on a
    bounded sample of rows."""
    W = R.W
    for i in range(3):
        R.step(i)
    R.torch.cuda.synchronize()
    h0 = time.perf_counter()
    for i in range(3):
        R.step(i)
    host_s = (time.perf_counter() - h0) / 3
    k_mean, _ = held(R.k_store, steps, host_s)
    s_mean, _ = held(R.score, steps, host_s)
    t_mean, _ = held(R.topk, steps, host_s)
    fused = R.fuses()
    L = R.replicas * max(1, -(-8 // R.replicas))
    graph_ms, _ = time_graph(R.torch, R.fused_step if fused else R.step, L, steps)
    ab = algorithmic_bytes(W, R.fmt, len(R.new))
    d = {"workload": W.name, "kv": R.kv, "B": W.B, "n_q": W.n_q, "H": W.H, "page_size": W.page_size,
         "max_ctx": W.max_ctx, "topk": W.topk, "cache": R.cache,
         "step_us": round(graph_ms * 1e3, 3),
         "path": "fused idx_decode_step" if fused else "idx_k_store + idx_logits_paged + idx_topk",
         "k_store_us": round(k_mean, 3), "score_us": round(s_mean, 3), "topk_us": round(t_mean, 3),
         "scorer_roofline": scorer_roof(R, ab, s_mean),
         "topk_roofline": topk_roof(R, ab, t_mean)}
    if with_cpu:
        d["cpu_baseline"] = cpu_baseline(W, R.fmt, cpu_budget_s, max_rows=32)
    return d


# The five workloads a default run reports beside the headline one (config index, K format).
ALL_CONFIGS = (("C0", 0, "mxfp4"), ("C1", 1, "mxfp4"), ("C2", 2, "mxfp4"), ("C3", 3, "mxfp4"),
               ("C4a", 4, "mxfp4"), ("C4b", 4, "fp8"))


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize, args.traffic_key, args.calib_mib)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; run with --gpus 1"}))
        sys.exit(2)
    import torch
    from sparse_attention_indexer_idx_amd import binding as bd
    from sparse_attention_indexer_idx_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    bd.load()
    if bd.idx_device_check() != bd.IDX_OK:
        raise SystemExit("device is not gfx950")
    held = make_held(torch)
    R = Run(torch, bd, wl, args.config, args.kv, warm=args.warm, heads=args.heads,
            calib_copy_mib=args.calib_copy_mib)
    W, fmt, P = R.W, R.fmt, R.W.page_size
    fused = not args.separate and R.fuses()
    if fused:
        R.fused_step(0)
        torch.cuda.synchronize()

    for i in range(args.warmup):
        R.step(i)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    for i in range(args.warmup):
        R.step(i)
    host_s = (time.perf_counter() - h0) / max(args.warmup, 1)  # host cost of enqueueing one step
    torch.cuda.synchronize()
    # Timed region: exactly K eager steps on the kernels' own (current) stream, then each
    # kernel alone K times back to back for its average duration.
    eager_us, _ = held(R.step, args.steps, host_s)
    eager_ms = eager_us * 1e-3
    k_mean, k_us = held(R.k_store, args.steps, host_s)
    s_mean, s_us = held(R.score, args.steps, host_s)
    t_mean, t_us = held(R.topk, args.steps, host_s)
    # the scorer on one pool replica over and over: K then sits in the last-level cache
    w_mean, _ = held(lambda i: R.score(0), args.steps, host_s)
    qprep_us = None
    if fmt == 0:
        # The Q-side preparation that feeds the scorer (rotation + MXFP4 packing + weight
        # fold of every query row's heads), timed alone; it is not part of the step.
        q3 = R.q_bf16.view(W.rows, W.H, 128)
        qpos = R.dev(np.array([max(W.valid_len(r) - 1, 0) for r in range(W.rows)], np.int32))
        qp2, qs2 = torch.empty_like(R.q), torch.empty_like(R.qs)
        w2 = torch.empty_like(R.w)
        qprep_us, _ = held(lambda i: bd.idx_q_prep_mxfp4(q3, qpos, R.cos_sin, R.w, 0.0625, qp2, qs2, w2), args.steps,
                           host_s)

    cand_us = None
    if decode_form(W):
        # The candidate-block scorer and its top-k (a two-level indexer's second level):
        # every row scores 16 blocks of its sequence drawn without replacement (seeded),
        # over the same rotated pool replicas; not part of the step.
        n_cand = min(16, W.page_table.shape[1])
        cand = R.dev(wl.candidate_blocks(np.random.default_rng(77), W, n_cand))
        clog = torch.empty((W.rows, n_cand * P), dtype=torch.float32, device="cuda")
        cout = torch.empty((W.rows, W.topk), dtype=torch.int32, device="cuda")
        cs_mean, _ = held(lambda i: bd.idx_logits_candidates(R.pool(i), R.q, R.qs, R.w, R.pt, R.ctx, W.B, W.n_q, W.H,
                                                             cand, clog), args.steps, host_s)
        ct_mean, _ = held(lambda i: bd.idx_topk_candidates(clog, cand, P, W.B, W.n_q, W.topk, cout), args.steps,
                          host_s)
        cells = W.rows * n_cand * P
        cbytes = cells * (68 if fmt == 0 else 132) // max(W.n_q, 1) + cells * 4 + W.rows * n_cand * 4
        cand_us = {"blocks_per_row": n_cand, "score": round(cs_mean, 3), "topk": round(ct_mean, 3),
                   "score_hbm_gbs": round(cbytes / (cs_mean * 1e-6) / 1e9, 1)}

    L = R.replicas * max(1, -(-8 // R.replicas))
    graph_ms, graph_wall_ms = time_graph(torch, R.step, L, args.steps)
    sep_graph_ms = graph_ms
    fused_us = None
    if fused:
        # The same step through the fused entry point (K store + scorer + top-k in one
        # launch); its result equals the separate calls bit for bit (tested).
        fused_us, _ = held(R.fused_step, args.steps, host_s)
        graph_ms, graph_wall_ms = time_graph(torch, R.fused_step, L, args.steps)
    ms_per_step = eager_ms if args.eager else graph_ms

    ab = algorithmic_bytes(W, fmt, len(R.new))
    roof = scorer_roof(R, ab, s_mean)
    fused_roof = None
    if fused_us is not None:
        fb = ab["scorer"] + ab["topk"] + ab["kstore"]
        fused_roof = {"bound": "hbm", "achieved": round(fb / (fused_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                      "unit": "GB/s", "frac": round(fb / (fused_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                      "kernel": "decode_step_kernel",
                      "traffic": traffic_from_profiles(f"cfg{args.config}_{args.kv}_fused", fused_source_hash()),
                      "algorithmic_bytes": fb, "source_hash": fused_source_hash(),
                      "note": "the whole step in one launch (K store + scorer + top-k), the top-k tail's "
                              "latency included"}
    step_us = ms_per_step * 1e3
    result = {
        "metric": "indexer score+top-k us/call; HBM TB/s (decode), FP4 TFLOPS (prefill)",
        "value": round(step_us, 3),
        "unit": "us/call",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4" if fmt == 0 else "fp8_e4m3",
        "data": "synthetic (seeded N(0,1) bf16 K/Q rows, shuffled physical pages)",
        "config": {"workload": W.name, "B": W.B, "n_q": W.n_q, "H": W.H, "D": 128, "page_size": P,
                   "max_ctx": W.max_ctx, "topk": W.topk, "kv": args.kv, "cache": R.cache},
        "step_us": {"graph": round(graph_ms * 1e3, 3), "eager": round(eager_ms * 1e3, 3),
                    "graph_wall": round(graph_wall_ms * 1e3, 3), "steps_per_graph": L,
                    "path": "fused idx_decode_step" if fused else "idx_k_store + idx_logits_paged + idx_topk",
                    "separate_graph": round(sep_graph_ms * 1e3, 3),
                    "fused_kernel": None if fused_us is None else round(fused_us, 3)},
        "breakdown_us": {"k_store": round(k_mean, 3), "score": round(s_mean, 3), "topk": round(t_mean, 3),
                         "score_p10_p90": [round(float(np.percentile(s_us, 10)), 3),
                                           round(float(np.percentile(s_us, 90)), 3)],
                         "score_plus_topk": round(s_mean + t_mean, 3),
                         "score_warm": round(w_mean, 3),
                         "note": "each kernel alone, back to back; per-call mean (p10/p90 over groups of 10 calls); "
                                 "score_warm: the scorer on one pool replica (K resident in the last-level cache)"},
        # the step's kernel: the fused decode step when the step runs through it, else the
        # scorer (the dominant one of the three); the scorer alone is always listed too
        "roofline": roof if fused_us is None else fused_roof,
        "scorer_roofline": roof,
        "topk_roofline": topk_roof(R, ab, t_mean),
        "q_prep_us": None if qprep_us is None else round(qprep_us, 3),
        "candidates_us": cand_us,
        "scorer_tflops": round(ab["flops"] / (s_mean * 1e-6) / 1e12, 2),
    }
    result["device"] = device_rates(torch, held, host_s)
    result["qk_prep_fp8_us"] = qk_prep_fp8_times(held, host_s, args.steps)
    if not args.no_cpu_baseline:
        # the CPU leg: the oracle timed on the host cores, and the same-run precision
        # comparison against the oracle's unquantised scorer
        result["cpu_baseline"] = cpu_baseline(W, fmt, args.cpu_budget_s)
        result["precision_vs_unquantized"] = precision_vs_unquantized(W, R.logits.cpu().numpy(), R.out.cpu().numpy())
    if not args.only:
        # Every workload of the set, measured the short way (the headline one included,
        # so the set reads as one table); each workload's buffers are freed before the next.
        head = (args.config, args.kv)
        del R
        torch.cuda.empty_cache()
        configs = {}
        for name, cfg, kv in ALL_CONFIGS:
            if args.warm or args.heads:
                break
            Rc = Run(torch, bd, wl, cfg, kv)
            configs[name] = summary(Rc, held, min(args.steps, 50), 3.0, not args.no_cpu_baseline)
            if (cfg, kv) != head and not args.no_cpu_baseline:
                pr = precision_vs_unquantized(Rc.W, Rc.logits.cpu().numpy(), Rc.out.cpu().numpy(), n_rows=2)
                configs[name]["precision_vs_unquantized"] = pr
            del Rc
            torch.cuda.empty_cache()
            print(f"[bench] {name} done", file=sys.stderr, flush=True)
        result["configs"] = configs
    print(json.dumps(result), flush=True)


def precision_vs_unquantized(W, logits, out, n_rows=4):
    """This arm's logits and top-k against the method on unquantised operands (bf16 K rows
    through RMSNorm and NeoX RoPE, bf16 Q, fp32 weights, all fp64, with no MXFP4 or e4m3
    rounding), computed by the oracle's unquantised K rows (oracle.k_rows_exact) and
    scorer (oracle.logits_exact).  Cosine over the valid cells and top-k recall, on
    n_rows sampled rows with more than k valid cells (part of the CPU leg)."""
    import oracle
    from sparse_attention_indexer_idx_amd import workloads as wl
    cand = [r for r in range(W.rows) if W.valid_len(r) > W.topk]
    if not cand:
        return None
    rows = sorted({cand[int(i)] for i in np.linspace(0, len(cand) - 1, n_rows)})
    offs = W.seq_row_offsets()
    cos, rec = [], []
    for r in rows:
        b, j = divmod(r, W.n_q)
        n = W.valid_len(r)
        z = oracle.k_rows_exact(W.k_rows[offs[b]: offs[b] + n], W.gamma, W.eps, W.positions[offs[b]: offs[b] + n],
                                W.cos_sin)                                       # [n, 128]
        q = wl.bf16_bits_to_f32(W.q_rows[b, j]).astype(np.float64)              # [H, 128]
        ref = oracle.logits_exact(q.reshape(1, W.H, 128), W.w[b, j], z.reshape(1, n, 128), np.array([n], np.int32),
                                  1, W.H, n, np.zeros(1, np.int64))[0]
        got = logits[r, :n].astype(np.float64)
        cos.append(float(got @ ref / (np.linalg.norm(got) * np.linalg.norm(ref))))
        top_ref = np.argsort(-ref, kind="stable")[:W.topk]
        rec.append(len(np.intersect1d(top_ref, out[r][out[r] >= 0])) / W.topk)
    return {"rows": rows, "cosine_min": round(min(cos), 7), "topk_recall_min": round(min(rec), 4),
            "topk_recall_mean": round(float(np.mean(rec)), 4),
            "reference": "the oracle's fp64 logits of the unquantised bf16 K (RMSNorm + NeoX RoPE) and Q"}


def qk_prep_fp8_times(held, host_s, steps):
    """idx_qk_prep_fp8 (LayerNorm k, interleaved RoPE on q and k, FP8 q with the scale
    folded into the weights, FP8 k to the pages) for 1 and 1024 tokens at 32 heads and
    page size 64, each timed alone back to back; not part of the step."""
    import torch
    from sparse_attention_indexer_idx_amd import binding as bd
    from sparse_attention_indexer_idx_amd import workloads as wl
    out = {}
    rng = np.random.default_rng(53)
    for T in (1, 1024):
        H, P, max_pos = 32, 64, 8192
        n_pages = (T + P - 1) // P + 1
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
        pool = torch.zeros(n_pages * 132 * P, dtype=torch.uint8, device="cuda")
        view = bd.make_pool(pool, 0, 132 * P, n_pages, P, wl.FP8)
        q = dev(wl.f32_to_bf16_bits(rng.standard_normal((T, H, 128), dtype=np.float32)).view(np.int16)).view(
            torch.bfloat16)
        k = dev(wl.f32_to_bf16_bits(rng.standard_normal((T, 128), dtype=np.float32)).view(np.int16)).view(
            torch.bfloat16)
        w = dev(rng.standard_normal((T, H), dtype=np.float32))
        pos = dev(rng.integers(0, max_pos, T).astype(np.int32))
        slots = dev(rng.permutation(n_pages * P)[:T].astype(np.int64))
        cs = dev(wl.rope_cos_sin(max_pos))
        g, b = torch.ones(128, device="cuda"), torch.zeros(128, device="cuda")
        q8 = torch.empty((T, H, 128), dtype=torch.uint8, device="cuda")
        wo = torch.empty((T, H), dtype=torch.float32, device="cuda")
        f = lambda i: bd.idx_qk_prep_fp8(view, q, k, w, pos, cs, False, g, b, 1e-6, slots, q8, wo)
        f(0)
        us, _ = held(f, steps, host_s)
        out[str(T)] = round(us, 3)
    return out


def device_rates(torch, held, host_s):
    """CU count and peak clock as the runtime reports them; the sustained rate of the
    scaled 16x16x128 MFMA on register operands (idx_diag_mfma) at 2, 4 and 8 waves per
    SIMD, next to the nominal peaks; and the rate of a plain streaming read
    (idx_diag_hbm_read) of the decode workload's K bytes (35,651,584) and of 1 GiB, each
    the best over a few grid sizes, next to the nominal 8 TB/s."""
    from sparse_attention_indexer_idx_amd import binding as bd
    cus, khz = bd.idx_device_info()
    rounds = 2000
    rates = {}
    for name, f in (("fp4", 0), ("fp8", 1)):
        sweep = {}
        for wps in (2, 4, 8):
            blocks = cus * wps  # 4 waves per block, 4 SIMDs per CU
            buf = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
            bd.idx_diag_mfma(f, blocks, rounds, buf)
            us, _ = held(lambda i: bd.idx_diag_mfma(f, blocks, rounds, buf), 5, host_s)
            sweep[str(wps)] = round(blocks * 4 * rounds * 8 * 2 * 16 * 16 * 128 / (us * 1e-6) / 1e12, 1)
            del buf
        rates[name] = {"best": max(sweep.values()), "by_waves_per_simd": sweep}
    reads = {}
    for label, nbytes in (("decode_k_35.65MB", 35651584), ("1GiB", 1 << 30)):
        # buffers rotated so that every read comes from HBM (their sum is twice the 256 MB
        # last-level cache); one read = one launch over one buffer
        nbuf = max(1, int(np.ceil(2 * LLC_BYTES / nbytes)) + 1) if nbytes < LLC_BYTES else 1
        srcs = [torch.ones(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(nbuf)]
        best = None
        for blocks in (1024, 2048, 4096, 8192):
            out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
            bd.idx_diag_hbm_read(srcs[0], blocks, out)
            us, _ = held(lambda i: bd.idx_diag_hbm_read(srcs[i % nbuf], blocks, out), max(10, 2 * nbuf), host_s)
            gbs = nbytes / (us * 1e-6) / 1e9
            if best is None or gbs > best[0]:
                best = (gbs, blocks, us)
            del out
        reads[label] = {"gbs": round(best[0], 1), "blocks": best[1], "us": round(best[2], 3), "buffers_rotated": nbuf}
        del srcs
    return {"cus": cus, "clock_mhz": round(khz / 1000), "mfma_measured_tflops": rates,
            "mfma_nominal_tflops": {"fp4": FP4_PEAK_TFLOPS, "fp8": FP8_PEAK_TFLOPS},
            "hbm_read_measured": reads, "hbm_nominal_gbs": HBM_PEAK_GBS}


if __name__ == "__main__":
    main()
