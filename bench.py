"""Benchmark of the lightning-indexer hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 1] [--kv mxfp4|fp8] [--warm]

One step is one pass of the whole hot path over one batch: the K-cache store of the
step's new rows (decode: the newest token of every sequence; prefill: every token),
the paged MQA scorer, and the per-row top-k.  Inputs are seeded synthetic data with
the shapes of the pages' isolated-scorer workloads, resident in HBM before timing.

By default the pool is rotated over enough replicas that every step reads its K cache
from HBM rather than from the 256 MB last-level cache ("cold"); --warm uses one pool.
Prints one JSON line.  Kernel durations come from HIP events recorded on the stream
the kernels run on, inside the timed loop.
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
    ap.add_argument("--eager", action="store_true",
                    help="report the eager step time as the value (default: HIP-graph replay of the step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0)
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


def cpu_baseline(W, fmt, budget_s):
    """The oracle, as it stands, on the host cores: one full step (K store of the new
    rows, logits of every row, top-k of every row) for the decode workloads; for the
    prefill workload a bounded sample of rows, scaled to one step."""
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
    if W.rows <= 4096:
        sample_rows = rows_all
    else:
        rng = np.random.default_rng(7)
        sample_rows = np.sort(rng.choice(W.rows, 256, replace=False)).astype(np.int64)
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
    return {"value": per_step * 1e6, "unit": "us/call", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": sample}


def main():
    args = parse()
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
    fmt = 0 if args.kv == "mxfp4" else 1
    W = wl.make_workload(args.config, kv_format=fmt)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    P = W.page_size
    page_bytes = (68 if fmt == 0 else 132) * P
    stride = max(W.page_stride_bytes, page_bytes)
    pool_bytes = W.offset_bytes + W.num_pages * stride
    used_bytes = int(np.minimum(W.ctx, W.max_ctx).sum()) * (68 if fmt == 0 else 132)
    # Prefill re-reads its small K from L2 by design and writes far more logits than
    # the last-level cache holds, so only decode rotates pool replicas.
    prefill_like = not decode_form(W)
    replicas = 1 if (args.warm or prefill_like) else max(2, int(np.ceil(2 * LLC_BYTES / max(used_bytes, 1))) + 1)
    replicas = min(replicas, 16, max(1, int((64 << 30) // pool_bytes)))

    # ---- inputs in HBM ----
    k_all = dev(W.k_rows.view(np.int16)).view(torch.bfloat16)
    gamma, cos_sin = dev(W.gamma), dev(W.cos_sin)
    positions, slots = dev(W.positions), dev(W.slots)
    pools = []
    for _ in range(replicas):
        t = torch.empty((pool_bytes + 256,), dtype=torch.uint8, device="cuda")
        shift = (-t.data_ptr()) % 256
        pools.append((t, bd.make_pool(t[shift:], W.offset_bytes, stride, W.num_pages, P, fmt)))
    store = bd.idx_k_store_mxfp4 if fmt == 0 else bd.idx_k_store_fp8
    for _, pv in pools:  # fill every replica's cache with the whole context (setup)
        store(pv, k_all, gamma, W.eps, positions, cos_sin, slots)
    q_bf16 = dev(W.q_rows.reshape(-1, 128).view(np.int16)).view(torch.bfloat16)
    nvec = q_bf16.shape[0]
    if fmt == 0:
        q = torch.empty((nvec, 64), dtype=torch.uint8, device="cuda")
        qs = torch.empty((nvec, 4), dtype=torch.uint8, device="cuda")
        bd.idx_q_quant_mxfp4(q_bf16, q, qs)
        w = dev(W.w.reshape(-1))
    else:
        q = torch.empty((nvec, 128), dtype=torch.uint8, device="cuda")
        qs = None
        w = torch.empty((nvec,), dtype=torch.float32, device="cuda")
        bd.idx_q_quant_fp8(q_bf16, dev(W.w.reshape(-1)), q, w)
    pt, ctx = dev(W.page_table), dev(W.ctx)
    logits = torch.empty((W.rows, W.max_ctx), dtype=torch.float32, device="cuda")
    out = torch.empty((W.rows, W.topk), dtype=torch.int32, device="cuda")
    new = step_rows(W)
    k_new, pos_new, slot_new = k_all[dev(new)], positions[dev(new)], slots[dev(new)]
    torch.cuda.synchronize()

    def step(i, ev=None):
        pv = pools[i % replicas][1]
        if ev:
            ev[0].record()
        store(pv, k_new, gamma, W.eps, pos_new, cos_sin, slot_new)
        if ev:
            ev[1].record()
        bd.idx_logits_paged(pv, q, qs, w, pt, ctx, W.B, W.n_q, W.H, W.max_ctx, logits)
        if ev:
            ev[2].record()
        bd.idx_topk(logits, ctx, W.B, W.n_q, W.max_ctx, W.topk, out)
        if ev:
            ev[3].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: exactly K steps, events on the kernels' own (current) stream
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    eager_ms = (t1 - t0) * 1e3 / args.steps
    k_us = np.array([e[0].elapsed_time(e[1]) for e in events]) * 1e3
    s_us = np.array([e[1].elapsed_time(e[2]) for e in events]) * 1e3
    t_us = np.array([e[2].elapsed_time(e[3]) for e in events]) * 1e3

    # The same step captured once per pool replica into a HIP graph and replayed, as a
    # serving loop runs the indexer; the timed region is exactly K replays.
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(replicas):
            step(i)  # warm the captured configuration eagerly on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i in range(replicas):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i)
        graphs.append(g)
    for i in range(args.warmup):
        graphs[i % replicas].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % replicas].replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    graph_ms = (t1 - t0) * 1e3 / args.steps
    ms_per_step = eager_ms if args.eager else graph_ms

    ab = algorithmic_bytes(W, fmt, len(new))
    src = [os.path.join(ROOT, "sparse_attention_indexer_idx_amd", "csrc", f) for f in
           ("logits.hip", "device_common.hpp", "launch.hpp")]
    shash = source_hash(src)
    prefill = not decode_form(W)
    if prefill:
        achieved = ab["flops"] / (s_us.mean() * 1e-6) / 1e12
        peak = FP4_PEAK_TFLOPS if fmt == 0 else FP8_PEAK_TFLOPS
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4)}
    else:
        achieved = ab["scorer"] / (s_us.mean() * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["kernel"] = "logits_prefill_kernel" if prefill else "logits_decode_kernel"
    roof["traffic"] = traffic_from_profiles(f"cfg{args.config}_{args.kv}", shash)
    roof["algorithmic_bytes"] = ab["scorer"]
    roof["source_hash"] = shash
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
                   "max_ctx": W.max_ctx, "topk": W.topk, "kv": args.kv,
                   "cache": "warm" if args.warm else f"cold ({replicas} pool replicas rotated)"},
        "step_us": {"graph": round(graph_ms * 1e3, 3), "eager": round(eager_ms * 1e3, 3)},
        "breakdown_us": {"k_store": round(float(np.median(k_us)), 3), "score": round(float(np.median(s_us)), 3),
                         "topk": round(float(np.median(t_us)), 3),
                         "score_p10_p90": [round(float(np.percentile(s_us, 10)), 3),
                                           round(float(np.percentile(s_us, 90)), 3)],
                         "score_plus_topk_mean": round(float(s_us.mean() + t_us.mean()), 3)},
        "roofline": roof,
        "topk_hbm_gbs": round(ab["topk"] / (t_us.mean() * 1e-6) / 1e9, 1),
        "scorer_tflops": round(ab["flops"] / (s_us.mean() * 1e-6) / 1e12, 2),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(W, fmt, args.cpu_budget_s)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
