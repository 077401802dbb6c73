"""Decode-attention throughput of the WISE path on one MI355X.

A step is one token of every row through the workload's depth schedule
(e.g. discover, discover-union, sparse, sparse) for every layer: each
(depth, layer) call is the split-KV decode kernel plus the finish kernel.
The timed region starts with every input resident in HBM.

Prints ONE JSON line (see the design doc for every field).
"""

from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from block_sparse_paged_split_amd import harness, synth  # noqa: E402
from block_sparse_paged_split_amd import wise as W  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def split_bytes(w, ctx, mode, support_words, bt_width):
    """Algorithmic bytes one split-KV launch moves for one (depth, layer).

    Per (row, head): K and V of every attended token (2 * d * e each), q
    (d * e), and per row the block-table entries of the attended pages.
    Discovery rows also write 8 bytes of tile stats per block; sparse rows
    read their support words.
    """
    e = 2 if w.dtype == "bf16" else 4
    d, H, P = w.head_dim, w.heads, w.page_size
    total = 0
    for r in range(w.rows):
        n = int(ctx[r])
        nb = (n + 31) // 32
        pages = (n + P - 1) // P
        total += pages * 4
        for h in range(H):
            if mode == W.WISE_SPARSE:
                bits = support_words[r, h]
                blocks = [b for b in range(nb) if (int(bits[b >> 5]) >> (b & 31)) & 1]
                toks = sum(min(32, n - 32 * b) for b in blocks)
                total += 4 * ((nb + 31) // 32)
            else:
                toks = n
                if mode != W.WISE_DENSE:
                    total += 8 * nb
            total += 2 * toks * d * e + d * e
    return total


def cpu_baseline(w, min_s=10.0, max_rows=32):
    """The fp64 oracle on a bounded sample of the same workload: up to
    max_rows rows through the whole depth schedule, repeated until at least
    min_s seconds of oracle time; single-threaded BLAS."""
    from threadpoolctl import threadpool_limits
    from oracle import wise_oracle as O
    R = w.rows
    sample_rows = list(range(min(R, max_rows)))
    inputs = [synth.layer_inputs(w, depth, 0, rows=sample_rows) for depth in range(len(w.schedule))]
    rows_done, t_total, tokens = 0, 0.0, 0
    with threadpool_limits(1):
        while t_total < min_s:
            sup = np.zeros((R, 1, w.heads, (w.max_ctx + 1023) // 1024), np.uint32)
            tags = np.zeros((R, 1), O.TAG_DTYPE)
            req = np.arange(R) + 1000
            pos = np.zeros(R, np.int64)
            for depth, mode in enumerate(w.schedule):
                li = inputs[depth]
                t0 = time.perf_counter()
                res = O.run_call(q=li.q, k_cache=li.k, v_cache=li.v, block_table=li.block_table,
                                 ctx_len=li.ctx_len, page_size=w.page_size, num_pages=li.num_pages,
                                 max_ctx=w.max_ctx, modes=[mode] * R, support=sup, tags=tags,
                                 row_request=req, row_position=pos, required=w.discoveries,
                                 eta=w.eta, rows=sample_rows)
                t_total += time.perf_counter() - t0
                sup, tags = res.support, res.tags
                rows_done += len(sample_rows)
            tokens += 1
    return {"value": round(rows_done / t_total, 2), "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(sample_rows)} of {R} rows x {len(w.schedule)} depths x {tokens} "
                      f"repeats = {rows_done} row-calls in {t_total:.1f} s (fp64 numpy, 1 BLAS thread)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ctx1k", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--replicas", type=int, default=2,
                    help="distinct KV sets per depth, rotated so the 256 MB MALL cannot serve repeats")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    W.lib()  # fails loudly if the HIP library is missing
    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- inputs: every (replica, depth) KV set resident in HBM ----
    t0 = time.time()
    layers = {}
    for rep in range(args.replicas):
        for depth in range(len(w.schedule)):
            li = synth.layer_inputs(dataclasses.replace(w, seed=w.seed + 1000 * rep), depth)
            layers[(rep, depth)] = harness.upload(li, device=dev)
            log(f"inputs: replica {rep} depth {depth} uploaded ({time.time() - t0:.1f} s)")
    ctx = synth.context_lengths(w)
    bt_width = layers[(0, 0)].block_table.shape[1]
    state = harness.SupportState(w.rows, w.heads, w.max_ctx, device=dev)
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx, device=dev)
    calls = len(w.schedule) * w.layers
    prepared = {(rep, depth): harness.PreparedCall(layers[(rep, depth)], ws, mode, state,
                                                   required=w.discoveries, eta=w.eta)
                for rep in range(args.replicas) for depth, mode in enumerate(w.schedule)}
    ev = harness.HipEvents(2 * calls * args.steps)

    def step(i, stream, timed=False):
        rep = i % args.replicas
        for depth in range(len(w.schedule)):
            pc = prepared[(rep, depth)]
            for layer in range(w.layers):
                c = 2 * (i * calls + depth * w.layers + layer)
                pc.set_events(ev.handle(c), ev.handle(c + 1)) if timed else pc.set_events(None, None)
                pc.run(stream)

    main_stream = torch.cuda.current_stream()
    sh = int(main_stream.cuda_stream)
    for i in range(args.warmup):
        step(i, sh)
    torch.cuda.synchronize()

    # ---- timed region 1 (eager): every split-KV launch bracketed by HIP events ----
    state.counters.zero_()
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record()
    for i in range(args.steps):
        step(i, sh, timed=True)
    t_end.record()
    torch.cuda.synchronize()
    eager_ms_per_step = t_start.elapsed_time(t_end) / args.steps
    ctr = state.counters.cpu().numpy().copy()

    # ---- timed region 2: the same steps replayed from HIP graphs ----
    graphs = []
    for rep in range(args.replicas):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(rep, int(torch.cuda.current_stream().cuda_stream))
        graphs.append(g)
    for i in range(args.warmup):
        graphs[i % args.replicas].replay()
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        graphs[i % args.replicas].replay()
    t_end.record()
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps

    # ---- per-mode split-kernel times and algorithmic bytes ----
    # the support a sparse depth reads is the one its replica's discovery
    # depths wrote in the same step: rebuild it per replica (untimed)
    sup_of = {}
    for rep in range(args.replicas):
        step(rep, sh)
        torch.cuda.synchronize()
        sup_of[rep] = state.support_numpy()[:, 0].copy()
    per_mode = {}
    for depth, mode in enumerate(w.schedule):
        key = {W.WISE_DENSE: "dense", W.WISE_DISCOVER: "discover",
               W.WISE_DISCOVER_UNION: "discover_union", W.WISE_SPARSE: "sparse"}[mode]
        m = per_mode.setdefault(key, {"ms": [], "bytes": []})
        nb_of = {rep: split_bytes(w, ctx, mode, sup_of[rep], bt_width) for rep in range(args.replicas)}
        for i in range(args.steps):
            for layer in range(w.layers):
                c = 2 * (i * calls + depth * w.layers + layer)
                m["ms"].append(ev.elapsed_ms(c, c + 1))
                m["bytes"].append(nb_of[i % args.replicas])
    modes_out = {}
    tot_bytes = tot_ms = 0.0
    for key, m in per_mode.items():
        ms = np.asarray(m["ms"])
        by = np.asarray(m["bytes"], dtype=np.float64)
        avg = float(ms.mean())
        modes_out[key] = {"split_us": round(avg * 1e3, 2),
                          "split_us_p10": round(float(np.percentile(ms, 10)) * 1e3, 2),
                          "split_us_p90": round(float(np.percentile(ms, 90)) * 1e3, 2),
                          "algorithmic_MB": round(float(by.mean()) / 1e6, 3),
                          "GBps": round(float(by.sum()) / (float(ms.sum()) * 1e-3) / 1e9, 1)}
        tot_bytes += float(by.sum())
        tot_ms += float(ms.sum())
    achieved = tot_bytes / (tot_ms * 1e-3) / 1e9
    rows_per_step = w.rows * calls
    out = {
        "metric": "decode-attn rows/s + achieved HBM GB/s (sparse vs dense), ctx 1K/4K/8K",
        "value": round(rows_per_step / (ms_per_step * 1e-3), 1),
        "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "eager_ms_per_step": round(eager_ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "rows": w.rows, "heads": w.heads, "head_dim": w.head_dim,
                   "ctx": w.ctx if w.ctx else "ragged", "page_size": w.page_size,
                   "layers": w.layers, "schedule": list(w.schedule), "eta": w.eta,
                   "row_calls_per_step": rows_per_step, "kv_replicas": args.replicas,
                   "timing": "HIP graph replay of whole steps",
                   "union_density": round(float(ctr[W.CTR_SELECTED] / max(1, ctr[W.CTR_CAUSAL])), 4),
                   "fallbacks": int(ctr[W.CTR_FALLBACKS]), "errors": int(ctr[W.CTR_ERRORS])},
        "modes": modes_out,
        "roofline": {"bound": "hbm", "kernel": "split_kernel", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
