"""Decode-attention throughput of the WISE path on one MI355X.

A step is one token of every row through the workload's whole hot path:
for the depth-schedule workloads, every depth (discover, discover-union,
sparse, sparse) of every layer; for the mixed workload, the one launch that
mixes dense, discover and sparse rows (after untimed setup depths).  Each
(depth, layer) call is the split-KV decode kernel (plus the plan kernel
for calls with sparse rows whose units span several split workgroups) and
the finish kernel.  Every input is resident in HBM before timing starts.

Prints ONE JSON line.  ``value`` = decode-attention rows per second, where a
row is one query row attended at one (depth, layer).
"""

from __future__ import annotations

import argparse
import ctypes
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
MODE_NAME = {W.WISE_DENSE: "dense", W.WISE_DISCOVER: "discover",
             W.WISE_DISCOVER_UNION: "discover_union", W.WISE_SPARSE: "sparse"}
LSE_ROUTE = -1  # split_bytes key of discovery by the LSE route


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def split_bytes(w, ctx, eff_modes, support_words):
    """Algorithmic bytes one split-KV launch moves.

    Per (row, head): K and V of every attended token (2 * d * e each) and q
    (d * e); per row the block-table entries of the pages it reads.
    Discovery rows also write 8 bytes of tile stats per block; sparse rows
    read their support words.  eff_modes[r] is the row's effective mode;
    support_words [rows, heads, words] is the support a sparse row reads.
    """
    e = 2 if w.dtype == "bf16" else 4
    d, H, P = w.head_dim, w.heads, w.page_size
    total = 0
    for r in range(w.rows):
        n = int(ctx[r])
        nb = (n + 31) // 32
        mode = int(eff_modes[r])
        if mode == W.WISE_SPARSE:
            b = np.arange(nb)
            bits = ((support_words[r][:, b >> 5] >> (b & 31).astype(np.uint32)) & 1).astype(bool)
            tok_per_block = np.minimum(32, n - 32 * b)
            toks = (bits * tok_per_block[None, :]).sum(axis=1)          # [H]
            pages = set()
            for blk in np.nonzero(bits.any(axis=0))[0]:
                pages.update(range((32 * blk) // P, (min(n, 32 * blk + 32) - 1) // P + 1))
            total += int(2 * toks.sum() * d * e) + H * d * e + H * 4 * ((nb + 31) // 32) + 4 * len(pages)
        elif mode == LSE_ROUTE:
            # discovery by the LSE route: K only, q, the tile stats written
            total += H * (n * d * e + d * e + 8 * nb) + 4 * ((n + P - 1) // P)
        else:
            total += H * (2 * n * d * e + d * e) + 4 * ((n + P - 1) // P)
            if mode != W.WISE_DENSE:
                total += H * 8 * nb
    return total


def external_lse(layer_dev, ctx, page_size, scale=None):
    """[R, H] fp32 log-sum-exp of every (row, head)'s scaled scores, computed
    with plain torch ops from the paged cache: the stand-in for the external
    dense kernel whose LSE the LSE route consumes (untimed setup)."""
    import torch
    q, k, bt = layer_dev.q, layer_dev.k, layer_dev.block_table
    R, H, d = q.shape
    scale = (1.0 / d ** 0.5) if scale is None else scale
    out = torch.empty((R, H), dtype=torch.float32, device=q.device)
    for r in range(R):
        n = int(ctx[r])
        t = torch.arange(n, device=q.device)
        pages = bt[r, t // page_size].long()
        K = k[pages, :, t % page_size, :].float()                  # [n, H, d]
        s = (K * q[r].float()[None]).sum(dim=-1).t() * scale        # [H, n]
        out[r] = torch.logsumexp(s, dim=1)
    return out


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
                                 row_request=req, row_position=pos, required=max(1, w.discoveries),
                                 eta=w.eta, rows=sample_rows)
                t_total += time.perf_counter() - t0
                sup, tags = res.support, res.tags
                rows_done += len(sample_rows)
            tokens += 1
    return {"value": round(rows_done / t_total, 2), "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(sample_rows)} of {R} rows x {len(w.schedule)} depths x {tokens} "
                      f"repeats = {rows_done} row-calls in {t_total:.1f} s (fp64 numpy, 1 BLAS thread)"}


def split_source_digest() -> str:
    from block_sparse_paged_split_amd.profile_summary import split_source_digest as digest
    return digest()


def measured_traffic(workload):
    """HBM bytes per split launch from the committed counter summary of this
    workload, or None when there is none or the split kernel's source has
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"split_kernel_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    try:
        block = text.split("```json", 1)[1].split("```", 1)[0]
        rec = json.loads(block)
    except (IndexError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != split_source_digest():
        return None
    return rec.get("traffic_bytes_per_launch")


class Plan:
    """The calls of one step, per replica, and how to account for them."""

    def __init__(self, w, args, dev):
        import torch
        self.w = w
        self.ctx = synth.context_lengths(w)
        self.mixed = w.mix is not None
        # distinct KV sets: replicas x depths x (layer groups)
        self.kv_layers = min(w.layers, args.kv_layers)
        self.replicas = args.replicas
        self.state = harness.SupportState(w.rows, w.heads, w.max_ctx, layers=w.layers, device=dev)
        self.ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx, device=dev)
        self.kv = {}
        t0 = time.time()
        depths = 3 if self.mixed else len(w.schedule)
        for rep in range(self.replicas):
            for depth in range(depths):
                for lg in range(self.kv_layers):
                    wl = dataclasses.replace(w, seed=w.seed + 1000 * rep)
                    self.kv[(rep, depth, lg)] = harness.upload(synth.layer_inputs(wl, depth, lg), device=dev)
                    log(f"inputs: replica {rep} depth {depth} layer-set {lg} ({time.time() - t0:.1f} s)")
        if self.mixed:
            modes, flagged = synth.mixed_row_modes(w)
            self.row_modes = modes
            self.flagged = flagged
            d0 = np.where(modes == W.WISE_DENSE, W.WISE_DENSE, W.WISE_DISCOVER).astype(np.uint8)
            d1 = np.where((modes == W.WISE_SPARSE) & ~flagged, W.WISE_DISCOVER_UNION,
                          W.WISE_DENSE).astype(np.uint8)
            self.setup_modes = [torch.from_numpy(d0).to(dev), torch.from_numpy(d1).to(dev)]
            self.mixed_modes = torch.from_numpy(modes.astype(np.uint8)).to(dev)
        # calls[rep] = list of (PreparedCall, key) for one step
        self.calls = {}
        for rep in range(self.replicas):
            lst = []
            if self.mixed:
                pc = harness.PreparedCall(self.kv[(rep, 2, 0)], self.ws, W.WISE_SPARSE, self.state,
                                          required=max(1, w.discoveries), eta=w.eta, row_mode=self.mixed_modes)
                lst.append((pc, ("mixed", 2, 0)))
            else:
                for depth, mode in enumerate(w.schedule):
                    for layer in range(w.layers):
                        pc = harness.PreparedCall(self.kv[(rep, depth, layer % self.kv_layers)], self.ws, mode,
                                                  self.state, layer_idx=layer, required=max(1, w.discoveries), eta=w.eta)
                        lst.append((pc, (MODE_NAME[mode], depth, layer)))
            self.calls[rep] = lst
        self.calls_per_step = len(self.calls[0])

    def setup(self, rep, stream):
        """Untimed work that precedes a step: the discovery depths of the
        mixed launch's rows, or the fixed random support of a kernel-bench
        workload (with tags that admit reuse)."""
        if self.w.fixed_density is not None:
            import torch
            w, st = self.w, self.state
            for layer in range(w.layers):
                bits = synth.random_support(w, w.fixed_density, self.ctx, st.words, layer=layer)
                st.support[:, layer] = torch.from_numpy(bits.view(np.int32)).to(st.support.device)
            st.tags[:, :, 0] = st.row_request[:, None]
            st.tags[:, :, 1] = st.row_position[:, None]
            st.tags[:, :, 2] = max(1, w.discoveries)
            return
        if not self.mixed:
            return
        for depth in (0, 1):
            harness.PreparedCall(self.kv[(rep, depth, 0)], self.ws, W.WISE_SPARSE, self.state,
                                 required=max(1, self.w.discoveries), eta=self.w.eta,
                                 row_mode=self.setup_modes[depth]).run(stream)

    def eff_modes(self, key):
        w = self.w
        if key[0] == "mixed":
            eff = self.row_modes.copy()
            eff[self.flagged] = W.WISE_DENSE
            return eff
        mode = {v: k for k, v in MODE_NAME.items()}[key[0]]
        return np.full(w.rows, mode)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ctx1k", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--replicas", type=int, default=None,
                    help="distinct KV sets per depth, rotated across steps so the 256 MB MALL cannot "
                         "serve repeats (default: 2 when one set is under 1 GB, else 1)")
    ap.add_argument("--kv-layers", type=int, default=3,
                    help="distinct KV sets per depth for multi-layer workloads, rotated over the layers")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense-reference", action="store_true")
    ap.add_argument("--no-lse-route", action="store_true",
                    help="skip the timing of discovery by the LSE route")
    ap.add_argument("--no-page-route", action="store_true",
                    help="skip the timing of the head-union page route")
    ap.add_argument("--no-state-copy", action="store_true",
                    help="skip the timing of the support/tag snapshot and restore")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (for counter-collection runs)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run one plain device-to-device copy of this many MiB (a known-size "
                         "reference for hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    W.lib()  # fails loudly if the HIP library is missing
    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.replicas is None:
        one_set = int(synth.context_lengths(w).sum()) * w.heads * w.head_dim * 2 * (2 if w.dtype == "bf16" else 4)
        args.replicas = 2 if one_set < (1 << 30) else 1
    if args.calibrate_copy:
        # a plain streaming kernel of known size (reads and writes MIB MiB)
        src = torch.zeros(args.calibrate_copy << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"calibration kernel (neg): {args.calibrate_copy} MiB read + {args.calibrate_copy} MiB written")
        del src, dst
    plan = Plan(w, args, dev)
    calls = plan.calls_per_step
    ev = harness.HipEvents(2 * calls * args.steps)
    main_stream = torch.cuda.current_stream()
    sh = int(main_stream.cuda_stream)

    def step(i, stream, timed=False):
        rep = i % plan.replicas
        for c, (pc, _) in enumerate(plan.calls[rep]):
            k = 2 * (i * calls + c)
            pc.set_events(ev.handle(k), ev.handle(k + 1)) if timed else pc.set_events(None, None)
            pc.run(stream)

    for rep in range(plan.replicas):
        plan.setup(rep, sh)
    for i in range(args.warmup):
        step(i, sh)
    torch.cuda.synchronize()

    # ---- timed region 1 (eager): every split-KV launch bracketed by HIP events ----
    plan.state.counters.zero_()
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record()
    for i in range(args.steps):
        step(i, sh, timed=True)
    t_end.record()
    torch.cuda.synchronize()
    eager_ms_per_step = t_start.elapsed_time(t_end) / args.steps
    ctr = plan.state.counters.cpu().numpy().copy()

    # ---- timed region 2: the same steps replayed from HIP graphs ----
    if args.no_graph:
        ms_per_step = eager_ms_per_step
    else:
        graphs = []
        for rep in range(plan.replicas):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(rep, int(torch.cuda.current_stream().cuda_stream))
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % plan.replicas].replay()
        torch.cuda.synchronize()
        t_start.record()
        for i in range(args.steps):
            graphs[i % plan.replicas].replay()
        t_end.record()
        torch.cuda.synchronize()
        ms_per_step = t_start.elapsed_time(t_end) / args.steps

    # ---- the same step with every call dense (no support state), replayed from
    # HIP graphs: the step-level comparison the page makes between WISE decode and
    # dense decode (its discovery depths cost a dense pass each; only the reuse
    # depths can save) ----
    dense_step_ms = None
    if not args.no_graph and not args.no_dense_reference and not plan.mixed:
        dgraphs = []
        for rep in range(plan.replicas):
            dcalls = [harness.PreparedCall(plan.kv[(rep, depth, layer % plan.kv_layers)], plan.ws, W.WISE_DENSE)
                      for _, (_, depth, layer) in plan.calls[rep]]
            for dc in dcalls:
                dc.run(sh)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                cs = int(torch.cuda.current_stream().cuda_stream)
                for dc in dcalls:
                    dc.run(cs)
            dgraphs.append(g)
        for i in range(args.warmup):
            dgraphs[i % plan.replicas].replay()
        torch.cuda.synchronize()
        t_start.record()
        for i in range(args.steps):
            dgraphs[i % plan.replicas].replay()
        t_end.record()
        torch.cuda.synchronize()
        dense_step_ms = t_start.elapsed_time(t_end) / args.steps

    # ---- per-mode split-kernel times and algorithmic bytes ----
    # the support a sparse call reads is the one its replica's discovery
    # depths wrote in the same step: rebuild it per replica (untimed)
    sup_of = {}
    for rep in range(plan.replicas):
        plan.setup(rep, sh)
        step(rep, sh)
        torch.cuda.synchronize()
        sup_of[rep] = plan.state.support_numpy().copy()
    per_mode = {}
    bytes_cache = {}
    for i in range(args.steps):
        rep = i % plan.replicas
        for c, (pc, key) in enumerate(plan.calls[rep]):
            name, depth, layer = key
            ck = (rep, name, layer)
            if ck not in bytes_cache:
                bytes_cache[ck] = split_bytes(w, plan.ctx, plan.eff_modes(key), sup_of[rep][:, layer])
            m = per_mode.setdefault(name, {"ms": [], "bytes": []})
            m["ms"].append(ev.elapsed_ms(2 * (i * calls + c), 2 * (i * calls + c) + 1))
            m["bytes"].append(bytes_cache[ck])
    modes_out = {}
    tot_bytes = tot_ms = 0.0
    for key, m in per_mode.items():
        ms = np.asarray(m["ms"])
        by = np.asarray(m["bytes"], dtype=np.float64)
        modes_out[key] = {"split_us": round(float(ms.mean()) * 1e3, 2),
                          "split_us_p10": round(float(np.percentile(ms, 10)) * 1e3, 2),
                          "split_us_p90": round(float(np.percentile(ms, 90)) * 1e3, 2),
                          "algorithmic_MB": round(float(by.mean()) / 1e6, 3),
                          "GBps": round(float(by.sum()) / (float(ms.sum()) * 1e-3) / 1e9, 1)}
        tot_bytes += float(by.sum())
        tot_ms += float(ms.sum())
    achieved = tot_bytes / (tot_ms * 1e-3) / 1e9

    # ---- dense reference: the dense decode of the same rows, back to back, rotating
    # over every KV set of the run (so that no call rereads what the last one left
    # in the 256 MB MALL; the sets hold the same shapes as the sparse calls' KV) ----
    if not args.no_dense_reference and any(key[0] in ("sparse", "mixed") for _, key in plan.calls[0]):
        dpcs = [harness.PreparedCall(plan.kv[k], plan.ws, W.WISE_DENSE) for k in sorted(plan.kv)]
        n_it = max(16, 2 * len(dpcs))
        ev2 = harness.HipEvents(2 * n_it)
        for dpc in dpcs[:2]:
            dpc.set_events(None, None)
            dpc.run(sh)
        for it in range(n_it):
            dpc = dpcs[it % len(dpcs)]
            dpc.set_events(ev2.handle(2 * it), ev2.handle(2 * it + 1))
            dpc.run(sh)
        torch.cuda.synchronize()
        dense_ms = [ev2.elapsed_ms(2 * it, 2 * it + 1) for it in range(n_it)]
        for dpc in dpcs:
            dpc.set_events(None, None)
        if dense_ms:
            dms = float(np.mean(dense_ms))
            dbytes = split_bytes(w, plan.ctx, np.full(w.rows, W.WISE_DENSE), None)
            key = "mixed" if plan.mixed else "sparse"
            modes_out["dense_same_kv"] = {"split_us": round(dms * 1e3, 2), "algorithmic_MB": round(dbytes / 1e6, 3),
                                          "GBps": round(dbytes / (dms * 1e-3) / 1e9, 1)}
            modes_out[key]["speedup_vs_dense"] = round(dms * 1e3 / modes_out[key]["split_us"], 3)

    # ---- discovery by the LSE route (K reread, no output), rotating over every KV set ----
    if not args.no_lse_route and not plan.mixed:
        sets = []
        for key, layer_dev in plan.kv.items():
            a = layer_dev.attn()
            lse = external_lse(layer_dev, plan.ctx, w.page_size)
            sets.append((a, lse))
        s = plan.state.view(0, 1, w.eta)
        n_it = 4 * len(sets)
        ev3 = harness.HipEvents(2 * n_it + 2)
        for a, lse in sets[:2]:
            W.wise_discover_lse(a, s, False, int(lse.data_ptr()), plan.ws.ptr, plan.ws.nbytes, sh)
        ev3.record(2 * n_it, sh)
        for it in range(n_it):       # back to back, like the timed steps
            a, lse = sets[it % len(sets)]
            a.ev_split_begin, a.ev_split_end = ev3.handle(2 * it), ev3.handle(2 * it + 1)
            W.wise_discover_lse(a, s, False, int(lse.data_ptr()), plan.ws.ptr, plan.ws.nbytes, sh)
        ev3.record(2 * n_it + 1, sh)
        torch.cuda.synchronize()
        split_ms = [ev3.elapsed_ms(2 * it, 2 * it + 1) for it in range(n_it)]
        call_ms = [ev3.elapsed_ms(2 * n_it, 2 * n_it + 1) / n_it]
        for a, _ in sets:
            a.ev_split_begin = a.ev_split_end = None
        lbytes = split_bytes(w, plan.ctx, np.full(w.rows, LSE_ROUTE), None)
        sms = float(np.mean(split_ms))
        modes_out["lse_discover"] = {"split_us": round(sms * 1e3, 2),
                                     "call_us": round(float(np.mean(call_ms)) * 1e3, 2),
                                     "algorithmic_MB": round(lbytes / 1e6, 3),
                                     "GBps": round(lbytes / (sms * 1e-3) / 1e9, 1),
                                     "note": "K-only split + LSE selection, eager back-to-back calls; "
                                             "not part of a step"}

    # ---- reuse depths by the head-union page route: compaction + dense decode over it ----
    if not args.no_page_route and not plan.mixed:
        sparse_keys = [key for _, key in plan.calls[0] if key[0] == "sparse"]
        if sparse_keys:
            plan.setup(0, sh)
            step(0, sh)                      # replica 0's discovery supports, untimed
            torch.cuda.synchronize()
            pus = [(harness.PageUnion(plan.kv[(0, depth, layer % plan.kv_layers)]), layer)
                   for _, depth, layer in sparse_keys]
            for pu, layer in pus:
                pu.compact(plan.state, layer, max(1, w.discoveries), stream=sh)
                pu.attend(plan.ws, stream=sh)
            n_it = max(20, 2 * len(pus))
            ev4 = harness.HipEvents(4 * n_it + 2)
            L = W.lib()
            prepared = []                    # ctypes arguments built once: issuing stays ahead of the GPU
            for pu, layer in pus:
                a_c, s_c, a_d = pu.layer.attn(), plan.state.view(layer, max(1, w.discoveries), w.eta), pu.attend_attn()
                prepared.append((a_c, s_c, a_d, int(pu.bt.data_ptr()), pu.bt.stride(0), int(pu.ctx.data_ptr())))
            ev4.record(4 * n_it, sh)
            for it in range(n_it):           # back to back
                a_c, s_c, a_d, bt_p, bt_s, ctx_p = prepared[it % len(prepared)]
                ev4.record(4 * it, sh)
                st = L.wise_compact_pages(ctypes.byref(a_c), ctypes.byref(s_c), None, bt_p, bt_s, ctx_p, sh)
                ev4.record(4 * it + 1, sh)
                a_d.ev_split_begin, a_d.ev_split_end = ev4.handle(4 * it + 2), ev4.handle(4 * it + 3)
                st |= L.wise_decode_dense(ctypes.byref(a_d), plan.ws.ptr, plan.ws.nbytes, sh)
                st |= L.wise_finish_select(ctypes.byref(a_d), None, plan.ws.ptr, plan.ws.nbytes, sh)
                if st != W.WISE_OK:
                    raise W.WiseError(st, "page route")
            ev4.record(4 * n_it + 1, sh)
            torch.cuda.synchronize()
            comp_ms = np.array([ev4.elapsed_ms(4 * it, 4 * it + 1) for it in range(n_it)])
            split_ms = np.array([ev4.elapsed_ms(4 * it + 2, 4 * it + 3) for it in range(n_it)])
            e = 2 if w.dtype == "bf16" else 4
            P, H, d = w.page_size, w.heads, w.head_dim
            by, kept_pages, all_pages = [], 0, 0
            for pu, _ in pus:
                c = pu.ctx.cpu().numpy().astype(np.int64)
                by.append(int((H * (2 * c * d * e + d * e) + 4 * ((c + P - 1) // P)).sum()))
                kept_pages += int(((c + P - 1) // P).sum())
                all_pages += int(((plan.ctx.astype(np.int64) + P - 1) // P).sum())
            sbytes = float(np.mean([by[it % len(pus)] for it in range(n_it)]))
            total_us = float(comp_ms.mean() + split_ms.mean()) * 1e3
            entry = {"compact_us": round(float(comp_ms.mean()) * 1e3, 2),
                     "split_us": round(float(split_ms.mean()) * 1e3, 2),
                     "call_us": round(ev4.elapsed_ms(4 * n_it, 4 * n_it + 1) / n_it * 1e3, 2),
                     "page_density": round(kept_pages / max(1, all_pages), 4),
                     "algorithmic_MB": round(sbytes / 1e6, 3),
                     "GBps": round(sbytes / (float(split_ms.mean()) * 1e-3) / 1e9, 1),
                     "note": "head-union pages of the reuse depths; compaction + dense decode over "
                             "the compacted table, eager back-to-back"}
            if "dense_same_kv" in modes_out:
                entry["speedup_vs_dense"] = round(modes_out["dense_same_kv"]["split_us"] / total_us, 3)
            modes_out["page_union"] = entry

    if dense_step_ms is not None:
        modes_out["dense_step"] = {"ms_per_step": round(dense_step_ms, 4),
                                   "wise_step_speedup": round(dense_step_ms / ms_per_step, 3),
                                   "note": "every call of the step dense, HIP graph replay; "
                                           "wise_step_speedup = dense step time / WISE step time"}

    # ---- support/tag snapshot and restore of every row's slot (KV offload and resume) ----
    if not args.no_state_copy:
        st_ = plan.state
        slots = torch.arange(w.rows, dtype=torch.int32, device=dev)
        rec = st_.record_bytes()
        records = torch.empty(w.rows * rec, dtype=torch.uint8, device=dev)
        n_it = 20
        ev5 = harness.HipEvents(4 * n_it)
        st_.snapshot(slots, records, sh)
        st_.restore(slots, records, sh)
        for it in range(n_it):
            ev5.record(4 * it, sh)
            st_.snapshot(slots, records, sh)
            ev5.record(4 * it + 1, sh)
            ev5.record(4 * it + 2, sh)
            st_.restore(slots, records, sh)
            ev5.record(4 * it + 3, sh)
        torch.cuda.synchronize()
        snap_ms = np.mean([ev5.elapsed_ms(4 * it, 4 * it + 1) for it in range(n_it)])
        rest_ms = np.mean([ev5.elapsed_ms(4 * it + 2, 4 * it + 3) for it in range(n_it)])
        modes_out["offload_state"] = {"snapshot_us": round(float(snap_ms) * 1e3, 2),
                                      "restore_us": round(float(rest_ms) * 1e3, 2),
                                      "bytes_per_slot": rec, "slots": w.rows,
                                      "note": "support words of every layer and head + tags, all rows' "
                                              "slots; each copy reads and writes slots x bytes_per_slot"}

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
                   "ctx": w.ctx if w.ctx else f"{int(plan.ctx.min())}..{int(plan.ctx.max())}",
                   "page_size": w.page_size, "layers": w.layers,
                   "schedule": "mixed launch" if plan.mixed else list(w.schedule), "eta": w.eta,
                   "row_calls_per_step": rows_per_step, "kv_replicas": plan.replicas,
                   "kv_sets_per_depth": plan.kv_layers,
                   "timing": "eager launches" if args.no_graph else "HIP graph replay of whole steps",
                   "union_density": round(float(ctr[W.CTR_SELECTED] / max(1, ctr[W.CTR_CAUSAL])), 4),
                   "fallbacks_per_step": round(float(ctr[W.CTR_FALLBACKS]) / args.steps, 2),
                   "errors": int(ctr[W.CTR_ERRORS])},
        "modes": modes_out,
        "roofline": {"bound": "hbm", "kernel": "split_kernel", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(w.name)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
