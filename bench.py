"""Decode-attention throughput of the WISE path on one MI355X.

A step is one token of every row through the workload's whole hot path:
for the depth-schedule workloads, every depth (discover, discover-union,
sparse, sparse) of every layer; for the mixed workloads, the one launch that
mixes dense, discover and sparse rows (after untimed setup depths).  Each
(depth, layer) call is the library's decode call plus its finish call.
Every input is resident in HBM before timing starts.

Prints ONE JSON line.  ``value`` = decode-attention rows per second of the
headline workload (ctx1k: 32 rows x 16 heads x 1K tokens), where a row is one
query row attended at one (depth, layer), timed over whole steps replayed
from HIP graphs.  ``contexts`` holds, for the 1K / 4K / 8K workloads and the
ragged batch, every call kind's time -- the split kernel alone (stamped with
its own start and stop) and the whole call (every kernel it launches, timed
by HIP-graph replay of back-to-back calls) -- its algorithmic bytes, GB/s,
fraction of the 8 TB/s HBM peak, sparse vs dense on the same KV, the time a
pure gather of the same K/V pages in items of the same length takes, the
all-dense step beside the WISE step, and the fp64 oracle's rows/s per mode
on a bounded sample of the same rows (``cpu_oracle``).

``roofline``: the split kernel of the headline's calls -- algorithmic bytes
over kernel-stamped durations against the 8 TB/s peak, the HBM bytes the
committed counter summary recorded for it (while its sources are unchanged),
the box's device-to-device copy rate and the read ceiling of the same
launches.  ``cpu_baseline``: the oracle on the headline rows in worker
processes (the host share of one GPU).  ``selection_parity``: the headline
step's selection beside the oracle's (ambiguity classes, union supports that
differ).
"""

from __future__ import annotations

import argparse
import ctypes
import dataclasses
import json
import math
import os
import subprocess
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
CALL_GRAPH_CALLS = 16   # back-to-back calls per captured graph (per-call time)
CONTEXT_WORKLOADS = ("ctx1k", "match1k", "kbench1k", "ctx4k_24l", "match4k", "mix4k", "ctx8k_mixed",
                     "match8k", "ragged")
CONTEXT_OF = {"ctx1k": "1K", "match1k": "1K", "kbench1k": "1K", "ctx4k_24l": "4K", "match4k": "4K",
              "mix4k": "4K", "ctx8k_mixed": "8K", "match8k": "8K", "ragged": "512-32K"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- bytes

def dtype_code(w):
    return W.WISE_BF16 if w.dtype == "bf16" else W.WISE_F32


def attended_blocks(n, mode, support_words_rh):
    """Blocks one (row, head) attends in a call of effective mode ``mode``."""
    nb = (n + 31) // 32
    if mode != W.WISE_SPARSE:
        return np.arange(nb)
    b = np.arange(nb)
    return b[((support_words_rh[b >> 5] >> (b & 31).astype(np.uint32)) & 1).astype(bool)]


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


# ----------------------------------------------------------------------------- CPU baseline

def _oracle_worker(w, rows, min_s):
    """One worker's share of the CPU baseline: the fp64 oracle on ``rows``
    through the whole depth schedule, repeated until at least ``min_s``
    seconds of oracle time; one BLAS thread.  Inputs are generated first and
    not timed."""
    from threadpoolctl import threadpool_limits
    from oracle import wise_oracle as O
    R = w.rows
    inputs = [synth.layer_inputs(w, depth, 0, rows=rows, workers=1) for depth in range(len(w.schedule))]
    done, t_total, passes = 0, 0.0, 0
    classes = {"discovery_units": 0, "class_a": 0, "class_b": 0}
    union = None
    discover_modes = (O.DISCOVER, O.DISCOVER_UNION)
    with threadpool_limits(1):
        while passes < 1 or t_total < min_s:   # pass 0 (first touch of the inputs) is not timed
            passes += 1
            sup = np.zeros((R, 1, w.heads, (w.max_ctx + 1023) // 1024), np.uint32)
            tags = np.zeros((R, 1), O.TAG_DTYPE)
            req, pos = np.arange(R) + 1000, np.zeros(R, np.int64)
            for depth, mode in enumerate(w.schedule):
                li = inputs[depth]
                t0 = time.perf_counter()
                res = O.run_call(q=li.q, k_cache=li.k, v_cache=li.v, block_table=li.block_table,
                                 ctx_len=li.ctx_len, page_size=w.page_size, num_pages=li.num_pages,
                                 max_ctx=w.max_ctx, modes=[mode] * R, support=sup, tags=tags,
                                 row_request=req, row_position=pos, required=max(1, w.discoveries),
                                 eta=w.eta, rows=rows)
                if passes > 1:
                    t_total += time.perf_counter() - t0
                    done += len(rows)
                elif mode in discover_modes:
                    # the selection's ambiguity classes, from the untimed pass
                    for u in res.units.values():
                        if u.selection is None:
                            continue
                        a = u.selection.near_eta(w.eta)
                        classes["discovery_units"] += 1
                        classes["class_a"] += int(a)
                        classes["class_b"] += int(not a and u.selection.near_tie())
                    union = res.support[rows].copy()
                sup, tags = res.support, res.tags
    return done, t_total, classes, union


def device_copy_gbs(dev, mib=1024, reps=10):
    """Bytes read + written per second by a plain device-to-device copy of
    ``mib`` MiB (torch's copy_), the mean over ``reps`` copies."""
    import torch
    src = torch.ones(mib << 18, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * (mib << 20) / (ms * 1e-3) / 1e9


def _oracle_modes_worker(w, rows):
    """The fp64 oracle on ``rows`` of workload ``w`` (its first KV set, layer
    0), one call per mode: dense and discover on depth 0, union on depth 1
    (after that discovery), sparse on depth 2 (over the union, or over the
    support set directly for a fixed-density workload).  Returns {mode:
    (row-calls, seconds)}; inputs are generated first and not timed."""
    from threadpoolctl import threadpool_limits
    from oracle import wise_oracle as O
    R = w.rows
    ctx = synth.context_lengths(w)
    words = (w.max_ctx + 1023) // 1024
    depths = [synth.layer_inputs(w, d, 0, rows=rows, workers=1) for d in range(3)]
    req, pos = np.arange(R) + 1000, np.zeros(R, np.int64)
    out = {}

    def call(li, mode, sup, tags, reps=3):
        ts = []
        for _ in range(reps):   # the median of a few calls from the same state
            t0 = time.perf_counter()
            res = O.run_call(q=li.q, k_cache=li.k, v_cache=li.v, block_table=li.block_table,
                             ctx_len=li.ctx_len, page_size=w.page_size, num_pages=li.num_pages,
                             max_ctx=w.max_ctx, modes=[mode] * R, support=sup, tags=tags, row_request=req,
                             row_position=pos, required=1, eta=w.eta, rows=rows)
            ts.append(time.perf_counter() - t0)
        return res, float(np.median(ts))

    with threadpool_limits(1):
        empty = lambda: (np.zeros((R, 1, w.heads, words), np.uint32), np.zeros((R, 1), O.TAG_DTYPE))
        call(depths[0], O.DENSE, *empty(), reps=1)               # first touch, not timed
        _, t = call(depths[0], O.DENSE, *empty())
        out["dense"] = (len(rows), t)
        if w.fixed_density is not None:
            sup, tags = empty()
            sup[:, 0] = synth.random_support(w, w.fixed_density, ctx, words)
            tags["request"][:, 0], tags["position"][:, 0], tags["discoveries"][:, 0] = req, pos, 1
        else:
            res, t = call(depths[0], O.DISCOVER, *empty())
            out["discover"] = (len(rows), t)
            res, t = call(depths[1], O.DISCOVER_UNION, res.support, res.tags)
            out["discover_union"] = (len(rows), t)
            sup, tags = res.support, res.tags
        _, t = call(depths[2], O.SPARSE, sup, tags)
        out["sparse"] = (len(rows), t)
    return out


def cpu_oracle_by_mode(w, pool, workers, max_rows=16):
    """Oracle rows/s per mode on a bounded sample of a workload: up to
    ``max_rows`` rows (spread over its context lengths), one row per worker
    process; rate = row-calls / the slowest worker's seconds for that mode."""
    R = w.rows
    pick = np.unique(np.linspace(0, R - 1, min(max_rows, R)).round().astype(int))
    res = [f.result() for f in [pool.submit(_oracle_modes_worker, w, [int(r)]) for r in pick]]
    rates = {}
    for mode in res[0]:
        calls = sum(r[mode][0] for r in res)
        slowest = max(r[mode][1] for r in res)
        rates[mode] = round(calls / slowest, 1)
    return {"rows_per_s": rates, "cores": min(workers, len(pick)),
            "sample": f"{len(pick)} rows of {w.name} (one per process), the median of 3 oracle calls per mode"}


def host_facts():
    model = "unknown"
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
    except Exception:
        pass
    return os.cpu_count() or 1, model


def cpu_baseline(w, pool, workers, facts, min_s=1.5):
    """The fp64 oracle on the headline workload's rows, split over ``workers``
    processes (rows are independent through the whole schedule), each
    repeating its rows' schedule for at least ``min_s`` s.  Throughput =
    all row-calls / the slowest worker's oracle time."""
    chunks = [list(map(int, c)) for c in np.array_split(np.arange(w.rows), min(workers, w.rows)) if len(c)]
    res = [f.result() for f in [pool.submit(_oracle_worker, w, c, min_s) for c in chunks]]
    done = sum(r[0] for r in res)
    wall = max(r[1] for r in res)
    cpu = sum(r[1] for r in res)
    nproc, model = facts
    classes = {k: sum(r[2][k] for r in res) for k in res[0][2]}
    union = None
    if all(r[3] is not None for r in res):
        union = np.concatenate([r[3] for r in res])   # rows in order: the chunks are consecutive
    baseline = {"value": round(done / wall, 2), "unit": "rows/s", "cores": len(chunks), "kind": "oracle",
                "sample": f"all {w.rows} rows of {w.name} x {len(w.schedule)} depths, repeated; {done} row-calls "
                          f"in {len(chunks)} processes ({cpu:.1f} s of oracle CPU time, slowest {wall:.2f} s); "
                          f"fp64 numpy, 1 BLAS thread per process",
                "nproc": nproc, "cpu_model": model, "blas_threads_per_process": 1}
    return baseline, classes, union


def selection_parity(classes, union_oracle, support_gpu, w):
    """The headline step's selection beside the oracle's: ambiguity classes
    of every discovery unit (class A: the oracle's cut within 1e-6 of eta;
    class B: its K-th and (K+1)-th masses tied within 1e-6), and the (row,
    head) units whose union support after the step differs from the
    oracle's, counted before any exemption."""
    out = dict(classes)
    if union_oracle is not None:
        gpu = support_gpu[:w.rows, 0]                    # [rows, heads, words] of replica 0
        orc = union_oracle[:, 0]
        out["union_units"] = int(w.rows * w.heads)
        out["union_mismatches"] = int((gpu != orc).any(axis=-1).sum())
    out["what"] = (f"fp64 oracle on the {w.name} step's inputs (replica 0) beside the GPU's union support "
                   f"after the timed steps")
    return out


# ----------------------------------------------------------------------------- counters

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


# ----------------------------------------------------------------------------- read-ceiling probe

class ReadProbe:
    """The benchmark's pure gather of K/V pages (libwise_probe.so)."""

    def __init__(self):
        from block_sparse_paged_split_amd import build
        self.L = ctypes.CDLL(build.PROBE_LIB)
        V, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        self.L.wise_read_probe.argtypes = [V, V, I64, I64, I64, I32, V, I64, V, I32, V, V, I32, V, V, V, V]
        self.L.wise_read_probe.restype = ctypes.c_int

    @staticmethod
    def items_for(w, ctx, eff_modes, support_words, waves, k_only=False):
        """(items [n, 4] int32, tiles int32, K/V bytes) of one call: every
        (row, head)'s attended blocks cut into items as the library cuts
        them -- a unit's tiles spread evenly over `waves` waves when the call
        runs one workgroup per unit (wise_fused_waves() > 0), else the
        call-wide rule (32 tiles when the launch keeps >= 4096 such items,
        else 16 on that condition, else 8)."""
        e = 2 if w.dtype == "bf16" else 4
        lists = []
        for r in range(w.rows):
            for h in range(w.heads):
                lists.append((r, h, attended_blocks(int(ctx[r]), int(eff_modes[r]),
                                                    None if support_words is None else support_words[r, h])))
        counts = np.array([len(b) for _, _, b in lists])
        T = 8
        for t in (32, 16):
            if int(((counts + t - 1) // t).sum()) >= 4096:
                T = t
                break
        items, tiles, nbytes = [], [], 0
        for (r, h, blocks), c in zip(lists, counts):
            n = int(ctx[r])
            toks = np.minimum(32, n - 32 * blocks)
            nbytes += int((1 if k_only else 2) * toks.sum() * w.head_dim * e)
            t = max(1, -(-c // waves)) if waves > 0 else T
            assert t <= 64 and (len(blocks) == 0 or (blocks.min() >= 0 and 32 * blocks.max() < n))
            for i in range(0, c, t):
                items.append((r, h, len(tiles) + i, min(t, c - i)))
            tiles.extend(blocks.tolist())
        return np.asarray(items, np.int32).reshape(-1, 4), np.asarray(tiles, np.int32), nbytes

    def time(self, launches, stream, n_it, ev):
        """Mean duration (ms) over n_it launches rotating over ``launches``."""
        for it in range(n_it):
            args = launches[it % len(launches)]
            st = self.L.wise_read_probe(*args, ctypes.c_void_p(stream), ctypes.c_void_p(ev.handle(2 * it)),
                                        ctypes.c_void_p(ev.handle(2 * it + 1)))
            if st != 0:
                raise RuntimeError(f"read probe failed ({st})")
        import torch
        torch.cuda.synchronize()
        return float(np.mean([ev.elapsed_ms(2 * it, 2 * it + 1) for it in range(n_it)]))


# ----------------------------------------------------------------------------- the calls of a step

class Plan:
    """The calls of one step, per replica (each replica with its own KV and
    its own support state), and how to account for them."""

    def __init__(self, w, replicas, kv_layers, dev):
        import torch
        self.w = w
        self.ctx = synth.context_lengths(w)
        self.mixed = w.mix is not None
        self.kv_layers = min(w.layers, kv_layers)
        self.replicas = replicas
        self.states = [harness.SupportState(w.rows, w.heads, w.max_ctx, layers=w.layers, device=dev)
                       for _ in range(replicas)]
        self.ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx, device=dev)
        self.kv = {}
        t0 = time.time()
        depths = 3 if self.mixed else len(w.schedule)
        for rep in range(replicas):
            for depth in range(depths):
                for lg in range(self.kv_layers):
                    wl = dataclasses.replace(w, seed=w.seed + 1000 * rep)
                    self.kv[(rep, depth, lg)] = harness.upload(synth.layer_inputs(wl, depth, lg), device=dev)
            log(f"  [{w.name}] inputs of replica {rep} ({time.time() - t0:.1f} s)")
        if self.mixed:
            modes, flagged = synth.mixed_row_modes(w)
            self.row_modes, self.flagged = modes, flagged
            d0 = np.where(modes == W.WISE_DENSE, W.WISE_DENSE, W.WISE_DISCOVER).astype(np.uint8)
            d1 = np.where((modes == W.WISE_SPARSE) & ~flagged, W.WISE_DISCOVER_UNION,
                          W.WISE_DENSE).astype(np.uint8)
            self.setup_modes = [torch.from_numpy(d0).to(dev), torch.from_numpy(d1).to(dev)]
            self.mixed_modes = torch.from_numpy(modes.astype(np.uint8)).to(dev)
        self.calls = {}
        req = max(1, w.discoveries)
        for rep in range(replicas):
            lst, st = [], self.states[rep]
            if self.mixed:
                pc = harness.PreparedCall(self.kv[(rep, 2, 0)], self.ws, W.WISE_SPARSE, st, required=req,
                                          eta=w.eta, row_mode=self.mixed_modes)
                lst.append((pc, ("mixed", 2, 0)))
            else:
                for depth, mode in enumerate(w.schedule):
                    for layer in range(w.layers):
                        pc = harness.PreparedCall(self.kv[(rep, depth, layer % self.kv_layers)], self.ws, mode, st,
                                                  layer_idx=layer, required=req, eta=w.eta)
                        lst.append((pc, (MODE_NAME[mode], depth, layer)))
            self.calls[rep] = lst
        self.calls_per_step = len(self.calls[0])

    def setup(self, rep, stream):
        """Untimed work that precedes a step: the discovery depths of the
        mixed launch's rows, or the fixed random support of a kernel-bench
        workload (with tags that admit reuse)."""
        w, st = self.w, self.states[rep]
        if w.fixed_density is not None:
            import torch
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
            harness.PreparedCall(self.kv[(rep, depth, 0)], self.ws, W.WISE_SPARSE, st,
                                 required=max(1, w.discoveries), eta=w.eta,
                                 row_mode=self.setup_modes[depth]).run(stream)

    def eff_modes(self, key):
        if key[0] == "mixed":
            eff = self.row_modes.copy()
            eff[self.flagged] = W.WISE_DENSE
            return eff
        mode = {v: k for k, v in MODE_NAME.items()}[key[0]]
        return np.full(self.w.rows, mode)

    def counters(self):
        return sum(st.counters.cpu().numpy() for st in self.states)

    def free(self):
        self.kv.clear()
        self.calls.clear()
        self.states.clear()


def graph_of(fn, torch):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(int(torch.cuda.current_stream().cuda_stream))
    return g


def replay_ms(graphs, n, warmup, torch):
    """Mean ms per replay over n replays rotating over ``graphs``."""
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0.record()
    for i in range(n):
        graphs[i % len(graphs)].replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / n


def measure(w, dev, *, steps, warmup, replicas, kv_layers, graphs=True, probe=None, headline=False,
            args=None, dense_reference=True):
    """Everything measured on one workload; returns (entry, extras) where
    extras holds what only the headline line reports."""
    import torch
    plan = Plan(w, replicas, kv_layers, dev)
    calls = plan.calls_per_step
    ev = harness.HipEvents(2 * calls * steps)
    sh = int(torch.cuda.current_stream().cuda_stream)

    def step(i, stream, timed=False):
        rep = i % plan.replicas
        for c, (pc, _) in enumerate(plan.calls[rep]):
            k = 2 * (i * calls + c)
            pc.set_events(ev.handle(k), ev.handle(k + 1)) if timed else pc.set_events(None, None)
            pc.run(stream)

    for rep in range(plan.replicas):
        plan.setup(rep, sh)
    for i in range(max(warmup, plan.replicas)):
        step(i, sh)
    torch.cuda.synchronize()

    # ---- eager steps: every split-KV launch stamped with its own start and stop ----
    for st in plan.states:
        st.counters.zero_()
    torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record()
    for i in range(steps):
        step(i, sh, timed=True)
    t_end.record()
    torch.cuda.synchronize()
    eager_ms = t_start.elapsed_time(t_end) / steps
    ctr = plan.counters()
    for rep in range(plan.replicas):
        for pc, _ in plan.calls[rep]:
            pc.set_events(None, None)

    # ---- whole steps replayed from HIP graphs ----
    step_ms = eager_ms
    if graphs:
        gs = [graph_of(lambda s, rep=rep: step(rep, s), torch) for rep in range(plan.replicas)]
        step_ms = replay_ms(gs, steps, warmup, torch)
        del gs

    # ---- per-kind split times and algorithmic bytes (each replica's own support) ----
    sup_of = {rep: plan.states[rep].support_numpy().copy() for rep in range(plan.replicas)}
    kinds, bytes_cache = {}, {}
    for i in range(steps):
        rep = i % plan.replicas
        for c, (pc, key) in enumerate(plan.calls[rep]):
            name, _, layer = key
            ck = (rep, name, layer)
            if ck not in bytes_cache:
                bytes_cache[ck] = split_bytes(w, plan.ctx, plan.eff_modes(key), sup_of[rep][:, layer])
            m = kinds.setdefault(name, {"ms": [], "bytes": []})
            m["ms"].append(ev.elapsed_ms(2 * (i * calls + c), 2 * (i * calls + c) + 1))
            m["bytes"].append(bytes_cache[ck])
    out = {}
    tot_bytes = tot_ms = 0.0
    for name, m in kinds.items():
        ms, by = np.asarray(m["ms"]), np.asarray(m["bytes"], np.float64)
        out[name] = {"split_us": round(float(ms.mean()) * 1e3, 2),
                     "split_us_median": round(float(np.median(ms)) * 1e3, 2),
                     "split_us_p10": round(float(np.percentile(ms, 10)) * 1e3, 2),
                     "split_us_p90": round(float(np.percentile(ms, 90)) * 1e3, 2),
                     "algorithmic_MB": round(float(by.mean()) / 1e6, 3),
                     "split_GBps": round(float(by.sum()) / (float(ms.sum()) * 1e-3) / 1e9, 1)}
        tot_bytes += float(by.sum())
        tot_ms += float(ms.sum())
    achieved = tot_bytes / (tot_ms * 1e-3) / 1e9

    # ---- whole calls: every kernel a call launches, by graph replay of back-to-back
    # calls (replicas rotate, each with its own state, so a reuse call reads the
    # support its own discovery depths wrote); kinds in schedule order ----
    dense_pcs = [harness.PreparedCall(plan.kv[k], plan.ws, W.WISE_DENSE) for k in sorted(plan.kv)]
    groups = []
    for name in kinds:
        pcs = [pc for rep in range(plan.replicas) for pc, key in plan.calls[rep] if key[0] == name]
        groups.append((name, pcs))
    if dense_reference:
        groups.append(("dense_same_kv", dense_pcs))
    dense_bytes = split_bytes(w, plan.ctx, np.full(w.rows, W.WISE_DENSE), None)
    if graphs:
        for name, pcs in groups:
            k = max(CALL_GRAPH_CALLS, len(pcs))

            def run_k(s, pcs=pcs, k=k):
                for j in range(k):
                    pcs[j % len(pcs)].run(s)
            run_k(sh)
            torch.cuda.synchronize()
            g = graph_of(run_k, torch)
            call_us = replay_ms([g], 3, 1, torch) / k * 1e3
            del g
            if name == "dense_same_kv":
                out[name] = {"algorithmic_MB": round(dense_bytes / 1e6, 3)}
            mb = out[name]["algorithmic_MB"]
            out[name].update({"call_us": round(call_us, 2), "call_rows_per_s": round(w.rows / (call_us * 1e-6), 1),
                              "call_GBps": round(mb * 1e6 / (call_us * 1e-6) / 1e9, 1),
                              "call_frac": round(mb * 1e6 / (call_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
    # split-stamped dense reference, rotating over every KV set of the run
    n_it = max(16, 2 * len(dense_pcs)) if dense_reference else 0
    ev2 = harness.HipEvents(2 * n_it)
    for it in range(n_it):
        pc = dense_pcs[it % len(dense_pcs)]
        pc.set_events(ev2.handle(2 * it), ev2.handle(2 * it + 1))
        pc.run(sh)
    torch.cuda.synchronize()
    for pc in dense_pcs:
        pc.set_events(None, None)
    if dense_reference:
        dms = float(np.mean([ev2.elapsed_ms(2 * it, 2 * it + 1) for it in range(n_it)]))
        out.setdefault("dense_same_kv", {"algorithmic_MB": round(dense_bytes / 1e6, 3)})
        out["dense_same_kv"].update({"split_us": round(dms * 1e3, 2),
                                     "split_GBps": round(dense_bytes / (dms * 1e-3) / 1e9, 1)})
    reuse = "mixed" if plan.mixed else ("sparse" if "sparse" in out else None)
    if reuse and dense_reference:
        out[reuse]["speedup_vs_dense_split"] = round(out["dense_same_kv"]["split_us"] / out[reuse]["split_us"], 3)
        if "call_us" in out[reuse]:
            out[reuse]["speedup_vs_dense_call"] = round(out["dense_same_kv"]["call_us"] / out[reuse]["call_us"], 3)

    # ---- read ceiling: a pure gather of the same K/V pages in items of the same length ----
    if probe is not None and reuse and dense_reference:
        e = 2 if w.dtype == "bf16" else 4
        ceil = {}
        for name, key_kind in ((reuse, reuse), ("dense_same_kv", None)):
            waves = W.wise_fused_waves(w.rows, w.heads, w.head_dim, w.max_ctx, dtype_code(w), key_kind is not None)
            launches, nbytes, keep = [], [], []
            for rep in range(plan.replicas):
                if key_kind is None:
                    lays = [(plan.kv[(rep, d, 0)], np.full(w.rows, W.WISE_DENSE), None)
                            for d in range(3 if plan.mixed else len(w.schedule))]
                else:
                    lays = [(pc_key_kv, plan.eff_modes(key), sup_of[rep][:, key[2]])
                            for pc, key in plan.calls[rep] if key[0] == key_kind
                            for pc_key_kv in [plan.kv[(rep, key[1], key[2] % plan.kv_layers)]]]
                for kv, eff, sw in lays:
                    items, tiles, nb = ReadProbe.items_for(w, plan.ctx, eff, sw, waves)
                    it_d = torch.from_numpy(items).to(dev)
                    ti_d = torch.from_numpy(tiles).to(dev)
                    sink = torch.empty(len(items), dtype=torch.int32, device=dev)
                    keep += [it_d, ti_d, sink]
                    sp, sh_, st_, _ = kv.k.stride()
                    launches.append((kv.k.data_ptr(), kv.v.data_ptr(), sp * e, sh_ * e, st_ * e, w.head_dim * e,
                                     kv.block_table.data_ptr(), kv.block_table.stride(0), kv.ctx_len.data_ptr(),
                                     int(math.log2(w.page_size)), it_d.data_ptr(), ti_d.data_ptr(), len(items),
                                     sink.data_ptr()))
                    nbytes.append(nb)
            n_it = max(16, 2 * len(launches))
            ev3 = harness.HipEvents(2 * n_it)
            probe.time(launches, sh, min(4, len(launches)), ev3)     # warm-up
            ms = probe.time(launches, sh, n_it, ev3)
            mb = float(np.mean([nbytes[i % len(nbytes)] for i in range(n_it)]))
            ceil[name] = {"us": round(ms * 1e3, 2), "kv_MB": round(mb / 1e6, 3),
                          "GBps": round(mb / (ms * 1e-3) / 1e9, 1)}
        out["read_ceiling"] = ceil

    if w.fixed_density is not None:
        # no discovery depth: the density of the support set directly
        nb = (plan.ctx.astype(np.int64) + 31) // 32
        sup = sup_of[0][:, 0]
        set_bits = sum(len(attended_blocks(int(plan.ctx[r]), W.WISE_SPARSE, sup[r, h]))
                       for r in range(w.rows) for h in range(w.heads))
        density = set_bits / float(nb.sum() * w.heads)
    else:
        density = float(ctr[W.CTR_SELECTED] / max(1, ctr[W.CTR_CAUSAL]))
    # the same step with every call dense (no support state), replayed from HIP
    # graphs: the step-level comparison of WISE decode with dense decode
    dense_step_ms = None
    if graphs and not plan.mixed and dense_reference:
        dgraphs = []
        for rep in range(plan.replicas):
            dcalls = [harness.PreparedCall(plan.kv[(rep, depth, layer % plan.kv_layers)], plan.ws, W.WISE_DENSE)
                      for _, (_, depth, layer) in plan.calls[rep]]

            def run_dense(s, dcalls=dcalls):
                for dc in dcalls:
                    dc.run(s)
            run_dense(sh)
            dgraphs.append(graph_of(run_dense, torch))
        dense_step_ms = replay_ms(dgraphs, steps, warmup, torch)
        del dgraphs
    entry = {"context": CONTEXT_OF.get(w.name, ""), "rows": w.rows,
             "ctx": w.ctx if w.ctx else f"{int(plan.ctx.min())}..{int(plan.ctx.max())}",
             "layers": w.layers, "union_density": round(density, 4),
             "fallbacks_per_step": round(float(ctr[W.CTR_FALLBACKS]) / steps, 2),
             "errors": int(ctr[W.CTR_ERRORS]),
             "ms_per_step": round(step_ms, 4), "rows_per_s": round(w.rows * calls / (step_ms * 1e-3), 1),
             "dense_ms_per_step": None if dense_step_ms is None else round(dense_step_ms, 4),
             "wise_step_speedup": None if dense_step_ms is None else round(dense_step_ms / step_ms, 3),
             "calls": out}
    extras = {"plan": plan, "eager_ms": eager_ms, "step_ms": step_ms, "achieved": achieved, "ctr": ctr,
              "calls": calls, "sh": sh, "support_r0": sup_of[0]}
    if headline:
        extras.update(headline_legs(w, plan, dev, sh, steps, warmup, args, out, graphs))
    return entry, extras


def headline_legs(w, plan, dev, sh, steps, warmup, args, out, graphs):
    """The legs only the headline line reports: the LSE route, the
    head-union page route and the support snapshot/restore."""
    import torch
    res = {}
    st0 = plan.states[0]
    if not args.no_lse_route and not plan.mixed:
        sets = [(layer_dev.attn(), external_lse(layer_dev, plan.ctx, w.page_size)) for layer_dev in plan.kv.values()]
        s = st0.view(0, 1, w.eta)
        n_it = 4 * len(sets)
        ev3 = harness.HipEvents(2 * n_it + 2)
        for a, lse in sets[:2]:
            W.wise_discover_lse(a, s, False, int(lse.data_ptr()), plan.ws.ptr, plan.ws.nbytes, sh)
        ev3.record(2 * n_it, sh)
        for it in range(n_it):
            a, lse = sets[it % len(sets)]
            a.ev_split_begin, a.ev_split_end = ev3.handle(2 * it), ev3.handle(2 * it + 1)
            W.wise_discover_lse(a, s, False, int(lse.data_ptr()), plan.ws.ptr, plan.ws.nbytes, sh)
        ev3.record(2 * n_it + 1, sh)
        torch.cuda.synchronize()
        sms = float(np.mean([ev3.elapsed_ms(2 * it, 2 * it + 1) for it in range(n_it)]))
        lbytes = split_bytes(w, plan.ctx, np.full(w.rows, LSE_ROUTE), None)
        ceiling = None
        if not args.no_read_ceiling:
            # a pure gather of the same K pages in items of the same length (K only)
            probe = ReadProbe()
            e = 2 if w.dtype == "bf16" else 4
            waves = W.wise_fused_waves(w.rows, w.heads, w.head_dim, w.max_ctx, dtype_code(w), True)
            launches, keep, kb = [], [], 0
            for layer_dev in plan.kv.values():
                items, tiles, kb = ReadProbe.items_for(w, plan.ctx, np.full(w.rows, W.WISE_DENSE), None, waves,
                                                       k_only=True)
                it_d, ti_d = torch.from_numpy(items).to(dev), torch.from_numpy(tiles).to(dev)
                sink = torch.empty(len(items), dtype=torch.int32, device=dev)
                keep += [it_d, ti_d, sink]
                sp, sh_, st_, _ = layer_dev.k.stride()
                launches.append((layer_dev.k.data_ptr(), None, sp * e, sh_ * e, st_ * e, w.head_dim * e,
                                 layer_dev.block_table.data_ptr(), layer_dev.block_table.stride(0),
                                 layer_dev.ctx_len.data_ptr(), int(math.log2(w.page_size)), it_d.data_ptr(),
                                 ti_d.data_ptr(), len(items), sink.data_ptr()))
            n_p = max(16, 2 * len(launches))
            evp = harness.HipEvents(2 * n_p)
            probe.time(launches, sh, min(4, len(launches)), evp)
            pms = probe.time(launches, sh, n_p, evp)
            ceiling = {"us": round(pms * 1e3, 2), "k_MB": round(kb / 1e6, 3), "GBps": round(kb / (pms * 1e-3) / 1e9, 1)}
        res["lse_discover"] = {"split_us": round(sms * 1e3, 2),
                               "call_us_eager": round(ev3.elapsed_ms(2 * n_it, 2 * n_it + 1) / n_it * 1e3, 2),
                               "algorithmic_MB": round(lbytes / 1e6, 3),
                               "split_GBps": round(lbytes / (sms * 1e-3) / 1e9, 1),
                               "read_ceiling_k_only": ceiling,
                               "note": "K-only split + LSE selection, eager back-to-back calls"}
        for a, _ in sets:
            a.ev_split_begin = a.ev_split_end = None
        # restore replica 0's own schedule state
        plan.setup(0, sh)
        for pc, _ in plan.calls[0]:
            pc.run(sh)
        torch.cuda.synchronize()
    if not args.no_page_route and not plan.mixed:
        sparse_keys = [key for _, key in plan.calls[0] if key[0] == "sparse"]
        if sparse_keys:
            pus = [(harness.PageUnion(plan.kv[(0, depth, layer % plan.kv_layers)]), layer)
                   for _, depth, layer in sparse_keys]
            for pu, layer in pus:
                pu.compact(st0, layer, max(1, w.discoveries), stream=sh)
                pu.attend(plan.ws, stream=sh)
            n_it = max(20, 2 * len(pus))
            ev4 = harness.HipEvents(4 * n_it + 2)
            L = W.lib()
            prepared = []
            for pu, layer in pus:
                a_c, s_c, a_d = pu.layer.attn(), st0.view(layer, max(1, w.discoveries), w.eta), pu.attend_attn()
                prepared.append((a_c, s_c, a_d, int(pu.bt.data_ptr()), pu.bt.stride(0), int(pu.ctx.data_ptr())))
            ev4.record(4 * n_it, sh)
            for it in range(n_it):
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
            res["page_union"] = {"compact_us": round(float(comp_ms.mean()) * 1e3, 2),
                                 "split_us": round(float(split_ms.mean()) * 1e3, 2),
                                 "call_us_eager": round(ev4.elapsed_ms(4 * n_it, 4 * n_it + 1) / n_it * 1e3, 2),
                                 "page_density": round(kept_pages / max(1, all_pages), 4),
                                 "algorithmic_MB": round(sbytes / 1e6, 3),
                                 "split_GBps": round(sbytes / (float(split_ms.mean()) * 1e-3) / 1e9, 1),
                                 "note": "head-union pages of the reuse depths; compaction + dense decode over "
                                         "the compacted table, eager back-to-back"}
    if not args.no_state_copy:
        slots = torch.arange(w.rows, dtype=torch.int32, device=dev)
        rec = st0.record_bytes()
        records = torch.empty(w.rows * rec, dtype=torch.uint8, device=dev)
        n_it = 20
        ev5 = harness.HipEvents(4 * n_it)
        st0.snapshot(slots, records, sh)
        st0.restore(slots, records, sh)
        for it in range(n_it):
            ev5.record(4 * it, sh)
            st0.snapshot(slots, records, sh)
            ev5.record(4 * it + 1, sh)
            ev5.record(4 * it + 2, sh)
            st0.restore(slots, records, sh)
            ev5.record(4 * it + 3, sh)
        torch.cuda.synchronize()
        res["offload_state"] = {
            "snapshot_us": round(float(np.mean([ev5.elapsed_ms(4 * i, 4 * i + 1) for i in range(n_it)])) * 1e3, 2),
            "restore_us": round(float(np.mean([ev5.elapsed_ms(4 * i + 2, 4 * i + 3) for i in range(n_it)])) * 1e3, 2),
            "bytes_per_slot": rec, "slots": w.rows}
    return res


def default_replicas(w):
    """Distinct KV sets per depth, rotated so the 256 MB MALL cannot serve
    repeats: 1K workloads read a few tens to a few hundred MB per call, so
    they rotate six; larger ones rotate one or two."""
    one_set = int(synth.context_lengths(w).sum()) * w.heads * w.head_dim * 2 * (2 if w.dtype == "bf16" else 4)
    if w.max_ctx <= 1024:
        return 6
    return 2 if one_set < (1 << 30) else 1


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ctx1k", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--replicas", type=int, default=None, help="distinct KV sets per depth (default: by size)")
    ap.add_argument("--kv-layers", type=int, default=3,
                    help="distinct KV sets per depth for multi-layer workloads, rotated over the layers")
    ap.add_argument("--contexts", default=",".join(CONTEXT_WORKLOADS),
                    help="workloads measured per call in the contexts block ('' for none)")
    ap.add_argument("--context-steps", type=int, default=6)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense-reference", action="store_true",
                    help="skip the dense calls on the same KV (counter runs of the headline's own launches)")
    ap.add_argument("--no-read-ceiling", action="store_true")
    ap.add_argument("--no-lse-route", action="store_true")
    ap.add_argument("--no-page-route", action="store_true")
    ap.add_argument("--no-state-copy", action="store_true")
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

    # the CPU baseline's worker processes fork from a server started before
    # this process touches the GPU
    pool, workers = None, 0
    facts = host_facts()
    if not args.no_cpu_baseline:
        import concurrent.futures
        import multiprocessing
        import multiprocessing.forkserver as fs
        ctx = multiprocessing.get_context("forkserver")
        ctx.set_forkserver_preload(["numpy", "oracle.wise_oracle", "block_sparse_paged_split_amd.synth"])
        fs.ensure_running()
        workers = max(1, min(16, os.cpu_count() or 1))   # the host share of one GPU
        pool = concurrent.futures.ProcessPoolExecutor(workers, mp_context=ctx)

    import torch
    W.lib()  # fails loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    graphs = not args.no_graph
    probe = None if args.no_read_ceiling else ReadProbe()
    if args.calibrate_copy:
        src = torch.zeros(args.calibrate_copy << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"calibration kernel (neg): {args.calibrate_copy} MiB read + {args.calibrate_copy} MiB written")
        del src, dst

    w = synth.WORKLOADS[args.workload]
    log(f"headline workload {w.name}")
    head, ex = measure(w, dev, steps=args.steps, warmup=args.warmup,
                       replicas=args.replicas or default_replicas(w), kv_layers=args.kv_layers, graphs=graphs,
                       probe=probe, headline=True, args=args, dense_reference=not args.no_dense_reference)
    plan = ex["plan"]
    rows_per_step = w.rows * ex["calls"]
    # the read ceiling of the step's split launches: the pure gather of the
    # same pages (reuse calls: their own supports; discovery calls: the dense
    # pages), weighted by how often each kind runs in a step
    step_ceiling = None
    ceil = head["calls"].get("read_ceiling")
    if ceil:
        kinds = [key[0] for _, key in plan.calls[0]]
        pick = [ceil[k] if k in ceil else ceil.get("dense_same_kv") for k in kinds]
        if all(c is not None for c in pick):
            step_ceiling = sum(c["kv_MB"] for c in pick) * 1e6 / (sum(c["us"] for c in pick) * 1e-6) / 1e9
    achieved = ex["achieved"]   # every timed split launch's algorithmic bytes / its stamped duration
    modes_out = dict(head["calls"])
    if head["dense_ms_per_step"] is not None:
        modes_out["dense_step"] = {"ms_per_step": head["dense_ms_per_step"],
                                   "wise_step_speedup": head["wise_step_speedup"],
                                   "note": "every call of the step dense, HIP graph replay"}
    for k in ("lse_discover", "page_union", "offload_state"):
        if k in ex:
            modes_out[k] = ex[k]
    ctr = ex["ctr"]
    config = {"workload": w.name, "rows": w.rows, "heads": w.heads, "head_dim": w.head_dim,
              "ctx": head["ctx"], "page_size": w.page_size, "layers": w.layers,
              "schedule": "mixed launch" if plan.mixed else list(w.schedule), "eta": w.eta,
              "row_calls_per_step": rows_per_step, "kv_replicas": plan.replicas,
              "kv_sets_per_depth": plan.kv_layers,
              "timing": "eager launches" if args.no_graph else "HIP graph replay of whole steps",
              "union_density": head["union_density"], "fallbacks_per_step": head["fallbacks_per_step"],
              "errors": head["errors"]}
    support_r0 = ex["support_r0"]
    plan.free()
    del ex, plan
    torch.cuda.empty_cache()

    contexts = {}
    for name in [x for x in args.contexts.split(",") if x]:
        if name == w.name:
            contexts[name] = head
            continue
        wc = synth.WORKLOADS[name]
        if wc.layers > 1:   # per-call figures need one layer of the same shape
            wc = dataclasses.replace(wc, layers=1)
        log(f"context workload {name}")
        entry, ex_c = measure(wc, dev, steps=args.context_steps, warmup=2, replicas=default_replicas(wc),
                              kv_layers=1, graphs=graphs, probe=probe)
        ex_c["plan"].free()
        del ex_c
        torch.cuda.empty_cache()
        contexts[name] = entry

    out = {
        "metric": "decode-attn rows/s + achieved HBM GB/s (sparse vs dense), ctx 1K/4K/8K",
        "value": round(rows_per_step / (head["ms_per_step"] * 1e-3), 1),
        "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": config,
        "modes": modes_out,
        "contexts": contexts,
        "roofline": None,
        "cpu_baseline": None,
    }
    # roofline of the dominant kernel: the split kernel of the headline's calls;
    # beside the published peak, the box's own device-to-device copy rate
    copy_gbs = device_copy_gbs(dev)
    out["roofline"] = {"bound": "hbm", "kernel": "split_kernel", "achieved": round(achieved, 1),
                       "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                       "traffic": measured_traffic(w.name),
                       "device_copy": round(copy_gbs, 1), "frac_of_device_copy": round(achieved / copy_gbs, 4)}
    if step_ceiling:
        out["roofline"].update({"read_ceiling": round(step_ceiling, 1),
                                "frac_of_read_ceiling": round(achieved / step_ceiling, 4)})
    if pool is not None:
        log("cpu baseline: the oracle on the headline rows, in worker processes")
        out["cpu_baseline"], classes, union = cpu_baseline(w, pool, workers, facts)
        for name, entry in contexts.items():
            wc = synth.WORKLOADS[name]
            if wc.layers > 1:
                wc = dataclasses.replace(wc, layers=1)
            log(f"cpu oracle by mode: {name}")
            entry["cpu_oracle"] = cpu_oracle_by_mode(wc, pool, workers)
        pool.shutdown()
        if w.mix is None and w.fixed_density is None:
            out["selection_parity"] = selection_parity(classes, union, support_r0, w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
