"""GPU-vs-oracle comparison of one (depth, layer) call.

The oracle is evaluated from the GPU's own pre-call state (support bitmask,
tags), so every call is checked on its own: outputs of dense / discover rows
against plain attention, outputs of sparse rows against masked attention
over the support the GPU itself holds, and the post-call support against
the oracle's selection, bit-exact.  A discovery unit's support may differ
from the oracle's only in two ways, each tied to a named ambiguity of fp32
masses against fp64 ones, and each counted:

  class A  the oracle's running sum lies within 1e-6 of eta at the cut:
           with c_{K-1} there, the GPU may stop one block early (the first
           K-1 blocks of the oracle's order); with c_K there, one block late
           (the first K+1);
  class B  the K-th and (K+1)-th masses of the oracle's order tie within
           1e-6 relative: the GPU may hold the first K-1 blocks and the
           (K+1)-th instead of the K-th.

Any other difference fails.  The density counters are checked exactly,
adjusted by the blocks the excused units really added.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

from oracle import wise_oracle as O
from block_sparse_paged_split_amd import harness, synth
from block_sparse_paged_split_amd import wise as W

TOL = {"bf16": (2e-3, 1e-2), "f32": (1e-5, 1e-5)}


# Every comparison made in this process, for the session summary (see conftest).
RECORDS = []


def record(kind: str, what: str, rep: "Report") -> "Report":
    RECORDS.append({"kind": kind, "what": what, "units": rep.units, "near_eta": rep.near_eta,
                    "near_tie": rep.near_tie, "mismatch": rep.support_mismatch,
                    "excused_a": rep.excused_a, "excused_b": rep.excused_b,
                    "max_abs": rep.max_abs, "max_rel": rep.max_rel})
    return rep


def allowed_supports(sel: O.Selection, eta: float, nb: int, words: int, old: np.ndarray,
                     union: bool):
    """The post-call support words a discovery unit may hold besides the
    oracle's own, as {class: words}: the cut moved by one block where the
    running sum is within 1e-6 of eta (class A), or the tied K-th and (K+1)-th
    blocks swapped (class B)."""
    order, K = sel.order, sel.K
    out = {}

    def words_of(blocks):
        new = O.blocks_to_bits(blocks, words)
        return (old | new) if union else new

    if K >= 2 and abs(sel.c_prev - eta) <= 1e-6:
        out.setdefault("A", []).append(words_of(order[:K - 1]))
    if K < nb and abs(sel.c_K - eta) <= 1e-6:
        out.setdefault("A", []).append(words_of(order[:K + 1]))
    if K < nb and sel.near_tie():
        out.setdefault("B", []).append(words_of(np.concatenate([order[:K - 1], order[K:K + 1]])))
    return out


def check_unit_support(got: np.ndarray, want: np.ndarray, sel: O.Selection, eta: float, nb: int,
                       old: np.ndarray, union: bool, rep: "Report", what: str) -> int:
    """Compare one discovery unit's post-call support; returns the blocks the
    GPU added minus the blocks the oracle added (0 unless excused)."""
    a = sel.near_eta(eta)
    b = sel.near_tie()
    rep.near_eta += int(a)
    rep.near_tie += int(b and not a)
    if np.array_equal(got, want):
        return 0
    rep.support_mismatch += 1
    words = len(want)
    for cls, cands in allowed_supports(sel, eta, nb, words, old, union).items():
        if any(np.array_equal(got, c) for c in cands):
            if cls == "A":
                rep.excused_a += 1
            else:
                rep.excused_b += 1
            pop = lambda x: int(sum(bin(int(v)).count("1") for v in x))  # noqa: E731
            if union:
                return pop(got & ~old) - pop(want & ~old)
            return pop(got) - pop(want)
    raise AssertionError(f"{what}: support differs beyond a moved cut or a tied swap: gpu "
                         f"{O.bits_to_blocks(got, 32 * words).tolist()} oracle {sel.blocks.tolist()} "
                         f"(K={sel.K}, c_K-1={sel.c_prev:.9f}, c_K={sel.c_K:.9f}, "
                         f"p_K={sel.p_K:.9g}, p_K+1={sel.p_next:.9g})")


# ----------------------------------------------------------------------------- oracle in worker processes

_POOL = None


def oracle_pool():
    """Worker processes for the fp64 oracle of full-size calls, forked from the
    fork server the test session starts before any GPU work (at most 16: the
    host share of one GPU)."""
    global _POOL
    if _POOL is None:
        import concurrent.futures
        import multiprocessing
        import os
        n = max(1, min(16, os.cpu_count() or 1))
        _POOL = concurrent.futures.ProcessPoolExecutor(n, mp_context=multiprocessing.get_context("forkserver"))
    return _POOL


def _oracle_rows(w, depth, layer, chunk, modes, kw):
    """One worker's share: regenerate the rows' inputs from the seeded
    generator and evaluate the oracle on them."""
    li = synth.layer_inputs(w, depth, layer, rows=chunk, workers=1)
    ref = O.run_call(q=li.q, k_cache=li.k, v_cache=li.v, block_table=li.block_table,
                     ctx_len=li.ctx_len, page_size=w.page_size, num_pages=li.num_pages,
                     max_ctx=w.max_ctx, modes=modes, rows=chunk, **kw)
    slot_of = kw.get("slot_of_row")
    slots = [r if slot_of is None else int(slot_of[r]) for r in chunk]
    sup = None if ref.support is None else {s: ref.support[s].copy() for s in slots
                                            if 0 <= s < ref.support.shape[0]}
    tags = None if ref.tags is None else {s: ref.tags[s].copy() for s in slots if 0 <= s < ref.tags.shape[0]}
    return ({r: ref.out[r] for r in chunk}, sup, tags, ref.counters, {r: ref.effective[r] for r in chunk},
            ref.units)


def run_call_parallel(w, depth, layer, modes, rows, kw) -> O.CallResult:
    """``O.run_call`` over ``rows`` of the seeded workload (w, depth, layer),
    split over worker processes.  Rows are independent (each owns its slot),
    so the merged result is the one a single call gives."""
    R = w.rows
    nw = max(1, min(len(rows), 4 * oracle_pool()._max_workers))
    chunks = [list(c) for c in np.array_split(np.asarray(rows), nw) if len(c)]
    futs = [oracle_pool().submit(_oracle_rows, w, depth, layer, [int(r) for r in c], modes, kw) for c in chunks]
    out = np.full((R, w.heads, w.head_dim), np.nan)
    sup = None if kw.get("support") is None else kw["support"].copy()
    tags = None if kw.get("tags") is None else kw["tags"].copy()
    counters = np.zeros(4, dtype=np.int64)
    eff = np.full(R, -1, dtype=np.int64)
    units = {}
    for f in futs:
        o, s, t, c, e, u = f.result()
        for r, v in o.items():
            out[r] = v
        if s is not None:
            for k, v in s.items():
                sup[k] = v
        if t is not None:
            for k, v in t.items():
                tags[k] = v
        counters += c
        for r, v in e.items():
            eff[r] = v
        units.update(u)
    return O.CallResult(out, sup, tags, counters, eff, units)


@dataclasses.dataclass
class Report:
    max_abs: float = 0.0
    max_rel: float = 0.0
    units: int = 0
    near_eta: int = 0          # units in class A (a mismatch would be excused)
    near_tie: int = 0          # units in class B and not in class A
    support_mismatch: int = 0  # units whose support differs (each one excused below)
    excused_a: int = 0         # mismatches that are exactly a class-A moved cut
    excused_b: int = 0         # mismatches that are exactly a class-B swap
    counters: Optional[np.ndarray] = None
    page_density: float = 0.0  # head-union page route: kept pages / causal pages


def assert_close(got, ref, dtype, what, report: Report):
    atol, rtol = TOL[dtype]
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), f"{what}: NaN pattern differs"
    g, r = got[~nan_ref], ref[~nan_ref]
    if g.size == 0:
        return
    err = np.abs(g - r)
    report.max_abs = max(report.max_abs, float(err.max()))
    report.max_rel = max(report.max_rel, float((err / np.maximum(np.abs(r), 1e-30)).max()))
    bad = err > atol + rtol * np.abs(r)
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of tolerance; "
                           f"max abs {err.max():.3e}")


def check_call(w: synth.Workload, li: synth.LayerInputs, dev: harness.DeviceLayer,
               ws: harness.Workspace, state: Optional[harness.SupportState], *, mode: int,
               row_modes: Optional[np.ndarray] = None, layer: int = 0,
               rows: Optional[Sequence[int]] = None, required: Optional[int] = None,
               eta: Optional[float] = None, check_stats: bool = True, pool: bool = False) -> Report:
    """One call on the GPU against the oracle on ``rows`` (all by default).
    With ``pool`` the oracle runs in worker processes that regenerate the
    inputs from (workload, depth, layer): ``li`` must then be the seeded
    generator's own output."""
    import torch
    R = li.q.shape[0]
    required = w.discoveries if required is None else required
    eta = w.eta if eta is None else eta
    rows = list(range(R)) if rows is None else list(rows)
    sup0 = state.support_numpy().copy() if state else None
    tags0 = state.tags_numpy() if state else None
    ctr0 = state.counters.cpu().numpy().copy() if state else None
    rm_dev = None
    if row_modes is not None:
        rm_dev = torch.from_numpy(row_modes.astype(np.uint8)).to(dev.q.device)
    harness.call(dev, ws, mode, state, layer_idx=layer, required=required, eta=eta, row_mode=rm_dev)
    torch.cuda.synchronize()
    out = dev.out.cpu().numpy()
    modes = row_modes if row_modes is not None else np.full(R, mode)
    kw = {}
    if state:
        kw = dict(support=sup0, tags=tags0, layer=layer,
                  slot_of_row=None if state.slot_of_row is None else state.slot_of_row.cpu().numpy(),
                  row_request=state.row_request.cpu().numpy(),
                  row_position=state.row_position.cpu().numpy(), required=required, eta=eta)
    if pool:
        ref = run_call_parallel(w, li.depth, li.layer, modes, rows, kw)
    else:
        ref = O.run_call(q=li.q, k_cache=li.k, v_cache=li.v, block_table=li.block_table,
                         ctx_len=li.ctx_len, page_size=w.page_size, num_pages=li.num_pages,
                         max_ctx=w.max_ctx, modes=modes, rows=rows, **kw)
    rep = Report()
    for r in rows:
        assert_close(out[r], ref.out[r], w.dtype, f"row {r} output", rep)
    rep.units = len(rows) * w.heads
    if state is None:
        return rep
    sup1 = state.support_numpy()
    tags1 = state.tags_numpy()
    ctr1 = state.counters.cpu().numpy()
    rep.counters = ctr1 - ctr0
    slot_of = (lambda r: r) if state.slot_of_row is None else (lambda r: int(state.slot_of_row[r]))
    selected_shift = 0
    for r in rows:
        s = slot_of(r)
        if ref.effective[r] < 0:
            continue
        for h in range(w.heads):
            unit = ref.units[(r, h)]
            if unit.selection is not None and not unit.error:
                nb = (int(li.ctx_len[r]) + 31) // 32
                selected_shift += check_unit_support(
                    sup1[s, layer, h], ref.support[s, layer, h], unit.selection, eta, nb,
                    sup0[s, layer, h], unit.effective == O.DISCOVER_UNION, rep, f"row {r} head {h}")
            else:
                assert np.array_equal(sup1[s, layer, h], sup0[s, layer, h]), f"row {r} head {h} support touched"
            if check_stats and dev.tile_stats is not None and not unit.error and unit.m is not None:
                st = dev.tile_stats[r, h].cpu().numpy().astype(np.float64)
                att = unit.attended
                # tile masses relative to the oracle's row (M, L) of the attended set
                M = np.max(unit.m)
                Lr = np.sum(unit.l * np.exp(unit.m - M))
                p_ref = unit.l * np.exp(unit.m - M) / Lr
                p_gpu = st[att, 1] * np.exp(st[att, 0] - M) / Lr
                err = np.abs(p_gpu - p_ref)
                assert (err <= 1e-6 + 1e-5 * p_ref).all(), f"tile masses of row {r} head {h}: max {err.max():.3e}"
        if int(modes[r]) != W.WISE_DENSE:
            for f in ("request", "position", "discoveries"):
                assert tags1[s, layer][f] == ref.tags[s, layer][f], f"tag {f} of row {r}"
    if len(rows) == R:
        assert rep.counters[W.CTR_FALLBACKS] == ref.counters[0]
        assert rep.counters[W.CTR_ERRORS] == ref.counters[3]
        assert rep.counters[W.CTR_SELECTED] == ref.counters[1] + selected_shift
        assert rep.counters[W.CTR_CAUSAL] == ref.counters[2]
    return record("call", f"{w.name} mode {mode}" + (" mixed" if row_modes is not None else ""), rep)


# ----------------------------------------------------------------------------- LSE route

def oracle_lse(w: synth.Workload, li: synth.LayerInputs, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """[R, H] fp32 log-sum-exp of every (row, head)'s scaled scores, from the
    oracle: the stand-in for an external dense kernel's LSE.  Rows whose
    context or pages are invalid (and rows not listed) get 0."""
    R, H, d = li.q.shape
    scale = O.default_scale(d)
    out = np.zeros((R, H), np.float32)
    for r in (range(R) if rows is None else rows):
        n = int(li.ctx_len[r])
        if not 1 <= n <= w.max_ctx:
            continue
        toks = np.arange(n)
        pages = li.block_table[r][toks // w.page_size]
        if np.any((pages < 0) | (pages >= li.num_pages)):
            continue
        qf = O.widen(li.q[r])
        for h in range(H):
            s = scale * (O.gather_tokens(li.k, li.block_table[r], toks, w.page_size, h) @ qf[h])
            out[r, h] = O.row_lse(s)
    return out


def check_lse_call(w: synth.Workload, li: synth.LayerInputs, dev: harness.DeviceLayer,
                   ws: harness.Workspace, state: harness.SupportState, lse: np.ndarray, *,
                   union: bool, layer: int = 0, rows: Optional[Sequence[int]] = None,
                   eta: Optional[float] = None) -> Report:
    """One LSE-route discovery depth on the GPU against ``O.run_lse_call`` on
    the same fp32 lse: supports (exact but for class A/B units), tile masses,
    tags, counters, and ``out`` left untouched."""
    import torch
    R, H = li.q.shape[:2]
    eta = w.eta if eta is None else eta
    rows = list(range(R)) if rows is None else list(rows)
    sup0 = state.support_numpy().copy()
    tags0 = state.tags_numpy()
    ctr0 = state.counters.cpu().numpy().copy()
    dev.out.fill_(123.0)
    lse_dev = torch.from_numpy(np.ascontiguousarray(lse, np.float32)).to(dev.q.device)
    harness.call_lse(dev, ws, lse_dev, union, state, layer_idx=layer, eta=eta)
    torch.cuda.synchronize()
    assert bool((dev.out == 123.0).all()), "the LSE route wrote the attention output"
    slot_of_row = None if state.slot_of_row is None else state.slot_of_row.cpu().numpy()
    ref = O.run_lse_call(q=li.q, k_cache=li.k, block_table=li.block_table, ctx_len=li.ctx_len,
                         page_size=w.page_size, num_pages=li.num_pages, max_ctx=w.max_ctx,
                         lse=lse.astype(np.float64), union=union, support=sup0, tags=tags0,
                         layer=layer, slot_of_row=slot_of_row,
                         row_request=state.row_request.cpu().numpy(),
                         row_position=state.row_position.cpu().numpy(), eta=eta, rows=rows)
    rep = Report(units=len(rows) * H)
    sup1 = state.support_numpy()
    tags1 = state.tags_numpy()
    rep.counters = state.counters.cpu().numpy() - ctr0
    selected_shift = 0
    for r in rows:
        if ref.effective[r] < 0:
            continue
        s = r if slot_of_row is None else int(slot_of_row[r])
        for h in range(H):
            unit = ref.units.get((r, h))
            if unit is not None and unit.selection is not None:
                nb = len(unit.mass)
                selected_shift += check_unit_support(
                    sup1[s, layer, h], ref.support[s, layer, h], unit.selection, eta, nb,
                    sup0[s, layer, h], unit.effective == O.DISCOVER_UNION, rep,
                    f"LSE route row {r} head {h}")
                if dev.tile_stats is not None:
                    st = dev.tile_stats[r, h].cpu().numpy().astype(np.float64)
                    nb = len(unit.mass)
                    p_gpu = st[:nb, 1] * np.exp(st[:nb, 0] - float(lse[r, h]))
                    err = np.abs(p_gpu - unit.mass)
                    assert (err <= 1e-6 + 1e-5 * unit.mass).all(), \
                        f"LSE block masses of row {r} head {h}: max {err.max():.3e}"
            else:
                assert np.array_equal(sup1[s, layer, h], sup0[s, layer, h]), \
                    f"row {r} head {h} support touched"
        for f in ("request", "position", "discoveries"):
            assert tags1[s, layer][f] == ref.tags[s, layer][f], f"tag {f} of row {r}"
    if len(rows) == R:
        assert rep.counters[W.CTR_FALLBACKS] == ref.counters[0]
        assert rep.counters[W.CTR_ERRORS] == ref.counters[3]
        assert rep.counters[W.CTR_SELECTED] == ref.counters[1] + selected_shift
        assert rep.counters[W.CTR_CAUSAL] == ref.counters[2]
    return record("lse", f"{w.name} {'union' if union else 'discover'}", rep)


# ----------------------------------------------------------------------------- head-union page route

def check_page_union(w: synth.Workload, li: synth.LayerInputs, dev: harness.DeviceLayer,
                     ws: harness.Workspace, state: harness.SupportState, *, layer: int = 0,
                     required: Optional[int] = None, row_modes: Optional[np.ndarray] = None,
                     rows: Optional[Sequence[int]] = None) -> Report:
    """One reuse depth by the head-union page route on the GPU (compaction,
    which counts fallbacks and data errors, then the dense decode over the
    compacted table) against ``O.run_page_union_call``: compacted tables and
    contexts exact, outputs within tolerance, fallback and error counts
    exact, the support state untouched."""
    import torch
    R, H = li.q.shape[:2]
    required = w.discoveries if required is None else required
    rows = list(range(R)) if rows is None else list(rows)
    sup0 = state.support_numpy().copy()
    tags_raw0 = state.tags.clone()
    tags0 = state.tags_numpy()
    ctr0 = state.counters.cpu().numpy().copy()
    rm_dev = None
    if row_modes is not None:
        rm_dev = torch.from_numpy(row_modes.astype(np.uint8)).to(dev.q.device)
    pu = harness.PageUnion(dev)
    pu.compact(state, layer_idx=layer, required=required, row_mode=rm_dev)
    pu.attend(ws)
    torch.cuda.synchronize()
    slot_of_row = None if state.slot_of_row is None else state.slot_of_row.cpu().numpy()
    ref = O.run_page_union_call(q=li.q, k_cache=li.k, v_cache=li.v, block_table=li.block_table,
                                ctx_len=li.ctx_len, page_size=w.page_size, num_pages=li.num_pages,
                                max_ctx=w.max_ctx, support=sup0, tags=tags0, layer=layer,
                                slot_of_row=slot_of_row, row_request=state.row_request.cpu().numpy(),
                                row_position=state.row_position.cpu().numpy(), required=required,
                                row_modes=row_modes, rows=rows)
    ctx = pu.ctx.cpu().numpy()
    bt = pu.bt.cpu().numpy()
    out = dev.out.cpu().numpy()
    rep = Report(units=len(rows) * H)
    for r in rows:
        assert int(ctx[r]) == int(ref.ctx[r]), f"row {r}: compacted context {ctx[r]} vs {ref.ctx[r]}"
        if r in ref.tables:
            k = len(ref.tables[r])
            assert bt[r, :k].tolist() == ref.tables[r].tolist(), f"row {r}: compacted table"
        assert_close(out[r], ref.out[r], w.dtype, f"row {r} output", rep)
    rep.counters = state.counters.cpu().numpy() - ctr0
    assert np.array_equal(state.support_numpy(), sup0), "support touched"
    assert torch.equal(state.tags, tags_raw0), "tags touched"
    if len(rows) == R:
        assert rep.counters[W.CTR_FALLBACKS] == ref.counters[0]
        assert rep.counters[W.CTR_ERRORS] == ref.counters[3]
    rep.page_density = (float(sum(len(ref.pages[r]) for r in rows if r in ref.pages)) /
                        max(1, sum(-(-int(li.ctx_len[r]) // w.page_size) for r in rows if r in ref.pages)))
    return rep
