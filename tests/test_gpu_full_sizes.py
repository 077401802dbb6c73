"""Parity at the workloads' full sizes, in the launch configuration bench.py
times: every row runs on the GPU and every row is checked against the fp64
oracle (outputs, supports, tags, tile masses, counters), the oracle running
in worker processes; the eta sweep's outer values and the LSE route check
sampled rows.
"""

import dataclasses

import numpy as np
import pytest

from block_sparse_paged_split_amd import harness, synth
from block_sparse_paged_split_amd import wise as W
from parity import check_call

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    W.lib()
    return t


def test_ctx4k_24_layers(torch):
    """64 rows at 4K, 24 layers per depth: every row of layers 0 and 23 of the
    4-depth schedule, each against its own support slice."""
    w = synth.WORKLOADS["ctx4k_24l"]
    state = harness.SupportState(w.rows, w.heads, w.max_ctx, layers=w.layers)
    state.row_position.fill_(3)
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    for layer in (0, 23):
        for depth, mode in enumerate(w.schedule):
            say(f"[ctx4k_24l] layer {layer} depth {depth} mode {mode}")
            li = synth.layer_inputs(w, depth, layer)
            dev = harness.upload(li, with_stats=True)
            rep = check_call(w, li, dev, ws, state, mode=mode, layer=layer, pool=True)
            say(f"   max_abs {rep.max_abs:.2e} near_eta {rep.near_eta} near_tie {rep.near_tie} "
                f"mismatch {rep.support_mismatch} counters {rep.counters}")
            assert rep.counters[W.CTR_FALLBACKS] == 0 and rep.counters[W.CTR_ERRORS] == 0
            del dev, li
    sup = state.support_numpy()
    assert sup[:, 0].any() and sup[:, 23].any() and not sup[:, 1:23].any()


def test_ctx8k_mixed_launch(torch):
    """One launch mixes 25% dense, 25% discover (fresh and union), 50% sparse
    rows; 5% of the sparse rows have an incomplete discovery and must run
    dense, counted as fallbacks."""
    w = synth.WORKLOADS["ctx8k_mixed"]
    modes, flagged = synth.mixed_row_modes(w)
    R = w.rows
    state = harness.SupportState(R, w.heads, w.max_ctx)
    state.row_position.fill_(9)
    ws = harness.Workspace(R, w.heads, w.head_dim, w.max_ctx)
    # setup depths: every non-dense row discovers at depth 0; sparse rows
    # that are not flagged complete their window with a union at depth 1
    d0 = np.where(modes == W.WISE_DENSE, W.WISE_DENSE, W.WISE_DISCOVER).astype(np.uint8)
    d1 = np.where((modes == W.WISE_SPARSE) & ~flagged, W.WISE_DISCOVER_UNION, W.WISE_DENSE).astype(np.uint8)
    for depth, rm in ((0, d0), (1, d1), (2, modes)):
        say(f"[ctx8k_mixed] depth {depth} modes {np.bincount(rm, minlength=4)}, every row")
        li = synth.layer_inputs(w, depth)
        dev = harness.upload(li, with_stats=True)
        fb0 = int(state.counters[W.CTR_FALLBACKS].item())
        rep = check_call(w, li, dev, ws, state, mode=W.WISE_SPARSE, row_modes=rm, pool=True)
        say(f"   max_abs {rep.max_abs:.2e} near_eta {rep.near_eta} near_tie {rep.near_tie} "
            f"mismatch {rep.support_mismatch} counters {rep.counters}")
        fallbacks = int(state.counters[W.CTR_FALLBACKS].item()) - fb0
        assert fallbacks == (int(flagged.sum()) if depth == 2 else 0)
        del dev, li


def test_ragged_eta_sweep(torch):
    """128 rows, contexts log-uniform over 512..32768, 1-16 planted blocks;
    the schedule at eta 0.9, 0.95 and 0.99 on identical data: every row at
    eta 0.95, sampled rows at 0.9 and 0.99.  Supports of one depth are nested
    across eta."""
    w = synth.WORKLOADS["ragged"]
    ctx = synth.context_lengths(w)
    order = np.argsort(ctx)
    rows = sorted({int(order[0]), int(order[-1]), int(order[len(order) // 2]), int(order[len(order) // 4]),
                   int(order[3 * len(order) // 4]), 5, 77, 100})
    say(f"[ragged] contexts {ctx.min()}..{ctx.max()} mean {ctx.mean():.0f}; checked rows {rows}")
    devs, samples = [], []
    for depth in range(len(w.schedule)):
        li = synth.layer_inputs(w, depth)
        devs.append(harness.upload(li, with_stats=True))
        del li
        samples.append(synth.layer_inputs(w, depth, rows=rows))
        say(f"   depth {depth} uploaded")
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    first_depth = {}
    for eta in (0.9, 0.95, 0.99):
        state = harness.SupportState(w.rows, w.heads, w.max_ctx)
        for depth, mode in enumerate(w.schedule):
            say(f"[ragged] eta {eta} depth {depth} mode {mode}")
            if eta == 0.95:
                # every row: the oracle's workers regenerate the rows they evaluate
                rep = check_call(w, samples[depth], devs[depth], ws, state, mode=mode, eta=eta, pool=True)
            else:
                rep = check_call(w, samples[depth], devs[depth], ws, state, mode=mode, rows=rows, eta=eta)
            say(f"   max_abs {rep.max_abs:.2e} near_eta {rep.near_eta} near_tie {rep.near_tie} "
                f"mismatch {rep.support_mismatch} counters {rep.counters}")
            if depth == 0:
                first_depth[eta] = state.support_numpy().copy()
        ctr = state.counters.cpu().numpy()
        say(f"   eta {eta}: union density {ctr[W.CTR_SELECTED] / ctr[W.CTR_CAUSAL]:.4f}")
    a, b, c = first_depth[0.9], first_depth[0.95], first_depth[0.99]
    assert ((a & ~b) == 0).all() and ((b & ~c) == 0).all()


def test_lse_route_ragged_full_size(torch):
    """Discovery and union by the LSE route on the 128-row ragged batch
    (contexts 512..32768): every row runs on the GPU, sampled rows (the
    shortest, the longest, the median and two others) are checked against
    the oracle; the LSE of the other rows is the same oracle's where sampled
    and 0 elsewhere (those rows are not checked)."""
    from parity import check_lse_call, oracle_lse
    w = synth.WORKLOADS["ragged"]
    ctx = synth.context_lengths(w)
    order = np.argsort(ctx)
    rows = sorted({int(order[0]), int(order[-1]), int(order[len(order) // 2]), 5, 77})
    say(f"[ragged lse] checked rows {rows} contexts {[int(ctx[r]) for r in rows]}")
    state = harness.SupportState(w.rows, w.heads, w.max_ctx)
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    for depth, union in ((0, False), (1, True)):
        li = synth.layer_inputs(w, depth)
        dev = harness.upload(li, with_stats=True)
        del li
        sample = synth.layer_inputs(w, depth, rows=rows)
        say(f"   depth {depth} union {union}")
        rep = check_lse_call(w, sample, dev, ws, state, oracle_lse(w, sample, rows), union=union, rows=rows)
        say(f"   near_eta {rep.near_eta} near_tie {rep.near_tie} mismatch {rep.support_mismatch}")
        del dev
    disc = state.tags_numpy()["discoveries"][:, 0]
    assert (disc[rows] == 2).all()
