"""Discovery by the LSE route (``wise_discover_lse``) on the GPU against the
fp64 oracle: block mass rebuilt from an external dense kernel's
log-sum-exp by rereading K, selection, union, tags and counters.  The LSE
handed to the GPU is the oracle's own (an input, rounded to fp32)."""

import dataclasses

import numpy as np
import pytest

from block_sparse_paged_split_amd import harness, synth
from block_sparse_paged_split_amd import wise as W
from parity import check_call, check_lse_call, oracle_lse

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    W.lib()
    return t


def test_lse_route_ctx1k_then_sparse(torch):
    """Depth 0 and 1 discover by the LSE route; depth 2 attends the resulting
    union through the sparse split, checked against masked attention."""
    w = synth.WORKLOADS["ctx1k"]
    state = harness.SupportState(w.rows, w.heads, w.max_ctx)
    state.row_position.fill_(4)
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    for depth, union in ((0, False), (1, True)):
        say(f"[lse ctx1k] depth {depth} union {union}")
        li = synth.layer_inputs(w, depth)
        dev = harness.upload(li, with_stats=True)
        rep = check_lse_call(w, li, dev, ws, state, oracle_lse(w, li), union=union)
        say(f"   near_eta {rep.near_eta} near_tie {rep.near_tie} mismatch {rep.support_mismatch} "
            f"counters {rep.counters}")
        assert rep.counters[W.CTR_ERRORS] == 0 and rep.counters[W.CTR_FALLBACKS] == 0
    tags = state.tags_numpy()
    assert (tags["discoveries"][:, 0] == 2).all()
    li = synth.layer_inputs(w, 2)
    dev = harness.upload(li, with_stats=True)
    say("[lse ctx1k] depth 2 sparse over the LSE-discovered union")
    rep = check_call(w, li, dev, ws, state, mode=W.WISE_SPARSE)
    say(f"   max_abs {rep.max_abs:.2e} counters {rep.counters}")
    assert rep.counters[W.CTR_FALLBACKS] == 0
    ctr = state.counters.cpu().numpy()
    say(f"   union density {ctr[W.CTR_SELECTED] / ctr[W.CTR_CAUSAL]:.4f}")


def test_lse_route_agrees_with_tile_route(torch):
    """Same data, two discovery routes: the supports differ only in units
    that one of the two comparisons exempts (cut within 1e-6 of eta, or a
    near tie at the cut)."""
    w = dataclasses.replace(synth.WORKLOADS["match1k"], rows=16, name="lse_vs_tile")
    li = synth.layer_inputs(w, 0)
    dev = harness.upload(li, with_stats=True)
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    say("[lse_vs_tile] tile-stat discovery, then LSE discovery on the same data")
    s_tile = harness.SupportState(w.rows, w.heads, w.max_ctx)
    rep_t = check_call(w, li, dev, ws, s_tile, mode=W.WISE_DISCOVER, required=1)
    s_lse = harness.SupportState(w.rows, w.heads, w.max_ctx)
    rep_l = check_lse_call(w, li, dev, ws, s_lse, oracle_lse(w, li), union=False)
    a, b = s_tile.support_numpy(), s_lse.support_numpy()
    differ = int((a != b).any(axis=-1).sum())
    exempt = rep_t.near_eta + rep_t.near_tie + rep_l.near_eta + rep_l.near_tie
    say(f"   units differing {differ}, exempt {exempt}")
    assert differ <= exempt
    assert np.array_equal(s_tile.tags.cpu().numpy(), s_lse.tags.cpu().numpy())


RAGGED = (1, 2, 31, 32, 33, 63, 64, 65, 100, 257, 1000, 2900)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_lse_route_ragged_and_errors(torch, dtype, d):
    """Ragged contexts (units spanning one to several split groups), then a
    union depth with a non-finite LSE in one unit, a bad page in one row and
    a broken window in another."""
    w = synth.Workload(name=f"lse_ragged_{dtype}{d}", rows=len(RAGGED), heads=3, head_dim=d,
                       dtype=dtype, page_size=16, shuffle=True, alpha=6.0, seed=31,
                       ctx_list=RAGGED, hot=3, schedule=(1, 2), eta=0.9)
    state = harness.SupportState(w.rows, w.heads, w.max_ctx)
    state.row_position.fill_(8)
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    say(f"[{w.name}] depth 0 LSE discovery")
    li = synth.layer_inputs(w, 0)
    dev = harness.upload(li, with_stats=True)
    rep = check_lse_call(w, li, dev, ws, state, oracle_lse(w, li), union=False)
    assert rep.counters[W.CTR_ERRORS] == 0
    say(f"[{w.name}] depth 1 LSE union with a NaN lse, a bad page and a broken window")
    li = synth.layer_inputs(w, 1)
    lse = oracle_lse(w, li)
    lse[4, 1] = np.nan                          # row 4 head 1: non-finite LSE
    li.block_table = li.block_table.copy()
    li.block_table[10, 3] = li.num_pages + 7    # row 10: a page id out of range
    state.row_position[7] = 9                   # row 7: the token moved on, window broken
    dev = harness.upload(li, with_stats=True)
    rep = check_lse_call(w, li, dev, ws, state, lse, union=True)
    say(f"   counters {rep.counters}")
    assert rep.counters[W.CTR_FALLBACKS] == 1
    assert rep.counters[W.CTR_ERRORS] == 1 + w.heads
    tags = state.tags_numpy()["discoveries"][:, 0]
    assert tags[4] == 0 and tags[7] == 0 and tags[10] == 0 and tags[0] == 2
