"""The head-union page route (``wise_compact_pages`` + a dense decode over
the compacted page table) on the GPU against the fp64 oracle: compacted
tables and contexts bit-exact, outputs against attention over the kept
pages, fallbacks and data errors counted exactly."""

import dataclasses

import numpy as np
import pytest

from block_sparse_paged_split_amd import harness, synth
from block_sparse_paged_split_amd import wise as W
from parity import check_call, check_page_union

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    W.lib()
    return t


def discover(w, state, ws, depths=(0, 1), layer=0):
    """Discovery depths through the tile-stat route (checked as usual)."""
    for depth, mode in zip(depths, (W.WISE_DISCOVER, W.WISE_DISCOVER_UNION)):
        li = synth.layer_inputs(w, depth, layer)
        dev = harness.upload(li)
        check_call(w, li, dev, ws, state, mode=mode, layer=layer)


@pytest.mark.parametrize("name", ["match1k", "shared8k"])
def test_page_union_after_discovery(torch, name):
    """Two discovery depths, then a reuse depth by the head-union page route.
    shared8k runs at full size with sampled rows checked."""
    w = synth.WORKLOADS[name]
    rows = None if w.rows * w.max_ctx <= 32 * 1024 else [0, 1, 17, 40, 63]
    state = harness.SupportState(w.rows, w.heads, w.max_ctx)
    state.row_position.fill_(6)
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    say(f"[{name}] discovery depths 0-1")
    if rows is None:
        discover(w, state, ws)
    else:
        for depth, mode in zip((0, 1), (W.WISE_DISCOVER, W.WISE_DISCOVER_UNION)):
            li = synth.layer_inputs(w, depth)
            dev = harness.upload(li)
            harness.call(dev, ws, mode, state, required=w.discoveries)
    say(f"[{name}] depth 2 head-union page route")
    li = synth.layer_inputs(w, 2)
    dev = harness.upload(li)
    rep = check_page_union(w, li, dev, ws, state, rows=rows)
    say(f"   max_abs {rep.max_abs:.2e} page density {rep.page_density:.3f} counters {rep.counters}")
    assert rep.counters[W.CTR_FALLBACKS] == 0 and rep.counters[W.CTR_ERRORS] == 0
    if name == "shared8k":
        assert rep.page_density < 0.5


@pytest.mark.parametrize("P", [8, 32, 64, 256])
def test_page_union_page_sizes_and_modes(torch, P):
    """Ragged contexts at page sizes 8..256 with one launch mixing DENSE rows,
    SPARSE rows, a stale tag (fallback), another mode, a slot out of range, a
    bad context and an empty union."""
    ctxs = (1, 2, 31, 32, 33, 63, 64, 65, 100, 257, 1000, 2900)
    w = synth.Workload(name=f"pages_P{P}", rows=len(ctxs), heads=3, head_dim=128, dtype="bf16",
                       page_size=P, shuffle=True, alpha=6.0, seed=51, ctx_list=ctxs, hot=2,
                       schedule=(1, 2, 3), eta=0.9)
    state = harness.SupportState(w.rows, w.heads, w.max_ctx, slots=w.rows + 2)
    state.row_position.fill_(3)
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    say(f"[{w.name}] discovery depths 0-1")
    discover(w, state, ws)
    say(f"[{w.name}] depth 2: page route, mixed modes and data errors")
    li = synth.layer_inputs(w, 2)
    li.ctx_len = li.ctx_len.copy()
    li.ctx_len[4] = w.max_ctx + 1                       # row 4: context out of range
    modes = np.full(w.rows, W.WISE_SPARSE, np.uint8)
    modes[[1, 8]] = W.WISE_DENSE
    modes[6] = 7                                        # row 6: not a mode
    state.row_position[9] = 4                           # row 9: stale position, fallback
    state.slot_of_row = torch.tensor([r if r != 3 else 99 for r in range(w.rows)], dtype=torch.int32,
                                     device="cuda")     # row 3: slot out of range
    sup = state.support.clone()
    sup[10, 0] = 0                                      # row 10: empty union
    state.support.copy_(sup)
    dev = harness.upload(li)
    rep = check_page_union(w, li, dev, ws, state, row_modes=modes)
    say(f"   max_abs {rep.max_abs:.2e} page density {rep.page_density:.3f} counters {rep.counters}")
    assert rep.counters[W.CTR_FALLBACKS] == 1
    assert rep.counters[W.CTR_ERRORS] == 4 * w.heads
    out = dev.out.cpu().numpy()
    assert np.isnan(out[[3, 4, 6, 10]]).all() and not np.isnan(out[[0, 1, 2, 5, 7, 8, 9, 11]]).any()


def test_page_union_all_blocks_is_dense_bitwise(torch):
    """Every block selected: the compacted table is the row's table and the
    output is bit for bit the dense decode's."""
    w = dataclasses.replace(synth.WORKLOADS["ctx1k"], rows=8, name="pages_all")
    li = synth.layer_inputs(w, 0)
    dev = harness.upload(li)
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    say("[pages_all] dense decode vs page route with every block set")
    harness.call(dev, ws, W.WISE_DENSE)
    torch.cuda.synchronize()
    dense = dev.out.clone()
    state = harness.SupportState(w.rows, w.heads, w.max_ctx)
    tags = state.tags.clone()
    tags[:, 0, 0] = state.row_request
    tags[:, 0, 2] = 2
    state.tags.copy_(tags)
    state.support.fill_(-1)
    pu = harness.PageUnion(dev)
    pu.compact(state, required=2)
    dev.out.fill_(float("nan"))
    pu.attend(ws)
    torch.cuda.synchronize()
    assert torch.equal(pu.ctx, dev.ctx_len)
    assert torch.equal(pu.bt, dev.block_table)
    assert torch.equal(dev.out, dense)
    assert int(state.counters[W.CTR_FALLBACKS].item()) == 0
