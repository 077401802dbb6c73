"""Exactly tied block masses on the GPU: every key of a (row, head) is the
same vector, so every full 32-token block carries the same softmax mass, in
fp32 on the GPU as in fp64 in the oracle.  The selection must then follow
the tie-break (mass descending, block index ascending) bit for bit: the
support is blocks 0..K-1 with no exemption at all, although every such unit
sits in the tied-boundary ambiguity class.  Contexts and eta are chosen so
that no running sum lies near eta.
"""

import dataclasses

import numpy as np
import pytest

from block_sparse_paged_split_amd import harness, synth
from block_sparse_paged_split_amd import wise as W
from oracle import wise_oracle as O
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


def tied(name, ctxs, eta, heads=4):
    return dataclasses.replace(synth.WORKLOADS["ctx1k"], name=name, rows=len(ctxs), heads=heads, ctx=None,
                               ctx_list=tuple(ctxs), hot=0, tied_keys=True, eta=eta)


# (contexts, eta): the fused path (every unit <= 1K tokens), the static grid
# with the finish kernel (up to 8K), a partial last block (1000 tokens: 31
# tied blocks, then a lighter one) and a row short enough to keep every block
CASES = [
    ((1024, 1000, 96, 320, 960, 1024), 0.95),
    ((1024, 1000, 96, 320, 960, 1024), 0.93),
    ((4096, 2048, 8192, 1000, 96, 8192), 0.95),
    ((4096, 2048, 8192, 1000, 96, 8192), 0.93),
]


def expected_blocks(n, eta):
    nb = (n + 31) // 32
    full = n // 32
    if full == nb:                               # every block tied
        k = int(np.ceil(eta * nb - 1e-12))
        return list(range(k))
    # full blocks first by index, then the lighter partial block
    c = np.cumsum([32.0 / n] * full + [(n - 32 * full) / n])
    k = int(np.nonzero(c >= eta)[0][0]) + 1
    return list(range(k))


@pytest.mark.parametrize("ctxs,eta", CASES)
def test_tied_masses_discover_union_sparse(torch, ctxs, eta):
    w = tied(f"tied_{max(ctxs)}_{eta}", ctxs, eta)
    say(f"[{w.name}] contexts {ctxs} eta {eta}: discover, union, sparse")
    state = harness.SupportState(w.rows, w.heads, w.max_ctx)
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    for depth, mode in enumerate((W.WISE_DISCOVER, W.WISE_DISCOVER_UNION, W.WISE_SPARSE)):
        li = synth.layer_inputs(w, depth)
        dev = harness.upload(li, with_stats=True)
        rep = check_call(w, li, dev, ws, state, mode=mode, required=2)
        say(f"   depth {depth}: units {rep.units} class B {rep.near_tie} mismatches {rep.support_mismatch}")
        assert rep.support_mismatch == 0, "a tied unit's support differs from the index-ascending tie-break"
        if mode == W.WISE_DISCOVER:
            sup = state.support_numpy()
            for r, n in enumerate(ctxs):
                for h in range(w.heads):
                    assert O.bits_to_blocks(sup[r, 0, h], (n + 31) // 32).tolist() == expected_blocks(n, eta)


def test_tied_masses_mixed_planned_launch(torch):
    """Discovery rows of a mixed launch (plan kernel, listed split, finish
    kernel) with tied masses."""
    ctxs = (4096, 2048, 8192, 1000, 96, 8192, 4096, 3000)
    w = tied("tied_mixed", ctxs, 0.95)
    say(f"[{w.name}] contexts {ctxs}: a mixed launch with discovery and sparse rows")
    state = harness.SupportState(w.rows, w.heads, w.max_ctx)
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    li = synth.layer_inputs(w, 0)
    dev = harness.upload(li, with_stats=True)
    rep = check_call(w, li, dev, ws, state, mode=W.WISE_DISCOVER, required=1)
    assert rep.support_mismatch == 0
    modes = np.array([1, 3, 2, 3, 1, 3, 0, 2], np.uint8)
    li = synth.layer_inputs(w, 1)
    dev = harness.upload(li, with_stats=True)
    rep = check_call(w, li, dev, ws, state, mode=W.WISE_SPARSE, row_modes=modes, required=1)
    say(f"   mixed: class B {rep.near_tie} mismatches {rep.support_mismatch}")
    assert rep.support_mismatch == 0


@pytest.mark.parametrize("ctxs", [(1024, 1000, 96, 320), (4096, 8192, 1000, 2048)])
def test_tied_masses_lse_route(torch, ctxs):
    w = tied(f"tied_lse_{max(ctxs)}", ctxs, 0.95)
    say(f"[{w.name}] contexts {ctxs}: LSE-route discovery and union")
    state = harness.SupportState(w.rows, w.heads, w.max_ctx)
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    for depth, union in ((0, False), (1, True)):
        li = synth.layer_inputs(w, depth)
        dev = harness.upload(li, with_stats=True)
        rep = check_lse_call(w, li, dev, ws, state, oracle_lse(w, li), union=union)
        say(f"   depth {depth}: class B {rep.near_tie} mismatches {rep.support_mismatch}")
        assert rep.support_mismatch == 0
