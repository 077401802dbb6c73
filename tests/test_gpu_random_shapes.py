"""Seeded random sweep of small shapes on the GPU, each call against the fp64
oracle: rows, heads, head size, dtype, page size, ragged contexts, planted
blocks, eta, a slot pool larger than the batch, and a final launch of random
per-row modes.  The dedicated tests pin one feature each; this sweep looks
for interactions between them.

Every case prints its parameters before touching the GPU, so a failure names
its case.
"""

import numpy as np
import pytest

from block_sparse_paged_split_amd import harness, synth
from block_sparse_paged_split_amd import wise as W
from parity import check_call

pytestmark = pytest.mark.gpu

CASES = 16


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    W.lib()
    return t


def draw_case(seed: int):
    """Shape and schedule of sweep case `seed` (host-side only)."""
    rng = np.random.default_rng(1000 + seed)
    heads = int(rng.choice([1, 2, 3, 4, 8, 16, 20]))
    rows = int(rng.integers(1, 25))
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "f32"]))
    page = int(rng.choice([8, 16, 32, 64, 128]))
    # contexts log-uniform over 1..6000, within a budget of tokens x heads
    budget = 300_000
    ctx = np.exp(rng.uniform(0.0, np.log(6000.0), size=rows)).round().astype(int).clip(1, 6000)
    while int(ctx.sum()) * heads > budget and rows > 1:
        rows -= 1
        ctx = ctx[:rows]
    while int(ctx.sum()) * heads > budget:
        ctx = (ctx // 2).clip(1)
    eta = float(rng.choice([0.5, 0.8, 0.9, 0.95, 0.99, 1.0]))
    w = synth.Workload(name=f"sweep{seed}", rows=rows, heads=heads, head_dim=d, dtype=dtype, page_size=page,
                       shuffle=bool(rng.integers(0, 2)), alpha=float(rng.uniform(2.0, 8.0)), seed=500 + seed,
                       ctx_list=tuple(int(c) for c in ctx), hot=int(rng.integers(1, 7)),
                       schedule=(W.WISE_DISCOVER, W.WISE_DISCOVER_UNION, W.WISE_SPARSE), eta=eta)
    slots = rows + int(rng.integers(0, 9))
    slot_of_row = rng.permutation(slots)[:rows].astype(np.int32)
    mixed = rng.choice([W.WISE_DENSE, W.WISE_DISCOVER, W.WISE_DISCOVER_UNION, W.WISE_SPARSE],
                       size=rows).astype(np.uint8)
    return w, slots, slot_of_row, mixed


@pytest.mark.parametrize("seed", range(CASES))
def test_random_shape_schedule(torch, seed):
    w, slots, slot_of_row, mixed = draw_case(seed)
    say(f"[{w.name}] rows {w.rows} heads {w.heads} d {w.head_dim} {w.dtype} P {w.page_size} "
        f"shuffle {w.shuffle} ctx {w.ctx_list} hot {w.hot} alpha {w.alpha:.2f} eta {w.eta} "
        f"slots {slots} slot_of_row {slot_of_row.tolist()} mixed {mixed.tolist()}")
    st = harness.SupportState(w.rows, w.heads, w.max_ctx, slots=slots)
    st.slot_of_row = torch.from_numpy(slot_of_row).cuda()
    st.row_position.fill_(11)
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    for depth, mode in enumerate(w.schedule):
        say(f"   depth {depth} mode {mode}")
        li = synth.layer_inputs(w, depth)
        dev = harness.upload(li, with_stats=True)
        rep = check_call(w, li, dev, ws, st, mode=mode, required=2)
        say(f"   max_abs {rep.max_abs:.2e} near_eta {rep.near_eta} near_tie {rep.near_tie} counters {rep.counters}")
        assert rep.counters[W.CTR_ERRORS] == 0
    # one launch of random per-row modes over the same state (a fourth depth)
    say(f"   mixed launch {mixed.tolist()}")
    li = synth.layer_inputs(w, 3)
    dev = harness.upload(li, with_stats=True)
    rep = check_call(w, li, dev, ws, st, mode=W.WISE_SPARSE, row_modes=mixed, required=2)
    say(f"   max_abs {rep.max_abs:.2e} counters {rep.counters}")
    assert rep.counters[W.CTR_ERRORS] == 0
