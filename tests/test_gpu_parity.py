"""HIP path vs the fp64 oracle, through the C ABI, on the GPU.

Every test prints what it runs before touching the GPU, so a failure names
its case.
"""

import dataclasses

import numpy as np
import pytest

from block_sparse_paged_split_amd import harness, synth
from block_sparse_paged_split_amd import wise as W
from oracle import wise_oracle as O
from parity import check_call

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    W.lib()  # fails loudly if libwise.so is missing
    return t


def run_schedule(w, rows=None, layer=0, eta=None, required=None, with_stats=True, pool=False):
    """All depths of w.schedule for one layer, each checked against the oracle
    (in worker processes with ``pool``)."""
    state = harness.SupportState(w.rows, w.heads, w.max_ctx, layers=max(w.layers, layer + 1))
    state.row_position.fill_(17)
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    reps = []
    for depth, mode in enumerate(w.schedule):
        say(f"[{w.name}] depth {depth} mode {mode} layer {layer} rows {'all' if rows is None else len(rows)}")
        li = synth.layer_inputs(w, depth, layer)
        dev = harness.upload(li, with_stats=with_stats)
        reps.append(check_call(w, li, dev, ws, state, mode=mode, layer=layer, rows=rows,
                               eta=eta, required=required, pool=pool))
        say(f"   max_abs {reps[-1].max_abs:.2e} near_eta {reps[-1].near_eta} "
            f"near_tie {reps[-1].near_tie} counters {reps[-1].counters}")
    return reps, state


def test_tiny_f32_schedule(torch):
    reps, state = run_schedule(synth.WORKLOADS["tiny_f32"])
    assert reps[0].counters[W.CTR_CAUSAL] == 4 * 8
    assert all(r.counters[W.CTR_FALLBACKS] == 0 for r in reps)


def test_ctx1k_schedule(torch):
    reps, state = run_schedule(synth.WORKLOADS["ctx1k"])
    ctr = state.counters.cpu().numpy()
    assert ctr[W.CTR_FALLBACKS] == 0 and ctr[W.CTR_ERRORS] == 0
    assert ctr[W.CTR_CAUSAL] == 32 * 16 * 32
    say(f"   union density {ctr[W.CTR_SELECTED] / ctr[W.CTR_CAUSAL]:.4f}")


def test_match1k_schedule(torch):
    """Density-matched supplement: supports far from dense."""
    reps, state = run_schedule(synth.WORKLOADS["match1k"])
    ctr = state.counters.cpu().numpy()
    dens = ctr[W.CTR_SELECTED] / ctr[W.CTR_CAUSAL]
    say(f"   union density {dens:.4f}")
    assert dens < 0.6


# ----------------------------------------------------------------------------- bitwise invariants

def _one_layer(w, depth=0):
    li = synth.layer_inputs(w, depth)
    return li, harness.upload(li, with_stats=True)


@pytest.mark.parametrize("ctx,rows", [(1024, 32), (4096, 8)])
def test_modes_agree_bitwise(torch, ctx, rows):
    """discover output == dense output; sparse with every block == dense;
    reruns are bitwise identical.  At 4K the sparse call runs the planned
    (listed) split and the dense call the static one."""
    w = dataclasses.replace(synth.WORKLOADS["ctx1k"], ctx=ctx, rows=rows, name=f"modes{ctx}")
    say(f"[{w.name}] dense / discover / all-blocks sparse, bitwise")
    li, dev = _one_layer(w)
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    harness.call(dev, ws, W.WISE_DENSE)
    torch.cuda.synchronize()
    dense = dev.out.clone()
    state = harness.SupportState(w.rows, w.heads, w.max_ctx)
    harness.call(dev, ws, W.WISE_DISCOVER, state, required=1)
    torch.cuda.synchronize()
    assert torch.equal(dev.out, dense)
    sup = state.support.clone()
    for _ in range(4):
        harness.call(dev, ws, W.WISE_DISCOVER, state, required=1)
        torch.cuda.synchronize()
        assert torch.equal(dev.out, dense)
        assert torch.equal(state.support, sup)
    state.support.fill_(-1)  # every bit set
    harness.call(dev, ws, W.WISE_SPARSE, state, required=1)
    torch.cuda.synchronize()
    assert torch.equal(dev.out, dense)
    assert state.counters[W.CTR_FALLBACKS].item() == 0


@pytest.mark.parametrize("ctx", [1024, 4096])
def test_mixed_launch_equals_uniform(torch, ctx):
    w = dataclasses.replace(synth.WORKLOADS["ctx1k"], rows=16, ctx=ctx, name=f"mixed16_{ctx}")
    say(f"[{w.name}] one mixed launch vs uniform launches")
    li0, dev0 = _one_layer(w, 0)
    li1, dev1 = _one_layer(w, 1)
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    # reference state: every row discovered at depth 0 (for the union and sparse rows)
    base = harness.SupportState(w.rows, w.heads, w.max_ctx)
    harness.call(dev0, ws, W.WISE_DISCOVER, base, required=1)
    modes = np.array([0, 1, 2, 3] * 4, dtype=np.uint8)
    outs = {}
    states = {}
    for m in range(4):
        st = harness.SupportState(w.rows, w.heads, w.max_ctx)
        st.support.copy_(base.support)
        st.tags.copy_(base.tags)
        harness.call(dev1, ws, m, st if m else None, required=1)
        torch.cuda.synchronize()
        outs[m] = dev1.out.clone()
        states[m] = st
    st = harness.SupportState(w.rows, w.heads, w.max_ctx)
    st.support.copy_(base.support)
    st.tags.copy_(base.tags)
    harness.call(dev1, ws, W.WISE_SPARSE, st, required=1,
                 row_mode=torch.from_numpy(modes).cuda())
    torch.cuda.synchronize()
    for r in range(w.rows):
        m = int(modes[r])
        assert torch.equal(dev1.out[r], outs[m][r]), f"row {r} mode {m}"
        if m:
            assert torch.equal(st.support[r], states[m].support[r])
            assert torch.equal(st.tags[r], states[m].tags[r])


# ----------------------------------------------------------------------------- ragged and layouts

RAGGED = (1, 2, 31, 32, 33, 63, 64, 65, 100, 257, 1000, 2900)  # 2900: units span several split groups


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
@pytest.mark.parametrize("P", [8, 16, 32, 64])
def test_ragged_contexts(torch, dtype, d, P):
    w = synth.Workload(name=f"ragged_{dtype}{d}_P{P}", rows=len(RAGGED), heads=3, head_dim=d,
                       dtype=dtype, page_size=P, shuffle=True, alpha=6.0, seed=21,
                       ctx_list=RAGGED, hot=3, schedule=(1, 2, 3), eta=0.9)
    run_schedule(w)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
@pytest.mark.parametrize("ctxs", [(1, 31, 33, 100, 257, 1000, 2048), (5, 40, 256)])
def test_small_launches(torch, dtype, d, ctxs):
    """Launches with few work items cut them to 1-4 tiles, and units of up
    to 16 items finish inside the split kernel (8 for fp32 at d 128)."""
    w = synth.Workload(name=f"small_{dtype}{d}_{len(ctxs)}", rows=len(ctxs), heads=3, head_dim=d,
                       dtype=dtype, page_size=16, shuffle=True, alpha=6.0, seed=71, ctx_list=ctxs, hot=2,
                       schedule=(1, 2, 3), eta=0.9)
    run_schedule(w)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f32", 128)])
def test_maximum_context(torch, dtype, d):
    """The longest supported context, 65536 tokens (2048 blocks: 64 support
    words, one per lane of a plan or split wave, and the finish's widest
    sort), beside a shorter row, through discover, union and sparse depths."""
    w = synth.Workload(name=f"maxctx_{dtype}{d}", rows=2, heads=4, head_dim=d, dtype=dtype, page_size=16,
                       shuffle=True, alpha=6.0, seed=101, ctx_list=(65536, 40001), hot=5,
                       schedule=(1, 2, 3), eta=0.9)
    assert w.max_ctx == 65536
    reps, state = run_schedule(w)
    assert all(r.counters[W.CTR_FALLBACKS] == 0 and r.counters[W.CTR_ERRORS] == 0 for r in reps)


@pytest.mark.parametrize("heads,ctxs", [(1, (200, 1000)), (20, (300, 1024)), (20, (700, 3000)),
                                        (255, (300, 2100)), (256, (64, 128))])
def test_head_counts(torch, heads, ctxs):
    """One head; 20 heads (a fused row of more than 16 heads at 1K and at
    3K); 255 heads (the most the fused kernel's 8-bit arrival count holds,
    long units); 256 heads (beyond it, so the two-kernel path)."""
    w = synth.Workload(name=f"heads{heads}_{max(ctxs)}", rows=len(ctxs), heads=heads, head_dim=64,
                       dtype="bf16", page_size=16, shuffle=True, alpha=6.0, seed=81, ctx_list=ctxs, hot=2,
                       schedule=(1, 2, 3), eta=0.9)
    run_schedule(w)


@pytest.mark.parametrize("max_ctx", [8192, 8224])
def test_fused_regime_boundary(torch, max_ctx):
    """The longest context the one-launch kernel takes (8192 tokens, 256
    blocks) and the first it does not (257 blocks: the static and listed
    grids with the finish kernel): rows of 8000 and 4500 tokens beside one
    of max_ctx, through discover, union and sparse depths, each against the
    oracle."""
    w = synth.Workload(name=f"boundary{max_ctx}", rows=3, heads=4, head_dim=128, dtype="bf16", page_size=16,
                       shuffle=True, alpha=5.0, seed=101, ctx_list=(max_ctx, 8000, 4500), hot=6,
                       schedule=(W.WISE_DISCOVER, W.WISE_DISCOVER_UNION, W.WISE_SPARSE))
    reps, _ = run_schedule(w)
    assert all(r.counters[W.CTR_FALLBACKS] == 0 and r.counters[W.CTR_ERRORS] == 0 for r in reps)


@pytest.mark.parametrize("rows,heads,tiles,dtype,d", [(8, 16, 16, "bf16", 128), (16, 16, 32, "bf16", 128),
                                                   (8, 16, 16, "f32", 64)])
def test_long_items(torch, rows, heads, tiles, dtype, d):
    """Calls with no sparse rows whose units outgrow the fused kernel (16K
    tokens) and whose launch stays large run 16- or 32-tile items on the
    static grid (a quarter or half of the partials); every row of every
    depth -- dense, discover, union, and the sparse depth on the listed grid
    -- against the oracle.  The same dense rows in a call with a per-row mode
    array (the listed grid, whose plan kernel picks the item length from the
    same tiles) are bitwise the dense call's."""
    w = synth.Workload(name=f"long{tiles}_{rows}x{heads}_{dtype}{d}", rows=rows, heads=heads, head_dim=d, dtype=dtype,
                       page_size=16, shuffle=True, alpha=2.5, seed=93, ctx=16384, hot=6,
                       schedule=(W.WISE_DENSE, W.WISE_DISCOVER, W.WISE_DISCOVER_UNION, W.WISE_SPARSE))
    units, nb = rows * heads, 16384 // 32
    assert units * (nb // tiles) >= 4096 and (tiles == 32 or units * (nb // 32) < 4096)
    reps, state = run_schedule(w, pool=True)
    assert all(r.counters[W.CTR_FALLBACKS] == 0 and r.counters[W.CTR_ERRORS] == 0 for r in reps)
    li, dev = _one_layer(w, 0)
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    harness.call(dev, ws, W.WISE_DENSE)
    torch.cuda.synchronize()
    long_out = dev.out.clone()
    st = harness.SupportState(w.rows, w.heads, w.max_ctx)
    harness.call(dev, ws, W.WISE_SPARSE, st, required=1,
                 row_mode=torch.full((w.rows,), W.WISE_DENSE, dtype=torch.uint8, device=dev.out.device))
    torch.cuda.synchronize()
    assert torch.equal(dev.out, long_out)


@pytest.mark.parametrize("rows,heads,ctx,tiles", [(32, 16, 16384, 32), (12, 16, 16384, 16), (2, 16, 16384, 8)])
def test_listed_long_items(torch, rows, heads, ctx, tiles):
    """Calls whose units outgrow the fused kernel (16K tokens) and that have
    sparse rows take their item length in the plan kernel from
    the tiles they attend, by the rule dense calls take on the host: 32 tiles
    when the launch keeps at least 4096 items of 32, else 16 on that
    condition, else 8.  With every block selected the attended tiles are the
    causal ones, so an all-blocks sparse call and a mixed call of dense and
    all-blocks sparse rows are bitwise the dense call; over the supports of a
    discovery depth (near dense) every row of a sparse and of a mixed call
    matches the oracle."""
    units, nb = rows * heads, ctx // 32
    assert tiles == (32 if units * (nb // 32) >= 4096 else 16 if units * (nb // 16) >= 4096 else 8)
    w = dataclasses.replace(synth.WORKLOADS["ctx1k"], rows=rows, heads=heads, ctx=ctx,
                            name=f"listed_long{tiles}_{rows}x{ctx}")
    say(f"[{w.name}] dense vs all-blocks sparse and mixed calls; sparse and mixed vs the oracle")
    li0, dev0 = _one_layer(w, 0)
    li2, dev2 = _one_layer(w, 2)
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    harness.call(dev2, ws, W.WISE_DENSE)
    torch.cuda.synchronize()
    dense = dev2.out.clone()
    st = harness.SupportState(w.rows, w.heads, w.max_ctx)
    harness.call(dev0, ws, W.WISE_DISCOVER, st, required=1)
    torch.cuda.synchronize()
    discovered = st.support.clone()
    st.support.fill_(-1)  # every bit set
    harness.call(dev2, ws, W.WISE_SPARSE, st, required=1)
    torch.cuda.synchronize()
    assert torch.equal(dev2.out, dense)
    modes = np.array([W.WISE_DENSE, W.WISE_SPARSE] * (rows // 2), dtype=np.uint8)
    harness.call(dev2, ws, W.WISE_SPARSE, st, required=1, row_mode=torch.from_numpy(modes).cuda())
    torch.cuda.synchronize()
    assert torch.equal(dev2.out, dense)
    assert int(st.counters[W.CTR_FALLBACKS].item()) == 0
    st.support.copy_(discovered)
    for row_modes in (None, modes):
        rep = check_call(w, li2, dev2, ws, st, mode=W.WISE_SPARSE, row_modes=row_modes, required=1, pool=True)
        say(f"   {'mixed' if row_modes is not None else 'sparse'}: max_abs {rep.max_abs:.2e}")


def test_plan_many_units(torch):
    """More than 4096 units (rows of 256 heads, more than the fused kernel's
    8-bit arrival count holds, take the plan kernel): the plan kernel's
    threads take five units each, the fifth keeping its tile count in the
    workspace between the passes (the first four stay in registers).
    Discovery, then a sparse and a mixed call (full-length items listed
    before the short last ones); every row against the oracle, counters
    exact."""
    w = synth.Workload(name="plan_many_units", rows=17, heads=256, head_dim=64, dtype="bf16", page_size=16,
                       shuffle=True, alpha=4.0, seed=97, ctx=1100, hot=6, schedule=(W.WISE_DISCOVER,))
    assert w.rows * w.heads > 4 * 1024
    say(f"[{w.name}] {w.rows * w.heads} units: discover, sparse, mixed")
    li0, dev0 = _one_layer(w, 0)
    li1, dev1 = _one_layer(w, 1)
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    st = harness.SupportState(w.rows, w.heads, w.max_ctx)
    rep = check_call(w, li0, dev0, ws, st, mode=W.WISE_DISCOVER, required=1, pool=True)
    say(f"   discover: max_abs {rep.max_abs:.2e} near_eta {rep.near_eta}")
    # every plan thread's units 5t .. 5t + 4 span several rows
    rep = check_call(w, li1, dev1, ws, st, mode=W.WISE_SPARSE, required=1, pool=True)
    say(f"   sparse: max_abs {rep.max_abs:.2e}")
    modes = np.array(([W.WISE_SPARSE, W.WISE_DENSE, W.WISE_SPARSE, W.WISE_DISCOVER_UNION] * w.rows)[:w.rows],
                     dtype=np.uint8)
    ctr0 = st.counters.cpu().numpy().copy()
    rep = check_call(w, li1, dev1, ws, st, mode=W.WISE_SPARSE, row_modes=modes, required=1, pool=True)
    say(f"   mixed: max_abs {rep.max_abs:.2e}")
    ctr = st.counters.cpu().numpy() - ctr0
    assert ctr[W.CTR_FALLBACKS] == 0 and ctr[W.CTR_ERRORS] == 0


def test_page_size_and_layout_invariance(torch):
    """Physical layout changes nothing: same bits for page sizes 8..4096 (from
    512 on every row sits in one page; 4096 is the largest supported), a
    shuffled or identity block table, and [pages, P, H, d] storage."""
    base = synth.Workload(name="layout", rows=6, heads=4, head_dim=128, dtype="bf16", page_size=8,
                          shuffle=True, alpha=4.0, seed=5, ctx_list=(5, 40, 64, 129, 300, 511),
                          hot=2, schedule=(1,))
    outs = []
    for P in (8, 16, 32, 64, 128, 512, 4096):
        for shuffle in (True, False):
            w = dataclasses.replace(base, page_size=P, shuffle=shuffle)
            say(f"[layout] P={P} shuffle={shuffle}")
            li = synth.layer_inputs(w, 0)
            dev = harness.upload(li)
            ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
            harness.call(dev, ws, W.WISE_DENSE)
            torch.cuda.synchronize()
            outs.append(dev.out.clone())
            # token-major storage [pages, P, H, d], viewed as [pages, H, P, d]
            dev.k = dev.k.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
            dev.v = dev.v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
            harness.call(dev, ws, W.WISE_DENSE)
            torch.cuda.synchronize()
            outs.append(dev.out.clone())
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


# ----------------------------------------------------------------------------- fallback and errors

def test_fallback_transitions(torch):
    w = dataclasses.replace(synth.WORKLOADS["ctx1k"], rows=8, name="fallback8")
    say("[fallback8] broken window, release, stale position, other request")
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    li0, dev0 = _one_layer(w, 0)
    li1, dev1 = _one_layer(w, 1)
    li2, dev2 = _one_layer(w, 2)
    st = harness.SupportState(w.rows, w.heads, w.max_ctx)
    st.row_position.fill_(5)
    check_call(w, li0, dev0, ws, st, mode=W.WISE_DISCOVER)
    # rows 1, 2: position moves on before the union depth (broken window)
    st.row_position[1] = 6
    st.row_position[2] = 6
    rep = check_call(w, li1, dev1, ws, st, mode=W.WISE_DISCOVER_UNION)
    assert rep.counters[W.CTR_FALLBACKS] == 2
    st.row_position[1] = 5
    st.row_position[2] = 5
    # row 3 released, row 4 stale, row 5 another request; rows 1, 2 broken above
    tags = st.tags.clone()
    tags[3, 0, 2] = 0
    tags[4, 0, 1] = 4
    tags[5, 0, 0] = 77
    st.tags.copy_(tags)
    rep = check_call(w, li2, dev2, ws, st, mode=W.WISE_SPARSE)
    assert rep.counters[W.CTR_FALLBACKS] == 5
    # incomplete window: only one discovery depth recorded of two
    st2 = harness.SupportState(w.rows, w.heads, w.max_ctx)
    check_call(w, li0, dev0, ws, st2, mode=W.WISE_DISCOVER)
    rep = check_call(w, li2, dev2, ws, st2, mode=W.WISE_SPARSE, required=2)
    assert rep.counters[W.CTR_FALLBACKS] == w.rows


def test_device_data_errors(torch):
    w = synth.Workload(name="errors", rows=6, heads=2, head_dim=128, dtype="bf16", page_size=16,
                       shuffle=True, alpha=6.0, seed=8, ctx_list=(64, 64, 64, 64, 64, 64), hot=1,
                       schedule=(1,), eta=0.9)
    say("[errors] bad ctx, bad page, bad mode, bad slot, empty support")
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    li = synth.layer_inputs(w, 0)
    st = harness.SupportState(w.rows, w.heads, w.max_ctx, slots=8)
    dev = harness.upload(li)
    check_call(w, li, dev, ws, st, mode=W.WISE_DISCOVER, required=1)
    li.ctx_len = li.ctx_len.copy()
    li.ctx_len[0] = 0                  # context outside [1, max_ctx]
    li.block_table = li.block_table.copy()
    li.block_table[1, 2] = li.num_pages + 5   # page id out of range, inside the context
    dev = harness.upload(li)
    modes = np.array([3, 3, 9, 3, 3, 3], np.uint8)   # row 2: invalid mode
    st.slot_of_row = torch.tensor([0, 1, 2, 3, 99, 5], dtype=torch.int32, device="cuda")  # row 4: bad slot
    sup = st.support.clone()
    sup[5, 0, 1] = 0                   # row 5 head 1: empty support
    st.support.copy_(sup)
    rep = check_call(w, li, dev, ws, st, mode=W.WISE_SPARSE, row_modes=modes, required=1)
    say(f"   counters {rep.counters}")
    out = dev.out.cpu().numpy()
    assert np.isnan(out[[0, 2, 4]]).all() and np.isnan(out[5, 1]).all()
    assert not np.isnan(out[3]).any() and not np.isnan(out[5, 0]).any()
    # row 1's bad page sits in block 1: NaN only for heads whose support holds it


@pytest.mark.parametrize("ctx", [1000, 3000])
def test_slot_indirection(torch, ctx):
    """Rows mapped to slots of a larger pool through slot_of_row (the state
    of each slot read after that one load): a full discover, union, sparse
    schedule against the oracle, fused (1K) and static + listed (3K) shapes;
    slots no row maps to keep their contents."""
    w = synth.Workload(name=f"slots_{ctx}", rows=6, heads=4, head_dim=128, dtype="bf16", page_size=16,
                       shuffle=True, alpha=4.0, seed=97, ctx=ctx, hot=3,
                       schedule=(W.WISE_DISCOVER, W.WISE_DISCOVER_UNION, W.WISE_SPARSE))
    st = harness.SupportState(w.rows, w.heads, w.max_ctx, slots=16)
    st.slot_of_row = torch.tensor([9, 3, 14, 0, 7, 12], dtype=torch.int32, device="cuda")
    st.row_position.fill_(23)
    st.support.fill_(0x5A5A5A5A)  # every slot starts with foreign bits
    free = [sl for sl in range(16) if sl not in (9, 3, 14, 0, 7, 12)]
    before = st.support[free].clone()
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    for depth, mode in enumerate(w.schedule):
        say(f"[{w.name}] depth {depth} mode {mode} through slot_of_row")
        li = synth.layer_inputs(w, depth)
        dev = harness.upload(li, with_stats=True)
        rep = check_call(w, li, dev, ws, st, mode=mode)
        say(f"   max_abs {rep.max_abs:.2e} counters {rep.counters}")
        assert rep.counters[W.CTR_FALLBACKS] == 0 and rep.counters[W.CTR_ERRORS] == 0
    assert torch.equal(st.support[free], before)


def test_graph_replay_matches_eager(torch):
    """A whole step captured in a HIP graph: every replay (with eager work and
    synchronisation in between) equals the eager step bit for bit."""
    w = dataclasses.replace(synth.WORKLOADS["ctx1k"], rows=8, name="graph8")
    say("[graph8] capture one step (4 depths), replay x3")
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    st = harness.SupportState(w.rows, w.heads, w.max_ctx)
    devs = [harness.upload(synth.layer_inputs(w, d)) for d in range(len(w.schedule))]
    calls = [harness.PreparedCall(devs[d], ws, m, st, required=w.discoveries, eta=w.eta)
             for d, m in enumerate(w.schedule)]

    def step(stream):
        for c in calls:
            c.run(stream)

    step(harness.stream_handle())
    torch.cuda.synchronize()
    ref_out = [d.out.clone() for d in devs]
    ref_sup, ref_tags = st.support.clone(), st.tags.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(int(torch.cuda.current_stream().cuda_stream))
    for it in range(3):
        for d in devs:
            d.out.fill_(float("nan"))
        st.support.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for d, r in zip(devs, ref_out):
            assert torch.equal(d.out, r), f"replay {it}"
        assert torch.equal(st.support, ref_sup) and torch.equal(st.tags, ref_tags)


def test_graph_replay_mixed_planned_launch(torch):
    """A mixed launch that takes the planned path (plan kernel + persistent
    split over the compact item list) replays from a HIP graph bit for bit."""
    w = dataclasses.replace(synth.WORKLOADS["ctx1k"], rows=8, ctx=4096, name="graph_mixed4k")
    say("[graph_mixed4k] capture discover + mixed launch, replay x3")
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    st = harness.SupportState(w.rows, w.heads, w.max_ctx)
    d0 = harness.upload(synth.layer_inputs(w, 0))
    d1 = harness.upload(synth.layer_inputs(w, 1))
    modes = torch.tensor([0, 1, 2, 3, 3, 3, 2, 1], dtype=torch.uint8, device="cuda")
    calls = [harness.PreparedCall(d0, ws, W.WISE_DISCOVER, st, required=1),
             harness.PreparedCall(d1, ws, W.WISE_SPARSE, st, required=1, row_mode=modes)]

    def step(stream):
        for c in calls:
            c.run(stream)

    step(harness.stream_handle())
    torch.cuda.synchronize()
    ref = (d0.out.clone(), d1.out.clone(), st.support.clone(), st.tags.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(int(torch.cuda.current_stream().cuda_stream))
    for it in range(3):
        d0.out.fill_(float("nan"))
        d1.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (d0.out, d1.out, st.support, st.tags)
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {it}"


def test_graph_replay_adapts_item_length(torch):
    """One captured sparse call whose plan kernel picks the item length from
    the support it finds on the device: replays over a full support (32-tile
    items) and over a sparse one (eight-tile items), alternating, each equal
    bit for bit to the same call run eagerly on the same state."""
    w = dataclasses.replace(synth.WORKLOADS["ctx1k"], rows=64, heads=16, head_dim=64, ctx=4096,
                            name="graph_item_length")
    say(f"[{w.name}] capture one sparse call; replay over full and sparse supports")
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    st = harness.SupportState(w.rows, w.heads, w.max_ctx)
    dev = harness.upload(synth.layer_inputs(w, 2))
    st.tags[:, :, 0] = st.row_request[:, None]
    st.tags[:, :, 1] = st.row_position[:, None]
    st.tags[:, :, 2] = 1
    rng = np.random.default_rng(5)
    nb = w.max_ctx // synth.BLOCK
    sparse_bits = np.zeros((w.rows, 1, w.heads, st.words), np.uint32)
    for r in range(w.rows):
        for h in range(w.heads):
            for b in rng.choice(nb, size=4, replace=False):
                sparse_bits[r, 0, h, b // 32] |= np.uint32(1) << np.uint32(b % 32)
    supports = {"full": torch.full_like(st.support, -1),
                "sparse": torch.from_numpy(sparse_bits.view(np.int32)).to(st.support.device)}
    call = harness.PreparedCall(dev, ws, W.WISE_SPARSE, st, required=1)
    eager = {}
    for name, sup in supports.items():
        st.support.copy_(sup)
        call.run(harness.stream_handle())
        torch.cuda.synchronize()
        eager[name] = dev.out.clone()
    assert not torch.equal(eager["full"], eager["sparse"])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call.run(int(torch.cuda.current_stream().cuda_stream))
    for it, name in enumerate(["sparse", "full", "sparse", "full"]):
        st.support.copy_(supports[name])
        dev.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dev.out, eager[name]), f"replay {it} ({name} support)"
    assert int(st.counters[W.CTR_FALLBACKS].item()) == 0 and int(st.counters[W.CTR_ERRORS].item()) == 0


def _oracle_chain_check(w, lis, devs, st, schedule, row_modes, required):
    """Check the results of one replayed step against the oracle run depth by
    depth from an empty state: outputs of every depth, the support after the
    discovery depths (exact but for the excused classes), tags and counters.
    Reuse depths are evaluated over the support the GPU holds, as in
    ``check_call``."""
    from parity import Report, assert_close, check_unit_support
    R, H = w.rows, w.heads
    words = st.words
    sup = np.zeros((R, 1, H, words), np.uint32)
    tags = np.zeros((R, 1), O.TAG_DTYPE)
    gpu_sup = st.support_numpy()
    rep = Report()
    counters = np.zeros(4, np.int64)
    for depth, (li, dev) in enumerate(zip(lis, devs)):
        modes = row_modes[depth] if row_modes[depth] is not None else np.full(R, schedule[depth])
        reuse = all(int(m) in (W.WISE_SPARSE, W.WISE_DENSE) for m in modes)
        ref = O.run_call(q=li.q, k_cache=li.k, v_cache=li.v, block_table=li.block_table, ctx_len=li.ctx_len,
                         page_size=w.page_size, num_pages=li.num_pages, max_ctx=w.max_ctx, modes=modes,
                         support=gpu_sup if reuse else sup, tags=tags, row_request=st.row_request.cpu().numpy(),
                         row_position=st.row_position.cpu().numpy(), required=required, eta=w.eta)
        out = dev.out.cpu().numpy()
        for r in range(R):
            assert_close(out[r], ref.out[r], w.dtype, f"depth {depth} row {r}", rep)
        if not reuse:
            for r in range(R):
                for h in range(H):
                    u = ref.units.get((r, h))
                    if u is not None and u.selection is not None:
                        rep.units += 1
                        nb = (int(li.ctx_len[r]) + 31) // 32
                        last = all(int(m) in (W.WISE_SPARSE, W.WISE_DENSE)
                                   for m in (row_modes[d][r] if row_modes[d] is not None else schedule[d]
                                             for d in range(depth + 1, len(lis))))
                        if last:   # the GPU's support after this depth is its final one
                            check_unit_support(gpu_sup[r, 0, h], ref.support[r, 0, h], u.selection, w.eta, nb,
                                               sup[r, 0, h], u.effective == O.DISCOVER_UNION, rep,
                                               f"depth {depth} row {r} head {h}")
        sup, tags = ref.support, ref.tags
        counters += ref.counters
    gt = st.tags_numpy()
    for f in ("request", "position", "discoveries"):
        np.testing.assert_array_equal(gt[f], tags[f])
    ctr = st.counters.cpu().numpy()
    assert ctr[W.CTR_FALLBACKS] == counters[0] and ctr[W.CTR_ERRORS] == counters[3]
    assert ctr[W.CTR_CAUSAL] == counters[2]
    if rep.support_mismatch == 0:
        assert ctr[W.CTR_SELECTED] == counters[1]
    return rep


@pytest.mark.parametrize("case", ["ctx1k", "mixed4k"])
def test_graph_replay_matches_oracle(torch, case):
    """A whole step captured in a HIP graph and replayed from an empty support
    state, twice, each replay checked against the oracle's own schedule: the
    ctx1k step (discover, union, sparse, sparse; the fused launch shape) and
    a discovery depth followed by a mixed launch at 4K (the plan kernel, the
    listed split and the finish kernel)."""
    if case == "ctx1k":
        w = synth.WORKLOADS["ctx1k"]
        schedule, row_modes, required = list(w.schedule), [None] * 4, w.discoveries
    else:
        w = dataclasses.replace(synth.WORKLOADS["ctx1k"], rows=8, ctx=4096, name="graph_mixed4k_oracle")
        schedule = [W.WISE_DISCOVER, W.WISE_SPARSE]
        row_modes = [None, np.array([0, 1, 2, 3, 3, 3, 2, 1], np.uint8)]
        required = 1
    say(f"[{w.name}] capture one step, replay x2 from an empty state, each against the oracle")
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    st = harness.SupportState(w.rows, w.heads, w.max_ctx)
    st.row_position.fill_(5)
    lis = [synth.layer_inputs(w, d) for d in range(len(schedule))]
    devs = [harness.upload(li) for li in lis]
    rm_dev = [None if m is None else torch.from_numpy(m).cuda() for m in row_modes]
    calls = [harness.PreparedCall(devs[d], ws, schedule[d], st, required=required, eta=w.eta, row_mode=rm_dev[d])
             for d in range(len(schedule))]

    def step(stream):
        for c in calls:
            c.run(stream)

    step(harness.stream_handle())       # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(int(torch.cuda.current_stream().cuda_stream))
    for it in range(2):
        st.support.zero_()
        st.tags.zero_()
        st.counters.zero_()
        for d in devs:
            d.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        rep = _oracle_chain_check(w, lis, devs, st, schedule, row_modes, required)
        say(f"   replay {it}: max_abs {rep.max_abs:.2e} units {rep.units} class A {rep.near_eta} "
            f"class B {rep.near_tie} mismatches {rep.support_mismatch}")
