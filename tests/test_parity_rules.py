"""The GPU-vs-oracle support comparison itself, on the CPU: which differing
supports it excuses (a moved cut at a running sum within 1e-6 of eta, a
swap of tied boundary blocks) and which it rejects (anything else)."""

import numpy as np
import pytest

from oracle import wise_oracle as O
from parity import Report, check_unit_support


def words(blocks, n=2):
    return O.blocks_to_bits(blocks, n)


def run(p, eta, got_blocks, old=None, union=False):
    sel = O.eta_select(np.asarray(p, float), eta)
    old = np.zeros(2, np.uint32) if old is None else old
    want = (old | words(sel.blocks)) if union else words(sel.blocks)
    got = (old | words(got_blocks)) if union else words(got_blocks)
    rep = Report()
    shift = check_unit_support(got, want, sel, eta, len(p), old, union, rep, "unit")
    return sel, rep, shift


def test_exact_match_counts_nothing():
    p = [0.5, 0.3, 0.15, 0.05]
    sel, rep, shift = run(p, 0.9, [0, 1, 2])
    assert (rep.support_mismatch, shift) == (0, 0)


def test_far_from_eta_any_difference_fails():
    p = [0.5, 0.3, 0.15, 0.05]                      # c = 0.5, 0.8, 0.95, 1.0; eta 0.9
    for got in ([0, 1], [0, 1, 2, 3], [0, 1, 3], [1, 2, 3]):
        with pytest.raises(AssertionError):
            run(p, 0.9, got)


def test_moved_cut_excused_only_on_its_side():
    p = [0.5, 0.3, 0.15, 0.05]                      # c_2 = 0.8 is 2e-7 below eta
    eta = 0.8 + 2e-7
    sel = O.eta_select(np.array(p), eta)
    assert sel.K == 3
    _, rep, shift = run(p, eta, [0, 1])             # stopped one block early: excused
    assert (rep.excused_a, shift) == (1, -1)
    with pytest.raises(AssertionError):            # one block late is not this unit's ambiguity
        run(p, eta, [0, 1, 2, 3])
    eta = 0.95 - 3e-7                               # c_3 = 0.95 is 3e-7 above eta
    _, rep, shift = run(p, eta, [0, 1, 2, 3])
    assert (rep.excused_a, shift) == (1, 1)
    with pytest.raises(AssertionError):
        run(p, eta, [0, 1])


def test_tied_swap_excused_only_when_tied():
    tied = [0.4, 0.3, 0.1, 0.1 * (1 - 5e-7), 0.1 * (1 + 5e-7) - 0.0]
    tied = list(np.array(tied) / np.sum(tied))
    sel = O.eta_select(np.array(tied), 0.8)
    assert sel.K == 3 and sel.near_tie()
    k3, k4 = int(sel.order[2]), int(sel.order[3])
    _, rep, shift = run(tied, 0.8, sorted([int(sel.order[0]), int(sel.order[1]), k4]))
    assert (rep.excused_b, shift) == (1, 0)
    with pytest.raises(AssertionError):            # swapping in the fifth block is not the tie
        run(tied, 0.8, sorted([int(sel.order[0]), int(sel.order[1]), int(sel.order[4])]))
    clear = [0.4, 0.3, 0.15, 0.1, 0.05]             # no tie: the same swap fails
    sel = O.eta_select(np.array(clear), 0.8)
    with pytest.raises(AssertionError):
        run(clear, 0.8, sorted([int(sel.order[0]), int(sel.order[1]), int(sel.order[3])]))


def test_equal_masses_have_no_exemption_beyond_the_boundary_pair():
    nb = 20
    p = [1.0 / nb] * nb
    sel = O.eta_select(np.array(p), 0.93)           # K = 19, blocks 0..18 by index
    assert sel.blocks.tolist() == list(range(19))
    # the index-descending tie-break picks blocks 1..19: a difference of the
    # boundary pair (18 <-> 19) only if it were block 18 alone; here block 0 is
    # swapped out, which no class excuses
    with pytest.raises(AssertionError):
        run(p, 0.93, list(range(1, 20)))


def test_union_difference_measured_against_old_bits():
    p = [0.5, 0.3, 0.15, 0.05]
    eta = 0.8 + 2e-7
    old = words([3])
    _, rep, shift = run(p, eta, [0, 1], old=old, union=True)
    assert (rep.excused_a, shift) == (1, -1)
    old = words([2])                                # the dropped block was already set
    _, rep, shift = run(p, eta, [0, 1], old=old, union=True)
    assert rep.support_mismatch == 0 and shift == 0


def test_parallel_oracle_equals_one_call():
    """The worker-process oracle of the full-size tests (inputs regenerated
    per worker from the seeded generator, rows merged) gives what one
    in-process call over the same rows gives, bit for bit."""
    import dataclasses
    from block_sparse_paged_split_amd import synth
    from parity import run_call_parallel
    w = dataclasses.replace(synth.WORKLOADS["ctx1k"], rows=6, heads=2, ctx=None,
                            ctx_list=(1024, 40, 700, 1024, 300, 999), name="par6")
    li = synth.layer_inputs(w, 0)
    words = 1
    sup = np.zeros((w.rows, 1, w.heads, words), np.uint32)
    tags = np.zeros((w.rows, 1), O.TAG_DTYPE)
    modes = np.array([1, 1, 0, 1, 1, 1])
    kw = dict(support=sup, tags=tags, layer=0, slot_of_row=None, row_request=np.arange(6) + 1000,
              row_position=np.zeros(6, np.int64), required=1, eta=0.95)
    rows = [0, 1, 2, 4, 5]
    one = O.run_call(q=li.q, k_cache=li.k, v_cache=li.v, block_table=li.block_table, ctx_len=li.ctx_len,
                     page_size=w.page_size, num_pages=li.num_pages, max_ctx=w.max_ctx, modes=modes,
                     rows=rows, **kw)
    par = run_call_parallel(w, 0, 0, modes, rows, kw)
    np.testing.assert_array_equal(one.out, par.out)
    np.testing.assert_array_equal(one.support, par.support)
    np.testing.assert_array_equal(one.tags, par.tags)
    np.testing.assert_array_equal(one.counters, par.counters)
    np.testing.assert_array_equal(one.effective, par.effective)
    assert sorted(one.units) == sorted(par.units)
    for k in one.units:
        assert one.units[k].selection is None or \
            one.units[k].selection.blocks.tolist() == par.units[k].selection.blocks.tolist()
