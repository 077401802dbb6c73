"""wise_decode_sparse_noalloc -- a whole (depth, layer) call on the library's
own static device workspace, for callers that cannot allocate -- against
the same call made with wise_decode_sparse + wise_finish_select on a caller
workspace: outputs, supports, tags and counters bit for bit, on two
workloads in a row, the second smaller (the static buffer keeps the first
call's contents), through every launch shape (planned mixed launch with its
finish kernel at 4K, the fused kernel at 1K).
"""

import ctypes
import dataclasses

import numpy as np
import pytest

from block_sparse_paged_split_amd import harness, synth
from block_sparse_paged_split_amd import wise as W

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    W.lib()
    return t


def twin_schedule(torch, w, schedule):
    """Run every depth of ``schedule`` (per-row mode arrays) twice from
    identical empty states -- through the no-allocation entry point and
    through the workspace entry points -- and compare after every depth."""
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    assert ws.nbytes <= W.SCRATCH_BYTES
    states = [harness.SupportState(w.rows, w.heads, w.max_ctx) for _ in range(2)]
    for st in states:
        st.row_position.fill_(7)
    for depth, modes in enumerate(schedule):
        say(f"[{w.name}] depth {depth} modes {np.bincount(modes, minlength=4).tolist()}")
        dev = harness.upload(synth.layer_inputs(w, depth))
        rm = torch.from_numpy(modes.astype(np.uint8)).cuda()
        outs = []
        for k, st in enumerate(states):
            dev.out.fill_(float("nan"))
            a = dev.attn()
            s = st.view(0, 1, w.eta)
            stream = harness.stream_handle()
            if k == 0:
                W.wise_decode_sparse_noalloc(a, s, int(rm.data_ptr()), stream)
            else:
                W.wise_decode_sparse(a, s, int(rm.data_ptr()), ws.ptr, ws.nbytes, stream)
                W.wise_finish_select(a, s, ws.ptr, ws.nbytes, stream)
            torch.cuda.synchronize()
            outs.append(dev.out.clone())
        assert torch.equal(outs[0], outs[1]), f"depth {depth}: outputs differ"
        assert not torch.isnan(outs[0]).any()
        assert torch.equal(states[0].support, states[1].support), f"depth {depth}: supports differ"
        assert torch.equal(states[0].tags, states[1].tags), f"depth {depth}: tags differ"
        assert torch.equal(states[0].counters, states[1].counters), f"depth {depth}: counters differ"
    return states[0]


def test_noalloc_matches_workspace_calls_larger_then_smaller(torch):
    big = dataclasses.replace(synth.WORKLOADS["ctx1k"], rows=16, ctx=4096, name="noalloc4k")
    R = big.rows
    disc = np.full(R, W.WISE_DISCOVER, np.uint8)
    mixed = np.array([W.WISE_DENSE, W.WISE_DISCOVER, W.WISE_DISCOVER_UNION, W.WISE_SPARSE] * (R // 4), np.uint8)
    st = twin_schedule(torch, big, [disc, mixed, np.full(R, W.WISE_SPARSE, np.uint8)])
    ctr = st.counters.cpu().numpy()
    assert ctr[W.CTR_FALLBACKS] == 0 and ctr[W.CTR_ERRORS] == 0
    small = dataclasses.replace(synth.WORKLOADS["ctx1k"], rows=4, name="noalloc1k")
    R = small.rows
    twin_schedule(torch, small, [np.full(R, W.WISE_DISCOVER, np.uint8),
                                 np.full(R, W.WISE_DISCOVER_UNION, np.uint8),
                                 np.full(R, W.WISE_SPARSE, np.uint8)])


def test_noalloc_rejects_oversized_calls(torch):
    """A call whose workspace would exceed the static buffer fails before
    anything is enqueued (the pointers below are never dereferenced)."""
    w = synth.WORKLOADS["ragged"]
    need = W.wise_workspace_size(w.rows, w.heads, w.head_dim, w.max_ctx)
    assert need > W.SCRATCH_BYTES
    fake = 0x10000
    a = W.WiseAttn(rows=w.rows, heads=w.heads, head_dim=w.head_dim, dtype=W.WISE_BF16, q=fake, k_cache=fake,
                   v_cache=fake, stride_page=w.heads * 16 * 128, stride_head=16 * 128, stride_token=128,
                   num_pages=8, page_size=16, block_table=fake, bt_stride=w.max_ctx // 16, ctx_len=fake,
                   max_ctx=w.max_ctx, scale=0.0, out=fake, tile_stats=None)
    s = W.WiseSupport(support=fake, slots=w.rows, layers=1, words=32, layer=0, slot_of_row=None, tags=fake,
                      row_request=fake, row_position=fake, discoveries_required=1, eta=0.95, counters=None)
    st = W.lib().wise_decode_sparse_noalloc(ctypes.byref(a), ctypes.byref(s), None, None)
    assert st == W.WISE_E_WORKSPACE
