"""Bitwise invariants on the GPU: twenty reruns of a whole schedule give the
same bits (a race detector for the in-kernel barriers and atomics), and the
rows that fall back to dense equal a dense call's rows bit for bit."""

import dataclasses
import os

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


RERUNS = int(os.environ.get("WISE_RERUNS", "20"))


@pytest.mark.parametrize("ctx,rows", [(1024, 16), (4096, 8), (4096, 20), (8192, 10), (16384, 4)])
def test_schedule_reruns_bitwise(torch, ctx, rows):
    """Discover, union, sparse and a mixed launch, rerun WISE_RERUNS times
    (20 by default) from the same state: outputs, supports, tags and counters
    identical every time.  Up to 8K every call is the one-launch split +
    finish (short units of four waves; long units of sixteen, the mixed
    launch taking its rows heaviest first; 320 units need a second round of
    workgroups); at 16K the static and the listed splits with the finish
    kernel (rows over several workgroups)."""
    w = dataclasses.replace(synth.WORKLOADS["ctx1k"], rows=rows, ctx=ctx, name=f"rerun{ctx}")
    devs = [harness.upload(synth.layer_inputs(w, d)) for d in range(4)]
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    modes = torch.tensor(([3, 1, 0, 2] * rows)[:rows], dtype=torch.uint8, device="cuda")
    ref = None
    for it in range(RERUNS):
        st = harness.SupportState(w.rows, w.heads, w.max_ctx)
        st.row_position.fill_(2)
        harness.call(devs[0], ws, W.WISE_DISCOVER, st, required=2)
        harness.call(devs[1], ws, W.WISE_DISCOVER_UNION, st, required=2)
        harness.call(devs[2], ws, W.WISE_SPARSE, st, required=2)
        out2 = devs[2].out.clone()
        harness.call(devs[3], ws, W.WISE_SPARSE, st, required=2, row_mode=modes)
        torch.cuda.synchronize()
        got = (devs[0].out.clone(), devs[1].out.clone(), out2, devs[3].out.clone(), st.support.clone(),
               st.tags.clone(), st.counters.clone())
        if ref is None:
            ref = got
            say(f"[rerun{ctx}] counters {st.counters.cpu().numpy()}")
            continue
        for a, b, what in zip(got, ref, ("discover", "union", "sparse", "mixed", "support", "tags", "counters")):
            assert torch.equal(a, b), f"rerun {it}: {what} differs"


@pytest.mark.parametrize("ctx", [1024, 4096])
def test_fallback_rows_equal_dense_bitwise(torch, ctx):
    """Sparse rows whose tag does not admit reuse (stale position, released,
    another request, incomplete window) attend densely: their outputs are
    bitwise the dense call's, and each is counted once."""
    w = dataclasses.replace(synth.WORKLOADS["ctx1k"], rows=8, ctx=ctx, name=f"fallback_bits{ctx}")
    d0 = harness.upload(synth.layer_inputs(w, 0))
    d2 = harness.upload(synth.layer_inputs(w, 2))
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    harness.call(d2, ws, W.WISE_DENSE)
    torch.cuda.synchronize()
    dense = d2.out.clone()
    st = harness.SupportState(w.rows, w.heads, w.max_ctx)
    st.row_position.fill_(5)
    harness.call(d0, ws, W.WISE_DISCOVER, st, required=1)
    tags = st.tags.clone()
    tags[1, 0, 1] = 4          # stale position
    tags[2, 0, 2] = 0          # released
    tags[3, 0, 0] = 77         # another request
    st.tags.copy_(tags)
    fb0 = int(st.counters[W.CTR_FALLBACKS].item())
    harness.call(d2, ws, W.WISE_SPARSE, st, required=1)
    torch.cuda.synchronize()
    assert int(st.counters[W.CTR_FALLBACKS].item()) - fb0 == 3
    for r in (1, 2, 3):
        assert torch.equal(d2.out[r], dense[r]), f"fallback row {r}"
    # an incomplete window (two discovery depths required, one recorded): every row falls back
    harness.call(d2, ws, W.WISE_SPARSE, st, required=2)
    torch.cuda.synchronize()
    assert int(st.counters[W.CTR_FALLBACKS].item()) - fb0 == 3 + w.rows
    assert torch.equal(d2.out, dense)


@pytest.mark.parametrize("ctx,rows", [(1024, 8), (4096, 4), (2112, 32)])
def test_one_launch_decode_completes_the_call(torch, ctx, rows):
    """For shapes with wise_fused_waves() > 0 the decode call alone writes the
    outputs, the supports, the tags and the counters; wise_finish_select adds
    nothing.  A schedule run without any finish call must equal, bit for
    bit, the same schedule with them (short units of a small launch; long
    units of sixteen waves; long units of eight waves in a launch of 512
    units)."""
    w = dataclasses.replace(synth.WORKLOADS["ctx1k"], rows=rows, ctx=ctx, name=f"decode_only{ctx}")
    waves = W.wise_fused_waves(w.rows, w.heads, w.head_dim, w.max_ctx, W.WISE_BF16, True)
    assert waves > 0
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    modes = torch.tensor(([3, 1, 0, 2] * rows)[:rows], dtype=torch.uint8, device="cuda")
    hosts = [synth.layer_inputs(w, d) for d in range(4)]
    runs = []
    for finish in (True, False):
        devs = [harness.upload(h) for h in hosts]
        st = harness.SupportState(w.rows, w.heads, w.max_ctx)
        st.row_position.fill_(2)
        harness.call(devs[0], ws, W.WISE_DISCOVER, st, required=2, finish=finish)
        harness.call(devs[1], ws, W.WISE_DISCOVER_UNION, st, required=2, finish=finish)
        harness.call(devs[2], ws, W.WISE_SPARSE, st, required=2, finish=finish)
        harness.call(devs[3], ws, W.WISE_SPARSE, st, required=2, row_mode=modes, finish=finish)
        torch.cuda.synchronize()
        runs.append([d.out.clone() for d in devs] + [st.support.clone(), st.tags.clone(), st.counters.clone()])
        say(f"[decode_only{ctx}] waves {waves} finish={finish} counters {st.counters.cpu().numpy()}")
        del devs
    for a, b, what in zip(runs[0], runs[1], ("discover", "union", "sparse", "mixed", "support", "tags",
                                             "counters")):
        assert torch.equal(a, b), f"{what} differs without the finish call"
    assert int(runs[0][6][W.CTR_SELECTED]) > 0 and not torch.isnan(runs[0][0]).any()
    if W.wise_fused_waves(w.rows, w.heads, w.head_dim, w.max_ctx, W.WISE_BF16, False) > 0:
        dev = harness.upload(hosts[0])
        harness.call(dev, ws, W.WISE_DENSE, finish=False)
        torch.cuda.synchronize()
        d_only = dev.out.clone()
        dev.out.fill_(float("nan"))
        harness.call(dev, ws, W.WISE_DENSE)
        torch.cuda.synchronize()
        assert torch.equal(d_only, dev.out), "dense decode alone differs"


def test_split_grid_calls_need_the_finish(torch):
    """Where wise_fused_waves() is 0 (contexts beyond 8K) the decode call only
    leaves partials in the workspace: the output stays untouched until
    wise_finish_select merges them."""
    w = dataclasses.replace(synth.WORKLOADS["ctx1k"], rows=2, ctx=9000, name="split_grid")
    assert W.wise_fused_waves(w.rows, w.heads, w.head_dim, w.max_ctx, W.WISE_BF16, True) == 0
    ws = harness.Workspace(w.rows, w.heads, w.head_dim, w.max_ctx)
    dev = harness.upload(synth.layer_inputs(w, 0))
    st = harness.SupportState(w.rows, w.heads, w.max_ctx)
    dev.out.fill_(float("nan"))
    harness.call(dev, ws, W.WISE_DISCOVER, st, required=1, finish=False)
    torch.cuda.synchronize()
    assert torch.isnan(dev.out).all(), "the decode call wrote the output"
    assert int(st.counters[W.CTR_SELECTED]) == 0 and int(st.support.abs().sum()) == 0
    harness.call(dev, ws, W.WISE_DISCOVER, st, required=1)
    torch.cuda.synchronize()
    assert not torch.isnan(dev.out).any()
    assert int(st.counters[W.CTR_SELECTED]) > 0
