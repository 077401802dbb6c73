"""No kernel writes outside its buffers: every output, state and workspace
buffer lives inside a larger allocation whose guard bands hold a sentinel,
and every launch shape and route runs over them (fused, static, listed,
LSE route, head-union page route, snapshot and restore)."""

import dataclasses

import numpy as np
import pytest

from block_sparse_paged_split_amd import harness, synth
from block_sparse_paged_split_amd import wise as W
from parity import oracle_lse

pytestmark = pytest.mark.gpu

GUARD_BYTES = 4096


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    W.lib()
    return t


class Guarded:
    """A view of `shape` inside an allocation with guard bands on both sides."""

    def __init__(self, torch, shape, dtype, fill_inside=0):
        esz = torch.empty((), dtype=dtype).element_size()
        self.g = GUARD_BYTES // esz
        n = int(np.prod(shape))
        self.base = torch.empty(n + 2 * self.g, dtype=dtype, device="cuda")
        self.base.view(torch.uint8).fill_(0xA5)
        self.view = self.base[self.g:self.g + n].view(shape)
        self.view.fill_(fill_inside)

    def intact(self, torch):
        b = self.base.view(torch.uint8)
        nb = self.g * self.base.element_size()
        return bool((b[:nb] == 0xA5).all()) and bool((b[-nb:] == 0xA5).all())


def guard_layer(torch, dev, w):
    R, H, d = dev.q.shape
    nbmax = (w.max_ctx + 31) // 32
    out = Guarded(torch, (R, H, d), torch.float32)
    stats = Guarded(torch, (R, H, nbmax, 2), torch.float32)
    dev.out, dev.tile_stats = out.view, stats.view
    return [out, stats]


def guard_state(torch, st):
    sup = Guarded(torch, tuple(st.support.shape), torch.int32)
    tags = Guarded(torch, tuple(st.tags.shape), torch.int64)
    ctr = Guarded(torch, tuple(st.counters.shape), torch.int64)
    st.support, st.tags, st.counters = sup.view, tags.view, ctr.view
    return [sup, tags, ctr]


@pytest.mark.parametrize("ctx,rows", [(1024, 8), (4096, 8)])
def test_no_writes_outside_buffers(torch, ctx, rows):
    w = dataclasses.replace(synth.WORKLOADS["ctx1k"], rows=rows, ctx=ctx, name=f"guards{ctx}")
    R, H = w.rows, w.heads
    guards = []
    lis = [synth.layer_inputs(w, d) for d in range(4)]
    devs = [harness.upload(li) for li in lis]
    for dev in devs:
        guards += guard_layer(torch, dev, w)
    st = harness.SupportState(R, H, w.max_ctx, slots=R + 4)
    st.row_position.fill_(3)
    guards += guard_state(torch, st)
    ws = harness.Workspace(R, H, w.head_dim, w.max_ctx)
    wsg = Guarded(torch, (ws.nbytes,), torch.uint8)
    ws.buf = wsg.view
    assert ws.ptr % 256 == 0
    guards.append(wsg)

    def check(stage):
        torch.cuda.synchronize()
        bad = [i for i, g in enumerate(guards) if not g.intact(torch)]
        say(f"[guards{ctx}] {stage}: {'ok' if not bad else f'guard bands hit: {bad}'}")
        assert not bad, stage

    harness.call(devs[0], ws, W.WISE_DISCOVER, st, required=2)
    check("discover")
    harness.call(devs[1], ws, W.WISE_DISCOVER_UNION, st, required=2)
    check("union")
    harness.call(devs[2], ws, W.WISE_SPARSE, st, required=2)
    check("sparse")
    modes = torch.tensor(([3, 0, 1, 3] * R)[:R], dtype=torch.uint8, device="cuda")
    harness.call(devs[3], ws, W.WISE_SPARSE, st, required=2, row_mode=modes)
    check("mixed")
    harness.call(devs[3], ws, W.WISE_DENSE)
    check("dense")
    lse = torch.from_numpy(oracle_lse(w, lis[0])).cuda()
    lseg = Guarded(torch, (R, H), torch.float32)
    lseg.view.copy_(lse)
    guards.append(lseg)
    harness.call_lse(devs[0], ws, lseg.view, False, st)
    check("lse route")
    # head-union page route over the discovered supports
    pu = harness.PageUnion(devs[2])
    btg = Guarded(torch, tuple(pu.bt.shape), torch.int32, fill_inside=-1)
    ctxg = Guarded(torch, tuple(pu.ctx.shape), torch.int32)
    pu.bt, pu.ctx = btg.view, ctxg.view
    guards += [btg, ctxg]
    st2 = harness.SupportState(R, H, w.max_ctx, slots=R + 4)
    guards += guard_state(torch, st2)
    st2.support.copy_(st.support)
    st2.tags.copy_(st.tags)
    pu.compact(st2, required=1)
    pu.attend(ws)
    check("page route")
    # snapshot and restore of every row's slot
    slots = torch.arange(R, dtype=torch.int32, device="cuda")
    recg = Guarded(torch, (R * st.record_bytes(),), torch.uint8)
    guards.append(recg)
    st.snapshot(slots, recg.view)
    check("snapshot")
    st.restore(torch.arange(4, 4 + R, dtype=torch.int32, device="cuda"), recg.view)
    check("restore")
