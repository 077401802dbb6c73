"""Support/tag snapshot and restore across a KV offload, on the GPU: records
byte-exact against the oracle's, and a request resumed into another slot
continues sparse reuse (no fallback) with bitwise the output it would have
had without the offload."""

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
    W.lib()
    return t


def parse_records(buf, count, layers, heads, words):
    rec = W.wise_snapshot_bytes(layers, heads, words)
    nwb = layers * heads * words * 4
    off = (nwb + 7) // 8 * 8
    out = []
    for i in range(count):
        r = buf[i * rec:(i + 1) * rec]
        sup = r[:nwb].view(np.uint32).reshape(layers, heads, words)
        raw = r[off:off + 24 * layers].view(np.int64).reshape(layers, 3)
        tags = np.zeros(layers, O.TAG_DTYPE)
        tags["request"], tags["position"] = raw[:, 0], raw[:, 1]
        tags["discoveries"] = (raw[:, 2] & 0xFFFFFFFF).astype(np.uint32).view(np.int32)
        out.append((sup, tags))
    return out


def test_offload_between_discovery_and_reuse_resumes_sparse(torch):
    w = dataclasses.replace(synth.WORKLOADS["ctx1k"], rows=8, layers=2, name="offload8")
    R, H, L = w.rows, w.heads, w.layers
    state = harness.SupportState(R, H, w.max_ctx, layers=L, slots=2 * R)
    state.row_position.fill_(5)
    ws = harness.Workspace(R, H, w.head_dim, w.max_ctx)
    devs = {}
    for layer in range(L):
        for depth, mode in enumerate(w.schedule[:2]):
            say(f"[offload8] layer {layer} depth {depth} mode {mode}")
            li = synth.layer_inputs(w, depth, layer)
            check_call(w, li, harness.upload(li), ws, state, mode=mode, layer=layer)
        li = synth.layer_inputs(w, 2, layer)
        devs[layer] = (li, harness.upload(li))
    # the outputs of the reuse depth without any offload
    never = {}
    for layer in range(L):
        li, dev = devs[layer]
        rep = check_call(w, li, dev, ws, state, mode=W.WISE_SPARSE, layer=layer)
        assert rep.counters[W.CTR_FALLBACKS] == 0
        never[layer] = dev.out.clone()

    say("[offload8] snapshot slots 0..7, release them, another request takes them")
    sup0, tags0 = state.support_numpy().copy(), state.tags_numpy()
    src_slots = torch.arange(R, dtype=torch.int32, device="cuda")
    rec_bytes = state.record_bytes()
    records = torch.zeros(R * rec_bytes, dtype=torch.uint8, device="cuda")
    state.snapshot(src_slots, records)
    torch.cuda.synchronize()
    got = parse_records(records.cpu().numpy(), R, L, H, state.words)
    for (gs, gt), (es, et) in zip(got, O.snapshot_slots(sup0, tags0, range(R))):
        assert np.array_equal(gs, es)
        assert gt.tobytes() == et.tobytes()
    state.support[:R] = 0
    state.tags[:R] = 0
    saved_request = state.row_request.clone()
    state.row_request += 5000
    li0 = synth.layer_inputs(w, 0, 0)
    check_call(w, li0, harness.upload(li0), ws, state, mode=W.WISE_DISCOVER, layer=0)
    state.row_request.copy_(saved_request)

    say("[offload8] restore into slots 8..15 and resume at the reuse depth")
    pre_sup, pre_tags = state.support_numpy().copy(), state.tags_numpy()
    dst_slots = torch.arange(R, 2 * R, dtype=torch.int32, device="cuda")
    ctr = state.counters.clone()
    state.restore(dst_slots, records)
    torch.cuda.synchronize()
    exp_sup, exp_tags, err = O.restore_slots(pre_sup, pre_tags, list(range(R, 2 * R)),
                                             O.snapshot_slots(sup0, tags0, range(R)))
    assert err == 0
    assert np.array_equal(state.support_numpy(), exp_sup)
    assert state.tags_numpy().tobytes() == exp_tags.tobytes()
    assert torch.equal(state.counters, ctr)
    state.slot_of_row = dst_slots
    for layer in range(L):
        li, dev = devs[layer]
        dev.out.fill_(float("nan"))
        rep = check_call(w, li, dev, ws, state, mode=W.WISE_SPARSE, layer=layer)
        assert rep.counters[W.CTR_FALLBACKS] == 0
        assert torch.equal(dev.out, never[layer]), f"layer {layer}"

    say("[offload8] control: resumed without a restore falls back to dense")
    state.slot_of_row = src_slots
    for layer in range(L):
        li, dev = devs[layer]
        rep = check_call(w, li, dev, ws, state, mode=W.WISE_SPARSE, layer=layer)
        assert rep.counters[W.CTR_FALLBACKS] == R

    say("[offload8] slots out of range: empty records, skipped restores counted")
    bad = torch.tensor([-1, 2 * R + 5], dtype=torch.int32, device="cuda")
    recs2 = torch.full((2 * rec_bytes,), 0xAB, dtype=torch.uint8, device="cuda")
    state.snapshot(bad, recs2)
    torch.cuda.synchronize()
    assert not recs2.any().item()
    before_sup, before_tags = state.support.clone(), state.tags.clone()
    err0 = int(state.counters[W.CTR_ERRORS].item())
    state.restore(torch.tensor([2 * R + 7], dtype=torch.int32, device="cuda"), records[:rec_bytes])
    torch.cuda.synchronize()
    assert int(state.counters[W.CTR_ERRORS].item()) == err0 + 1
    assert torch.equal(state.support, before_sup) and torch.equal(state.tags, before_tags)
