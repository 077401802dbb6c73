"""Device-side plumbing around the binding: upload synthetic inputs, hold the
support state, run one (depth, layer) call, time with HIP events.

PyTorch supplies device memory and the stream; every computation of the
method runs in libwise's kernels.
"""

from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import numpy as np

from . import synth
from . import wise as W


def _torch():
    import torch
    return torch


def to_device(x: np.ndarray, device, dtype: Optional[str] = None):
    """numpy -> torch on device; bf16 bit patterns (uint16) become bfloat16."""
    torch = _torch()
    if x.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device)


@dataclasses.dataclass
class DeviceLayer:
    """Encoded inputs and outputs of one (depth, layer) call on the device."""

    q: object
    k: object
    v: object
    block_table: object
    ctx_len: object
    out: object
    tile_stats: Optional[object]
    page_size: int
    max_ctx: int

    def attn(self, events=None) -> W.WiseAttn:
        return W.attn_from(self.q, self.k, self.v, self.block_table, self.ctx_len, self.out,
                           page_size=self.page_size, max_ctx=self.max_ctx,
                           tile_stats=self.tile_stats, events=events)

    @property
    def kv_bytes(self) -> int:
        return int(self.k.numel() * self.k.element_size() * 2)


def upload(li: synth.LayerInputs, device="cuda", with_stats: bool = False) -> DeviceLayer:
    torch = _torch()
    w = li.workload
    R, H, d = li.q.shape
    nbmax = (w.max_ctx + synth.BLOCK - 1) // synth.BLOCK
    return DeviceLayer(
        q=to_device(li.q, device), k=to_device(li.k, device), v=to_device(li.v, device),
        block_table=to_device(li.block_table, device), ctx_len=to_device(li.ctx_len, device),
        out=torch.empty((R, H, d), dtype=torch.float32, device=device),
        tile_stats=(torch.full((R, H, nbmax, 2), float("nan"), dtype=torch.float32, device=device)
                    if with_stats else None),
        page_size=w.page_size, max_ctx=w.max_ctx)


class SupportState:
    """Support bitmask, tags and counters of a workload (the pages' WiseState)."""

    def __init__(self, rows: int, heads: int, max_ctx: int, layers: int = 1, device="cuda",
                 slots: Optional[int] = None):
        torch = _torch()
        self.slots = rows if slots is None else slots
        nb = (max_ctx + synth.BLOCK - 1) // synth.BLOCK
        self.words = (nb + 31) // 32
        self.support = torch.zeros((self.slots, layers, heads, self.words), dtype=torch.int32, device=device)
        self.tags = torch.zeros((self.slots, layers, 3), dtype=torch.int64, device=device)
        self.counters = torch.zeros(W.NUM_COUNTERS, dtype=torch.int64, device=device)
        self.row_request = torch.arange(rows, dtype=torch.int64, device=device) + 1000
        self.row_position = torch.zeros(rows, dtype=torch.int64, device=device)
        self.slot_of_row = None

    def view(self, layer: int, required: int, eta: float) -> W.WiseSupport:
        return W.support_from(self.support, self.tags, layer=layer, row_request=self.row_request,
                              row_position=self.row_position, required=required, eta=eta,
                              counters=self.counters, slot_of_row=self.slot_of_row)

    def tags_numpy(self):
        """Tags as the oracle's structured dtype."""
        raw = self.tags.cpu().numpy().copy()
        out = np.zeros(raw.shape[:2], dtype=[("request", "<i8"), ("position", "<i8"),
                                             ("discoveries", "<i4"), ("reserved", "<i4")])
        out["request"] = raw[..., 0]
        out["position"] = raw[..., 1]
        out["discoveries"] = (raw[..., 2] & 0xFFFFFFFF).astype(np.uint32).view(np.int32)
        return out

    def support_numpy(self):
        return self.support.cpu().numpy().view(np.uint32)

    def record_bytes(self) -> int:
        layers, heads = self.support.shape[1], self.support.shape[2]
        return W.wise_snapshot_bytes(layers, heads, self.words)

    def snapshot(self, slots, records, stream: Optional[int] = None) -> None:
        """Records of the given slots (device int32 tensor) into ``records``
        (device uint8 tensor of len(slots) * record_bytes())."""
        st = stream_handle() if stream is None else stream
        W.wise_support_snapshot(self.view(0, 1, 0.95), self.support.shape[2], int(slots.data_ptr()),
                                int(slots.numel()), int(records.data_ptr()), int(records.numel()), st)

    def restore(self, slots, records, stream: Optional[int] = None) -> None:
        st = stream_handle() if stream is None else stream
        W.wise_support_restore(self.view(0, 1, 0.95), self.support.shape[2], int(slots.data_ptr()),
                               int(slots.numel()), int(records.data_ptr()), int(records.numel()), st)


class Workspace:
    def __init__(self, rows, heads, head_dim, max_ctx, device="cuda"):
        torch = _torch()
        self.nbytes = W.wise_workspace_size(rows, heads, head_dim, max_ctx)
        if self.nbytes == 0:
            raise ValueError("unsupported sizes for libwise")
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        assert self.buf.data_ptr() % 256 == 0

    @property
    def ptr(self) -> int:
        return int(self.buf.data_ptr())


def stream_handle() -> int:
    return int(_torch().cuda.current_stream().cuda_stream)


def call(layer: DeviceLayer, ws: Workspace, mode: int, state: Optional[SupportState] = None,
         layer_idx: int = 0, required: int = 2, eta: float = 0.95, row_mode=None,
         events=None, stream: Optional[int] = None, finish: bool = True) -> None:
    """One (depth, layer) call: decode (split-KV kernel) + finish (left out
    with finish=False, for the tests of what the decode call alone does)."""
    st = stream_handle() if stream is None else stream
    a = layer.attn(events)
    s = state.view(layer_idx, required, eta) if state is not None else None
    if row_mode is not None:
        W.wise_decode_sparse(a, s, int(row_mode.data_ptr()), ws.ptr, ws.nbytes, st)
    elif mode == W.WISE_DENSE:
        W.wise_decode_dense(a, ws.ptr, ws.nbytes, st)
    elif mode in (W.WISE_DISCOVER, W.WISE_DISCOVER_UNION):
        W.wise_decode_discover(a, s, mode == W.WISE_DISCOVER_UNION, ws.ptr, ws.nbytes, st)
    else:
        W.wise_decode_sparse(a, s, None, ws.ptr, ws.nbytes, st)
    if finish:
        W.wise_finish_select(a, s, ws.ptr, ws.nbytes, st)


def call_lse(layer: DeviceLayer, ws: Workspace, lse, union: bool, state: SupportState,
             layer_idx: int = 0, eta: float = 0.95, events=None,
             stream: Optional[int] = None) -> None:
    """One discovery depth by the LSE route: ``lse`` [R, H] fp32 on the device
    is the external dense kernel's log-sum-exp."""
    st = stream_handle() if stream is None else stream
    a = layer.attn(events)
    s = state.view(layer_idx, 1, eta)
    W.wise_discover_lse(a, s, union, int(lse.data_ptr()), ws.ptr, ws.nbytes, st)


class PageUnion:
    """Compacted page table and context of one reuse depth by the head-union
    page route, and the dense attention call over them."""

    def __init__(self, layer: DeviceLayer, device="cuda"):
        torch = _torch()
        R = layer.q.shape[0]
        width = layer.block_table.shape[1]
        self.bt = torch.full((R, width), -1, dtype=torch.int32, device=device)
        self.ctx = torch.zeros(R, dtype=torch.int32, device=device)
        self.layer = layer

    def compact(self, state: SupportState, layer_idx: int = 0, required: int = 2, row_mode=None,
                stream: Optional[int] = None) -> None:
        st = stream_handle() if stream is None else stream
        a = self.layer.attn()
        s = state.view(layer_idx, required, 0.95)
        W.wise_compact_pages(a, s, None if row_mode is None else int(row_mode.data_ptr()),
                             int(self.bt.data_ptr()), self.bt.stride(0), int(self.ctx.data_ptr()), st)

    def attend_attn(self, events=None) -> W.WiseAttn:
        """The attention call's operands: the layer's, over the compacted table."""
        a = self.layer.attn(events)
        a.block_table = int(self.bt.data_ptr())
        a.bt_stride = self.bt.stride(0)
        a.ctx_len = int(self.ctx.data_ptr())
        return a

    def attend(self, ws: "Workspace", events=None, stream: Optional[int] = None) -> None:
        """Dense decode over the compacted table (data errors were counted by
        the compaction)."""
        st = stream_handle() if stream is None else stream
        a = self.attend_attn(events)
        W.wise_decode_dense(a, ws.ptr, ws.nbytes, st)
        W.wise_finish_select(a, None, ws.ptr, ws.nbytes, st)


class PreparedCall:
    """One (depth, layer) call with its ctypes arguments built once, so that
    issuing it costs two foreign calls (decode, finish)."""

    def __init__(self, layer: DeviceLayer, ws: Workspace, mode: int,
                 state: Optional[SupportState] = None, layer_idx: int = 0, required: int = 2,
                 eta: float = 0.95, row_mode=None):
        self.a = layer.attn()
        self.s = state.view(layer_idx, required, eta) if state is not None else None
        self.mode = mode
        self.row_mode = None if row_mode is None else int(row_mode.data_ptr())
        self.ws, self.nbytes = ws.ptr, ws.nbytes
        self.L = W.lib()
        self.pa = ctypes.byref(self.a)
        self.ps = None if self.s is None else ctypes.byref(self.s)

    def set_events(self, begin: Optional[int], end: Optional[int]) -> None:
        self.a.ev_split_begin = begin
        self.a.ev_split_end = end

    def run(self, stream: int) -> None:
        L, m = self.L, self.mode
        if self.row_mode is not None or m == W.WISE_SPARSE:
            st = L.wise_decode_sparse(self.pa, self.ps, self.row_mode, self.ws, self.nbytes, stream)
        elif m == W.WISE_DENSE:
            st = L.wise_decode_dense(self.pa, self.ws, self.nbytes, stream)
        else:
            st = L.wise_decode_discover(self.pa, self.ps, int(m == W.WISE_DISCOVER_UNION), self.ws,
                                        self.nbytes, stream)
        if st != W.WISE_OK:
            raise W.WiseError(st, "decode")
        st = L.wise_finish_select(self.pa, self.ps, self.ws, self.nbytes, stream)
        if st != W.WISE_OK:
            raise W.WiseError(st, "finish")


class HipEvents:
    """Raw HIP events (hipEventCreate) usable as the library's timing hook."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e)

    def handle(self, i: int) -> int:
        return int(self.ev[i].value)

    def record(self, i: int, stream: int) -> None:
        if self.hip.hipEventRecord(self.ev[i], ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        try:
            for e in self.ev:
                self.hip.hipEventDestroy(e)
        except Exception:
            pass


class EventPair:
    """(begin, end) handles in the shape attn_from expects (``.cuda_event``)."""

    class _H:
        def __init__(self, h):
            self.cuda_event = h

    def __init__(self, events: HipEvents, i: int, j: int):
        self.pair = (self._H(events.handle(i)), self._H(events.handle(j)))

    def __getitem__(self, k):
        return self.pair[k]
