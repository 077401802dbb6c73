"""Python binding of libwise (the C ABI declared in include/wise.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libwise.so.  There is no fallback: if the library is missing, importing the
functions raises, so nothing silently runs elsewhere.

Functions carry the C names (``wise_decode_dense`` ...) and take the ctypes
structures below; ``attn_from`` / ``support_from`` fill those structures
from torch tensors (device memory and streams come from PyTorch).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwise.so")

WISE_OK, WISE_E_ARG, WISE_E_UNSUPPORTED, WISE_E_WORKSPACE, WISE_E_HIP = range(5)
WISE_DENSE, WISE_DISCOVER, WISE_DISCOVER_UNION, WISE_SPARSE = range(4)
WISE_BF16, WISE_F32 = 0, 1
CTR_FALLBACKS, CTR_SELECTED, CTR_CAUSAL, CTR_ERRORS = range(4)
NUM_COUNTERS = 4
BLOCK = 32

EXPORTED = ("wise_workspace_size", "wise_decode_dense", "wise_decode_discover",
            "wise_decode_sparse", "wise_finish_select", "wise_discover_lse", "wise_compact_pages",
            "wise_snapshot_bytes", "wise_support_snapshot", "wise_support_restore", "wise_status_string",
            "wise_decode_sparse_noalloc", "wise_fused_waves")
SCRATCH_BYTES = 32 << 20  # WISE_SCRATCH_BYTES


class WiseTag(ctypes.Structure):
    _fields_ = [("request", ctypes.c_int64), ("position", ctypes.c_int64),
                ("discoveries", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class WiseAttn(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("stride_page", ctypes.c_int64), ("stride_head", ctypes.c_int64),
                ("stride_token", ctypes.c_int64),
                ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("bt_stride", ctypes.c_int32),
                ("ctx_len", ctypes.c_void_p), ("max_ctx", ctypes.c_int32),
                ("scale", ctypes.c_float), ("out", ctypes.c_void_p),
                ("tile_stats", ctypes.c_void_p),
                ("ev_split_begin", ctypes.c_void_p), ("ev_split_end", ctypes.c_void_p)]


class WiseSupport(ctypes.Structure):
    _fields_ = [("support", ctypes.c_void_p), ("slots", ctypes.c_int32),
                ("layers", ctypes.c_int32), ("words", ctypes.c_int32), ("layer", ctypes.c_int32),
                ("slot_of_row", ctypes.c_void_p), ("tags", ctypes.c_void_p),
                ("row_request", ctypes.c_void_p), ("row_position", ctypes.c_void_p),
                ("discoveries_required", ctypes.c_int32), ("eta", ctypes.c_float),
                ("counters", ctypes.c_void_p)]


class WiseError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded libwise.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libwise.so not built ({LIB_PATH}); run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.wise_workspace_size.restype = ctypes.c_size_t
        L.wise_workspace_size.argtypes = [ctypes.c_int32] * 4
        L.wise_fused_waves.restype = ctypes.c_int32
        L.wise_fused_waves.argtypes = [ctypes.c_int32] * 6
        P, S, V = ctypes.POINTER(WiseAttn), ctypes.POINTER(WiseSupport), ctypes.c_void_p
        L.wise_decode_dense.argtypes = [P, V, ctypes.c_size_t, V]
        L.wise_decode_discover.argtypes = [P, S, ctypes.c_int32, V, ctypes.c_size_t, V]
        L.wise_decode_sparse.argtypes = [P, S, V, V, ctypes.c_size_t, V]
        L.wise_finish_select.argtypes = [P, S, V, ctypes.c_size_t, V]
        L.wise_discover_lse.argtypes = [P, S, ctypes.c_int32, V, V, ctypes.c_size_t, V]
        L.wise_compact_pages.argtypes = [P, S, V, V, ctypes.c_int32, V, V]
        L.wise_snapshot_bytes.restype = ctypes.c_size_t
        L.wise_snapshot_bytes.argtypes = [ctypes.c_int32] * 3
        L.wise_support_snapshot.argtypes = [S, ctypes.c_int32, V, ctypes.c_int32, V, ctypes.c_size_t, V]
        L.wise_support_restore.argtypes = [S, ctypes.c_int32, V, ctypes.c_int32, V, ctypes.c_size_t, V]
        L.wise_decode_sparse_noalloc.argtypes = [P, S, V, V]
        for f in ("wise_decode_sparse_noalloc", "wise_decode_dense", "wise_decode_discover", "wise_decode_sparse",
                  "wise_finish_select", "wise_discover_lse", "wise_compact_pages",
                  "wise_support_snapshot", "wise_support_restore"):
            getattr(L, f).restype = ctypes.c_int
        L.wise_status_string.restype = ctypes.c_char_p
        L.wise_status_string.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().wise_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != WISE_OK:
        raise WiseError(status, where)


def _ref(x):
    return None if x is None else ctypes.byref(x)


# ----------------------------------------------------------------------------- C names

def wise_workspace_size(rows: int, heads: int, head_dim: int, max_ctx: int) -> int:
    return int(lib().wise_workspace_size(rows, heads, head_dim, max_ctx))


def wise_fused_waves(rows: int, heads: int, head_dim: int, max_ctx: int, dtype: int, stateful: bool) -> int:
    return int(lib().wise_fused_waves(rows, heads, head_dim, max_ctx, dtype, 1 if stateful else 0))


def wise_decode_dense(a: WiseAttn, ws: int, ws_bytes: int, stream: int = 0) -> None:
    _check(lib().wise_decode_dense(ctypes.byref(a), ws, ws_bytes, stream), "wise_decode_dense")


def wise_decode_discover(a: WiseAttn, s: WiseSupport, union_with_previous: bool, ws: int,
                         ws_bytes: int, stream: int = 0) -> None:
    _check(lib().wise_decode_discover(ctypes.byref(a), ctypes.byref(s), int(bool(union_with_previous)),
                                      ws, ws_bytes, stream), "wise_decode_discover")


def wise_decode_sparse(a: WiseAttn, s: WiseSupport, row_mode: Optional[int], ws: int,
                       ws_bytes: int, stream: int = 0) -> None:
    _check(lib().wise_decode_sparse(ctypes.byref(a), ctypes.byref(s), row_mode, ws, ws_bytes, stream),
           "wise_decode_sparse")


def wise_finish_select(a: WiseAttn, s: Optional[WiseSupport], ws: int, ws_bytes: int,
                       stream: int = 0) -> None:
    _check(lib().wise_finish_select(ctypes.byref(a), _ref(s), ws, ws_bytes, stream),
           "wise_finish_select")


def wise_discover_lse(a: WiseAttn, s: WiseSupport, union_with_previous: bool, lse: int, ws: int,
                      ws_bytes: int, stream: int = 0) -> None:
    _check(lib().wise_discover_lse(ctypes.byref(a), ctypes.byref(s), int(bool(union_with_previous)),
                                   lse, ws, ws_bytes, stream), "wise_discover_lse")


def wise_compact_pages(a: WiseAttn, s: WiseSupport, row_mode: Optional[int], bt_out: int,
                       bt_out_stride: int, ctx_out: int, stream: int = 0) -> None:
    _check(lib().wise_compact_pages(ctypes.byref(a), ctypes.byref(s), row_mode, bt_out, bt_out_stride,
                                    ctx_out, stream), "wise_compact_pages")


def wise_decode_sparse_noalloc(a: WiseAttn, s: WiseSupport, row_mode: Optional[int], stream: int = 0) -> None:
    _check(lib().wise_decode_sparse_noalloc(ctypes.byref(a), ctypes.byref(s), row_mode, stream),
           "wise_decode_sparse_noalloc")


def wise_snapshot_bytes(layers: int, heads: int, words: int) -> int:
    return int(lib().wise_snapshot_bytes(layers, heads, words))


def wise_support_snapshot(s: WiseSupport, heads: int, slots: int, count: int, dst: int, dst_bytes: int,
                          stream: int = 0) -> None:
    _check(lib().wise_support_snapshot(ctypes.byref(s), heads, slots, count, dst, dst_bytes, stream),
           "wise_support_snapshot")


def wise_support_restore(s: WiseSupport, heads: int, slots: int, count: int, src: int, src_bytes: int,
                         stream: int = 0) -> None:
    _check(lib().wise_support_restore(ctypes.byref(s), heads, slots, count, src, src_bytes, stream),
           "wise_support_restore")


# ----------------------------------------------------------------------------- torch marshalling

def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def attn_from(q, k_cache, v_cache, block_table, ctx_len, out, *, page_size: int, max_ctx: int,
              scale: float = 0.0, tile_stats=None, events=None) -> WiseAttn:
    """Fill a WiseAttn from torch tensors.

    q [rows, heads, d] (bf16 or fp32, contiguous); k_cache / v_cache with
    element strides (page, head, slot, dim) taken from the tensors, dim
    contiguous; block_table int32 [rows, >= ceil(max_ctx/P)]; ctx_len int32
    [rows]; out fp32 [rows, heads, d]; tile_stats optional fp32
    [rows, heads, ceil(max_ctx/32), 2]; events optional (begin, end)
    torch.cuda.Event pair recorded around the split-KV kernel.
    """
    import torch
    rows, heads, d = q.shape
    dt = {torch.bfloat16: WISE_BF16, torch.float32: WISE_F32}[q.dtype]
    assert k_cache.dtype == q.dtype and v_cache.dtype == q.dtype
    assert k_cache.stride() == v_cache.stride() and k_cache.stride(3) == 1
    assert q.is_contiguous() and out.is_contiguous() and out.dtype == torch.float32
    assert block_table.dtype == torch.int32 and ctx_len.dtype == torch.int32
    sp, sh, st, _ = k_cache.stride()
    a = WiseAttn(rows=rows, heads=heads, head_dim=d, dtype=dt, q=_ptr(q), k_cache=_ptr(k_cache),
                 v_cache=_ptr(v_cache), stride_page=sp, stride_head=sh, stride_token=st,
                 num_pages=k_cache.shape[0], page_size=page_size, block_table=_ptr(block_table),
                 bt_stride=block_table.stride(0), ctx_len=_ptr(ctx_len), max_ctx=max_ctx,
                 scale=scale, out=_ptr(out), tile_stats=_ptr(tile_stats))
    if events is not None:
        a.ev_split_begin = events[0].cuda_event
        a.ev_split_end = events[1].cuda_event
    return a


def support_from(support, tags, *, layer: int, row_request, row_position, required: int,
                 eta: float, counters=None, slot_of_row=None) -> WiseSupport:
    """Fill a WiseSupport from torch tensors.

    support int32 [slots, layers, heads, words] (uint32 bits); tags int64
    [slots, layers, 3] (request, position, discoveries | reserved << 32);
    row_request / row_position int64 [rows]; counters int64 [4] or None;
    slot_of_row int32 [rows] or None.
    """
    import torch
    assert support.dtype == torch.int32 and support.is_contiguous()
    assert tags.dtype == torch.int64 and tags.is_contiguous() and tags.shape[-1] == 3
    slots, layers, _, words = support.shape
    return WiseSupport(support=_ptr(support), slots=slots, layers=layers, words=words, layer=layer,
                       slot_of_row=_ptr(slot_of_row), tags=_ptr(tags),
                       row_request=_ptr(row_request), row_position=_ptr(row_position),
                       discoveries_required=required, eta=eta, counters=_ptr(counters))
