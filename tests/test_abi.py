"""The C-ABI library loads, exports every entry point include/wise.h
declares, sizes its workspace, and rejects bad host arguments before any
work is enqueued (no GPU needed: every case below fails validation)."""

import ctypes
import os
import re
import subprocess

import pytest

from block_sparse_paged_split_amd import wise as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(W.LIB_PATH):
        from block_sparse_paged_split_amd import build
        build.build()
    return W.lib()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "wise.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wise_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(W.EXPORTED)
    dyn = subprocess.run(["nm", "-D", "--defined-only", W.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (wise_\w+)", dyn))
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_status_strings(lib):
    for st in range(5):
        assert W.status_string(st)
    assert W.status_string(0) == "ok"


def test_workspace_size(lib):
    s1 = W.wise_workspace_size(32, 16, 128, 1024)
    assert s1 > 0 and s1 % 256 == 0
    assert W.wise_workspace_size(64, 16, 128, 1024) > s1
    assert W.wise_workspace_size(32, 16, 128, 4096) > s1
    assert W.wise_workspace_size(32, 16, 64, 1024) < s1
    # partial results + tile stats dominate: at least (d + 2) floats per item slot
    items = 32 * 16 * (32 // 8)
    assert s1 >= items * (128 + 2) * 4 + 32 * 16 * 32 * 8
    for bad in [(0, 16, 128, 1024), (32, 0, 128, 1024), (32, 16, 96, 1024), (32, 16, 128, 0),
                (32, 16, 128, 65537), (1 << 20, 16, 128, 64)]:
        assert W.wise_workspace_size(*bad) == 0


def test_fused_waves_regimes(lib):
    """The host-side launch query: one-launch workgroups of 4-16 waves up to
    8K tokens and 255 heads, the split grid + finish kernel beyond, and -1
    for sizes or dtypes the library rejects."""
    fw = W.wise_fused_waves
    bf, f32 = W.WISE_BF16, W.WISE_F32
    assert fw(32, 16, 128, 1024, bf, True) == 4        # four 8-tile items per 1K unit
    assert fw(32, 16, 128, 1024, bf, False) == 4
    assert fw(2, 16, 128, 1024, bf, True) in (8, 16)   # small launch: shorter items, more waves
    assert fw(64, 16, 128, 4096, bf, True) == 8        # >= 512 units: 8 waves
    assert fw(20, 16, 128, 4096, bf, True) == 16       # fewer units: 16 waves
    assert fw(20, 16, 128, 4096, f32, True) == 8       # fp32 d128 waves need more registers
    assert fw(20, 16, 128, 4096, bf, False) == 0       # small plain dense call: split grid
    assert fw(64, 16, 128, 8192, bf, True) == 8
    assert fw(64, 16, 128, 8224, bf, True) == 0        # 257 blocks: beyond the one-launch kernel
    assert fw(4, 256, 128, 1024, bf, True) == 0        # row arrivals are counted in 8 bits
    assert fw(4, 255, 128, 1024, bf, True) == 4
    for bad in [(32, 16, 96, 1024, bf, True), (32, 16, 128, 1024, 7, True), (0, 16, 128, 1024, bf, True),
                (32, 16, 128, 65537, bf, True)]:
        assert fw(*bad) == -1


FAKE = 0x10000  # never dereferenced: every call below fails host validation


def good_attn(**kw):
    a = W.WiseAttn(rows=2, heads=2, head_dim=128, dtype=W.WISE_BF16, q=FAKE, k_cache=FAKE,
                   v_cache=FAKE, stride_page=2 * 16 * 128, stride_head=16 * 128, stride_token=128,
                   num_pages=8, page_size=16, block_table=FAKE, bt_stride=4, ctx_len=FAKE,
                   max_ctx=64, scale=0.0, out=FAKE, tile_stats=None)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def good_support(**kw):
    s = W.WiseSupport(support=FAKE, slots=2, layers=1, words=1, layer=0, slot_of_row=None,
                      tags=FAKE, row_request=FAKE, row_position=FAKE, discoveries_required=1,
                      eta=0.95, counters=None)
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def call(lib, fn, a, s=None, ws=None, ws_bytes=None, extra=None):
    ws = 0 if ws is None else ws
    wsb = 0 if ws_bytes is None else ws_bytes
    pa = ctypes.byref(a) if a is not None else None
    ps = ctypes.byref(s) if s is not None else None
    if fn == "dense":
        return lib.wise_decode_dense(pa, ws, wsb, None)
    if fn == "discover":
        return lib.wise_decode_discover(pa, ps, 0, ws, wsb, None)
    if fn == "sparse":
        return lib.wise_decode_sparse(pa, ps, extra, ws, wsb, None)
    if fn == "lse":
        return lib.wise_discover_lse(pa, ps, 0, FAKE if extra is None else extra, ws, wsb, None)
    return lib.wise_finish_select(pa, ps, ws, wsb, None)


CASES = [
    ("null attn", dict(), "dense", W.WISE_E_ARG, "attn_none"),
    ("head_dim 96", dict(head_dim=96), "dense", W.WISE_E_UNSUPPORTED, None),
    ("dtype 7", dict(dtype=7), "dense", W.WISE_E_UNSUPPORTED, None),
    ("rows 0", dict(rows=0), "dense", W.WISE_E_ARG, None),
    ("page 12", dict(page_size=12), "dense", W.WISE_E_UNSUPPORTED, None),
    ("page 4", dict(page_size=4), "dense", W.WISE_E_UNSUPPORTED, None),
    ("max_ctx 70000", dict(max_ctx=70000, bt_stride=5000), "dense", W.WISE_E_UNSUPPORTED, None),
    ("null q", dict(q=None), "dense", W.WISE_E_ARG, None),
    ("null out", dict(out=None), "finish", W.WISE_E_ARG, None),
    ("misaligned k", dict(k_cache=FAKE + 8), "dense", W.WISE_E_ARG, None),
    ("stride not 16B", dict(stride_token=132), "dense", W.WISE_E_ARG, None),
    ("short bt", dict(bt_stride=3), "dense", W.WISE_E_ARG, None),
    ("negative scale", dict(scale=-1.0), "dense", W.WISE_E_ARG, None),
    ("one event", dict(ev_split_begin=FAKE), "dense", W.WISE_E_ARG, None),
    ("no workspace", dict(), "dense", W.WISE_E_WORKSPACE, None),
]


@pytest.mark.parametrize("name,kw,fn,expect,special", CASES, ids=[c[0] for c in CASES])
def test_attn_validation(lib, name, kw, fn, expect, special):
    assert expect != W.WISE_OK
    a = None if special == "attn_none" else good_attn(**kw)
    assert call(lib, fn, a) == expect


SUPPORT_CASES = [
    ("no support", None, W.WISE_E_ARG),
    ("eta 0", dict(eta=0.0), W.WISE_E_ARG),
    ("eta 1.5", dict(eta=1.5), W.WISE_E_ARG),
    ("layer out of range", dict(layer=1), W.WISE_E_ARG),
    ("too few words", dict(words=0), W.WISE_E_ARG),
    ("required 0", dict(discoveries_required=0), W.WISE_E_ARG),
    ("null tags", dict(tags=None), W.WISE_E_ARG),
]


@pytest.mark.parametrize("name,kw,expect", SUPPORT_CASES, ids=[c[0] for c in SUPPORT_CASES])
@pytest.mark.parametrize("fn", ["discover", "sparse", "lse"])
def test_support_validation(lib, name, kw, expect, fn):
    s = None if kw is None else good_support(**kw)
    assert call(lib, fn, good_attn(), s) == expect


def test_workspace_validation(lib):
    need = W.wise_workspace_size(2, 2, 128, 64)
    # too small (a fake, aligned address is never touched: the size check fails first)
    assert call(lib, "dense", good_attn(), ws=1 << 20, ws_bytes=need - 1) == W.WISE_E_WORKSPACE
    assert call(lib, "finish", good_attn(), ws=(1 << 20) + 64, ws_bytes=need) == W.WISE_E_WORKSPACE


def test_lse_route_validation(lib):
    """wise_discover_lse: the LSE array is required and 4-byte aligned, V and
    out are optional (only the workspace check is left to fail), K is not."""
    a, s = good_attn(), good_support()
    assert call(lib, "lse", a, s, extra=None) == W.WISE_E_WORKSPACE      # FAKE lse, no workspace
    assert lib.wise_discover_lse(ctypes.byref(a), ctypes.byref(s), 0, None, 0, 0, None) == W.WISE_E_ARG
    assert call(lib, "lse", a, s, extra=FAKE + 2) == W.WISE_E_ARG
    assert call(lib, "lse", good_attn(v_cache=None, out=None), s) == W.WISE_E_WORKSPACE
    assert call(lib, "lse", good_attn(k_cache=None), s) == W.WISE_E_ARG
    assert call(lib, "lse", a, None) == W.WISE_E_ARG
    # the other entry points still need V and out
    assert call(lib, "dense", good_attn(v_cache=None)) == W.WISE_E_ARG
    assert call(lib, "finish", good_attn(out=None)) == W.WISE_E_ARG


def test_compact_pages_validation(lib):
    """wise_compact_pages: outputs required, 4-byte aligned, wide enough, and
    never the input table or contexts (every case fails before a launch)."""
    a, s = good_attn(), good_support()
    B, C = FAKE + 4096, FAKE + 8192

    def cp(a=a, s=s, bt=B, stride=4, ctx=C):
        return lib.wise_compact_pages(ctypes.byref(a), None if s is None else ctypes.byref(s), None,
                                      bt, stride, ctx, None)
    assert cp(bt=None) == W.WISE_E_ARG
    assert cp(ctx=None) == W.WISE_E_ARG
    assert cp(bt=B + 2) == W.WISE_E_ARG
    assert cp(stride=3) == W.WISE_E_ARG                 # ceil(64 / 16) = 4 pages needed
    assert cp(bt=FAKE) == W.WISE_E_ARG                  # the input block table itself
    assert cp(ctx=FAKE) == W.WISE_E_ARG                 # the input contexts themselves
    assert cp(s=None) == W.WISE_E_ARG
    assert cp(s=good_support(words=0)) == W.WISE_E_ARG
    assert cp(a=good_attn(page_size=12)) == W.WISE_E_UNSUPPORTED


def test_snapshot_bytes_and_validation(lib):
    # [layers][heads][words] uint32 padded to 8 bytes, then [layers] 24-byte tags
    assert W.wise_snapshot_bytes(24, 16, 4) == 24 * 16 * 4 * 4 + 24 * 24
    assert W.wise_snapshot_bytes(1, 3, 1) == 16 + 24
    assert W.wise_snapshot_bytes(0, 16, 4) == 0 and W.wise_snapshot_bytes(1, 1, 0) == 0
    s = good_support(layers=2, words=1)
    need = W.wise_snapshot_bytes(2, 2, 1)
    D = FAKE + 4096

    def snap(s=s, heads=2, slots=FAKE, count=3, dst=D, nbytes=3 * need):
        return lib.wise_support_snapshot(None if s is None else ctypes.byref(s), heads, slots, count, dst,
                                         nbytes, None)
    assert snap(s=None) == W.WISE_E_ARG
    assert snap(slots=None) == W.WISE_E_ARG
    assert snap(dst=None) == W.WISE_E_ARG
    assert snap(dst=D + 4) == W.WISE_E_ARG              # records are 8-byte aligned
    assert snap(nbytes=3 * need - 1) == W.WISE_E_ARG
    assert snap(heads=0) == W.WISE_E_ARG
    assert snap(count=-1) == W.WISE_E_ARG
    assert snap(s=good_support(tags=None)) == W.WISE_E_ARG
    assert snap(count=0, nbytes=0) == W.WISE_OK         # nothing to copy, nothing enqueued
    assert lib.wise_support_restore(ctypes.byref(s), 2, FAKE, 3, D, 3 * need - 8, None) == W.WISE_E_ARG
    assert lib.wise_support_restore(ctypes.byref(s), 2, FAKE, 0, D, 0, None) == W.WISE_OK


def test_missing_library_fails_loudly(monkeypatch):
    """Without libwise.so the binding raises; nothing falls back to a CPU path."""
    monkeypatch.setattr(W, "_lib", None)
    monkeypatch.setattr(W, "LIB_PATH", os.path.join(ROOT, "_no_such_dir", "libwise.so"))
    with pytest.raises(RuntimeError, match="not built"):
        W.lib()
    with pytest.raises(RuntimeError, match="not built"):
        W.wise_workspace_size(1, 1, 128, 64)


def test_noalloc_validation(lib):
    """wise_decode_sparse_noalloc checks every host argument, and that the
    call fits the library's static workspace, before it touches a device."""
    a, s = good_attn(), good_support()

    def na(a=a, s=s):
        return lib.wise_decode_sparse_noalloc(None if a is None else ctypes.byref(a),
                                              None if s is None else ctypes.byref(s), None, None)
    assert na(a=None) == W.WISE_E_ARG
    assert na(s=None) == W.WISE_E_ARG
    assert na(a=good_attn(head_dim=96)) == W.WISE_E_UNSUPPORTED
    assert na(s=good_support(eta=0.0)) == W.WISE_E_ARG
    big = good_attn(rows=128, heads=16, max_ctx=32768, bt_stride=2048)
    assert W.wise_workspace_size(128, 16, 128, 32768) > W.SCRATCH_BYTES
    assert na(a=big, s=good_support(slots=128, words=32)) == W.WISE_E_WORKSPACE
