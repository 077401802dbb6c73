"""bench.py's algorithmic bytes per split launch (the numerator of the
roofline figure), against closed forms written out per case."""

import dataclasses

import numpy as np

import bench
from block_sparse_paged_split_amd import synth
from block_sparse_paged_split_amd import wise as W

CTX1K = synth.WORKLOADS["ctx1k"]  # 32 rows, 16 heads, d 128, bf16, page 16


def _modes(w, m):
    return np.full(w.rows, m)


def test_dense_ctx1k_closed_form():
    w = CTX1K
    ctx = np.full(w.rows, 1024)
    # per (row, head): K and V of 1024 tokens x 128 x 2 B, and q; per row 64 block-table entries
    per_row = 16 * (2 * 1024 * 128 * 2 + 128 * 2) + 4 * 64
    assert bench.split_bytes(w, ctx, _modes(w, W.WISE_DENSE), None) == 32 * per_row == 268_574_720


def test_discovery_adds_tile_stats():
    w = CTX1K
    ctx = np.full(w.rows, 1024)
    dense = bench.split_bytes(w, ctx, _modes(w, W.WISE_DENSE), None)
    for m in (W.WISE_DISCOVER, W.WISE_DISCOVER_UNION):
        assert bench.split_bytes(w, ctx, _modes(w, m), None) - dense == 32 * 16 * 8 * 32


def test_sparse_all_blocks_is_dense_plus_support_words():
    w = CTX1K
    ctx = np.full(w.rows, 1024)
    sup = np.full((w.rows, w.heads, 1), 0xFFFFFFFF, dtype=np.uint32)
    dense = bench.split_bytes(w, ctx, _modes(w, W.WISE_DENSE), None)
    assert bench.split_bytes(w, ctx, _modes(w, W.WISE_SPARSE), sup) == dense + 32 * 16 * 4


def test_sparse_single_block_and_partial_tail():
    w = dataclasses.replace(CTX1K, rows=2)
    ctx = np.array([1024, 100])   # row 1: blocks 0..3, the last holds 4 tokens
    sup = np.zeros((2, w.heads, 1), dtype=np.uint32)
    sup[0, :, 0] = 1 << 5         # row 0: block 5 in every head (tokens 160..191, pages 10 and 11)
    sup[1, 0, 0] = 1 << 3         # row 1: head 0 only, the 4-token last block (page 6)
    got = bench.split_bytes(w, ctx, _modes(w, W.WISE_SPARSE), sup)
    row0 = 16 * (2 * 32 * 128 * 2) + 16 * 128 * 2 + 16 * 4 + 4 * 2
    row1 = 2 * 4 * 128 * 2 + 16 * 128 * 2 + 16 * 4 + 4 * 1
    assert got == row0 + row1


def test_sparse_pages_shared_by_heads_count_once():
    w = dataclasses.replace(CTX1K, rows=1, heads=2)
    ctx = np.array([64])
    sup = np.zeros((1, 2, 1), dtype=np.uint32)
    sup[0, 0, 0] = 0b01           # head 0: block 0 (pages 0, 1)
    sup[0, 1, 0] = 0b11           # head 1: blocks 0 and 1 (pages 0..3)
    got = bench.split_bytes(w, ctx, _modes(w, W.WISE_SPARSE), sup)
    assert got == 2 * (32 + 64) * 128 * 2 + 2 * 128 * 2 + 2 * 4 + 4 * 4


def test_lse_route_reads_k_only():
    w = CTX1K
    ctx = np.full(w.rows, 1024)
    per_row = 16 * (1024 * 128 * 2 + 128 * 2 + 8 * 32) + 4 * 64
    assert bench.split_bytes(w, ctx, _modes(w, bench.LSE_ROUTE), None) == 32 * per_row


def test_fp32_element_size():
    w = synth.WORKLOADS["tiny_f32"]  # 1 row, 4 heads, d 64, fp32, page 32
    ctx = np.array([256])
    assert bench.split_bytes(w, ctx, _modes(w, W.WISE_DENSE), None) == 4 * (2 * 256 * 64 * 4 + 64 * 4) + 4 * 8
