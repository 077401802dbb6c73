"""Seeded synthetic inputs for working-set paged decode attention.

This module only *draws* inputs: queries, paged key/value caches, block
tables, context lengths and planted "hot" blocks.  It holds none of the
method's arithmetic (no scores, no softmax, no selection), so both the HIP
path and the CPU oracle can consume what it produces without sharing any
computation.

Workload recipes follow the decode-attention shapes that the WISE pull
request (vllm-rlt #143, "Results") measures on: 16 heads of head_dim 128 in
bf16, contexts of 1K / 4K / 8K tokens, and a tiny fp32 case.  Their prompts
are not available, so every tensor is N(0, 1) noise with a few 32-token
blocks made "hot" by adding ``alpha * q / |q|`` to their keys.

Every random stream is keyed by ``numpy.random.SeedSequence(seed,
spawn_key=...)`` so that one row of one (depth, layer) can be regenerated
on its own: the oracle side can rebuild only the rows it samples.

Encodings
---------
* bf16 tensors are carried as ``uint16`` bit patterns, rounded from fp32
  with round-to-nearest-even (NaN never occurs: inputs are finite).
* fp32 tensors are carried as ``float32``.
* Unused cache slots (past a row's context, and spare pages) are filled with
  a quiet-NaN pattern, so a kernel that reads them poisons its output.
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
import threading
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

BLOCK = 32  # tokens per selection block (the method's B)

# stream identifiers for SeedSequence spawn keys
_S_QKV = 1
_S_HOT = 2
_S_CTX = 3
_S_TABLE = 4
_S_MODES = 5
_S_SUPPORT = 6

BF16_QNAN = np.uint16(0x7FC0)

# mode codes (mirrors the C ABI's wise_mode enumeration)
DENSE, DISCOVER, DISCOVER_UNION, SPARSE = 0, 1, 2, 3


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); return bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic decode-attention workload.

    ``ctx`` is a fixed context length, or ``None`` with ``ctx_range`` for a
    log-uniform ragged batch.  ``hot`` is the number of planted blocks per
    (row, head), or ``None`` with ``hot_range`` for a uniform draw.
    ``schedule`` lists the requested mode of every depth.
    """

    name: str
    rows: int
    heads: int
    head_dim: int
    dtype: str                      # "bf16" | "f32"
    page_size: int
    shuffle: bool
    alpha: float
    seed: int
    ctx: Optional[int] = None
    ctx_range: Optional[Tuple[int, int]] = None
    ctx_list: Optional[Tuple[int, ...]] = None
    hot: Optional[int] = None
    hot_range: Optional[Tuple[int, int]] = None
    layers: int = 1
    schedule: Tuple[int, ...] = (DISCOVER, DISCOVER_UNION, SPARSE, SPARSE)
    eta: float = 0.95
    spare_pages: int = 3
    shared_hot: bool = False        # one set of planted blocks per (row, layer), shared by the heads
    # one-launch mixed batch: fractions of (dense, discover, sparse) rows and
    # the fraction of sparse rows left with an incomplete discovery
    mix: Optional[Tuple[float, float, float]] = None
    mix_flagged: float = 0.0
    # reuse depths read a random support of this density set directly
    # (no discovery), as a kernel benchmark does
    fixed_density: Optional[float] = None
    # every key of a (row, head) is the same draw (exactly tied scores, so
    # every full block carries the same softmax mass); no planting
    tied_keys: bool = False
    note: str = ""

    @property
    def max_ctx(self) -> int:
        if self.ctx is not None:
            return self.ctx
        if self.ctx_list is not None:
            return max(self.ctx_list)
        return self.ctx_range[1]

    @property
    def discoveries(self) -> int:
        return sum(1 for m in self.schedule if m in (DISCOVER, DISCOVER_UNION))


# The five workloads named by the task, plus density-matched supplements.
WORKLOADS: Dict[str, Workload] = {
    "tiny_f32": Workload(
        name="tiny_f32", rows=1, heads=4, head_dim=64, dtype="f32", page_size=32,
        shuffle=False, alpha=3.0, seed=0, ctx=256, hot=2,
        schedule=(DISCOVER, SPARSE, SPARSE),
        note="1 sequence, 4 heads, d=64, 256 tokens, contiguous KV"),
    "ctx1k": Workload(
        name="ctx1k", rows=32, heads=16, head_dim=128, dtype="bf16", page_size=16,
        shuffle=True, alpha=2.5, seed=1, ctx=1024, hot=4,
        note="32 rows, 16 heads, d=128, bf16, page 16, shuffled table"),
    "ctx4k_24l": Workload(
        name="ctx4k_24l", rows=64, heads=16, head_dim=128, dtype="bf16", page_size=16,
        shuffle=True, alpha=2.5, seed=2, ctx=4096, hot=8, layers=24,
        note="64 rows at 4K, 24 layers looped per depth"),
    "ctx8k_mixed": Workload(
        name="ctx8k_mixed", rows=64, heads=16, head_dim=128, dtype="bf16", page_size=16,
        shuffle=True, alpha=2.5, seed=3, ctx=8192, hot=4, mix=(0.25, 0.25, 0.5), mix_flagged=0.05,
        note="64 rows at 8K; one launch mixes dense/discover/sparse rows"),
    "ragged": Workload(
        name="ragged", rows=128, heads=16, head_dim=128, dtype="bf16", page_size=16,
        shuffle=True, alpha=2.5, seed=4, ctx_range=(512, 32768), hot_range=(1, 16),
        note="128 rows, contexts log-uniform 512..32768, eta swept"),
    # supplementary, density-matched to the reuse densities the pull request reports
    "match1k": Workload(
        name="match1k", rows=32, heads=16, head_dim=128, dtype="bf16", page_size=16,
        shuffle=True, alpha=8.0, seed=11, ctx=1024, hot=9,
        note="supplementary: ~0.28 union density at 1K"),
    "match4k": Workload(
        name="match4k", rows=64, heads=16, head_dim=128, dtype="bf16", page_size=16,
        shuffle=True, alpha=8.0, seed=12, ctx=4096, hot=23,
        note="supplementary: ~0.18 union density at 4K"),
    "match8k": Workload(
        name="match8k", rows=64, heads=16, head_dim=128, dtype="bf16", page_size=16,
        shuffle=True, alpha=8.0, seed=13, ctx=8192, hot=38,
        note="supplementary: ~0.15 union density at 8K"),
    # supplementary analogs of the pull request's kernel benchmark ("Results"):
    # 1K x 64 with the support set directly to a random 0.13 of the blocks,
    # and a 4K x 20 launch of half discovery and half sparse rows
    "kbench1k": Workload(
        name="kbench1k", rows=64, heads=16, head_dim=128, dtype="bf16", page_size=16,
        shuffle=True, alpha=2.5, seed=15, ctx=1024, hot=4, schedule=(SPARSE,), fixed_density=0.13,
        note="supplementary: kernel benchmark, 1K x 64, random support density 0.13"),
    "mix4k": Workload(
        name="mix4k", rows=20, heads=16, head_dim=128, dtype="bf16", page_size=16,
        shuffle=True, alpha=8.0, seed=16, ctx=4096, hot=23, mix=(0.0, 0.5, 0.5),
        note="supplementary: kernel benchmark, 4K x 20, half discovery and half sparse rows"),
    # supplementary: a small batch (two rows), latency-bound
    "small1k": Workload(
        name="small1k", rows=2, heads=16, head_dim=128, dtype="bf16", page_size=16,
        shuffle=True, alpha=2.5, seed=17, ctx=1024, hot=4,
        note="supplementary: 2 rows at 1K, a latency-bound small batch"),
    # supplementary, for the head-union page-granular route: the heads of a row
    # share their planted blocks (heads attending the same positions)
    "shared8k": Workload(
        name="shared8k", rows=64, heads=16, head_dim=128, dtype="bf16", page_size=16,
        shuffle=True, alpha=8.0, seed=14, ctx=8192, hot=38, shared_hot=True,
        note="supplementary: match8k with planted blocks shared by a row's heads"),
}


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def context_lengths(w: Workload) -> np.ndarray:
    """Per-row context lengths (tokens attended, including the current one)."""
    if w.ctx is not None:
        return np.full(w.rows, w.ctx, dtype=np.int32)
    if w.ctx_list is not None:
        assert len(w.ctx_list) == w.rows
        return np.asarray(w.ctx_list, dtype=np.int32)
    lo, hi = w.ctx_range
    u = _rng(w.seed, _S_CTX).uniform(math.log(lo), math.log(hi), size=w.rows)
    return np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int32)


def block_table(w: Workload, ctx: np.ndarray) -> Tuple[np.ndarray, int]:
    """Block table [rows, ceil(max_ctx / P)] (int32, -1 past each row) and page count."""
    P = w.page_size
    need = (ctx.astype(np.int64) + P - 1) // P
    total = int(need.sum())
    num_pages = total + w.spare_pages
    if w.shuffle:
        phys = _rng(w.seed, _S_TABLE).permutation(num_pages)[:total]
    else:
        phys = np.arange(total)
    width = (w.max_ctx + P - 1) // P
    bt = np.full((w.rows, width), -1, dtype=np.int32)
    off = 0
    for r in range(w.rows):
        bt[r, : need[r]] = phys[off: off + need[r]]
        off += int(need[r])
    return bt, num_pages


def hot_blocks(w: Workload, layer: int, row: int, nb: int) -> np.ndarray:
    """Planted block indices for each head of one (layer, row): list of arrays.

    Fixed across depths (only the offset direction follows each depth's q).
    """
    g = _rng(w.seed, _S_HOT, layer, row)
    out = []
    for _ in range(1 if w.shared_hot else w.heads):
        k = w.hot if w.hot is not None else int(g.integers(w.hot_range[0], w.hot_range[1] + 1))
        k = min(k, nb)
        out.append(np.sort(g.choice(nb, size=k, replace=False)).astype(np.int64))
    return out * w.heads if w.shared_hot else out


def row_qkv(w: Workload, depth: int, layer: int, row: int, n: int):
    """Logical fp32 draws for one row: q [H, d], K [H, n, d], V [H, n, d].

    Hot blocks of each head get ``alpha * q_h / |q_h|`` added to every key.
    """
    g = _rng(w.seed, _S_QKV, depth, layer, row)
    H, d = w.heads, w.head_dim
    q = g.standard_normal((H, d), dtype=np.float32)
    K = g.standard_normal((H, n, d), dtype=np.float32)
    V = g.standard_normal((H, n, d), dtype=np.float32)
    if w.tied_keys:
        K[:] = K[:, :1]
        return q, K, V
    nb = (n + BLOCK - 1) // BLOCK
    hb = hot_blocks(w, layer, row, nb)
    for h in range(H):
        qh = q[h] / np.float32(np.linalg.norm(q[h]))
        off = np.float32(w.alpha) * qh
        for b in hb[h]:
            K[h, b * BLOCK: min(b * BLOCK + BLOCK, n)] += off
    return q, K, V


def _encode(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


@dataclasses.dataclass
class LayerInputs:
    """Encoded inputs of one (depth, layer) call.

    q        [rows, H, d]            bf16 bits (uint16) or float32
    k, v     [pages, H, P, d]        same encoding, physical page order
    block_table [rows, width] int32; ctx_len [rows] int32
    """

    workload: Workload
    depth: int
    layer: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    block_table: np.ndarray
    ctx_len: np.ndarray
    num_pages: int


class _Scratch(threading.local):
    """Per-thread reusable buffers (large fresh temporaries in many threads
    serialize on page faults)."""

    def get(self, name: str, shape, dtype) -> np.ndarray:
        n = int(np.prod(shape))
        buf = getattr(self, name, None)
        if buf is None or buf.size < n or buf.dtype != dtype:
            buf = np.empty(n, dtype=dtype)
            setattr(self, name, buf)
        return buf[:n].reshape(shape)


_scratch = _Scratch()


def _round_bf16(x: np.ndarray, name: str) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even; the same rounding as
    f32_to_bf16_bits), overwriting x; return the bit patterns in a contiguous
    per-thread uint16 buffer."""
    u = x.view(np.uint32)
    t = _scratch.get("round_tmp", u.shape, np.uint32)
    np.right_shift(u, np.uint32(16), out=t)
    np.bitwise_and(t, np.uint32(1), out=t)
    np.add(t, np.uint32(0x7FFF), out=t)
    np.add(u, t, out=u)
    np.right_shift(u, np.uint32(16), out=t)
    b = _scratch.get(name, u.shape, np.uint16)
    np.copyto(b, t, casting="unsafe")
    return b


def _fill_row(w: Workload, depth: int, layer: int, r: int, n: int, bt_row, q, k, v) -> None:
    """Draw row r (same streams as row_qkv) and write it into q and the pages of k, v."""
    g = _rng(w.seed, _S_QKV, depth, layer, r)
    H, d, P = w.heads, w.head_dim, w.page_size
    qf = g.standard_normal((H, d), dtype=np.float32)
    K = _scratch.get("K", (H, n, d), np.float32)
    V = _scratch.get("V", (H, n, d), np.float32)
    g.standard_normal(out=K, dtype=np.float32)
    g.standard_normal(out=V, dtype=np.float32)
    nb = (n + BLOCK - 1) // BLOCK
    hb = [] if w.tied_keys else hot_blocks(w, layer, r, nb)
    if w.tied_keys:
        K[:] = K[:, :1]
    for h in range(len(hb)):
        off = np.float32(w.alpha) * (qf[h] / np.float32(np.linalg.norm(qf[h])))
        for b in hb[h]:
            K[h, b * BLOCK: min(b * BLOCK + BLOCK, n)] += off
    q[r] = _encode(qf, w.dtype)
    for name, src, dst in (("K16", K, k), ("V16", V, v)):
        e = _round_bf16(src, name) if w.dtype == "bf16" else src
        for j in range((n + P - 1) // P):
            lo, hi = j * P, min(n, j * P + P)
            dst[bt_row[j], :, : hi - lo] = e[:, lo:hi]


def layer_inputs(w: Workload, depth: int, layer: int = 0,
                 rows: Optional[Sequence[int]] = None, workers: Optional[int] = None) -> LayerInputs:
    """Build the encoded paged inputs of one (depth, layer).

    ``rows`` limits the *filled* rows (others have zero q and pages whose
    content is undefined); shapes and the block table are those of the full
    workload either way.  Slots past a filled row's context and spare pages
    hold the poison pattern.
    Rows are drawn in parallel threads; every row has its own random stream,
    so the result does not depend on ``workers``.
    """
    ctx = context_lengths(w)
    bt, num_pages = block_table(w, ctx)
    H, d, P = w.heads, w.head_dim, w.page_size
    enc = np.uint16 if w.dtype == "bf16" else np.float32
    poison = BF16_QNAN if w.dtype == "bf16" else np.float32(np.nan)
    # Pages of unfilled rows are never read; only the slots no filled row
    # writes (tails of last pages, spare pages) need the poison pattern.
    k = np.empty((num_pages, H, P, d), dtype=enc)
    v = np.empty((num_pages, H, P, d), dtype=enc)
    used = bt[bt >= 0]
    spare = np.setdiff1d(np.arange(num_pages), used)
    k[spare] = poison
    v[spare] = poison
    q = np.zeros((w.rows, H, d), dtype=enc)
    todo = list(range(w.rows)) if rows is None else list(rows)

    def fill(r: int) -> None:
        n = int(ctx[r])
        _fill_row(w, depth, layer, r, n, bt[r], q, k, v)
        if n % P:
            last = bt[r, n // P]
            k[last, :, n % P:] = poison
            v[last, :, n % P:] = poison

    nw = workers if workers is not None else min(16, os.cpu_count() or 1, max(1, len(todo)))
    if nw <= 1:
        for r in todo:
            fill(r)
    else:
        with concurrent.futures.ThreadPoolExecutor(nw) as ex:
            list(ex.map(fill, todo))
    return LayerInputs(w, depth, layer, q, k, v, bt, ctx, num_pages)


def mixed_row_modes(w: Workload, discover_union_alt: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """Row modes of the one-launch mixed batch: fractions ``w.mix`` of dense,
    discover and sparse rows (25% / 25% / 50% for the 8K mixed batch).

    Discover rows alternate DISCOVER / DISCOVER_UNION.  A fraction
    ``w.mix_flagged`` of the sparse rows (rounded, at least one when it is
    positive) are returned as ``flagged``: their discovery is to be left
    incomplete, so they must fall back to dense.
    Returns (modes uint8 [rows], flagged bool [rows]).
    """
    R = w.rows
    g = _rng(w.seed, _S_MODES)
    perm = g.permutation(R)
    nd, nc = int(R * w.mix[0]), int(R * w.mix[1])
    modes = np.empty(R, dtype=np.uint8)
    modes[perm[:nd]] = DENSE
    disc = perm[nd: nd + nc]
    for i, r in enumerate(disc):
        modes[r] = DISCOVER_UNION if (discover_union_alt and i % 2) else DISCOVER
    sparse = perm[nd + nc:]
    modes[sparse] = SPARSE
    flagged = np.zeros(R, dtype=bool)
    if w.mix_flagged > 0:
        nflag = max(1, int(round(w.mix_flagged * len(sparse))))
        flagged[np.sort(g.choice(sparse, size=nflag, replace=False))] = True
    return modes, flagged


def random_support(w: Workload, density: float, ctx: np.ndarray, words: int,
                   layer: int = 0) -> np.ndarray:
    """A support bitmask [rows, H, words] (uint32) with round(density*nb) >= 1
    random blocks set per (row, head): the fixed-density kernel-bench setup."""
    g = _rng(w.seed, _S_SUPPORT, layer)
    sup = np.zeros((w.rows, w.heads, words), dtype=np.uint32)
    for r in range(w.rows):
        nb = (int(ctx[r]) + BLOCK - 1) // BLOCK
        k = max(1, int(round(density * nb)))
        for h in range(w.heads):
            for b in g.choice(nb, size=k, replace=False):
                sup[r, h, b >> 5] |= np.uint32(1) << np.uint32(b & 31)
    return sup
