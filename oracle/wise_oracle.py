"""Plain fp64 CPU oracle for WISE working-set paged decode attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or run anything in this package.  It shares no code with the HIP
library and does not import it; it reads only the raw arrays produced by
the seeded input generator (bf16 bit patterns are widened exactly).

Source: the WISE pull request page (InferMatrixLab/vllm-rlt pull 143).
"Summary": the early recurrent depths determine, per query, which 32-token
blocks hold its attention (an eta = 0.95 cumulative-mass rule); the later
depths attend those blocks only, recomputing q, K, V and the softmax inside
them.  "What changes": a split kernel whose rows are dense, discovering
(dense, plus each 32-token tile's score max and exp-sum) or sparse (the
support's tiles only); a second step that merges the splits and selects for
discovering rows; the support as a [slot, layer, head, block] bitmask tagged
with its (request, position); a token without a complete discovery runs
dense for the rest of its depths and is counted.  "Tests": sparse output is
masked attention, and the selection follows the rule and the union over
discovery depths.  Review thread and author's replies: the second discovery
depth ORs into the first; the density count takes the first depth's pick
and causal blocks, then only the bits a union depth newly sets.

Where the page is silent, this oracle takes these readings:
  * softmax scale defaults to 1/sqrt(head_dim);
  * a tile is the logical token range [32b, 32b+32) clipped to the context;
    its "max and sum" are max_t s_t and sum_t exp(s_t - max) over it;
  * block mass is normalised by the full causal row, so masses sum to one;
  * blocks are ordered by mass descending, then block index ascending;
  * the support is the shortest such prefix whose running fp64 sum reaches
    (>=) eta; at least one block; all blocks if rounding never reaches eta;
  * sparse attention renormalises within the support (masked attention);
  * tags count recorded discovery depths; see ``plan_row``;
  * the page's second discovery route (rebuild block mass from a dense
    kernel's LSE, rereading K) takes lse = log sum_t exp(s_t) in natural-log
    units over the row's whole context; a block's mass is then the sum of
    exp(s_t - lse) over its tokens, selection as above; a non-finite lse is a
    data error of its unit;
  * the page's head-union support at page granularity keeps a KV page when
    it holds a valid token of any block selected for any head of the row's
    (slot, layer); every head then attends all tokens of the kept pages.

Every function here has a pin in ``tests/test_oracle_pins.py``.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

BLOCK = 32
DENSE, DISCOVER, DISCOVER_UNION, SPARSE = 0, 1, 2, 3

TAG_DTYPE = np.dtype([("request", "<i8"), ("position", "<i8"),
                      ("discoveries", "<i4"), ("reserved", "<i4")])


# ----------------------------------------------------------------------------
# O1 gather: logical token t of a row lives in physical page
#            block_table[t // P], slot t % P (paged KV cache).
# ----------------------------------------------------------------------------

def widen(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) or fp32 values -> fp64, exactly."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def gather_tokens(cache: np.ndarray, bt_row: np.ndarray, tokens, page_size: int,
                  head: int) -> np.ndarray:
    """Keys (or values) of one (row, head) at the given logical token
    positions, in that order: [len(tokens), d] fp64.

    ``cache`` is [pages, heads, page_size, head_dim].
    """
    t = np.asarray(tokens, dtype=np.int64)
    pages = np.asarray(bt_row)[t // page_size]
    return widen(cache[pages, head, t % page_size, :])


# ----------------------------------------------------------------------------
# O2 dense attention of one decode query over its n causal keys.
# ----------------------------------------------------------------------------

def default_scale(head_dim: int) -> float:
    return 1.0 / np.sqrt(float(head_dim))


def dense_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> Dict:
    """softmax(scale * K q) V in fp64.

    Returns o [d], scores s [n], the max M and the sum L = sum exp(s - M).
    """
    s = scale * (K @ q)
    M = float(s.max())
    w = np.exp(s - M)
    L = float(w.sum())
    o = (w @ V) / L
    return {"o": o, "s": s, "M": M, "L": L}


# ----------------------------------------------------------------------------
# O3 tile statistics (what discover mode records per 32-token tile).
# ----------------------------------------------------------------------------

def num_blocks(n: int) -> int:
    return (n + BLOCK - 1) // BLOCK


def tile_stats(s: np.ndarray):
    """Per tile b: m_b = max score in the tile, l_b = sum exp(s - m_b) over it."""
    n = len(s)
    nb = num_blocks(n)
    m = np.empty(nb)
    l = np.empty(nb)
    for b in range(nb):
        seg = s[b * BLOCK: min(n, b * BLOCK + BLOCK)]
        m[b] = seg.max()
        l[b] = np.exp(seg - m[b]).sum()
    return m, l


def tile_stats_of(s: np.ndarray, tokens: np.ndarray):
    """Tile stats of the blocks that ``tokens`` (ascending positions, whole
    blocks clipped to the context) cover; ``s`` holds their scores."""
    blk = np.asarray(tokens) // BLOCK
    ids = np.unique(blk)
    m = np.array([s[blk == b].max() for b in ids])
    l = np.array([np.exp(s[blk == b] - mb).sum() for b, mb in zip(ids, m)])
    return m, l


# ----------------------------------------------------------------------------
# O4 block mass: the share of the row's softmax that falls in each tile,
#    rebuilt from the tile stats and the row's (M, L).
# ----------------------------------------------------------------------------

def block_mass(m: np.ndarray, l: np.ndarray, M: float, L: float) -> np.ndarray:
    return l * np.exp(m - M) / L


# ----------------------------------------------------------------------------
# O5 eta selection: the fewest blocks, heaviest first, whose mass reaches eta.
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class Selection:
    order: np.ndarray        # block indices, mass descending, index ascending
    K: int                   # number of selected blocks
    blocks: np.ndarray       # selected block indices, ascending
    c_prev: float            # running sum before the K-th block (0 if K == 1)
    c_K: float               # running sum including the K-th block
    p_K: float               # mass of the K-th block in the order
    p_next: float            # mass of the (K+1)-th block (0 if none)

    def near_eta(self, eta: float, tol: float = 1e-6) -> bool:
        """The cut sits within tol of eta (fp32 and fp64 may pick differently)."""
        return abs(self.c_prev - eta) <= tol or abs(self.c_K - eta) <= tol

    def near_tie(self, tol: float = 1e-6) -> bool:
        """The K-th and (K+1)-th masses nearly tie (the swap may differ)."""
        return self.p_next > 0 and abs(self.p_K - self.p_next) <= tol * self.p_K


def eta_select(p: np.ndarray, eta: float) -> Selection:
    p = np.asarray(p, dtype=np.float64)
    nb = len(p)
    idx = np.arange(nb)
    order = np.lexsort((idx, -p))          # primary: -p ascending; secondary: index
    c = np.cumsum(p[order])                # sequential fp64 running sum
    hit = np.nonzero(c >= eta)[0]
    K = int(hit[0]) + 1 if len(hit) else nb
    K = max(1, min(K, nb))
    return Selection(order=order, K=K, blocks=np.sort(order[:K]),
                     c_prev=float(c[K - 2]) if K >= 2 else 0.0, c_K=float(c[K - 1]),
                     p_K=float(p[order[K - 1]]),
                     p_next=float(p[order[K]]) if K < nb else 0.0)


# ----------------------------------------------------------------------------
# O7 masked (sparse) attention: attention over the tokens of the selected
#    blocks only, renormalised within them.
# ----------------------------------------------------------------------------

def token_mask(blocks: Sequence[int], n: int) -> np.ndarray:
    mask = np.zeros(n, dtype=bool)
    for b in blocks:
        mask[b * BLOCK: min(n, b * BLOCK + BLOCK)] = True
    return mask


def masked_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                     blocks: Sequence[int]) -> np.ndarray:
    mask = token_mask(blocks, K.shape[0])
    return dense_attention(q, K[mask], V[mask], scale)["o"]


# ----------------------------------------------------------------------------
# Support bitmask helpers: bit b of a (slot, layer, head) lives in word b//32,
# bit b%32.
# ----------------------------------------------------------------------------

def bits_to_blocks(words: np.ndarray, nb: int) -> np.ndarray:
    words = np.asarray(words, dtype=np.uint32)
    b = np.arange(nb)
    return b[((words[b >> 5] >> (b & 31).astype(np.uint32)) & 1).astype(bool)]


def blocks_to_bits(blocks: Sequence[int], words: int) -> np.ndarray:
    out = np.zeros(words, dtype=np.uint32)
    for b in blocks:
        out[b >> 5] |= np.uint32(1) << np.uint32(b & 31)
    return out


# ----------------------------------------------------------------------------
# O8 support state: tags, effective mode, dense fallback.
# ----------------------------------------------------------------------------

def plan_row(requested: int, tag, request: int, position: int, required: int):
    """Effective mode of one row and whether it is a fallback.

    A tag holds (request, position, discoveries) for one (slot, layer).
    * DENSE and DISCOVER always run as requested (DISCOVER opens a window).
    * DISCOVER_UNION needs a window opened for this very (request, position);
      otherwise the window is broken and the row runs dense (fallback).
    * SPARSE needs this (request, position) with at least ``required``
      discovery depths recorded; a stale position, a released slot
      (discoveries == 0) or an incomplete window runs dense (fallback).
    """
    if requested in (DENSE, DISCOVER):
        return requested, False
    same = int(tag["request"]) == request and int(tag["position"]) == position
    if requested == DISCOVER_UNION:
        ok = same and int(tag["discoveries"]) >= 1
        return (DISCOVER_UNION, False) if ok else (DENSE, True)
    ok = same and int(tag["discoveries"]) >= required
    return (SPARSE, False) if ok else (DENSE, True)


def update_tag(tag, requested: int, effective: int, request: int, position: int,
               row_error: bool):
    """Tag after the call (returns a new record)."""
    t = np.zeros((), dtype=TAG_DTYPE)
    t[()] = tag
    if effective == DISCOVER:
        t["request"], t["position"], t["discoveries"] = request, position, 1
    elif effective == DISCOVER_UNION:
        t["discoveries"] = int(t["discoveries"]) + 1
    if (requested == DISCOVER_UNION and effective == DENSE) or \
            (effective in (DISCOVER, DISCOVER_UNION) and row_error):
        t["discoveries"] = 0        # broken window: the rest of this token runs dense
    return t


# ----------------------------------------------------------------------------
# One (depth, layer) call over every row: plan, attention, finish, bookkeeping.
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class UnitResult:
    out: np.ndarray
    error: bool
    effective: int
    attended: np.ndarray                     # block indices attended
    m: Optional[np.ndarray] = None           # tile stats of the attended blocks
    l: Optional[np.ndarray] = None
    mass: Optional[np.ndarray] = None        # block masses (discover units)
    selection: Optional[Selection] = None


@dataclasses.dataclass
class CallResult:
    out: Optional[np.ndarray]                # [R, H, d] fp64 (NaN for error units); None
                                             # for the LSE route, which makes no output
    support: np.ndarray                      # updated copy
    tags: np.ndarray                         # updated copy
    counters: np.ndarray                     # delta: fallback, selected, causal, errors
    effective: np.ndarray                    # [R] effective mode (-1 = error row)
    units: Dict                              # (r, h) -> UnitResult


def run_call(*, q, k_cache, v_cache, block_table, ctx_len, page_size: int, num_pages: int,
             max_ctx: int, scale: float = 0.0, modes: Sequence[int],
             support: Optional[np.ndarray] = None, tags: Optional[np.ndarray] = None,
             layer: int = 0, slot_of_row: Optional[Sequence[int]] = None,
             row_request: Optional[Sequence[int]] = None,
             row_position: Optional[Sequence[int]] = None,
             required: int = 1, eta: float = 0.95,
             rows: Optional[Sequence[int]] = None) -> CallResult:
    """Evaluate one (depth, layer) call of the method for the given rows.

    ``modes[r]`` is the requested mode of row r.  ``support`` is
    [slots, layers, heads, words] uint32 and ``tags`` [slots, layers] of
    TAG_DTYPE; both are copied, never modified in place.
    Bad device data (context outside [1, max_ctx], slot out of range, a page
    id outside [0, num_pages), an invalid mode, or an empty sparse support)
    makes the affected (row, head) output NaN and counts one error per unit.
    """
    R, H, d = q.shape
    scale = scale if scale else default_scale(d)
    sup = None if support is None else support.copy()
    tg = None if tags is None else tags.copy()
    out = np.full((R, H, d), np.nan)
    counters = np.zeros(4, dtype=np.int64)
    eff_all = np.full(R, -1, dtype=np.int64)
    units = {}
    slots = 0 if sup is None else sup.shape[0]
    words = 0 if sup is None else sup.shape[3]
    todo = range(R) if rows is None else rows
    for r in todo:
        n = int(ctx_len[r])
        req = int(modes[r])
        slot = r if slot_of_row is None else int(slot_of_row[r])
        bad_row = not (1 <= n <= max_ctx) or req not in (DENSE, DISCOVER, DISCOVER_UNION, SPARSE)
        if req != DENSE and not bad_row:
            bad_row = not (0 <= slot < slots)
        if bad_row:
            counters[3] += H
            continue
        nb = num_blocks(n)
        eff, fb = req, False
        if req != DENSE:
            eff, fb = plan_row(req, tg[slot, layer], int(row_request[r]), int(row_position[r]),
                               required)
        counters[0] += int(fb)
        eff_all[r] = eff
        qf = widen(q[r])
        row_err = False
        for h in range(H):
            if eff == SPARSE:
                attended = bits_to_blocks(sup[slot, layer, h], nb)
            else:
                attended = np.arange(nb)
            toks = np.nonzero(token_mask(attended, n))[0]
            pages = np.asarray(block_table[r])[toks // page_size] if len(toks) else np.zeros(0, int)
            err = len(attended) == 0 or bool(np.any((pages < 0) | (pages >= num_pages)))
            if err:
                counters[3] += 1
                row_err = True
                units[(r, h)] = UnitResult(out[r, h], True, eff, attended)
                continue
            Kf = gather_tokens(k_cache, block_table[r], toks, page_size, h)
            Vf = gather_tokens(v_cache, block_table[r], toks, page_size, h)
            att = dense_attention(qf[h], Kf, Vf, scale)
            if eff == SPARSE:
                # attention over the support's tokens only: masked attention
                m, l = tile_stats_of(att["s"], toks)
                res = UnitResult(att["o"], False, eff, attended, m=m, l=l)
            else:
                m, l = tile_stats(att["s"])
                res = UnitResult(att["o"], False, eff, attended, m=m, l=l)
            if eff in (DISCOVER, DISCOVER_UNION):
                p = block_mass(m, l, att["M"], att["L"])
                sel = eta_select(p, eta)
                res.mass, res.selection = p, sel
                new = blocks_to_bits(sel.blocks, words)
                old = sup[slot, layer, h].copy()
                if eff == DISCOVER:
                    sup[slot, layer, h] = new
                    counters[1] += sel.K
                    counters[2] += nb
                else:
                    sup[slot, layer, h] = old | new
                    added = new & ~old
                    counters[1] += int(sum(bin(int(x)).count("1") for x in added))
            out[r, h] = res.out
            units[(r, h)] = res
        if req != DENSE:
            tg[slot, layer] = update_tag(tg[slot, layer], req, eff, int(row_request[r]),
                                         int(row_position[r]), row_err)
    return CallResult(out, sup, tg, counters, eff_all, units)


# ----------------------------------------------------------------------------
# O9 discovery after an external dense kernel: the page's FlashAttention
#    route ("What changes", second bullet) rereads K once and rebuilds every
#    block's mass from the log-sum-exp the dense kernel reported.  With
#    lse = log sum_t exp(s_t), the mass of block b is sum over its tokens of
#    exp(s_t - lse), i.e. its share of the row's softmax.
# ----------------------------------------------------------------------------

def row_lse(s: np.ndarray) -> float:
    """log sum_t exp(s_t) of one row's scores (what a dense kernel reports)."""
    M = float(np.max(s))
    return M + float(np.log(np.exp(s - M).sum()))


def lse_block_mass(s: np.ndarray, lse: float) -> np.ndarray:
    """Per block b: sum over the block's valid tokens of exp(s_t - lse)."""
    n = len(s)
    return np.array([np.exp(s[b * BLOCK: min(n, b * BLOCK + BLOCK)] - lse).sum()
                     for b in range(num_blocks(n))])


def run_lse_call(*, q, k_cache, block_table, ctx_len, page_size: int, num_pages: int,
                 max_ctx: int, lse, union: bool, support: np.ndarray, tags: np.ndarray,
                 scale: float = 0.0, layer: int = 0,
                 slot_of_row: Optional[Sequence[int]] = None,
                 row_request: Optional[Sequence[int]] = None,
                 row_position: Optional[Sequence[int]] = None, eta: float = 0.95,
                 rows: Optional[Sequence[int]] = None) -> CallResult:
    """One discovery depth by the LSE route, every row DISCOVER (or
    DISCOVER_UNION when ``union``).  ``lse`` [R, H] is the dense kernel's
    log-sum-exp of the scaled scores.  No attention output is produced (the
    dense kernel made it); selection, support, tags and counters follow
    ``run_call``.  A non-finite lse, like a bad page, is a data error of its
    (row, head) unit and breaks the row's discovery window.
    """
    R, H, d = q.shape
    scale = scale if scale else default_scale(d)
    sup, tg = support.copy(), tags.copy()
    counters = np.zeros(4, dtype=np.int64)
    eff_all = np.full(R, -1, dtype=np.int64)
    units = {}
    slots, words = sup.shape[0], sup.shape[3]
    req = DISCOVER_UNION if union else DISCOVER
    for r in (range(R) if rows is None else rows):
        n = int(ctx_len[r])
        slot = r if slot_of_row is None else int(slot_of_row[r])
        if not (1 <= n <= max_ctx) or not (0 <= slot < slots):
            counters[3] += H
            continue
        nb = num_blocks(n)
        eff, fb = plan_row(req, tg[slot, layer], int(row_request[r]), int(row_position[r]), 1)
        counters[0] += int(fb)
        eff_all[r] = eff
        row_err = False
        if eff != DENSE:
            qf = widen(q[r])
            toks = np.arange(n)
            pages = np.asarray(block_table[r])[toks // page_size]
            page_bad = bool(np.any((pages < 0) | (pages >= num_pages)))
            for h in range(H):
                lse_rh = float(lse[r][h])
                if page_bad or not np.isfinite(lse_rh):
                    counters[3] += 1
                    row_err = True
                    units[(r, h)] = UnitResult(None, True, eff, np.arange(nb))
                    continue
                s = scale * (gather_tokens(k_cache, block_table[r], toks, page_size, h) @ qf[h])
                m, l = tile_stats(s)
                p = lse_block_mass(s, lse_rh)
                sel = eta_select(p, eta)
                new = blocks_to_bits(sel.blocks, words)
                old = sup[slot, layer, h].copy()
                if eff == DISCOVER:
                    sup[slot, layer, h] = new
                    counters[1] += sel.K
                    counters[2] += nb
                else:
                    sup[slot, layer, h] = old | new
                    counters[1] += int(sum(bin(int(x)).count("1") for x in (new & ~old)))
                units[(r, h)] = UnitResult(None, False, eff, np.arange(nb), m=m, l=l, mass=p,
                                           selection=sel)
        tg[slot, layer] = update_tag(tg[slot, layer], req, eff, int(row_request[r]),
                                     int(row_position[r]), row_err)
    return CallResult(None, sup, tg, counters, eff_all, units)


# ----------------------------------------------------------------------------
# O10 head-union, page-granular support through a compacted page table: the
#     page's FlashAttention route ("What changes", second bullet) lets a sparse
#     row attend the union over its heads of the layer's support, widened to
#     whole KV pages and handed to the attention kernel as a shorter page table.
# ----------------------------------------------------------------------------

def head_union_blocks(words: np.ndarray, nb: int) -> np.ndarray:
    """Blocks set for any head: words is [heads, W] of one (slot, layer)."""
    u = set()
    for h in range(words.shape[0]):
        u.update(int(b) for b in bits_to_blocks(words[h], nb))
    return np.array(sorted(u), dtype=np.int64)


def union_pages(blocks: Sequence[int], n: int, page_size: int) -> np.ndarray:
    """Logical pages j < ceil(n/P) holding a token of a selected block."""
    pages = set()
    for b in blocks:
        lo, hi = b * BLOCK, min(n, b * BLOCK + BLOCK) - 1      # the block's valid tokens
        pages.update(range(lo // page_size, hi // page_size + 1))
    return np.array(sorted(pages), dtype=np.int64)


def page_tokens(pages: Sequence[int], n: int, page_size: int) -> np.ndarray:
    """Logical token positions of the given pages, in order (clipped to n)."""
    return np.array([t for j in pages for t in range(j * page_size, min(n, j * page_size + page_size))],
                    dtype=np.int64)


@dataclasses.dataclass
class PageUnionResult:
    out: np.ndarray                          # [R, H, d] fp64, NaN for error rows
    tables: Dict                             # r -> compacted physical page list
    ctx: np.ndarray                          # [R] compacted context length
    counters: np.ndarray                     # fallback, -, -, errors (per (row, head))
    pages: Dict                              # r -> kept logical pages


def run_page_union_call(*, q, k_cache, v_cache, block_table, ctx_len, page_size: int,
                        num_pages: int, max_ctx: int, support: np.ndarray, tags: np.ndarray,
                        scale: float = 0.0, layer: int = 0,
                        slot_of_row: Optional[Sequence[int]] = None,
                        row_request: Optional[Sequence[int]] = None,
                        row_position: Optional[Sequence[int]] = None, required: int = 1,
                        row_modes: Optional[Sequence[int]] = None,
                        rows: Optional[Sequence[int]] = None) -> PageUnionResult:
    """One reuse depth by the head-union page route.  Row modes: SPARSE
    (default) attends the pages holding any block of the union over its heads
    of the (slot, layer) support, when the tag admits reuse (as ``plan_row``);
    otherwise, and for DENSE rows, every causal page.  The compacted table
    lists the kept pages' physical ids in logical order and the compacted
    context is the number of tokens they hold, so every kept page but the
    last is full.  Every head of a row attends the same tokens, renormalised
    within them.  Data errors (context outside [1, max_ctx], another mode, a
    slot out of range, an empty union, a kept page id out of range) give a
    compacted context of 0, NaN for every head of the row and one error per
    head.
    """
    R, H, d = q.shape
    P = page_size
    scale = scale if scale else default_scale(d)
    out = np.full((R, H, d), np.nan)
    ctx_out = np.zeros(R, dtype=np.int64)
    tables, kept = {}, {}
    counters = np.zeros(4, dtype=np.int64)
    slots = support.shape[0]
    for r in (range(R) if rows is None else rows):
        n = int(ctx_len[r])
        req = SPARSE if row_modes is None else int(row_modes[r])
        if req not in (DENSE, SPARSE):
            counters[3] += H
            continue
        if not 1 <= n <= max_ctx:
            counters[3] += H
            continue
        npg = (n + P - 1) // P
        pages = np.arange(npg)
        if req == SPARSE:
            slot = r if slot_of_row is None else int(slot_of_row[r])
            if not 0 <= slot < slots:
                counters[3] += H
                continue
            eff, fb = plan_row(SPARSE, tags[slot, layer], int(row_request[r]), int(row_position[r]),
                               required)
            counters[0] += int(fb)
            if eff == SPARSE:
                blocks = head_union_blocks(support[slot, layer], num_blocks(n))
                if len(blocks) == 0:
                    counters[3] += H
                    continue
                pages = union_pages(blocks, n, P)
        phys = np.asarray(block_table[r])[pages]
        if np.any((phys < 0) | (phys >= num_pages)):
            counters[3] += H
            continue
        kept[r] = pages
        tables[r] = phys
        ctx_out[r] = len(page_tokens(pages, n, P))
        toks = page_tokens(pages, n, P)
        qf = widen(q[r])
        for h in range(H):
            Kf = gather_tokens(k_cache, block_table[r], toks, P, h)
            Vf = gather_tokens(v_cache, block_table[r], toks, P, h)
            out[r, h] = dense_attention(qf[h], Kf, Vf, scale)["o"]
    return PageUnionResult(out, tables, ctx_out, counters, kept)


# ----------------------------------------------------------------------------
# O11 support snapshot and restore across a KV offload: the review's first
#     finding asks for the support and tags of a request to be saved with
#     its KV and recurrent state and restored on resume, so that reuse after
#     the resume continues instead of failing.  A record holds one slot's
#     support words of every (layer, head) and its tag of every layer.
# ----------------------------------------------------------------------------

def snapshot_slots(support: np.ndarray, tags: np.ndarray, slots: Sequence[int]):
    """Records of the given slots: (support [layers, heads, words], tags
    [layers]) copies; a slot out of range gives an empty record (zero words,
    zero tags, so that reuse from it falls back)."""
    recs = []
    for sl in slots:
        if 0 <= sl < support.shape[0]:
            recs.append((support[sl].copy(), tags[sl].copy()))
        else:
            recs.append((np.zeros(support.shape[1:], support.dtype), np.zeros(tags.shape[1:], tags.dtype)))
    return recs


def restore_slots(support: np.ndarray, tags: np.ndarray, slots: Sequence[int], recs):
    """Support and tags with record i written into slot slots[i] (new copies).
    A destination out of range is skipped and counted as a data error."""
    sup, tg = support.copy(), tags.copy()
    errors = 0
    for sl, (words, t) in zip(slots, recs):
        if 0 <= sl < sup.shape[0]:
            sup[sl] = words
            tg[sl] = t
        else:
            errors += 1
    return sup, tg, errors


def density(counters: Sequence[int]) -> float:
    """Reuse-union support density: selected blocks over causal blocks."""
    return float(counters[1]) / float(counters[2]) if counters[2] else 0.0
