"""Pins of the fp64 oracle against facts that do not come from the oracle.

Brute force on tiny inputs (pure-Python loops with math.fsum), closed forms,
invariants of the mathematics, exhaustive subset search for the selection
rule, the worked counting example the WISE pull request page prints, and
the fallback transitions it names.  The last test plants mistakes in the
oracle and checks that these pins catch them.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import wise_oracle as O
from block_sparse_paged_split_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- helpers

def brute_softmax_attention(q, K, V, scale):
    """Textbook softmax attention with Python floats and math.fsum."""
    n, d = len(K), len(q)
    s = [scale * math.fsum(q[i] * K[t][i] for i in range(d)) for t in range(n)]
    mx = max(s)
    w = [math.exp(x - mx) for x in s]
    Z = math.fsum(w)
    o = [math.fsum(w[t] * V[t][j] for t in range(n)) / Z for j in range(len(V[0]))]
    return o, [wt / Z for wt in w]


def rand_qkv(rng, n, d):
    return rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d))


def paged_case(rng, n, d=8, H=2, P=16, shuffle=True, spare=2):
    """A tiny paged layout (fp32 encoded) with a known logical K/V per head."""
    npg = (n + P - 1) // P
    num_pages = npg + spare
    phys = rng.permutation(num_pages)[:npg] if shuffle else np.arange(npg)
    Kl = rng.standard_normal((H, n, d)).astype(np.float32)
    Vl = rng.standard_normal((H, n, d)).astype(np.float32)
    k = np.full((num_pages, H, P, d), np.nan, np.float32)
    v = np.full((num_pages, H, P, d), np.nan, np.float32)
    for j in range(npg):
        lo, hi = j * P, min(n, j * P + P)
        k[phys[j], :, : hi - lo] = Kl[:, lo:hi]
        v[phys[j], :, : hi - lo] = Vl[:, lo:hi]
    bt = np.full((1, npg + 1), -1, np.int32)
    bt[0, :npg] = phys
    q = rng.standard_normal((1, H, d)).astype(np.float32)
    return dict(q=q, k_cache=k, v_cache=v, block_table=bt, ctx_len=np.array([n], np.int32),
                page_size=P, num_pages=num_pages, max_ctx=(npg + 1) * P), Kl, Vl


def state(slots=1, layers=1, heads=2, words=1):
    return (np.zeros((slots, layers, heads, words), np.uint32),
            np.zeros((slots, layers), O.TAG_DTYPE))


# ----------------------------------------------------------------------------- O2 dense

@pytest.mark.parametrize("n,d", [(1, 4), (7, 3), (33, 8), (64, 5)])
def test_dense_matches_brute_force(n, d):
    rng = np.random.default_rng(n * 100 + d)
    q, K, V = rand_qkv(rng, n, d)
    scale = 0.7
    ref, _ = brute_softmax_attention(q.tolist(), K.tolist(), V.tolist(), scale)
    got = O.dense_attention(q, K, V, scale)
    np.testing.assert_allclose(got["o"], ref, rtol=0, atol=1e-12)
    # (M, L) are the max and the normaliser of exp(s - M)
    s = scale * (K @ q)
    assert got["M"] == pytest.approx(max(s), abs=1e-12)
    assert got["L"] == pytest.approx(math.fsum(math.exp(x - max(s)) for x in s), rel=1e-13)


def test_dense_closed_forms():
    rng = np.random.default_rng(1)
    d, n = 6, 40
    q = rng.standard_normal(d)
    V = rng.standard_normal((n, d))
    K = np.tile(rng.standard_normal(d), (n, 1))            # all keys equal
    np.testing.assert_allclose(O.dense_attention(q, K, V, 1.0)["o"], V.mean(0), atol=1e-14)
    K = rng.standard_normal((n, d)) * 1e-3                   # one key +60 logits above the rest
    K[17] = q * (60.0 / (q @ q))
    np.testing.assert_allclose(O.dense_attention(q, K, V, 1.0)["o"], V[17], atol=1e-20)


def test_default_scale():
    assert O.default_scale(64) == 0.125
    assert O.default_scale(128) == pytest.approx(1 / math.sqrt(128), rel=1e-16)


# ----------------------------------------------------------------------------- O3/O4 tile stats

@pytest.mark.parametrize("n", [1, 31, 32, 33, 95, 200])
def test_tile_stats_and_mass(n):
    rng = np.random.default_rng(n)
    q, K, V = rand_qkv(rng, n, 4)
    att = O.dense_attention(q, K, V, 0.9)
    m, l = O.tile_stats(att["s"])
    nb = (n + 31) // 32
    assert len(m) == nb
    # recombining the tiles reproduces the row's (M, L)
    M = m.max()
    assert M == att["M"]
    assert float(np.sum(l * np.exp(m - M))) == pytest.approx(att["L"], rel=1e-13)
    # masses are the brute-force block sums of the full softmax and sum to one
    _, probs = brute_softmax_attention(q.tolist(), K.tolist(), V.tolist(), 0.9)
    p = O.block_mass(m, l, att["M"], att["L"])
    brute = [math.fsum(probs[32 * b: min(n, 32 * b + 32)]) for b in range(nb)]
    np.testing.assert_allclose(p, brute, rtol=0, atol=1e-14)
    assert float(p.sum()) == pytest.approx(1.0, abs=1e-13)
    # per-tile definition, brute force
    for b in range(nb):
        seg = att["s"][32 * b: min(n, 32 * b + 32)]
        assert m[b] == max(seg)
        assert l[b] == pytest.approx(math.fsum(math.exp(x - max(seg)) for x in seg), rel=1e-14)


def test_tile_stats_of_subset_brute_force():
    """Tile stats of a token subset (what a sparse unit attends): the blocks
    are the absolute 32-token ranges the tokens fall in, not runs of 32
    entries of the gathered list; a partial last block is a block."""
    rng = np.random.default_rng(21)
    n = 200                                          # blocks 0..6, block 6 holds 8 tokens
    s_all = rng.standard_normal(n) * 3
    for blocks in ([6], [0, 2, 6], [1, 3, 4], [5], list(range(7))):
        toks = np.nonzero(O.token_mask(blocks, n))[0]
        m, l = O.tile_stats_of(s_all[toks], toks)
        assert len(m) == len(blocks)
        for i, b in enumerate(blocks):
            seg = [float(s_all[t]) for t in range(32 * b, min(n, 32 * b + 32))]
            assert m[i] == max(seg)
            assert l[i] == pytest.approx(math.fsum(math.exp(x - max(seg)) for x in seg), rel=1e-14)
    # the whole context gives the dense tile stats, bit for bit
    toks = np.arange(n)
    m, l = O.tile_stats_of(s_all, toks)
    m2, l2 = O.tile_stats(s_all)
    np.testing.assert_array_equal(m, m2)
    np.testing.assert_allclose(l, l2, rtol=1e-15, atol=0)


def test_widen_bf16_bit_patterns():
    """bf16 bits -> fp64 by the format's definition (1 sign, 8 exponent bits
    with bias 127, 7 mantissa bits; exponent 0 is subnormal), evaluated here
    with exact binary arithmetic, never by the oracle's own shift."""
    def bf16_value(bits):
        sign = -1.0 if bits >> 15 else 1.0
        e, m = (bits >> 7) & 0xFF, bits & 0x7F
        if e == 0:
            return sign * math.ldexp(m, -126 - 7)
        assert e != 0xFF
        return sign * math.ldexp(128 + m, e - 127 - 7)

    cases = {0x3F80: 1.0, 0xC020: -2.5, 0x4049: 3.140625, 0x3F81: 1.0 + 2 ** -7,
             0x0001: 2.0 ** -133, 0x807F: -(127 * 2.0 ** -133), 0x0080: 2.0 ** -126,
             0x7F7F: (2 - 2 ** -7) * 2.0 ** 127, 0xFF7F: -(2 - 2 ** -7) * 2.0 ** 127,
             0x0000: 0.0, 0x8000: -0.0}
    bits = np.array(sorted(cases), dtype=np.uint16)
    got = O.widen(bits)
    assert got.dtype == np.float64
    for b, g in zip(bits.tolist(), got.tolist()):
        assert g == cases[b] == bf16_value(b), hex(b)
        assert math.copysign(1.0, g) == math.copysign(1.0, cases[b]), hex(b)   # -0.0 keeps its sign
    rng = np.random.default_rng(8)
    rnd = rng.integers(0, 0x7F80, size=500).astype(np.uint16) | (rng.integers(0, 2, 500) << 15).astype(np.uint16)
    np.testing.assert_array_equal(O.widen(rnd), np.array([bf16_value(int(b)) for b in rnd]))
    # fp32 input passes through exactly; shape is kept
    x = np.array([[1.5, -2.0 ** -149], [3.0e38, 0.1]], np.float32)
    np.testing.assert_array_equal(O.widen(x), x.astype(np.float64))
    assert O.widen(bits.reshape(1, -1)).shape == (1, len(bits))


# ----------------------------------------------------------------------------- O5 selection

def brute_select(p, eta):
    """Smallest cardinality subset with mass >= eta; among those, the heaviest."""
    nb = len(p)
    for k in range(1, nb + 1):
        best = None
        for c in itertools.combinations(range(nb), k):
            mass = math.fsum(p[i] for i in c)
            if mass >= eta and (best is None or mass > best[0]):
                best = (mass, c)
        if best is not None:
            return k, sorted(best[1])
    return nb, list(range(nb))


@pytest.mark.parametrize("nb", [1, 2, 5, 9, 12])
@pytest.mark.parametrize("eta", [0.5, 0.9, 0.95, 0.99])
def test_selection_brute_force(nb, eta):
    rng = np.random.default_rng(nb * 7 + int(eta * 100))
    for _ in range(3):
        w = rng.exponential(size=nb) ** 3
        p = w / w.sum()
        k, blocks = brute_select(p.tolist(), eta)
        sel = O.eta_select(p, eta)
        assert sel.K == k
        assert sel.blocks.tolist() == blocks
        assert sel.c_prev < eta <= sel.c_K or (sel.K == nb and sel.c_K < eta)


def test_selection_tie_break_equal_masses():
    # identical keys: every full 32-token block has the same mass; the order
    # among equals is by block index, so the support is blocks 0..ceil(eta*nb)-1
    nb, d = 30, 4
    rng = np.random.default_rng(3)
    q = rng.standard_normal(d)
    K = np.tile(rng.standard_normal(d), (32 * nb, 1))
    att = O.dense_attention(q, K, K, 1.0)
    p = O.block_mass(*O.tile_stats(att["s"]), att["M"], att["L"])
    for eta in (0.91, 0.95, 0.47):               # eta * nb is not an integer
        sel = O.eta_select(p, eta)
        assert sel.blocks.tolist() == list(range(math.ceil(eta * nb)))


def test_selection_dominant_and_single_block():
    p = np.full(10, 0.004)
    p[6] = 1 - 0.036
    assert O.eta_select(p, 0.95).blocks.tolist() == [6]
    assert O.eta_select(np.array([1.0]), 0.95).blocks.tolist() == [0]     # n <= 32
    assert O.eta_select(np.array([1.0]), 1.0).K == 1
    # equality reaches eta
    assert O.eta_select(np.array([0.5, 0.25, 0.25]), 0.75).blocks.tolist() == [0, 1]


def test_selection_nesting():
    rng = np.random.default_rng(9)
    for _ in range(20):
        w = rng.standard_normal(64) * 2
        p = np.exp(w) / np.exp(w).sum()
        s90, s95, s99 = (set(O.eta_select(p, e).blocks.tolist()) for e in (0.9, 0.95, 0.99))
        assert s90 <= s95 <= s99


def test_bitmask_roundtrip():
    blocks = [0, 1, 31, 32, 63, 100]
    bits = O.blocks_to_bits(blocks, 4)
    assert bits[0] == (1 | 2 | (1 << 31)) and bits[1] == (1 | (1 << 31)) and bits[3] == (1 << 4)
    assert O.bits_to_blocks(bits, 128).tolist() == blocks
    assert O.bits_to_blocks(bits, 64).tolist() == [0, 1, 31, 32, 63]


# ----------------------------------------------------------------------------- O7 masked

def test_masked_attention():
    rng = np.random.default_rng(5)
    n, d = 100, 5
    q, K, V = rand_qkv(rng, n, d)
    np.testing.assert_allclose(O.masked_attention(q, K, V, 0.5, range(4)),
                               O.dense_attention(q, K, V, 0.5)["o"], atol=1e-15)
    ref, _ = brute_softmax_attention(q.tolist(), K[64:96].tolist(), V[64:96].tolist(), 0.5)
    np.testing.assert_allclose(O.masked_attention(q, K, V, 0.5, [2]), ref, atol=1e-12)
    ref, _ = brute_softmax_attention(q.tolist(), K[96:].tolist(), V[96:].tolist(), 0.5)
    np.testing.assert_allclose(O.masked_attention(q, K, V, 0.5, [3]), ref, atol=1e-12)


# ----------------------------------------------------------------------------- whole call

def test_call_dense_discover_sparse_and_page_permutation():
    rng = np.random.default_rng(11)
    case, Kl, Vl = paged_case(rng, 150, H=2)
    sup, tags = state(heads=2)
    common = dict(layer=0, row_request=[7], row_position=[42], required=1, eta=0.9)
    d = O.run_call(**case, modes=[O.DENSE])
    for h in range(2):
        np.testing.assert_allclose(
            d.out[0, h], O.dense_attention(case["q"][0, h].astype(float), Kl[h].astype(float),
                                           Vl[h].astype(float), 1 / math.sqrt(8))["o"], atol=1e-14)
    c = O.run_call(**case, modes=[O.DISCOVER], support=sup, tags=tags, **common)
    assert np.array_equal(c.out, d.out)                      # discover output is the dense output
    assert c.tags[0, 0]["discoveries"] == 1 and c.tags[0, 0]["position"] == 42
    s = O.run_call(**case, modes=[O.SPARSE], support=c.support, tags=c.tags, **common)
    assert s.counters[0] == 0
    for h in range(2):
        blocks = c.units[(0, h)].selection.blocks
        assert O.bits_to_blocks(c.support[0, 0, h], 5).tolist() == blocks.tolist()
        ref = O.masked_attention(case["q"][0, h].astype(float), Kl[h].astype(float),
                                 Vl[h].astype(float), 1 / math.sqrt(8), blocks)
        np.testing.assert_allclose(s.out[0, h], ref, atol=1e-14)
    # all blocks selected: sparse equals dense
    full = c.support.copy()
    full[...] = 0x1F
    s_all = O.run_call(**case, modes=[O.SPARSE], support=full, tags=c.tags, **common)
    np.testing.assert_allclose(s_all.out, d.out, atol=1e-14)
    # a different physical page order gives the same results
    perm = rng.permutation(case["num_pages"])
    inv = np.argsort(perm)
    case2 = dict(case)
    case2["k_cache"] = case["k_cache"][inv]
    case2["v_cache"] = case["v_cache"][inv]
    bt = case["block_table"].copy()
    bt[bt >= 0] = perm[bt[bt >= 0]]
    case2["block_table"] = bt
    c2 = O.run_call(**case2, modes=[O.DISCOVER], support=sup, tags=tags, **common)
    np.testing.assert_allclose(c2.out, c.out, atol=1e-14)
    assert np.array_equal(c2.support, c.support)


def _two_block_row(rng, hot_block, d=8):
    """n = 64 (two causal blocks) where one block holds nearly all the mass."""
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = 1.0
    K = rng.standard_normal((1, 64, d)).astype(np.float32) * 0.01
    K[0, 32 * hot_block: 32 * hot_block + 32, 0] = 40.0
    k = K.reshape(1, 2, 32, d).transpose(1, 0, 2, 3).copy()
    v = rng.standard_normal(k.shape).astype(np.float32)
    return dict(q=q, k_cache=k, v_cache=v, block_table=np.array([[0, 1]], np.int32),
                ctx_len=np.array([64], np.int32), page_size=32, num_pages=2, max_ctx=64)


def test_union_density_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "union_density_example.json")))
    rng = np.random.default_rng(2)
    sup, tags = state(heads=1)
    common = dict(layer=0, row_request=[1], row_position=[5], required=2, eta=0.9)
    c0 = O.run_call(**_two_block_row(rng, 0), modes=[O.DISCOVER], support=sup, tags=tags, **common)
    assert c0.units[(0, 0)].selection.blocks.tolist() == g["depth0_selection"]
    c1 = O.run_call(**_two_block_row(rng, 1), modes=[O.DISCOVER_UNION], support=c0.support,
                    tags=c0.tags, **common)
    assert c1.units[(0, 0)].selection.blocks.tolist() == g["depth1_selection"]
    total = c0.counters + c1.counters
    assert total[2] == g["causal_blocks"]
    assert O.density(total) == g["expected_union_density"]
    indiv = (c0.units[(0, 0)].selection.K + c1.units[(0, 0)].selection.K) / (2 * g["causal_blocks"])
    assert indiv == g["density_of_individual_selections"]
    assert O.bits_to_blocks(c1.support[0, 0, 0], 2).tolist() == [0, 1]
    assert c1.tags[0, 0]["discoveries"] == 2
    # the reuse depth attends the union: with every block in it, sparse equals dense
    case = _two_block_row(rng, 1)
    s = O.run_call(**case, modes=[O.SPARSE], support=c1.support, tags=c1.tags, **common)
    d = O.run_call(**case, modes=[O.DENSE])
    assert s.counters[0] == 0
    np.testing.assert_allclose(s.out, d.out, atol=1e-14)


# ----------------------------------------------------------------------------- O8 fallback

def _discovered(rng, required=2):
    case, _, _ = paged_case(rng, 96, H=2)
    sup, tags = state(heads=2)
    common = dict(layer=0, row_request=[3], row_position=[10], required=required, eta=0.95)
    c0 = O.run_call(**case, modes=[O.DISCOVER], support=sup, tags=tags, **common)
    return case, common, c0


def test_fallback_transitions():
    rng = np.random.default_rng(4)
    case, common, c0 = _discovered(rng)
    dense = O.run_call(**case, modes=[O.DENSE]).out
    # complete window: union then sparse, no fallback
    c1 = O.run_call(**case, modes=[O.DISCOVER_UNION], support=c0.support, tags=c0.tags, **common)
    ok = O.run_call(**case, modes=[O.SPARSE], support=c1.support, tags=c1.tags, **common)
    assert c1.counters[0] == 0 and ok.counters[0] == 0 and ok.effective[0] == O.SPARSE
    # incomplete window: one discovery of the two required -> dense, counted
    r = O.run_call(**case, modes=[O.SPARSE], support=c0.support, tags=c0.tags, **common)
    assert r.counters[0] == 1 and r.effective[0] == O.DENSE
    assert np.array_equal(r.out, dense)
    # stale position: the tag belongs to the previous token
    stale = dict(common, row_position=[11])
    r = O.run_call(**case, modes=[O.SPARSE], support=c1.support, tags=c1.tags, **stale)
    assert r.counters[0] == 1 and np.array_equal(r.out, dense)
    # released slot: discoveries cleared by the owner
    rel = c1.tags.copy()
    rel[0, 0]["discoveries"] = 0
    r = O.run_call(**case, modes=[O.SPARSE], support=c1.support, tags=rel, **common)
    assert r.counters[0] == 1 and np.array_equal(r.out, dense)
    # another request's support in this slot
    other = dict(common, row_request=[4])
    r = O.run_call(**case, modes=[O.SPARSE], support=c1.support, tags=c1.tags, **other)
    assert r.counters[0] == 1
    # broken window: the union depth sees no discovery for this position; it
    # runs dense, invalidates the tag, and the reuse depths fall back too
    b = O.run_call(**case, modes=[O.DISCOVER_UNION], support=c0.support, tags=c0.tags, **stale)
    assert b.counters[0] == 1 and np.array_equal(b.out, dense)
    assert b.tags[0, 0]["discoveries"] == 0
    assert np.array_equal(b.support, c0.support)             # nothing recorded
    r = O.run_call(**case, modes=[O.SPARSE], support=b.support, tags=b.tags, **stale)
    assert r.counters[0] == 1
    # a dense row never touches the state
    r = O.run_call(**case, modes=[O.DENSE], support=c1.support, tags=c1.tags, **common)
    assert r.counters.tolist() == [0, 0, 0, 0] and np.array_equal(r.tags, c1.tags)


def test_data_errors():
    rng = np.random.default_rng(6)
    case, common, c0 = _discovered(rng, required=1)
    bad = dict(case, ctx_len=np.array([case["max_ctx"] + 1], np.int32))
    r = O.run_call(**bad, modes=[O.DENSE])
    assert np.isnan(r.out).all() and r.counters[3] == 2
    bad = dict(case, ctx_len=np.array([0], np.int32))
    assert O.run_call(**bad, modes=[O.DENSE]).counters[3] == 2
    # a bad page id inside the attended range
    bt = case["block_table"].copy()
    bt[0, 1] = case["num_pages"]
    r = O.run_call(**dict(case, block_table=bt), modes=[O.DENSE])
    assert np.isnan(r.out).all() and r.counters[3] == 2
    # outside every head's support it is harmless for a sparse row
    sup = c0.support.copy()
    sup[...] = 0b001                                          # block 0 only (tokens 0..31, page 0..1)
    bt = case["block_table"].copy()
    bt[0, 5] = -7                                             # tokens 80..95 -> block 2
    r = O.run_call(**dict(case, block_table=bt), modes=[O.SPARSE], support=sup, tags=c0.tags, **common)
    assert r.counters[3] == 0 and not np.isnan(r.out).any()
    # an empty support
    sup[0, 0, 1] = 0
    r = O.run_call(**case, modes=[O.SPARSE], support=sup, tags=c0.tags, **common)
    assert r.counters[3] == 1 and np.isnan(r.out[0, 1]).all() and not np.isnan(r.out[0, 0]).any()
    # slot out of range for a stateful row; invalid mode
    r = O.run_call(**case, modes=[O.SPARSE], support=sup, tags=c0.tags, slot_of_row=[5], **common)
    assert r.counters[3] == 2
    r = O.run_call(**case, modes=[9], support=sup, tags=c0.tags, **common)
    assert r.counters[3] == 2


# ----------------------------------------------------------------------------- generator sanity

def test_synth_encodings_and_layout():
    x = np.array([1.0, -2.5, 3.140625, 1.00390625, 1.01171875, 65504.0], np.float32)
    b = synth.f32_to_bf16_bits(x)
    # 1.00390625 = 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins (1.0)
    # 1.01171875 = 1 + 3*2^-8 ties between 1+2^-7 and 1+2^-6: even is 1+2^-6
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(b),
                                  np.array([1.0, -2.5, 3.140625, 1.0, 1.015625, 65536.0], np.float32))
    w = synth.WORKLOADS["tiny_f32"]
    li = synth.layer_inputs(w, depth=0)
    assert li.k.shape == (8 + w.spare_pages, 4, 32, 64)
    assert li.block_table[0].tolist() == list(range(8))
    q, K, V = synth.row_qkv(w, 0, 0, 0, 256)
    np.testing.assert_array_equal(li.k[3, 2, 5], K[2, 3 * 32 + 5])
    w = synth.WORKLOADS["ctx1k"]
    li = synth.layer_inputs(w, depth=1, rows=[3])
    q, K, V = synth.row_qkv(w, 1, 0, 3, 1024)
    page = li.block_table[3, 10]
    np.testing.assert_array_equal(li.k[page, 7, 4], synth.f32_to_bf16_bits(K[7, 164]))
    assert len(set(li.block_table[li.block_table >= 0].tolist())) == (li.block_table >= 0).sum()
    ctx = synth.context_lengths(synth.WORKLOADS["ragged"])
    assert ctx.min() >= 512 and ctx.max() <= 32768


# ----------------------------------------------------------------------------- O9 LSE route

def brute_lse(s):
    mx = max(s)
    return mx + math.log(math.fsum(math.exp(x - mx) for x in s))


@pytest.mark.parametrize("n", [1, 32, 33, 95, 200])
def test_lse_block_mass_is_softmax_block_sums(n):
    """Block masses rebuilt from the row's log-sum-exp are the block sums of
    the brute-force softmax; a larger lse scales them by exp(-delta)."""
    rng = np.random.default_rng(500 + n)
    q, K, V = rand_qkv(rng, n, 4)
    _, probs = brute_softmax_attention(q.tolist(), K.tolist(), V.tolist(), 0.8)
    s_py = [0.8 * math.fsum(q[i] * K[t][i] for i in range(4)) for t in range(n)]
    lse = brute_lse(s_py)
    s = 0.8 * (K @ q)
    assert O.row_lse(s) == pytest.approx(lse, abs=1e-12)
    nb = (n + 31) // 32
    brute = np.array([math.fsum(probs[32 * b: min(n, 32 * b + 32)]) for b in range(nb)])
    p = O.lse_block_mass(s, lse)
    assert len(p) == nb
    np.testing.assert_allclose(p, brute, rtol=0, atol=1e-14)
    np.testing.assert_allclose(O.lse_block_mass(s, lse + 0.25), brute * math.exp(-0.25), rtol=1e-13)


def test_lse_block_mass_closed_form():
    """Equal scores c over n tokens: lse = c + ln n and each block holds its
    token count over n (the partial last block included)."""
    n = 75
    s = np.full(n, 1.7)
    assert O.row_lse(s) == pytest.approx(1.7 + math.log(n), abs=1e-14)
    np.testing.assert_allclose(O.lse_block_mass(s, 1.7 + math.log(n)), [32 / n, 32 / n, 11 / n],
                               rtol=1e-14)


def test_lse_call_matches_tile_route_and_unions():
    """The LSE route picks the supports, tags and counts that discovery from
    the tile stats picks; a second LSE depth ORs like DISCOVER_UNION; a union
    without a window falls back; a non-finite lse is a data error."""
    rng = np.random.default_rng(21)
    case, Kl, Vl = paged_case(rng, 150, H=2)
    sup, tags = state(heads=2)
    common = dict(layer=0, row_request=[7], row_position=[42], eta=0.9)
    lse = np.array([[brute_lse((case["q"][0, h].astype(float) @ Kl[h].astype(float).T
                                / math.sqrt(8)).tolist()) for h in range(2)]])
    kw = {k: case[k] for k in ("q", "k_cache", "block_table", "ctx_len", "page_size", "num_pages",
                               "max_ctx")}
    ref = O.run_call(**case, modes=[O.DISCOVER], support=sup, tags=tags, required=1, **common)
    got = O.run_lse_call(**kw, lse=lse, union=False, support=sup, tags=tags, **common)
    assert got.out is None
    for h in range(2):
        assert not ref.units[(0, h)].selection.near_eta(0.9)
        np.testing.assert_allclose(got.units[(0, h)].mass, ref.units[(0, h)].mass, atol=1e-14)
    assert np.array_equal(got.support, ref.support)
    assert got.tags.tobytes() == ref.tags.tobytes()
    assert got.counters.tolist() == ref.counters.tolist()
    # second discovery depth with fresh queries: the LSE union equals the tile-stat union
    case2 = dict(case)
    case2["q"] = rng.standard_normal(case["q"].shape).astype(np.float32)
    kw2 = dict(kw, q=case2["q"])
    lse2 = np.array([[brute_lse((case2["q"][0, h].astype(float) @ Kl[h].astype(float).T
                                 / math.sqrt(8)).tolist()) for h in range(2)]])
    ref_u = O.run_call(**case2, modes=[O.DISCOVER_UNION], support=ref.support, tags=ref.tags,
                       required=1, **common)
    got_u = O.run_lse_call(**kw2, lse=lse2, union=True, support=got.support, tags=got.tags, **common)
    assert np.array_equal(got_u.support, ref_u.support)
    assert got_u.tags[0, 0]["discoveries"] == 2 and got_u.counters.tolist() == ref_u.counters.tolist()
    # a union with no window: dense fallback, window invalidated, support untouched
    fb = O.run_lse_call(**kw2, lse=lse2, union=True, support=sup, tags=tags, **common)
    assert fb.counters.tolist() == [1, 0, 0, 0]
    assert fb.tags[0, 0]["discoveries"] == 0 and np.array_equal(fb.support, sup)
    # a non-finite lse: one error, the window breaks
    bad = lse.copy()
    bad[0, 1] = np.nan
    e = O.run_lse_call(**kw, lse=bad, union=False, support=sup, tags=tags, **common)
    assert e.counters[3] == 1 and e.tags[0, 0]["discoveries"] == 0
    assert np.array_equal(e.support[0, 0, 0], ref.support[0, 0, 0])


# ----------------------------------------------------------------------------- O10 head-union page route

@pytest.mark.parametrize("P", [8, 16, 32, 64, 256])
def test_union_pages_brute_force(P):
    """Kept pages are exactly the pages holding a valid token of a selected
    block (token-by-token enumeration), and the compacted token sequence is
    the kept tokens in order, every kept page but the last full."""
    rng = np.random.default_rng(P)
    for n in (1, 31, 33, 100, 257, 1000):
        nb = (n + 31) // 32
        for _ in range(5):
            blocks = np.sort(rng.choice(nb, size=int(rng.integers(1, nb + 1)), replace=False))
            brute = sorted({t // P for t in range(n) if (t // 32) in set(blocks.tolist())})
            got = O.union_pages(blocks, n, P)
            assert got.tolist() == brute
            toks = O.page_tokens(got, n, P)
            assert toks.tolist() == [t for t in range(n) if t // P in set(brute)]
            # compacted position i is token kept_pages[i // P] * P + i % P
            i = np.arange(len(toks))
            assert np.array_equal(got[i // P] * P + i % P, toks)


def test_head_union_blocks():
    words = np.array([[0b1001, 0], [0b0110, 1 << 3], [0, 0]], dtype=np.uint32)
    assert O.head_union_blocks(words, 40).tolist() == [0, 1, 2, 3, 35]
    assert O.head_union_blocks(words, 35).tolist() == [0, 1, 2, 3]     # bits past nb ignored
    assert O.head_union_blocks(np.zeros((2, 1), np.uint32), 5).tolist() == []


def test_page_union_call():
    """All blocks set: the compacted table is the row's table and the output
    is dense attention.  A sparse union: every head attends exactly the kept
    pages' tokens (brute-force softmax).  A stale tag falls back to every
    page.  A large page turns one selected block into its whole page."""
    rng = np.random.default_rng(41)
    case, Kl, Vl = paged_case(rng, 150, H=2, P=16)
    sup, tags = state(heads=2)
    tags[0, 0] = (7, 42, 2, 0)
    common = dict(layer=0, row_request=[7], row_position=[42], required=2)
    d = O.run_call(**case, modes=[O.DENSE])
    full = sup.copy()
    full[...] = 0x1F
    res = O.run_page_union_call(**case, support=full, tags=tags, **common)
    assert res.tables[0].tolist() == case["block_table"][0, :10].tolist() and res.ctx[0] == 150
    np.testing.assert_allclose(res.out, d.out, atol=1e-14)
    # head 0 selects block 1, head 1 selects block 4 (tokens 128..149)
    part = sup.copy()
    part[0, 0, 0, 0] = 1 << 1
    part[0, 0, 1, 0] = 1 << 4
    res = O.run_page_union_call(**case, support=part, tags=tags, **common)
    assert res.pages[0].tolist() == [2, 3, 8, 9] and res.ctx[0] == 16 * 3 + 6
    assert res.tables[0].tolist() == case["block_table"][0, [2, 3, 8, 9]].tolist()
    toks = list(range(32, 64)) + list(range(128, 150))
    for h in range(2):
        ref, _ = brute_softmax_attention(case["q"][0, h].astype(float).tolist(),
                                         Kl[h][toks].astype(float).tolist(),
                                         Vl[h][toks].astype(float).tolist(), 1 / math.sqrt(8))
        np.testing.assert_allclose(res.out[0, h], ref, atol=1e-12)
    assert res.counters.tolist() == [0, 0, 0, 0]
    # stale position: dense fallback over every page
    stale = O.run_page_union_call(**case, support=part, tags=tags,
                                  **dict(common, row_position=[43]))
    assert stale.counters[0] == 1 and stale.ctx[0] == 150
    np.testing.assert_allclose(stale.out, d.out, atol=1e-14)
    # empty union: a data error for every head
    empty = O.run_page_union_call(**case, support=sup, tags=tags, **common)
    assert empty.counters[3] == 2 and np.isnan(empty.out).all() and empty.ctx[0] == 0
    # a bad id in a kept page poisons every head of the row; in a dropped page it does nothing
    bad = dict(case)
    bad["block_table"] = case["block_table"].copy()
    bad["block_table"][0, 5] = case["num_pages"] + 3
    ok = O.run_page_union_call(**bad, support=part, tags=tags, **common)
    assert ok.counters[3] == 0 and not np.isnan(ok.out).any()
    bad["block_table"][0, 8] = -2
    hit = O.run_page_union_call(**bad, support=part, tags=tags, **common)
    assert hit.counters[3] == 2 and np.isnan(hit.out).all() and hit.ctx[0] == 0
    # one selected block inside a 256-token page keeps the whole page
    case2, _, _ = paged_case(rng, 600, H=1, P=256)
    one = np.zeros((1, 1, 1, 1), np.uint32)
    one[0, 0, 0, 0] = 1 << 9                                 # tokens 288..319, page 1
    r2 = O.run_page_union_call(**case2, support=one, tags=tags[:, :1], layer=0,
                               row_request=[7], row_position=[42], required=2)
    assert r2.pages[0].tolist() == [1] and r2.ctx[0] == 256


# ----------------------------------------------------------------------------- O11 snapshot / restore

def test_snapshot_restore_resumes_reuse():
    """Discovery, offload (snapshot, then the slot is released and reused by
    another request), resume into another slot (restore): the reuse depth
    runs sparse with no fallback and gives exactly the never-offloaded
    output; without the restore it falls back to dense."""
    rng = np.random.default_rng(61)
    case, Kl, Vl = paged_case(rng, 150, H=2)
    sup, tags = state(slots=3, heads=2)
    common = dict(layer=0, row_request=[7], row_position=[42], required=1, eta=0.9)
    c = O.run_call(**case, modes=[O.DISCOVER], support=sup, tags=tags, **common)
    never = O.run_call(**case, modes=[O.SPARSE], support=c.support, tags=c.tags, **common)
    assert never.counters[0] == 0
    recs = O.snapshot_slots(c.support, c.tags, [0])
    # offload: slot 0 released, then taken by another request's discovery
    freed_sup, freed_tags = c.support.copy(), c.tags.copy()
    freed_sup[0] = 0
    freed_tags[0] = np.zeros((), O.TAG_DTYPE)
    other = O.run_call(**case, modes=[O.DISCOVER], support=freed_sup, tags=freed_tags,
                       **dict(common, row_request=[8]))
    # resume into slot 2
    sup2, tags2, err = O.restore_slots(other.support, other.tags, [2], recs)
    assert err == 0 and np.array_equal(sup2[2], c.support[0]) and sup2[2].any()
    assert np.array_equal(sup2[0], other.support[0])          # the other request is untouched
    resumed = O.run_call(**case, modes=[O.SPARSE], support=sup2, tags=tags2, slot_of_row=[2], **common)
    assert resumed.counters[0] == 0
    assert np.array_equal(resumed.out, never.out)
    # no restore: the resumed request finds no discovery for its token and runs dense
    lost = O.run_call(**case, modes=[O.SPARSE], support=other.support, tags=other.tags,
                      slot_of_row=[2], **common)
    dense = O.run_call(**case, modes=[O.DENSE])
    assert lost.counters[0] == 1 and np.array_equal(lost.out, dense.out)
    # a record of a slot out of range is empty; a destination out of range is an error
    empty = O.snapshot_slots(c.support, c.tags, [5])[0]
    assert not empty[0].any() and int(empty[1]["discoveries"][0]) == 0
    _, _, err = O.restore_slots(c.support, c.tags, [3], recs)
    assert err == 1


# ----------------------------------------------------------------------------- planted mistakes

def test_pins_catch_planted_mistakes(monkeypatch):
    """Each plausible slip in the oracle makes at least one pin above fail."""
    real_select, real_mass, real_stats = O.eta_select, O.block_mass, O.tile_stats

    def strict_cut(p, eta):                     # '>' instead of '>=' at the cut
        sel = real_select(p, eta)
        c = np.cumsum(np.asarray(p)[sel.order])
        K = int(np.nonzero(c > eta)[0][0]) + 1 if np.any(c > eta) else len(p)
        return O.Selection(sel.order, K, np.sort(sel.order[:K]), 0, c[K - 1], 0, 0)

    def index_desc(p, eta):                     # ties broken by descending index
        p = np.asarray(p)
        order = np.lexsort((-np.arange(len(p)), -p))
        c = np.cumsum(p[order])
        K = int(np.nonzero(c >= eta)[0][0]) + 1
        return O.Selection(order, K, np.sort(order[:K]), 0, c[K - 1], 0, 0)

    def no_norm(m, l, M, L):                    # forgot to divide by L
        return l * np.exp(m - M)

    def last_tile_full(s):                      # tile stats over a padded last tile
        m, l = real_stats(np.concatenate([s, np.zeros((-len(s)) % 32)]))
        return m, l

    real_lse_mass = O.lse_block_mass

    def lse_sign(s, lse):                       # exp(s + lse) instead of exp(s - lse)
        return real_lse_mass(s, -lse)

    def lse_full_blocks(s, lse):                # the partial last block dropped
        return real_lse_mass(s[: 32 * (len(s) // 32)] if len(s) >= 32 else s, lse)

    real_union_pages = O.union_pages

    def pages_whole_block(blocks, n, P):        # the block's end not clipped to the context
        return np.array(sorted({j for b in blocks for j in range(32 * b // P, (32 * b + 31) // P + 1)}),
                        dtype=np.int64)

    real_widen, real_stats_of = O.widen, O.tile_stats_of

    def widen_as_integers(x):                   # bf16 bit patterns taken as integer values
        x = np.asarray(x)
        return x.astype(np.float64)

    def widen_shift15(x):                       # one bit short of the fp32 layout
        x = np.asarray(x)
        if x.dtype == np.uint16:
            return (x.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
        return x.astype(np.float64)

    def stats_of_row_max(s, tokens):            # every block's max taken as the subset's max
        blk = np.asarray(tokens) // 32
        ids = np.unique(blk)
        mx = float(np.max(s))
        return np.full(len(ids), mx), np.array([np.exp(s[blk == b] - mx).sum() for b in ids])

    def stats_of_unclipped(s, tokens):          # sum over the block's first token only
        blk = np.asarray(tokens) // 32
        ids = np.unique(blk)
        m = np.array([s[blk == b].max() for b in ids])
        return m, np.array([np.exp(s[blk == b][:1] - mb).sum() for b, mb in zip(ids, m)])

    planted = [
        ("widen", widen_as_integers, lambda: test_widen_bf16_bit_patterns()),
        ("widen", widen_shift15, lambda: test_widen_bf16_bit_patterns()),
        ("tile_stats_of", stats_of_row_max, lambda: test_tile_stats_of_subset_brute_force()),
        ("tile_stats_of", stats_of_unclipped, lambda: test_tile_stats_of_subset_brute_force()),
        ("union_pages", pages_whole_block, lambda: test_union_pages_brute_force(8)),
        ("eta_select", strict_cut, lambda: test_selection_dominant_and_single_block()),
        ("eta_select", index_desc, lambda: test_selection_tie_break_equal_masses()),
        ("block_mass", no_norm, lambda: test_tile_stats_and_mass(95)),
        ("tile_stats", last_tile_full, lambda: test_tile_stats_and_mass(33)),
        ("lse_block_mass", lse_sign, lambda: test_lse_block_mass_is_softmax_block_sums(95)),
        ("lse_block_mass", lse_full_blocks, lambda: test_lse_block_mass_closed_form()),
    ]
    reals = {"eta_select": real_select, "block_mass": real_mass, "tile_stats": real_stats,
             "lse_block_mass": real_lse_mass, "union_pages": real_union_pages,
             "widen": real_widen, "tile_stats_of": real_stats_of}
    for name, fn, pin in planted:
        monkeypatch.setattr(O, name, fn)
        with pytest.raises(AssertionError):
            pin()
        monkeypatch.setattr(O, name, reals[name])
