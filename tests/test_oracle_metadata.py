"""Pins for the integer metadata oracle (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle import metadata as OM
from decode_attention_paged_gqa_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "metadata_hand.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("mode,key,extra", [
    (OM.Q_STRIDED, "cu_seqlens_q_strided", {}),
    (OM.Q_CUMSUM, "cu_seqlens_q_cumsum", {"q_in": "q_lens"}),
    (OM.Q_PRESET, "cu_seqlens_q_preset", {"q_in": "cu_q_preset"}),
])
def test_hand_built_batch(mode, key, extra):
    g = _golden()
    q_in = np.array(g[extra["q_in"]]) if "q_in" in extra else None
    md = OM.metadata(g["seq_lens"], g["req_pool_indices"], np.array(g["req_to_token"]),
                     g["page_size"], g["max_pages"], q_mode=mode, q_in=q_in, q_stride=g["q_stride"])
    e = g["expect"]
    assert md["cache_seqlens"].tolist() == e["cache_seqlens"]
    assert md["cu_seqlens_k"].tolist() == e["cu_seqlens_k"]
    assert md["page_table"].tolist() == e["page_table"]
    assert md["cu_seqlens_q"].tolist() == e[key]
    assert md["batch_order"].tolist() == e["batch_order"]


def test_paged_layout_predicate_rejects_broken_layouts():
    """paged_layout_holds must say False whenever one token slot is not where
    the page table puts it: a moved slot, two swapped pages, a shifted
    offset inside a page, or a request row read through the wrong index."""
    w = W.BF16_B16.scaled(batch=4, length=200)
    rng = np.random.Generator(np.random.PCG64(1000 + w.seed))
    L = W.draw_lengths(w, rng)
    pt, r2t, rpi, P = W.build_layout(w, L, rng)
    S = w.page_size
    assert OM.paged_layout_holds(pt, L, rpi, r2t, S)
    r = r2t.copy()
    r[rpi[2], 137] += 1  # one slot of request 2 moved by one
    assert not OM.paged_layout_holds(pt, L, rpi, r, S)
    p = pt.copy()
    p[1, [0, 2]] = p[1, [2, 0]]  # two pages of request 1 swapped in the table
    assert not OM.paged_layout_holds(p, L, rpi, r2t, S)
    r = r2t.copy()
    r[rpi[0], :S] = r[rpi[0], :S][::-1]  # offsets inside the first page reversed
    assert not OM.paged_layout_holds(pt, L, rpi, r, S)
    assert not OM.paged_layout_holds(pt, L, rpi[::-1].copy(), r2t, S)  # rows crossed
    # tokens past a request's length do not matter
    r = r2t.copy()
    r[rpi[3], int(L[3]):] = -7
    assert OM.paged_layout_holds(pt, L, rpi, r, S)


@pytest.mark.parametrize("w", [W.TINY_FP32, W.BF16_B16.scaled(batch=5, length=300),
                               W.RAGGED_B64.scaled(batch=9, length_lo=3, length_hi=500)],
                         ids=lambda w: w.name)
def test_closed_forms_on_generated_batches(w):
    rng = np.random.Generator(np.random.PCG64(1000 + w.seed))
    L = W.draw_lengths(w, rng)
    pt, r2t, rpi, P = W.build_layout(w, L, rng)
    assert OM.paged_layout_holds(pt, L, rpi, r2t, w.page_size)
    md = OM.metadata(L, rpi, r2t, w.page_size, pt.shape[1], q_mode=OM.Q_STRIDED, q_stride=3)
    # cu_k differences are the lengths; starts at 0
    assert md["cu_seqlens_k"][0] == 0
    assert np.array_equal(np.diff(md["cu_seqlens_k"]), L)
    # page table equals the page assignment the generator scattered (tail 0)
    assert np.array_equal(md["page_table"], pt)
    n = (L + w.page_size - 1) // w.page_size
    for b in range(len(L)):
        assert np.all(md["page_table"][b, n[b]:] == 0)
    assert md["cu_seqlens_q"].tolist() == [3 * b for b in range(len(L) + 1)]
    order = md["batch_order"]
    assert sorted(order.tolist()) == list(range(len(L)))          # a permutation
    Ls = L[order]
    assert np.all(Ls[:-1] >= Ls[1:])                               # non-increasing lengths
    for a, b in zip(order[:-1], order[1:]):                        # ties keep index order
        if L[a] == L[b]:
            assert a < b


def test_sentinels_never_produce_negative_or_out_of_range_ids():
    rng = np.random.default_rng(0)
    R, W_, S = 6, 40, 8
    r2t = rng.integers(-3, 200, size=(R, W_)).astype(np.int32)
    seq = np.array([-5, 0, 40, 17, 41, 3])
    rpi = np.array([-1, 2, 5, 6, 0, -7])
    md = OM.metadata(seq, rpi, r2t, S, 6)
    assert np.all(md["page_table"] >= 0)
    assert md["cache_seqlens"].tolist() == [0, 0, 40, 17, 41, 3]
    # rpi 6 is past the table (R = 6) and rpi -1 / -7 are sentinels -> zero rows
    assert np.all(md["page_table"][[0, 3, 5]] == 0)
    # b=4 has L=41 -> 6 pages, column 40 is past the table width -> 0
    assert md["page_table"][4, 5] == 0
    for j in range(5):
        slot = r2t[0, j * S]
        assert md["page_table"][4, j] == (slot // S if slot >= 0 else 0)


def test_cumsum_and_preset_modes():
    seq = np.array([3, 4])
    r2t = np.zeros((2, 8), dtype=np.int32)
    md = OM.metadata(seq, [0, 1], r2t, 4, 2, q_mode=OM.Q_CUMSUM, q_in=np.array([2, 5]))
    assert md["cu_seqlens_q"].tolist() == [0, 2, 7]
    md = OM.metadata(seq, [0, 1], r2t, 4, 2, q_mode=OM.Q_PRESET, q_in=np.array([0, 9, 11]))
    assert md["cu_seqlens_q"].tolist() == [0, 9, 11]


# ---------------------------------------------------------------- SWA translation
def _swa_golden():
    with open(os.path.join(GOLDEN, "metadata_swa_hand.json")) as f:
        return json.load(f)


def test_swa_hand_built_batch():
    g, s = _golden(), _swa_golden()
    args = (g["seq_lens"], g["req_pool_indices"], np.array(g["req_to_token"]), g["page_size"],
            g["max_pages"])
    md = OM.metadata(*args, full_to_swa=np.array(s["full_to_swa"]))
    assert md["swa_page_table"].tolist() == s["expect"]["swa_page_table"]
    assert md["page_table"].tolist() == g["expect"]["page_table"]  # the full table is unchanged
    cut = OM.swa_page_table(*args, np.array(s["full_to_swa"][:40]))
    assert cut.tolist() == s["expect"]["swa_page_table_mapping40"]


def _generated(w):
    rng = np.random.Generator(np.random.PCG64(1000 + w.seed))
    L = W.draw_lengths(w, rng)
    pt, r2t, rpi, P = W.build_layout(w, L, rng)
    return L, pt, r2t, rpi, P, rng


SWA_CASES = [W.TINY_FP32, W.RAGGED_B64.scaled(batch=9, length_lo=3, length_hi=500)]


@pytest.mark.parametrize("w", SWA_CASES, ids=lambda w: w.name)
def test_swa_identity_mapping_gives_the_full_table(w):
    L, pt, r2t, rpi, P, _ = _generated(w)
    ident = np.arange(P * w.page_size)
    swa = OM.swa_page_table(L, rpi, r2t, w.page_size, pt.shape[1], ident)
    assert np.array_equal(swa, pt)


@pytest.mark.parametrize("w", SWA_CASES, ids=lambda w: w.name)
def test_swa_page_permutation_and_evictions(w):
    """A page-aligned SWA pool: full page p lives in SWA page pi(p), or is not
    resident (-1).  The SWA table must be pi applied to the full table, 0 where
    the page is evicted and in the tail."""
    L, pt, r2t, rpi, P, rng = _generated(w)
    ps = w.page_size
    pi = rng.permutation(P + 5)[:P]                # SWA pool is a bit larger
    evicted = rng.random(P) < 0.3
    f2s = np.empty(P * ps, dtype=np.int64)
    for p in range(P):
        f2s[p * ps:(p + 1) * ps] = -1 if evicted[p] else pi[p] * ps + np.arange(ps)
    swa = OM.swa_page_table(L, rpi, r2t, ps, pt.shape[1], f2s)
    n = (L + ps - 1) // ps
    for b in range(len(L)):
        for j in range(pt.shape[1]):
            want = 0 if j >= n[b] or evicted[pt[b, j]] else pi[pt[b, j]]
            assert swa[b, j] == want


def test_swa_guards():
    """Sentinel slots are not looked up (mapping[-1] would be the last entry),
    slots past the mapping give 0, negative mapped slots give 0."""
    r2t = np.array([[-1, -1, 8, 9, 4, 5]], dtype=np.int32)  # pages: sentinel, 4, 2
    f2s = np.array([100, 101, 102, 103, -4, -4, 40, 41, 77])  # slot 4 -> -4, slot 8 -> 77
    swa = OM.swa_page_table([6], [0], r2t, 2, 4, f2s)
    assert swa.tolist() == [[0, 77 // 2, 0, 0]]
    swa = OM.swa_page_table([6], [0], r2t, 2, 4, f2s[:8])       # slot 8 now past the end
    assert swa.tolist() == [[0, 0, 0, 0]]
    # the tail past ceil(L / page_size) is 0 even where the row holds valid slots
    r2t = np.arange(8, dtype=np.int32)[None]
    swa = OM.swa_page_table([3], [0], r2t, 2, 4, np.arange(8) + 10)
    assert swa.tolist() == [[5, 6, 0, 0]]
