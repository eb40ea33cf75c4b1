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
