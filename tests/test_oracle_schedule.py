"""Pins for the per-request split schedule oracle and for split/merge with
per-request split counts (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle import attention as OA
from oracle import schedule as OS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "schedule_hand.json")) as f:
        return json.load(f)


def test_hand_built_schedule():
    g = _golden()
    sc = OS.request_splits(g["seq_lens"], g["page_size"], g["table"], g["bucket_tokens"],
                           g["max_splits"])
    assert sc.tolist() == g["expect"]["split_counts"]
    wl = OS.work_list(g["seq_lens"], sc, g["capacity"])
    assert wl.tolist() == g["expect"]["work_list"]


def test_capacity_too_small_is_an_error():
    g = _golden()
    sc = OS.request_splits(g["seq_lens"], g["page_size"], g["table"], g["bucket_tokens"],
                           g["max_splits"])
    with pytest.raises(ValueError):
        OS.work_list(g["seq_lens"], sc, int(sc.sum()) - 1)


def test_constant_table_is_the_batch_wide_split():
    """A table holding one value S, requests of at least S pages: every request
    gets S splits and the list is batch_order x range(S)."""
    L = np.array([700, 1300, 640, 2000, 999])
    for S in (1, 3, 8):
        sc = OS.request_splits(L, 64, [S] * 5, 512, 64)
        assert sc.tolist() == [S] * len(L)
        wl = OS.work_list(L, sc, len(L) * S)
        order = [3, 1, 4, 0, 2]
        assert wl.tolist() == [b * 256 + s for b in order for s in range(S)]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_generated_schedule_invariants(seed):
    rng = np.random.default_rng(seed)
    B, ps, bt = 40, 16, 256
    L = rng.integers(-3, 3000, size=B)
    table = rng.integers(1, 20, size=6)
    smax = 12
    sc = OS.request_splits(L, ps, table, bt, smax)
    cap = B * smax + 7
    wl = OS.work_list(L, sc, cap)
    items = [int(x) for x in wl if x >= 0]
    assert len(items) == int(sc.sum()) and np.all(wl[len(items):] == -1)
    # every (b, s < S_b) exactly once
    assert sorted(items) == sorted(b * 256 + s for b in range(B) for s in range(sc[b]))
    # requests appear in non-increasing length, each as one run of ascending splits
    Lc = np.maximum(L, 0)
    runs = [items[0] // 256]
    for a, c in zip(items[:-1], items[1:]):
        if c // 256 != a // 256:
            runs.append(c // 256)
            assert c % 256 == 0
        else:
            assert c == a + 1
    assert len(runs) == B and all(Lc[x] >= Lc[y] for x, y in zip(runs[:-1], runs[1:]))
    # the count against its definition, written as range checks
    for b in range(B):
        n = int(np.ceil(Lc[b] / ps))
        k = min(max(int(np.ceil(Lc[b] / bt)), 1), len(table)) - 1
        assert 1 <= sc[b] <= max(1, n) and sc[b] <= smax and sc[b] <= max(1, table[k])
        assert sc[b] == max(1, min(table[k], n, smax))


@pytest.mark.parametrize("causal,qn", [(False, 1), (True, 3)])
def test_per_request_splits_merge_to_the_unsplit_result(causal, qn):
    """Splitting each request into its own number of page-aligned splits and
    merging only those reproduces un-split attention; slots past a request's
    count hold garbage that the merge must not read."""
    rng = np.random.Generator(np.random.PCG64(7))
    B, Hq, Hkv, D, ps = 3, 4, 2, 16, 4
    L = np.array([37, 23, 0])
    P = 24
    perm = rng.permutation(P)
    pt = np.zeros((B, 10), dtype=np.int64)
    k = 0
    for b in range(B):
        n = -(-L[b] // ps)
        pt[b, :n] = perm[k:k + n]
        k += n
    q = rng.standard_normal((B, qn, Hq, D))
    kp = rng.standard_normal((P, ps, Hkv, D))
    vp = rng.standard_normal((P, ps, Hkv, D))
    full, flse = OA.decode_attention(q, kp, vp, pt, L, ps, 0.3, causal=causal)
    S = 7
    counts = np.array([7, 2, 1])
    o, lse = OA.split_partials(q, kp, vp, pt, L, ps, 0.3, S, causal=causal, split_counts=counts)
    for b in range(B):                                # unused slots: garbage
        o[b, :, :, counts[b]:] = 1e30
        lse[b, :, :, counts[b]:] = 50.0
    out, olse = OA.merge(o, lse, split_counts=counts)
    assert np.allclose(out, full, rtol=0, atol=1e-12)
    fin = np.isfinite(flse)
    assert np.array_equal(fin, np.isfinite(olse))
    assert np.allclose(olse[fin], flse[fin], rtol=0, atol=1e-12)
