"""Pins for the fp64 attention oracle (CPU only).

Each check ties the oracle to something other than itself: hand-derived
closed-form cases (tests/golden/attention_hand.json), a library routine
(torch's fp64 CPU scaled_dot_product_attention) on dense inputs generated
before they are scattered into pages, and closed forms / invariances of
softmax attention.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as OA

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lnparse(x):
    if isinstance(x, str):
        return {"-inf": -math.inf, "0": 0.0}.get(x, None) if not x.startswith("ln") else math.log(float(x[2:]))
    return x


def _load_attention_golden():
    with open(os.path.join(GOLDEN, "attention_hand.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _load_attention_golden()["cases"], ids=lambda c: c["name"])
def test_hand_derived_cases(case):
    q = np.array(case["q"], dtype=np.float64)
    k = np.array(case["k_pool"], dtype=np.float64)
    v = np.array(case["v_pool"], dtype=np.float64)
    out, lse = OA.decode_attention(q, k, v, np.array(case["page_table"]), np.array(case["seq_lens"]),
                                   case["page_size"], case["scale"], causal=case["causal"])
    np.testing.assert_allclose(out, np.array(case["out"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(case["lse"]), rtol=0, atol=1e-12)


def test_hand_derived_split_case():
    g = _load_attention_golden()
    base = {c["name"]: c for c in g["cases"]}
    for sc in g["split_cases"]:
        case = base[sc["base"]]
        q = np.array(case["q"], dtype=np.float64)
        k = np.array(case["k_pool"], dtype=np.float64)
        v = np.array(case["v_pool"], dtype=np.float64)
        o, l = OA.split_partials(q, k, v, np.array(case["page_table"]), np.array(case["seq_lens"]),
                                 case["page_size"], case["scale"], sc["num_splits"], causal=case["causal"])
        np.testing.assert_allclose(o, np.array(sc["o_partial"]), rtol=0, atol=1e-12)
        want = np.vectorize(_lnparse, otypes=[np.float64])(np.array(sc["lse_partial"], dtype=object))
        assert np.array_equal(np.isinf(l), np.isinf(want))
        np.testing.assert_allclose(l[~np.isinf(l)], want[~np.isinf(want)], rtol=0, atol=1e-12)
        out, lse = OA.merge(o, l)
        np.testing.assert_allclose(out, np.array(case["out"]), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, np.array(case["lse"]), rtol=0, atol=1e-12)


def _dense_problem(rng, B, qn, Hq, Hkv, D, page_size, lengths, extra_pages=3):
    """Dense K/V per request first, then scattered into a permuted pool by this test
    (independently of the oracle's gather)."""
    lengths = np.asarray(lengths)
    dense_k = [rng.standard_normal((L, Hkv, D)) for L in lengths]
    dense_v = [rng.standard_normal((L, Hkv, D)) for L in lengths]
    n = (lengths + page_size - 1) // page_size
    P = int(n.sum()) + extra_pages
    perm = rng.permutation(P)
    kpool = rng.standard_normal((P, page_size, Hkv, D)) * 100.0  # junk where unused
    vpool = rng.standard_normal((P, page_size, Hkv, D)) * 100.0
    pt = np.zeros((B, max(1, int(n.max()))), dtype=np.int64)
    off = 0
    for b in range(B):
        for j in range(n[b]):
            p = perm[off]
            off += 1
            pt[b, j] = p
            lo, hi = j * page_size, min((j + 1) * page_size, lengths[b])
            kpool[p, : hi - lo] = dense_k[b][lo:hi]
            vpool[p, : hi - lo] = dense_v[b][lo:hi]
    q = rng.standard_normal((B, qn, Hq, D))
    return q, kpool, vpool, pt, dense_k, dense_v


@pytest.mark.parametrize("causal,qn", [(False, 1), (True, 4), (False, 3)])
def test_matches_library_sdpa_on_dense_inputs(causal, qn):
    rng = np.random.default_rng(7)
    B, Hq, Hkv, D, S = 3, 8, 2, 16, 4
    lengths = [1, 13, 29]
    scale = 0.37
    q, kp, vp, pt, dk, dv = _dense_problem(rng, B, qn, Hq, Hkv, D, S, lengths)
    out, lse = OA.decode_attention(q, kp, vp, pt, np.array(lengths), S, scale, causal=causal)
    for b, L in enumerate(lengths):
        qq = torch.from_numpy(q[b]).permute(1, 0, 2).unsqueeze(0)           # [1, Hq, qn, D]
        kk = torch.from_numpy(dk[b]).permute(1, 0, 2).unsqueeze(0)          # [1, Hkv, L, D]
        vv = torch.from_numpy(dv[b]).permute(1, 0, 2).unsqueeze(0)
        mask = None
        if causal:
            i = torch.arange(qn).unsqueeze(1)
            t = torch.arange(L).unsqueeze(0)
            mask = t < (L - (qn - 1 - i))                                    # [qn, L]
        ref = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=scale, enable_gqa=True)
        ref = ref[0].permute(1, 0, 2).numpy()                                # [qn, Hq, D]
        if causal:
            # rows with nothing visible: the oracle defines them as 0; SDPA gives NaN
            for i in range(qn):
                if L - (qn - 1 - i) <= 0:
                    ref[i] = 0.0
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-12)
        # lse against an independent logsumexp of the same scores
        Gs = Hq // Hkv
        for i in range(qn):
            nvis = L - (qn - 1 - i) if causal else L
            for h in range(Hq):
                if nvis <= 0:
                    assert lse[b, i, h] == -math.inf
                    continue
                s = scale * dk[b][:nvis, h // Gs] @ q[b, i, h]
                want = torch.logsumexp(torch.from_numpy(s), 0).item()
                assert abs(lse[b, i, h] - want) < 1e-12


def test_length_one_gives_v0_exactly():
    rng = np.random.default_rng(1)
    q, kp, vp, pt, dk, dv = _dense_problem(rng, 2, 1, 4, 2, 8, 4, [1, 1])
    out, lse = OA.decode_attention(q, kp, vp, pt, np.array([1, 1]), 4, 0.5)
    for b in range(2):
        for h in range(4):
            assert np.array_equal(out[b, 0, h], dv[b][0, h // 2])
            assert lse[b, 0, h] == pytest.approx(0.5 * dk[b][0, h // 2] @ q[b, 0, h], abs=1e-14)


def test_equal_scores_give_mean_of_v():
    rng = np.random.default_rng(2)
    L = [5, 17]
    q, kp, vp, pt, dk, dv = _dense_problem(rng, 2, 1, 2, 1, 8, 4, L)
    q[:] = 0.0
    out, lse = OA.decode_attention(q, kp, vp, pt, np.array(L), 4, 1.0)
    for b in range(2):
        np.testing.assert_allclose(out[b, 0, 0], dv[b][:, 0].mean(axis=0), rtol=0, atol=1e-13)
        assert lse[b, 0, 0] == pytest.approx(math.log(L[b]), abs=1e-13)
    # all K rows equal, q arbitrary: scores equal too -> mean, lse = s + ln L
    q, kp, vp, pt, dk, dv = _dense_problem(rng, 1, 1, 1, 1, 8, 4, [9])
    krow = rng.standard_normal(8)
    for p in range(kp.shape[0]):
        kp[p, :, 0] = krow
    out, lse = OA.decode_attention(q, kp, vp, pt, np.array([9]), 4, 0.25)
    np.testing.assert_allclose(out[0, 0, 0], dv[0][:, 0].mean(axis=0), rtol=0, atol=1e-13)
    assert lse[0, 0, 0] == pytest.approx(0.25 * krow @ q[0, 0, 0] + math.log(9), abs=1e-12)


def test_two_tokens_closed_form():
    rng = np.random.default_rng(3)
    q, kp, vp, pt, dk, dv = _dense_problem(rng, 1, 1, 1, 1, 8, 4, [2])
    out, _ = OA.decode_attention(q, kp, vp, pt, np.array([2]), 4, 0.3)
    s0 = 0.3 * dk[0][0, 0] @ q[0, 0, 0]
    s1 = 0.3 * dk[0][1, 0] @ q[0, 0, 0]
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    want = sig(s0 - s1) * dv[0][0, 0] + sig(s1 - s0) * dv[0][1, 0]
    np.testing.assert_allclose(out[0, 0, 0], want, rtol=0, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(4)
    B, Hq, Hkv, D, S = 2, 6, 2, 8, 4
    L = [7, 12]
    q, kp, vp, pt, _, _ = _dense_problem(rng, B, 1, Hq, Hkv, D, S, L)
    out, lse = OA.decode_attention(q, kp, vp, pt, np.array(L), S, 0.4)
    G = Hq // Hkv
    kp_mha = np.repeat(kp, G, axis=2)  # head h of the MHA pool = kv-head h // G
    vp_mha = np.repeat(vp, G, axis=2)
    out2, lse2 = OA.decode_attention(q, kp_mha, vp_mha, pt, np.array(L), S, 0.4)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_mtp_query_equals_single_query_decode_on_shorter_cache():
    rng = np.random.default_rng(5)
    qn, L = 4, 11
    q, kp, vp, pt, _, _ = _dense_problem(rng, 1, qn, 4, 2, 8, 4, [L])
    out, lse = OA.decode_attention(q, kp, vp, pt, np.array([L]), 4, 0.2, causal=True)
    for i in range(qn):
        o1, l1 = OA.decode_attention(q[:, i:i + 1], kp, vp, pt, np.array([L - (qn - 1 - i)]), 4, 0.2)
        np.testing.assert_array_equal(out[:, i], o1[:, 0])
        np.testing.assert_array_equal(lse[:, i], l1[:, 0])


@pytest.mark.parametrize("S", [1, 2, 3, 4, 7, 8, 16])
def test_split_then_merge_equals_unsplit(S):
    rng = np.random.default_rng(6)
    L = [0, 1, 5, 16, 37, 100]
    q, kp, vp, pt, _, _ = _dense_problem(rng, len(L), 2, 4, 1, 8, 16 // 4, L)
    for causal in (False, True):
        out, lse = OA.decode_attention(q, kp, vp, pt, np.array(L), 4, 0.3, causal=causal)
        o, l = OA.split_partials(q, kp, vp, pt, np.array(L), 4, 0.3, S, causal=causal)
        m_out, m_lse = OA.merge(o, l)
        np.testing.assert_allclose(m_out, out, rtol=0, atol=1e-12)
        assert np.array_equal(np.isinf(m_lse), np.isinf(lse))
        np.testing.assert_allclose(m_lse[np.isfinite(lse)], lse[np.isfinite(lse)], rtol=0, atol=1e-12)
        # empty splits are exactly (0, -inf)
        emp = np.isinf(l)
        assert np.all(o[emp] == 0.0)


def test_split_ranges_partition_the_tokens():
    for L in [0, 1, 15, 16, 17, 37, 100, 1000]:
        for S in [1, 2, 3, 4, 5, 8, 32]:
            rs = [OA.split_token_range(L, 16, S, s) for s in range(S)]
            cover = []
            for a, b in rs:
                assert a <= b
                cover.extend(range(a, b))
                if a < b:
                    assert a % 16 == 0  # page aligned starts
            assert cover == list(range(L))


def test_page_permutation_invariance_is_exact():
    rng = np.random.default_rng(8)
    L = [9, 33, 64]
    q, kp, vp, pt, _, _ = _dense_problem(rng, 3, 1, 4, 2, 8, 8, L)
    out, lse = OA.decode_attention(q, kp, vp, pt, np.array(L), 8, 0.5)
    P = kp.shape[0]
    perm = rng.permutation(P)        # new physical position of old page p is perm[p]
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    pt2 = perm[pt]
    out2, lse2 = OA.decode_attention(q, kp2, vp2, pt2, np.array(L), 8, 0.5)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)

