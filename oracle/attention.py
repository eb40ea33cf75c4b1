"""fp64 CPU oracle for paged GQA decode attention (split-KV stage 1, LSE merge).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and never calls it.

What is computed, and where the pages fix it:

* The kernels being reproduced are the decode kernels listed in LightLLM
  PR #1549 "feat(autotune): separate general and decode attention warmup",
  section "Covered decode kernels": a KV-cache decode attention whose tunable
  is ``num_splits``, a GQA flash-decode "stage 1", INT8 / INT4 KV stage-1
  variants and a two-stage MTP attention.  The pages do not print the
  attention formula; the plainest reading, used here, is softmax attention
  ``out = softmax(scale * q K^T) V`` per query head, with the query head ``h``
  reading kv-head ``h // G`` (``G = Hq / Hkv``, contiguous GQA groups).
* Split-KV followed by a log-sum-exp merge reaches that same result exactly
  (up to rounding order), so the un-split oracle is the definition written
  out; the split/merge functions below exist to check stage outputs on their
  own.
* MTP verify rows (several query tokens per request; SGLang PR #36219 digest,
  section "Key source snippets", TARGET_VERIFY with
  ``decode_num_tokens_per_req`` tokens per request) are causal within the
  request: query ``i`` of ``q`` sees tokens ``t < L - (q - 1 - i)``
  (bottom-right alignment, the new tokens already being in the cache).
* Logical token ``t`` of request ``b`` lives in physical page
  ``page_table[b, t // page_size]`` at slot ``t % page_size``.

Everything is float64.  Inputs are numpy arrays already widened exactly from
their storage type (see ``oracle.quant`` for the quantised caches).
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -math.inf


def gather_tokens(pool: np.ndarray, page_row: np.ndarray, length: int, page_size: int) -> np.ndarray:
    """Dense copy of the first ``length`` logical tokens of one request.

    ``pool`` is ``[num_pages, page_size, ...]``; the result is ``[length, ...]``.
    """
    t = np.arange(int(length))
    return pool[page_row[t // page_size], t % page_size]


def visible_length(L: int, q_per_req: int, i: int, causal: bool) -> int:
    """Number of cache tokens query ``i`` (of ``q_per_req``) attends to."""
    if not causal:
        return int(L)
    return max(0, int(L) - (q_per_req - 1 - i))


def attend(qvec: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """softmax(scale * K qvec) V and its natural-log normaliser, in fp64.

    ``qvec`` [D], ``K`` [n, D], ``V`` [n, D].  With ``n == 0`` the result is the
    zero vector and ``lse = -inf`` (nothing to attend to).
    """
    n = K.shape[0]
    if n == 0:
        return np.zeros(V.shape[1], dtype=np.float64), NEG_INF
    s = scale * (K @ qvec)
    m = s.max()
    w = np.exp(s - m)
    l = w.sum()
    return (w @ V) / l, m + math.log(l)


def decode_attention(q, k_pool, v_pool, page_table, seq_lens, page_size, scale,
                     causal=False):
    """Full decode attention for a batch.

    q          [B, qn, Hq, D]  float64
    k_pool     [P, page_size, Hkv, D] float64 (already dequantised)
    v_pool     [P, page_size, Hkv, D] float64
    page_table [B, max_pages] int
    seq_lens   [B] int   (negative treated as 0)
    Returns (out [B, qn, Hq, D], lse [B, qn, Hq]).
    """
    B, qn, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, qn, Hq, D), dtype=np.float64)
    lse = np.full((B, qn, Hq), NEG_INF, dtype=np.float64)
    for b in range(B):
        L = max(0, int(seq_lens[b]))
        Kb = gather_tokens(k_pool, page_table[b], L, page_size)
        Vb = gather_tokens(v_pool, page_table[b], L, page_size)
        for i in range(qn):
            n = visible_length(L, qn, i, causal)
            for h in range(Hq):
                g = h // G
                out[b, i, h], lse[b, i, h] = attend(q[b, i, h], Kb[:n, g], Vb[:n, g], scale)
    return out, lse


def split_token_range(L: int, page_size: int, num_splits: int, s: int):
    """Token range [t0, t1) handled by split ``s``.

    The pages name ``num_splits`` as the tunable of the KV-cache decode kernel
    and a separate "stage 1" but fix no partition.  Reading used here:
    page-aligned, ``c = ceil(n / S)`` whole pages per split where
    ``n = ceil(L / page_size)``; split ``s`` covers pages [s*c, min((s+1)*c, n))
    clipped to ``L`` tokens.  Splits past the last page are empty.
    """
    L = max(0, int(L))
    n = -(-L // page_size)
    c = -(-n // num_splits) if n else 0
    p0 = min(s * c, n)
    p1 = min((s + 1) * c, n)
    return min(p0 * page_size, L), min(p1 * page_size, L)


def split_partials(q, k_pool, v_pool, page_table, seq_lens, page_size, scale,
                   num_splits, causal=False, split_counts=None):
    """Stage 1: per-split normalised partial outputs and their LSE.

    o_partial [B, qn, Hq, S, D] = softmax over the split's visible tokens, V-weighted;
    lse_partial [B, qn, Hq, S]  = log-sum-exp of the split's scaled scores.
    An empty split (no visible token) gives (0, -inf).  With ``split_counts``
    ([B], each <= S), request b is partitioned into ``split_counts[b]`` splits
    and its slots from ``split_counts[b]`` on stay (0, -inf).
    """
    B, qn, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    G = Hq // Hkv
    S = num_splits
    o = np.zeros((B, qn, Hq, S, D), dtype=np.float64)
    lse = np.full((B, qn, Hq, S), NEG_INF, dtype=np.float64)
    for b in range(B):
        L = max(0, int(seq_lens[b]))
        Kb = gather_tokens(k_pool, page_table[b], L, page_size)
        Vb = gather_tokens(v_pool, page_table[b], L, page_size)
        Sb = S if split_counts is None else int(split_counts[b])
        for s in range(Sb):
            t0, t1 = split_token_range(L, page_size, Sb, s)
            for i in range(qn):
                n = visible_length(L, qn, i, causal)
                a, e = t0, min(t1, n)
                if e <= a:
                    continue
                for h in range(Hq):
                    g = h // G
                    o[b, i, h, s], lse[b, i, h, s] = attend(q[b, i, h], Kb[a:e, g], Vb[a:e, g], scale)
    return o, lse


def merge(o_partial: np.ndarray, lse_partial: np.ndarray, split_counts=None):
    """Stage 2: combine split partials by their log-sum-exp.

    out = sum_s w_s O_s / sum_s w_s with w_s = exp(lse_s - max_s lse_s);
    lse = max + ln(sum_s w_s).  Rows whose splits are all empty give (0, -inf).
    The pages name the two stages and the reuse of stage-2 inputs (LightLLM
    PR #1549, sections "Covered decode kernels" and "Validation"); this is the
    standard recombination of softmax over a partition of the keys.
    With ``split_counts`` ([B]; the partials' leading axis is B), the rows of
    request b combine only their first ``split_counts[b]`` slots.
    """
    S = lse_partial.shape[-1]
    lead = lse_partial.shape[:-1]
    D = o_partial.shape[-1]
    o2 = o_partial.reshape(-1, S, D)
    l2 = lse_partial.reshape(-1, S)
    rows_per_req = o2.shape[0] // lead[0]
    out = np.zeros((o2.shape[0], D), dtype=np.float64)
    lse = np.full(o2.shape[0], NEG_INF, dtype=np.float64)
    for r in range(o2.shape[0]):
        n = S if split_counts is None else int(split_counts[r // rows_per_req])
        m = l2[r, :n].max()
        if m == NEG_INF:
            continue
        w = np.exp(l2[r, :n] - m)
        tot = w.sum()
        out[r] = (w @ o2[r, :n]) / tot
        lse[r] = m + math.log(tot)
    return out.reshape(*lead, D), lse.reshape(lead)
