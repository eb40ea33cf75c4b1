"""Integer oracle for the per-batch decode metadata prelude.  TEST INFRASTRUCTURE ONLY.

SGLang PR #29843 digest (fused TRT-LLM MHA CUDA-graph metadata kernel),
sections "Features and motivation" and "Implementation breakdown": at every
graph replay the backend rebuilds ``cache_seqlens``, ``cu_seqlens_k/q`` and
``page_table``; the fused kernel computes all of them in one launch with one
program per batch row, supports three q modes (preset / cumsum / strided)
and guards a -1 sentinel; its tests cover a zero-padded page-table tail.

Readings taken where the page is silent:
* ``cache_seqlens[b] = max(seq_lens[b], 0)``  (a negative length is a sentinel).
* ``cu_seqlens_k`` is the exclusive prefix sum of ``cache_seqlens``, length B+1.
* ``cu_seqlens_q``: strided -> ``b * q_stride`` for b = 0..B; cumsum -> exclusive
  prefix of ``max(q_lens[b], 0)``; preset -> copy of the caller's B+1 values.
* ``page_table[b, j] = req_to_token[rpi[b], j * page_size] // page_size`` for
  ``j < ceil(cache_seqlens[b] / page_size)``; every other entry (the tail) is 0.
  A negative / out-of-range ``rpi[b]``, a slot column past the table width, or
  a negative slot gives 0 instead of an index.
* ``batch_order`` (a scheduling aid the pages do not have): request indices
  sorted by descending ``cache_seqlens``, ties by ascending index.
* SWA translation (same section: the fused kernel performs it, fed by a
  full-to-SWA slot mapping the backend prepares): layers with a sliding
  window keep their K/V in a second pool, and ``full_to_swa[slot]`` is the
  SWA-pool slot holding the token of full-pool ``slot``.  The SWA page table
  is built like the full one from the translated first slot of every page:
  ``swa_page_table[b, j] = full_to_swa[slot] // page_size``.  A guarded full
  slot (the cases that give 0 above), a slot past the end of the mapping, or
  a negative mapped slot (a token no longer resident in the SWA pool) gives 0.
All arithmetic is exact integer arithmetic (Python ints).
"""
from __future__ import annotations

import numpy as np

Q_STRIDED = 0
Q_CUMSUM = 1
Q_PRESET = 2


def _first_slot(r2t, rpi_b, j, page_size):
    """Full-pool slot of logical page ``j`` of a request, or None when guarded
    (invalid pool row, column past the table, negative slot)."""
    R, W = r2t.shape
    if rpi_b < 0 or rpi_b >= R:
        return None
    col = j * page_size
    if col >= W:
        return None
    slot = int(r2t[rpi_b, col])
    return slot if slot >= 0 else None


def swa_page_table(seq_lens, req_pool_indices, req_to_token, page_size, max_pages, full_to_swa):
    """[B, max_pages] page table of the SWA pool, through the full-to-SWA slot map."""
    r2t = np.asarray(req_to_token)
    f2s = [int(x) for x in np.asarray(full_to_swa).reshape(-1)]
    rpi = [int(x) for x in np.asarray(req_pool_indices).reshape(-1)]
    seq = [max(int(x), 0) for x in np.asarray(seq_lens).reshape(-1)]
    pt = np.zeros((len(seq), max_pages), dtype=np.int64)
    for b, L in enumerate(seq):
        n = -(-L // page_size)
        for j in range(min(n, max_pages)):
            slot = _first_slot(r2t, rpi[b], j, page_size)
            if slot is None or slot >= len(f2s):
                continue
            swa = f2s[slot]
            pt[b, j] = swa // page_size if swa >= 0 else 0
    return pt


def metadata(seq_lens, req_pool_indices, req_to_token, page_size, max_pages,
             q_mode=Q_STRIDED, q_in=None, q_stride=1, full_to_swa=None):
    """Returns dict(cache_seqlens [B], cu_seqlens_k [B+1], cu_seqlens_q [B+1],
    page_table [B, max_pages], batch_order [B]) as int64 numpy arrays, plus
    swa_page_table [B, max_pages] when ``full_to_swa`` is given."""
    seq_lens = [int(x) for x in np.asarray(seq_lens).reshape(-1)]
    rpi = [int(x) for x in np.asarray(req_pool_indices).reshape(-1)]
    r2t = np.asarray(req_to_token)
    R, W = r2t.shape
    B = len(seq_lens)

    cache = [max(L, 0) for L in seq_lens]
    cu_k = [0]
    for L in cache:
        cu_k.append(cu_k[-1] + L)

    if q_mode == Q_STRIDED:
        cu_q = [b * int(q_stride) for b in range(B + 1)]
    elif q_mode == Q_CUMSUM:
        ql = [max(int(x), 0) for x in np.asarray(q_in).reshape(-1)[:B]]
        cu_q = [0]
        for x in ql:
            cu_q.append(cu_q[-1] + x)
    elif q_mode == Q_PRESET:
        cu_q = [int(x) for x in np.asarray(q_in).reshape(-1)[: B + 1]]
    else:
        raise ValueError("unknown q_mode")

    pt = np.zeros((B, max_pages), dtype=np.int64)
    for b in range(B):
        n = -(-cache[b] // page_size)
        r = rpi[b]
        if r < 0 or r >= R:
            continue
        for j in range(min(n, max_pages)):
            col = j * page_size
            if col >= W:
                continue
            slot = int(r2t[r, col])
            pt[b, j] = slot // page_size if slot >= 0 else 0

    order = sorted(range(B), key=lambda b: (-cache[b], b))

    extra = {}
    if full_to_swa is not None:
        extra["swa_page_table"] = swa_page_table(seq_lens, rpi, r2t, page_size, max_pages,
                                                 full_to_swa)
    return dict(
        **extra,
        batch_order=np.asarray(order, dtype=np.int64),
        cache_seqlens=np.asarray(cache, dtype=np.int64),
        cu_seqlens_k=np.asarray(cu_k, dtype=np.int64),
        cu_seqlens_q=np.asarray(cu_q, dtype=np.int64),
        page_table=pt,
    )


def paged_layout_holds(page_table, seq_lens, req_pool_indices, req_to_token, page_size):
    """True when every token slot of every request sits where its page-table
    entry says: ``req_to_token[rpi[b], t] == page_table[b, t // S] * S + t % S``.

    This is the assumption under which a page table alone addresses the KV
    pool; tests assert it on generated inputs.
    """
    pt = np.asarray(page_table)
    r2t = np.asarray(req_to_token)
    for b, L in enumerate(np.asarray(seq_lens).reshape(-1)):
        L = max(int(L), 0)
        t = np.arange(L)
        want = pt[b, t // page_size].astype(np.int64) * page_size + (t % page_size)
        if not np.array_equal(r2t[int(req_pool_indices[b]), :L].astype(np.int64), want):
            return False
    return True
