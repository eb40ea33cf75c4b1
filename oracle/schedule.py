"""Integer oracle for per-request split counts and the flattened stage-1
work list.  TEST INFRASTRUCTURE ONLY.

LightLLM PR #1549, section "Covered decode kernels": the decode kernels'
``num_splits`` is tuned at a representative KV length with run keys
bucketed by KV length, while normal execution selects configurations from
the real request length.  Taken per request, that is a table indexed by the
request's own length bucket.  Readings used (the page fixes neither the
bucket width nor the table; both are arguments here):

* bucket of a request: ``k = clamp(ceil(L / bucket_tokens), 1, n_buckets) - 1``
  (a request of length 0 falls in the first bucket);
* its split count: ``S_b = max(1, min(table[k], n_b, max_splits))`` with
  ``n_b = ceil(L / page_size)`` pages -- more splits than pages would only
  add empty splits, and one split is kept for an empty request so that it
  still writes its (0, -inf) partial;
* the work list holds one item per (request, split): requests in
  ``batch_order`` (descending length, ties by index), splits ascending.  An
  item is the integer ``b * 256 + s``; entries past the last item up to the
  list's capacity are -1.

Within a request, split ``s`` of ``S_b`` covers the same page-aligned token
range as for a batch-wide split count (``oracle.attention.split_token_range``).
"""
from __future__ import annotations

import numpy as np

ITEM_SHIFT = 256  # item = b * ITEM_SHIFT + s; s < 256


def request_splits(cache_seqlens, page_size, table, bucket_tokens, max_splits):
    """[B] per-request split counts."""
    table = [int(x) for x in np.asarray(table).reshape(-1)]
    out = []
    for L in np.asarray(cache_seqlens).reshape(-1):
        L = max(int(L), 0)
        k = min(max(-(-L // bucket_tokens), 1), len(table)) - 1
        n = -(-L // page_size)
        out.append(max(1, min(table[k], n, max_splits)))
    return np.asarray(out, dtype=np.int64)


def batch_order(cache_seqlens):
    seq = [max(int(x), 0) for x in np.asarray(cache_seqlens).reshape(-1)]
    return sorted(range(len(seq)), key=lambda b: (-seq[b], b))


def work_list(cache_seqlens, split_counts, capacity):
    """[capacity] work items (b * 256 + s) in dispatch order, -1 past the end."""
    items = []
    for b in batch_order(cache_seqlens):
        for s in range(int(split_counts[b])):
            items.append(b * ITEM_SHIFT + s)
    if len(items) > capacity:
        raise ValueError("work list capacity too small")
    return np.asarray(items + [-1] * (capacity - len(items)), dtype=np.int64)
