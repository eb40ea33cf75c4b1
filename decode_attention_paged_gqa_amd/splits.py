"""num_splits per KV-length bucket.

LightLLM PR #1549 ("Covered decode kernels") tunes the split count of the
KV-cache decode kernel once, at startup, with KV-length run keys grouped into
buckets; the real request length picks the bucket at run time, an untuned key
falls back to the nearest tuned one, and nothing is tuned on live requests.
Here the tuned values live in ``splits_table.json`` (written by
``bench.py --tune`` on the GPU), keyed by kernel variant, then by batch key,
then by 4096-token bucket; the lookup itself is the C helper
``decode_attn_pick_splits``.  Under graph capture, where lengths are not
known on the host, callers key on the representative length 32768.

Per-request split counts (the metadata prelude's schedule option) take a
per-bucket table too.  It is derived from one tuned number per variant and
batch key, the target split size in pages: bucket k (1-based) gets
ceil(k * bucket_pages / chunk_pages) splits, so every request's splits come
out near that size whatever the batch's length mix, and the device picks
each request's count from its own length -- also inside a captured graph.
"""
from __future__ import annotations

import json
import os
from dataclasses import dataclass, field
from typing import Dict, List

from ._binding import decode_attn_pick_splits

TABLE_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "splits_table.json")
REPRESENTATIVE_KV_LEN = 32768
BUCKET_TOKENS = 4096
N_BUCKETS = 8
BATCH_KEYS = (1, 4, 16, 32, 64)
CANDIDATES = (1, 2, 4, 8, 16, 32, 64, 128)
CHUNK_CANDIDATES = (8, 16, 24, 32, 48, 64, 96, 128, 192)
DEFAULT_CHUNK_PAGES = 64


def kernel_key(kv: str, rows: int, head_dim: int, page_size: int, kv_layout: str = "NHD") -> str:
    """Table key of a stage-1 variant: cache format, query rows per kv-head, D, page size,
    pool layout."""
    return f"{kv}_r{rows}_d{head_dim}_p{page_size}_{kv_layout.lower()}"


def heads_per_workgroup(key: str) -> int:
    """kv-heads one stage-1 workgroup covers for variant ``key`` (with Hkv a
    multiple of 4): 4 where the kernel takes a token-major pool four kv-heads at
    a time (INT8 and INT4 at any row count, dense bf16 and fp32 at D = 64), else 1."""
    kv, _rows, d, _page, layout = key.split("_")
    if layout != "nhd":
        return 1
    if kv in ("int8", "int4"):
        return 4
    if kv in ("bf16", "fp32") and d == "d64":
        return 4
    return 1


def _heuristic(batch_key: int, bucket: int, num_kv_heads: int = 8, cus: int = 256) -> int:
    pages = bucket * BUCKET_TOKENS // 64
    want = max(1, (4 * cus) // max(1, batch_key * num_kv_heads))
    s = 1
    while s < want and s * 2 <= min(32, max(1, pages // 4)):
        s *= 2
    return s


@dataclass
class SplitTable:
    bucket_tokens: int = BUCKET_TOKENS
    batch_keys: List[int] = field(default_factory=lambda: list(BATCH_KEYS))
    tables: Dict[str, List[List[int]]] = field(default_factory=dict)
    chunk_pages: Dict[str, List[int]] = field(default_factory=dict)  # per batch key

    @classmethod
    def load(cls, path: str = None) -> "SplitTable":
        path = path or os.environ.get("DECODE_ATTN_SPLITS_TABLE") or TABLE_PATH
        if not os.path.exists(path):
            return default_table()
        with open(path) as f:
            d = json.load(f)
        return cls(bucket_tokens=d["bucket_tokens"], batch_keys=list(d["batch_keys"]),
                   tables={k: [list(r) for r in v] for k, v in d["tables"].items()},
                   chunk_pages={k: list(v) for k, v in d.get("chunk_pages", {}).items()})

    def save(self, path: str = None):
        path = path or os.environ.get("DECODE_ATTN_SPLITS_TABLE") or TABLE_PATH
        lines = ['{', f' "bucket_tokens": {self.bucket_tokens},',
                 f' "batch_keys": {json.dumps(self.batch_keys)},', ' "tables": {']
        keys = sorted(self.tables)
        for i, k in enumerate(keys):
            rows = ",\n   ".join(json.dumps(r) for r in self.tables[k])
            lines.append(f'  "{k}": [\n   {rows}\n  ]' + ("," if i + 1 < len(keys) else ""))
        lines.append(' },' if self.chunk_pages else ' }')
        if self.chunk_pages:
            ck = sorted(self.chunk_pages)
            lines.append(' "chunk_pages": {')
            for i, k in enumerate(ck):
                lines.append(f'  "{k}": {json.dumps(self.chunk_pages[k])}' +
                             ("," if i + 1 < len(ck) else ""))
            lines.append(' }')
        lines.append('}')
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")

    def table_for(self, key: str) -> List[List[int]]:
        """The variant's [batch key][bucket] counts; the heuristic when it is not
        tuned, or was tuned for another set of batch keys."""
        rows = self.tables.get(key)
        if rows is not None and len(rows) == len(self.batch_keys):
            return rows
        units = 8 // heads_per_workgroup(key)  # workgroups per request and split (Hkv = 8)
        return [[_heuristic(b, k + 1, units) for k in range(N_BUCKETS)] for b in self.batch_keys]

    def pick(self, key: str, batch: int, kv_len: int = REPRESENTATIVE_KV_LEN) -> int:
        """num_splits for variant ``key`` at this batch size and (max) KV length."""
        return decode_attn_pick_splits(self.table_for(key), self.batch_keys, self.bucket_tokens,
                                       batch, kv_len)

    def chunk_for(self, key: str, batch: int) -> int:
        """Tuned split size in pages for per-request counts (nearest batch key)."""
        row = self.chunk_pages.get(key)
        if not row or len(row) != len(self.batch_keys):
            return DEFAULT_CHUNK_PAGES
        return decode_attn_pick_splits([[c] for c in row], self.batch_keys, 1, batch, 1)

    def request_table(self, key: str, batch: int, page_size: int) -> List[int]:
        """Per-bucket split counts for the metadata prelude's per-request schedule."""
        return per_request_table(self.chunk_for(key, batch), page_size, self.bucket_tokens)


def per_request_table(chunk_pages: int, page_size: int, bucket_tokens: int = BUCKET_TOKENS,
                      n_buckets: int = N_BUCKETS) -> List[int]:
    """Bucket k (1-based) -> ceil(k * bucket_pages / chunk_pages) splits, capped at 256."""
    per = max(1, bucket_tokens // page_size)
    return [min(256, max(1, -(-k * per // chunk_pages))) for k in range(1, n_buckets + 1)]


def default_table() -> SplitTable:
    return SplitTable()
