"""Plain fp64 / integer CPU oracle for paged GQA decode attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``, never by the library.  It shares no
code with the HIP path (``decode_attention_paged_gqa_amd``), and the HIP path
never imports it.

Modules:
  attention -- gather, softmax attention, split partials, LSE merge (float64)
  metadata  -- cache_seqlens / cu_seqlens_k / cu_seqlens_q / page_table (exact ints)
  quant     -- fp64 decoders of the INT8 / INT4 KV formats
  kvcache   -- appending new tokens at their slots, with the INT8 / INT4 encoders
  schedule  -- per-request split counts and the flattened stage-1 work list (exact ints)
"""
from . import attention, kvcache, metadata, quant, schedule  # noqa: F401
