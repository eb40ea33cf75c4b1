"""Paged GQA decode attention for MI355X (gfx950): HIP kernels behind a C ABI.

The C ABI (include/decode_attn.h) is exported by ``libdecode_attn.so``, built
in-tree by ``python -m decode_attention_paged_gqa_amd.build``.  The binding
loads it on first use and raises if it is missing; there is no fallback path.
"""
from ._binding import (  # noqa: F401
    CACHE_FORMATS, DA_BF16, DA_CACHE_DENSE, DA_CACHE_INT4, DA_CACHE_INT8, DA_FP32, DA_KV_HND,
    DA_KV_NHD, DA_Q_CUMSUM, DA_Q_PRESET, DA_Q_STRIDED, DA_MAX_SPLITS, DA_STATIC_SCRATCH_BYTES,
    EXPORTS, KV_LAYOUTS, LIB_PATH, CHECKED_LIB_PATH,
    DA_CHECK_COUNTS, DA_CHECK_ORDER, DA_CHECK_PAGE_ID, DA_CHECK_REQ_ROW, DA_CHECK_SEQLEN,
    DA_CHECK_TOO_LONG, DA_CHECK_WORK,
    DecodeAttnError, decode_attn_append_kv, decode_attn_checks, decode_attn_gather_kv,
    decode_attn_decode_static, decode_attn_merge, decode_attn_metadata,
    decode_attn_pick_splits, decode_attn_split, decode_attn_split_int4, decode_attn_split_int8,
    decode_attn_version, load,
)
from .splits import SplitTable, default_table  # noqa: F401
