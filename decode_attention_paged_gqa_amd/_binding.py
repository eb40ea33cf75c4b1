"""ctypes binding of libdecode_attn.so.

Argument marshalling only: these wrappers check tensor devices, dtypes,
shapes and contiguity, allocate outputs with torch when the caller passes
none, and hand raw device pointers plus torch's current HIP stream to the C
entry points of the same names.  Every computation runs in the HIP kernels;
there is no fallback, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdecode_attn.so")
# the same library with the device-data contract checks (decode_attn_checks)
CHECKED_LIB_PATH = os.path.join(_HERE, "libdecode_attn_checked.so")
# the same library with AddressSanitizer on its host code (build.py --asan)
ASAN_LIB_PATH = os.path.join(_HERE, "libdecode_attn_asan.so")

DA_OK, DA_ERR_INVALID_ARG, DA_ERR_UNSUPPORTED, DA_ERR_LAUNCH, DA_ERR_TOO_LARGE = 0, 1, 2, 3, 4
DA_FP32, DA_BF16 = 0, 1
DA_KV_NHD, DA_KV_HND = 0, 1
DA_CACHE_DENSE, DA_CACHE_INT8, DA_CACHE_INT4 = 0, 1, 2
CACHE_FORMATS = {"dense": DA_CACHE_DENSE, "int8": DA_CACHE_INT8, "int4": DA_CACHE_INT4}
KV_LAYOUTS = {"NHD": DA_KV_NHD, "HND": DA_KV_HND}
DA_Q_STRIDED, DA_Q_CUMSUM, DA_Q_PRESET = 0, 1, 2
DA_MAX_SPLITS = 256
DA_STATIC_SCRATCH_BYTES = 64 << 20  # scratch of decode_attn_decode_static, per GPU
# decode_attn_checks flag bits
DA_CHECK_PAGE_ID, DA_CHECK_SEQLEN, DA_CHECK_ORDER, DA_CHECK_WORK = 0x01, 0x02, 0x04, 0x08
DA_CHECK_COUNTS, DA_CHECK_REQ_ROW, DA_CHECK_TOO_LONG = 0x10, 0x20, 0x40

_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F32 = ctypes.c_float

_SIGS = {
    "decode_attn_metadata": [_P, _P, _P, _I64, _I64, _I64, _I32, _I32, _I32, _I32, _P, _I32,
                             _P, _P, _P, _P, _P, _P],
    "decode_attn_metadata_ex": [_P, _P, _P, _I64, _I64, _I64, _I32, _I32, _I32, _I32, _P, _I32,
                                _P, _P, _P, _P, _P, _P, _I64, _P, _P, _I32, _I32, _I32, _P, _P,
                                _I32, _P],
    "decode_attn_split": [_P, _I32, _P, _P, _P, _I32, _I32, _P, _P, _I32, _I32, _I32, _I32,
                          _I32, _I32, _I32, _I32, _I32, _P, _P, _I32, _F32, _I32, _P, _P, _P],
    "decode_attn_split_int8": [_P, _I32, _P, _P, _P, _P, _P, _I32, _I32, _P, _P, _I32, _I32,
                               _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _I32, _F32,
                               _I32, _P, _P, _P],
    "decode_attn_split_int4": [_P, _I32, _P, _P, _P, _P, _P, _I32, _I32, _P, _P, _I32, _I32,
                               _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _I32, _F32,
                               _I32, _P, _P, _P],
    "decode_attn_decode_static": [_P, _I32, _I32, _P, _P, _P, _P, _P, _I32, _I32, _P, _P, _I32,
                                  _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _I32,
                                  _F32, _I32, _P, _I32, _P, _P],
    "decode_attn_merge": [_P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _I32, _P, _P],
    "decode_attn_append_kv": [_P, _P, _I32, _P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _I32, _I32,
                              _I32, _P],
    "decode_attn_pick_splits": [_P, _P, _I32, _I32, _I32, _I32, _I32],
    "decode_attn_gather_kv": [_P, _I64, _I32, _I32, _I32, _I32, _P, _I32, _I32, _P, _P, _I32,
                              _P, _P],
    "decode_attn_checks": [_P, _P, _I32],
    "decode_attn_strerror": [_I32],
    "decode_attn_version": [],
}

EXPORTS = tuple(_SIGS)


class DecodeAttnError(ValueError):
    """A C entry point returned a non-zero status."""


def load(path: Optional[str] = None, reload: bool = False):
    """Load the HIP library (once; ``reload`` switches to ``path``, e.g.
    CHECKED_LIB_PATH).  Without ``path``: $DECODE_ATTN_LIB if set (one of the
    built variants), else LIB_PATH.  Raises if it has not been built."""
    global _lib
    if _lib is not None and not reload:
        return _lib
    path = path or os.environ.get("DECODE_ATTN_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m decode_attention_paged_gqa_amd.build`")
    lib = ctypes.CDLL(path)
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "decode_attn_strerror" else ctypes.c_int32
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != DA_OK:
        msg = load().decode_attn_strerror(status).decode()
        raise DecodeAttnError(f"{what}: status {status} ({msg})")


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype=None, device=None, ndim=None, shape=None):
    """Type, dtype, device, rank, exact shape and contiguity of one tensor
    (that it lives on a GPU is checked last, by _gpu, after every shape)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, has {t.dim()}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, has {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _gpu(**tensors):
    """Every named tensor (None skipped) is a GPU tensor."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")


# ------------------------------------------------------------------ metadata
def decode_attn_metadata(seq_lens, req_pool_indices, req_to_token, page_size, max_pages,
                         q_mode=DA_Q_STRIDED, q_in=None, q_stride=1, out=None,
                         full_to_swa=None, split_table=None, bucket_tokens=4096,
                         max_splits=None, work_capacity=None):
    """cache_seqlens, cu_seqlens_k, cu_seqlens_q, page_table, batch_order in one launch.

    Options, computed in the same launch (``decode_attn_metadata_ex``):
    ``full_to_swa`` (int64 [n] slot map) adds "swa_page_table"; ``split_table``
    (a host list of per-bucket split counts) adds "split_counts" and
    "work_list" (``work_capacity`` entries, default batch * max_splits), for
    the split calls' per-request scheduling.  ``max_splits`` defaults to
    max(split_table).  Returns a dict of int32 tensors (those in ``out`` are
    reused)."""
    lib = load()
    dev = seq_lens.device
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    _need(req_pool_indices, "req_pool_indices", torch.int64, dev, 1)
    _need(req_to_token, "req_to_token", torch.int32, dev, 2)
    B = seq_lens.shape[0]
    if req_pool_indices.shape[0] != B:
        raise ValueError("req_pool_indices length != batch")
    if q_mode not in (DA_Q_STRIDED, DA_Q_CUMSUM, DA_Q_PRESET):
        raise ValueError(f"unknown q_mode {q_mode}")
    if q_in is not None:
        _need(q_in, "q_in", torch.int32, dev, 1)
    # CUMSUM reads q_in[0 .. B-1], PRESET q_in[0 .. B]
    q_need = {DA_Q_STRIDED: 0, DA_Q_CUMSUM: B, DA_Q_PRESET: B + 1}[q_mode]
    if q_need and (q_in is None or q_in.shape[0] < q_need):
        raise ValueError(f"q_in needs at least {q_need} entries for q_mode {q_mode}")
    out = dict(out or {})
    mk = lambda k, n: out.get(k) if out.get(k) is not None else torch.empty(n, dtype=torch.int32, device=dev)
    out["cache_seqlens"] = mk("cache_seqlens", (B,))
    out["cu_seqlens_k"] = mk("cu_seqlens_k", (B + 1,))
    out["cu_seqlens_q"] = mk("cu_seqlens_q", (B + 1,))
    out["page_table"] = mk("page_table", (B, max_pages))
    out["batch_order"] = mk("batch_order", (B,))
    shapes = {"cache_seqlens": (B,), "cu_seqlens_k": (B + 1,), "cu_seqlens_q": (B + 1,),
              "page_table": (B, max_pages), "batch_order": (B,)}
    for k, shp in shapes.items():
        _need(out[k], k, torch.int32, dev, shape=shp)
    if full_to_swa is not None or split_table is not None:
        return _metadata_ex(lib, dev, B, seq_lens, req_pool_indices, req_to_token, page_size,
                            max_pages, q_mode, q_in, q_stride, out, mk, full_to_swa,
                            split_table, bucket_tokens, max_splits, work_capacity)
    _gpu(seq_lens=seq_lens, req_pool_indices=req_pool_indices, req_to_token=req_to_token,
         q_in=q_in, **{k: out[k] for k in shapes})
    st = lib.decode_attn_metadata(
        _ptr(seq_lens), _ptr(req_pool_indices), _ptr(req_to_token), req_to_token.shape[0],
        req_to_token.shape[1], req_to_token.stride(0), B, page_size, max_pages, q_mode,
        _ptr(q_in), q_stride, _ptr(out["cache_seqlens"]), _ptr(out["cu_seqlens_k"]),
        _ptr(out["cu_seqlens_q"]), _ptr(out["page_table"]), _ptr(out["batch_order"]),
        _stream(dev))
    _check(st, "decode_attn_metadata")
    return out


def _metadata_ex(lib, dev, B, seq_lens, rpi, r2t, page_size, max_pages, q_mode, q_in, q_stride,
                 out, mk, full_to_swa, split_table, bucket_tokens, max_splits, work_capacity):
    f2s_len = 0
    if full_to_swa is not None:
        _need(full_to_swa, "full_to_swa", torch.int64, dev, 1)
        f2s_len = full_to_swa.shape[0]
        out["swa_page_table"] = mk("swa_page_table", (B, max_pages))
        _need(out["swa_page_table"], "swa_page_table", torch.int32, dev, shape=(B, max_pages))
    table_host, nb, smax = None, 0, 0
    if split_table is not None:
        vals = [int(x) for x in split_table]
        nb = len(vals)
        smax = int(max_splits) if max_splits is not None else max(vals)
        table_host = (ctypes.c_int32 * nb)(*vals)
        cap = int(work_capacity) if work_capacity is not None else B * min(smax, max(vals))
        out["split_counts"] = mk("split_counts", (B,))
        out["work_list"] = mk("work_list", (cap,))
        for k in ("split_counts", "work_list"):
            _need(out[k], k, torch.int32, dev, 1)
        if out["work_list"].shape[0] != cap or out["split_counts"].shape[0] != B:
            raise ValueError("split_counts / work_list sized for another batch or capacity")
    _gpu(seq_lens=seq_lens, req_pool_indices=rpi, req_to_token=r2t, q_in=q_in,
         full_to_swa=full_to_swa, **{k: v for k, v in out.items() if k in (
             "cache_seqlens", "cu_seqlens_k", "cu_seqlens_q", "page_table", "batch_order",
             "swa_page_table", "split_counts", "work_list")})
    st = lib.decode_attn_metadata_ex(
        _ptr(seq_lens), _ptr(rpi), _ptr(r2t), r2t.shape[0], r2t.shape[1], r2t.stride(0), B,
        page_size, max_pages, q_mode, _ptr(q_in), q_stride, _ptr(out["cache_seqlens"]),
        _ptr(out["cu_seqlens_k"]), _ptr(out["cu_seqlens_q"]), _ptr(out["page_table"]),
        _ptr(out["batch_order"]), _ptr(full_to_swa), f2s_len,
        _ptr(out["swa_page_table"]) if full_to_swa is not None else None,
        table_host, nb, int(bucket_tokens), smax,
        _ptr(out["split_counts"]) if table_host is not None else None,
        _ptr(out["work_list"]) if table_host is not None else None,
        out["work_list"].shape[0] if table_host is not None else 0,
        _stream(dev))
    _check(st, "decode_attn_metadata_ex")
    return out


# ------------------------------------------------------------------ stage 1
def _layout_code(kv_layout) -> int:
    if isinstance(kv_layout, str):
        if kv_layout.upper() not in KV_LAYOUTS:
            raise ValueError(f"kv_layout must be one of {tuple(KV_LAYOUTS)}")
        return KV_LAYOUTS[kv_layout.upper()]
    if int(kv_layout) not in (DA_KV_NHD, DA_KV_HND):
        raise ValueError("kv_layout must be DA_KV_NHD or DA_KV_HND")
    return int(kv_layout)


def _pool_dims(pool, code):
    """(num_pages, page_size, Hkv) of a pool [P, ps, Hkv, ...] (NHD) or [P, Hkv, ps, ...] (HND)."""
    P, a, b = pool.shape[:3]
    return (P, a, b) if code == DA_KV_NHD else (P, b, a)


def _partials(q, num_splits, o_partial, lse_partial):
    B, qn, Hq, D = q.shape
    if o_partial is None:
        o_partial = torch.empty((B, qn, Hq, num_splits, D), dtype=torch.float32, device=q.device)
    if lse_partial is None:
        lse_partial = torch.empty((B, qn, Hq, num_splits), dtype=torch.float32, device=q.device)
    _need(o_partial, "o_partial", torch.float32, q.device, shape=(B, qn, Hq, num_splits, D))
    _need(lse_partial, "lse_partial", torch.float32, q.device, shape=(B, qn, Hq, num_splits))
    return o_partial, lse_partial


def _pool_geometry(fmt, q, k_pool, v_pool, k_scale, v_scale, lay):
    """Checks the pools (and scales) of a cache format against each other and
    against q; returns (num_pages, page_size, Hkv, D)."""
    dev = q.device
    if fmt == DA_CACHE_DENSE:
        _need(k_pool, "k_pool", q.dtype, dev, 4)
        _need(v_pool, "v_pool", q.dtype, dev, 4)
        if k_pool.shape != v_pool.shape:
            raise ValueError("k_pool / v_pool shapes differ")
        D = k_pool.shape[3]
    elif fmt == DA_CACHE_INT8:
        _need(k_pool, "k_pool", torch.int8, dev, 4)
        _need(v_pool, "v_pool", torch.int8, dev, 4)
        _need(k_scale, "k_scale", torch.float16, dev, 3)
        _need(v_scale, "v_scale", torch.float16, dev, 3)
        D = k_pool.shape[3]
        if v_pool.shape != k_pool.shape or tuple(k_scale.shape) != tuple(k_pool.shape[:3]) \
                or k_scale.shape != v_scale.shape:
            raise ValueError("int8 pool / scale shapes inconsistent")
    elif fmt == DA_CACHE_INT4:
        _need(k_pool, "k_pool", torch.uint8, dev, 4)
        _need(v_pool, "v_pool", torch.uint8, dev, 4)
        _need(k_scale, "k_scale_zero", torch.float16, dev, 5)
        _need(v_scale, "v_scale_zero", torch.float16, dev, 5)
        D = 2 * k_pool.shape[3]
        if v_pool.shape != k_pool.shape or \
                tuple(k_scale.shape) != tuple(k_pool.shape[:3]) + (D // 32, 2) \
                or k_scale.shape != v_scale.shape:
            raise ValueError("int4 pool / scale-zero shapes inconsistent")
    else:
        raise ValueError(f"cache_format must be one of {tuple(CACHE_FORMATS)}")
    if q.shape[3] != D:
        raise ValueError("head_dim mismatch")
    P, S_p, Hkv = _pool_dims(k_pool, lay)
    return P, S_p, Hkv, D


def _q_code(q):
    if q.dtype == torch.bfloat16:
        return DA_BF16
    if q.dtype == torch.float32:
        return DA_FP32
    raise TypeError(f"q dtype {q.dtype} unsupported")


def _split_common(q, page_table, cache_seqlens, batch_order, split_counts=None,
                  work_list=None):
    _need(q, "q", (torch.bfloat16, torch.float32), ndim=4)
    dev = q.device
    _need(page_table, "page_table", torch.int32, dev, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, dev, 1)
    if page_table.shape[0] != q.shape[0] or cache_seqlens.shape[0] != q.shape[0]:
        raise ValueError("batch mismatch between q, page_table and cache_seqlens")
    if batch_order is not None:
        _need(batch_order, "batch_order", torch.int32, dev, 1)
        if batch_order.shape[0] != q.shape[0]:
            raise ValueError("batch_order length != batch")
    if (work_list is None) != (split_counts is None):
        raise ValueError("work_list and split_counts go together")
    if work_list is not None:
        _need(work_list, "work_list", torch.int32, dev, 1)
        _need(split_counts, "split_counts", torch.int32, dev, 1)
        if split_counts.shape[0] != q.shape[0]:
            raise ValueError("split_counts length != batch")
    return dev


def _sched_args(split_counts, work_list):
    return (_ptr(split_counts), _ptr(work_list), 0 if work_list is None else work_list.shape[0])


def decode_attn_split(q, k_pool, v_pool, page_table, cache_seqlens, num_splits,
                      softmax_scale=None, causal=False, o_partial=None, lse_partial=None,
                      batch_order=None, kv_layout="NHD", split_counts=None, work_list=None):
    """Stage 1 over a dense bf16 / fp32 cache.  Returns (o_partial, lse_partial).

    Pools are [P, page_size, Hkv, D] (kv_layout "NHD") or [P, Hkv, page_size, D] ("HND").
    With ``work_list`` / ``split_counts`` (from ``decode_attn_metadata(split_table=...)``)
    request b has split_counts[b] splits and ``num_splits`` is the slots per row."""
    return _split(DA_CACHE_DENSE, "decode_attn_split", q, k_pool, v_pool, None, None,
                  page_table, cache_seqlens, num_splits, softmax_scale, causal, o_partial,
                  lse_partial, batch_order, kv_layout, split_counts, work_list)


def decode_attn_split_int8(q, k_pool, v_pool, k_scale, v_scale, page_table, cache_seqlens,
                           num_splits, softmax_scale=None, causal=False, o_partial=None,
                           lse_partial=None, batch_order=None, kv_layout="NHD",
                           split_counts=None, work_list=None):
    """Stage 1 over an INT8 cache (fp16 scale per token and kv-head).

    Pools [P, page_size, Hkv, D] with scales [P, page_size, Hkv] ("NHD"), or
    [P, Hkv, page_size, D] with [P, Hkv, page_size] ("HND")."""
    return _split(DA_CACHE_INT8, "decode_attn_split_int8", q, k_pool, v_pool, k_scale, v_scale,
                  page_table, cache_seqlens, num_splits, softmax_scale, causal, o_partial,
                  lse_partial, batch_order, kv_layout, split_counts, work_list)


def decode_attn_split_int4(q, k_pool, v_pool, k_scale_zero, v_scale_zero, page_table,
                           cache_seqlens, num_splits, softmax_scale=None, causal=False,
                           o_partial=None, lse_partial=None, batch_order=None, kv_layout="NHD",
                           split_counts=None, work_list=None):
    """Stage 1 over an INT4 cache (fp16 (scale, zero) per 32-group along D).

    Pools [P, page_size, Hkv, D/2] with (scale, zero) [P, page_size, Hkv, D/32, 2]
    ("NHD"), or the first three dims as [P, Hkv, page_size] ("HND")."""
    return _split(DA_CACHE_INT4, "decode_attn_split_int4", q, k_pool, v_pool, k_scale_zero,
                  v_scale_zero, page_table, cache_seqlens, num_splits, softmax_scale, causal,
                  o_partial, lse_partial, batch_order, kv_layout, split_counts, work_list)


def _split(fmt, name, q, k_pool, v_pool, k_scale, v_scale, page_table, cache_seqlens,
           num_splits, softmax_scale, causal, o_partial, lse_partial, batch_order, kv_layout,
           split_counts, work_list):
    lib = load()
    dev = _split_common(q, page_table, cache_seqlens, batch_order, split_counts, work_list)
    lay = _layout_code(kv_layout)
    P, S_p, Hkv, D = _pool_geometry(fmt, q, k_pool, v_pool, k_scale, v_scale, lay)
    B, qn, Hq, _ = q.shape
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    o_partial, lse_partial = _partials(q, num_splits, o_partial, lse_partial)
    _gpu(q=q, k_pool=k_pool, v_pool=v_pool, k_scale=k_scale, v_scale=v_scale,
         page_table=page_table, cache_seqlens=cache_seqlens, batch_order=batch_order,
         split_counts=split_counts, work_list=work_list, o_partial=o_partial,
         lse_partial=lse_partial)
    pools = (_ptr(k_pool), _ptr(v_pool)) + (() if fmt == DA_CACHE_DENSE else
                                            (_ptr(k_scale), _ptr(v_scale)))
    st = getattr(lib, name)(
        _ptr(q), _q_code(q), *pools, _ptr(page_table), page_table.stride(0),
        page_table.shape[1], _ptr(cache_seqlens), _ptr(batch_order), B, qn, Hq, Hkv, D, S_p, P,
        lay, num_splits, *_sched_args(split_counts, work_list), scale, int(bool(causal)),
        _ptr(o_partial), _ptr(lse_partial), _stream(dev))
    _check(st, name)
    return o_partial, lse_partial


def decode_attn_decode_static(q, k_pool, v_pool, page_table, cache_seqlens, num_splits,
                              softmax_scale=None, causal=False, k_scale=None, v_scale=None,
                              cache_format="dense", out=None, out_dtype=torch.bfloat16,
                              lse_out=None, want_lse=False, batch_order=None, kv_layout="NHD",
                              split_counts=None, work_list=None):
    """Stage 1 and the merge in one call, the split partials in the library's
    per-GPU scratch array (the C call allocates nothing; pass ``out`` to
    allocate nothing here either).  Same arguments and result as
    decode_attn_split[_int8|_int4] followed by decode_attn_merge; ``k_scale`` /
    ``v_scale`` are the quantised formats' scales or (scale, zero) pairs.
    Returns out (and lse if requested)."""
    lib = load()
    fmt = CACHE_FORMATS.get(cache_format) if isinstance(cache_format, str) else int(cache_format)
    if fmt not in (DA_CACHE_DENSE, DA_CACHE_INT8, DA_CACHE_INT4):
        raise ValueError(f"cache_format must be one of {tuple(CACHE_FORMATS)}")
    dev = _split_common(q, page_table, cache_seqlens, batch_order, split_counts, work_list)
    lay = _layout_code(kv_layout)
    P, S_p, Hkv, D = _pool_geometry(fmt, q, k_pool, v_pool, k_scale, v_scale, lay)
    B, qn, Hq, _ = q.shape
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, qn, Hq, D), dtype=out_dtype, device=dev)
    _need(out, "out", (torch.bfloat16, torch.float32), dev, shape=(B, qn, Hq, D))
    if want_lse and lse_out is None:
        lse_out = torch.empty((B, qn, Hq), dtype=torch.float32, device=dev)
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, dev, shape=(B, qn, Hq))
    _gpu(q=q, k_pool=k_pool, v_pool=v_pool, k_scale=k_scale, v_scale=v_scale,
         page_table=page_table, cache_seqlens=cache_seqlens, batch_order=batch_order,
         split_counts=split_counts, work_list=work_list, out=out, lse_out=lse_out)
    st = lib.decode_attn_decode_static(
        _ptr(q), _q_code(q), fmt, _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
        _ptr(page_table), page_table.stride(0), page_table.shape[1], _ptr(cache_seqlens),
        _ptr(batch_order), B, qn, Hq, Hkv, D, S_p, P, lay, num_splits,
        *_sched_args(split_counts, work_list), scale, int(bool(causal)), _ptr(out),
        DA_BF16 if out.dtype == torch.bfloat16 else DA_FP32, _ptr(lse_out), _stream(dev))
    _check(st, "decode_attn_decode_static")
    return (out, lse_out) if (want_lse or lse_out is not None) else out


# ------------------------------------------------------------------ KV append
def decode_attn_append_kv(k_new, v_new, out_cache_loc, k_pool, v_pool, k_scale=None,
                          v_scale=None, cache_format="dense", kv_layout="NHD"):
    """Write the new tokens' K/V [N, Hkv, D] into the pools at ``out_cache_loc`` (int64
    token slots), encoding them for "int8" / "int4" caches.  Pools and scales are
    updated in place, in the layout the split calls read (kv_layout)."""
    lib = load()
    _need(k_new, "k_new", (torch.bfloat16, torch.float32), ndim=3)
    dev = k_new.device
    _need(v_new, "v_new", k_new.dtype, dev, 3)
    _need(out_cache_loc, "out_cache_loc", torch.int64, dev, 1)
    if v_new.shape != k_new.shape or out_cache_loc.shape[0] != k_new.shape[0]:
        raise ValueError("k_new / v_new / out_cache_loc sizes differ")
    N, Hkv, D = k_new.shape
    fmt = CACHE_FORMATS.get(cache_format) if isinstance(cache_format, str) else int(cache_format)
    if fmt is None:
        raise ValueError(f"cache_format must be one of {tuple(CACHE_FORMATS)}")
    lay = _layout_code(kv_layout)
    pool_dtype = {DA_CACHE_DENSE: k_new.dtype, DA_CACHE_INT8: torch.int8,
                  DA_CACHE_INT4: torch.uint8}[fmt]
    row = {DA_CACHE_DENSE: (D,), DA_CACHE_INT8: (D,), DA_CACHE_INT4: (D // 2,)}[fmt]
    _need(k_pool, "k_pool", pool_dtype, dev, 4)
    _need(v_pool, "v_pool", pool_dtype, dev, 4)
    P, S_p, Hp = _pool_dims(k_pool, lay)
    if v_pool.shape != k_pool.shape or Hp != Hkv or tuple(k_pool.shape[3:]) != row:
        raise ValueError("pool shape does not match the new rows")
    if fmt != DA_CACHE_DENSE:
        nd = 3 if fmt == DA_CACHE_INT8 else 5
        _need(k_scale, "k_scale", torch.float16, dev, nd)
        _need(v_scale, "v_scale", torch.float16, dev, nd)
        want = tuple(k_pool.shape[:3]) + (() if fmt == DA_CACHE_INT8 else (D // 32, 2))
        if tuple(k_scale.shape) != want or v_scale.shape != k_scale.shape:
            raise ValueError(f"scale shape must be {want}")
    _gpu(k_new=k_new, v_new=v_new, out_cache_loc=out_cache_loc, k_pool=k_pool, v_pool=v_pool,
         k_scale=k_scale, v_scale=v_scale)
    st = lib.decode_attn_append_kv(_ptr(k_new), _ptr(v_new), _q_code(k_new), _ptr(out_cache_loc),
                                   N, Hkv, D, fmt, _ptr(k_pool), _ptr(v_pool), _ptr(k_scale),
                                   _ptr(v_scale), S_p, P, lay, _stream(dev))
    _check(st, "decode_attn_append_kv")


# ------------------------------------------------------------------ stage 2
def decode_attn_merge(o_partial, lse_partial, out_dtype=torch.bfloat16, out=None, lse_out=None,
                      want_lse=False, split_counts=None):
    """LSE merge of the split partials.  Returns out (and lse if requested).
    With ``split_counts`` ([B] int32) request b merges only its first split_counts[b] slots."""
    lib = load()
    _need(o_partial, "o_partial", torch.float32, ndim=5)
    dev = o_partial.device
    _need(lse_partial, "lse_partial", torch.float32, dev, 4)
    B, qn, Hq, S, D = o_partial.shape
    if tuple(lse_partial.shape) != (B, qn, Hq, S):
        raise ValueError("lse_partial shape mismatch")
    if out is None:
        out = torch.empty((B, qn, Hq, D), dtype=out_dtype, device=dev)
    _need(out, "out", (torch.bfloat16, torch.float32), dev, shape=(B, qn, Hq, D))
    if want_lse and lse_out is None:
        lse_out = torch.empty((B, qn, Hq), dtype=torch.float32, device=dev)
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, dev, shape=(B, qn, Hq))
    if split_counts is not None:
        _need(split_counts, "split_counts", torch.int32, dev, shape=(B,))
    _gpu(o_partial=o_partial, lse_partial=lse_partial, out=out, lse_out=lse_out,
         split_counts=split_counts)
    code = DA_BF16 if out.dtype == torch.bfloat16 else DA_FP32
    st = lib.decode_attn_merge(_ptr(o_partial), _ptr(lse_partial), B, qn, Hq, D, S,
                               _ptr(split_counts), _ptr(out), code, _ptr(lse_out), _stream(dev))
    _check(st, "decode_attn_merge")
    return (out, lse_out) if (want_lse or lse_out is not None) else out


# ------------------------------------------------------------------ helpers
def decode_attn_pick_splits(table, batch_keys, bucket_tokens, batch, kv_len) -> int:
    """Host lookup of num_splits from a [n_batch_keys, n_buckets] table."""
    lib = load()
    t = (ctypes.c_int32 * (len(table) * len(table[0])))(*[int(x) for row in table for x in row])
    k = (ctypes.c_int32 * len(batch_keys))(*[int(x) for x in batch_keys])
    s = lib.decode_attn_pick_splits(ctypes.cast(t, _P), ctypes.cast(k, _P), len(batch_keys),
                                    len(table[0]), int(bucket_tokens), int(batch), int(kv_len))
    if s < 1:
        _check(-s, "decode_attn_pick_splits")
    return int(s)


def decode_attn_gather_kv(pool, page_table, cache_seqlens, cu_seqlens_k, total_tokens, out=None,
                          kv_layout="NHD"):
    """Dense [total_tokens, Hkv, *row] copy of every request's tokens (test hook).

    pool is [P, page_size, Hkv, *row] ("NHD") or [P, Hkv, page_size, *row] ("HND")."""
    lib = load()
    dev = pool.device
    lay = _layout_code(kv_layout)
    _need(pool, "pool", None, dev)
    _need(page_table, "page_table", torch.int32, dev, 2)
    Bt = page_table.shape[0]
    _need(cache_seqlens, "cache_seqlens", torch.int32, dev, shape=(Bt,))
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, dev, shape=(Bt + 1,))
    if pool.dim() < 3:
        raise ValueError("pool needs at least [pages, slots, heads] dims")
    P, S_p, Hkv = _pool_dims(pool, lay)
    row = tuple(pool.shape[3:])
    row_bytes = pool[0, 0, 0].numel() * pool.element_size()
    if out is None:
        out = torch.empty((total_tokens, Hkv) + row, dtype=pool.dtype, device=dev)
    _need(out, "out", pool.dtype, dev, shape=(total_tokens, Hkv) + row)
    _gpu(pool=pool, page_table=page_table, cache_seqlens=cache_seqlens,
         cu_seqlens_k=cu_seqlens_k, out=out)
    st = lib.decode_attn_gather_kv(_ptr(pool), row_bytes, Hkv, lay, S_p, P, _ptr(page_table),
                                   page_table.stride(0), page_table.shape[1], _ptr(cache_seqlens),
                                   _ptr(cu_seqlens_k), page_table.shape[0], _ptr(out), _stream(dev))
    _check(st, "decode_attn_gather_kv")
    return out


def decode_attn_version() -> int:
    return int(load().decode_attn_version())


def decode_attn_checks(reset: bool = False):
    """(flags, count) of the checked library's contract-check words (see
    DA_CHECK_*); synchronises the device.  Raises DecodeAttnError with the
    normal library, which has no checks."""
    lib = load()
    flags, count = ctypes.c_uint32(0), ctypes.c_uint64(0)
    st = lib.decode_attn_checks(ctypes.byref(flags), ctypes.byref(count), 1 if reset else 0)
    _check(st, "decode_attn_checks")
    return int(flags.value), int(count.value)
