"""Oracle for appending new tokens' K/V to the paged cache, with
quantise-on-write.  TEST INFRASTRUCTURE ONLY.

SGLang PR #29843 digest, test listing of the fused metadata kernel: every
decode step carries ``out_cache_loc``, one int64 token slot per new token,
and the new tokens' K/V are written there before attention runs (the
metadata's KV lengths already include them).  A slot addresses page
``slot // page_size``, offset ``slot % page_size`` of the pool.  LightLLM
PR #1549, "Covered decode kernels", lists INT8-KV and INT4-KV caches; their
encoders are not given on the pages.  Readings used (the encoders are the
plainest ones that produce the formats ``oracle/quant.py`` decodes; every
rounding decision is taken in IEEE fp32, as a kernel would take it):

* INT8, per (token, kv-head) row of D values x (the fp32 values of the
  bf16 / fp32 input):  s = fp16(max|x| / 127), and s = 1 if that fp16 value
  is 0;  code = clamp(rne(x / s), -127, 127).
* INT4, per group of 32 along D:  s = fp16((max - min) / 15), and s = 1 if
  that fp16 value is 0;  z = fp16(clamp(rne(-min / s), 0, 15)), an integer
  code stored as +0 when it is zero (rounding a small positive min gives -0);
  nib = clamp(rne(x / s) + z, 0, 15);  byte j = nib[2j] | nib[2j+1] << 4.
* dense (bf16 / fp32): the values are stored unchanged.
* A negative slot, or one at or past ``num_pages * page_size``, writes
  nothing (the -1 sentinel of padded batches).  Slots are assumed distinct;
  with repeats the last token in order wins.

fp32 arithmetic here is numpy float32, whose +, -, / are IEEE correctly
rounded; ``np.rint`` rounds half to even; float32 -> float16 rounds to
nearest even.
"""
from __future__ import annotations

import numpy as np

INT4_GROUP = 32
_F32 = np.float32


def _fp16_scale(v32: np.ndarray) -> np.ndarray:
    """fp16(v) with 0 replaced by 1 (the reading for an all-equal row / group)."""
    s = v32.astype(np.float16)
    return np.where(s == 0, np.float16(1.0), s)


def quantize_int8(x: np.ndarray):
    """x [..., D] (values exactly representable in fp32) -> (codes int8 [..., D], s fp16 [...])."""
    xf = np.asarray(x, dtype=_F32)
    amax = np.max(np.abs(xf), axis=-1)
    s = _fp16_scale(amax / _F32(127.0))
    q = np.rint(xf / s.astype(_F32)[..., None])
    return np.clip(q, -127, 127).astype(np.int8), s


def quantize_int4(x: np.ndarray):
    """x [..., D] -> (packed uint8 [..., D/2], scale_zero fp16 [..., D/32, 2])."""
    xf = np.asarray(x, dtype=_F32)
    D = xf.shape[-1]
    g = xf.reshape(xf.shape[:-1] + (D // INT4_GROUP, INT4_GROUP))
    mn = g.min(axis=-1)
    mx = g.max(axis=-1)
    s = _fp16_scale((mx - mn) / _F32(15.0))
    sf = s.astype(_F32)
    z = (np.clip(np.rint(-mn / sf), 0, 15) + _F32(0.0)).astype(np.float16)  # -0 -> +0
    nib = np.clip(np.rint(g / sf[..., None]) + z.astype(_F32)[..., None], 0, 15)
    nib = nib.astype(np.uint8).reshape(xf.shape)
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return packed, np.stack([s, z], axis=-1)


def append_kv(pool: np.ndarray, new: np.ndarray, out_cache_loc, page_size: int,
              fmt: str, scale: np.ndarray = None):
    """Write ``new`` [N, Hkv, D] into ``pool`` (in place) at the given token slots.

    pool: dense [P, page, Hkv, D]; int8 codes [P, page, Hkv, D] with ``scale``
    [P, page, Hkv] fp16; int4 packed [P, page, Hkv, D/2] with ``scale``
    [P, page, Hkv, D/32, 2] fp16.  fmt is "dense", "int8" or "int4".
    """
    P = pool.shape[0]
    for n, slot in enumerate(np.asarray(out_cache_loc, dtype=np.int64)):
        if slot < 0 or slot >= P * page_size:
            continue
        p, t = int(slot) // page_size, int(slot) % page_size
        if fmt == "dense":
            pool[p, t] = new[n]
        elif fmt == "int8":
            codes, s = quantize_int8(new[n])
            pool[p, t] = codes
            scale[p, t] = s
        elif fmt == "int4":
            packed, sz = quantize_int4(new[n])
            pool[p, t] = packed
            scale[p, t] = sz
        else:
            raise ValueError(fmt)
