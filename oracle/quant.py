"""fp64 decoders for the quantised KV caches.  TEST INFRASTRUCTURE ONLY.

LightLLM PR #1549 "feat(autotune): separate general and decode attention
warmup", section "Covered decode kernels", lists INT8-KV and INT4-KV
flash-decode stage-1 kernels but does not give their storage formats.  The
formats decoded here are the plainest ones that fit the workload description
(symmetric int8 with one fp16 scale per (token, kv-head); 4-bit codes packed
two per byte with an fp16 scale and zero point per group of 32 along D):

* INT8:  x = code * s            (code int8, s fp16)
* INT4:  x = (nib - z) * s       per 32-group; byte j holds element 2j in its
                                 low nibble and element 2j+1 in its high nibble;
                                 (s, z) are stored as an fp16 pair per group.

fp16 values are widened to fp64 exactly (numpy's IEEE half decoder).
"""
from __future__ import annotations

import numpy as np

INT4_GROUP = 32


def fp16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Raw IEEE binary16 bit patterns (uint16) -> exact float64."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def dequant_int8(codes: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """codes [..., D] int8, scale_bits [...] uint16 (fp16) -> [..., D] float64."""
    return codes.astype(np.float64) * fp16_bits_to_f64(scale_bits)[..., None]


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """[..., D/2] uint8 -> [..., D] integer nibbles, element 2j from the low nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.int64)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def dequant_int4(packed: np.ndarray, scale_zero_bits: np.ndarray) -> np.ndarray:
    """packed [..., D/2] uint8, scale_zero_bits [..., D/32, 2] uint16 -> [..., D] float64."""
    nib = unpack_nibbles(packed).astype(np.float64)
    D = nib.shape[-1]
    sz = fp16_bits_to_f64(scale_zero_bits)
    s = sz[..., 0]
    z = sz[..., 1]
    g = nib.reshape(nib.shape[:-1] + (D // INT4_GROUP, INT4_GROUP))
    x = (g - z[..., None]) * s[..., None]
    return x.reshape(nib.shape)
