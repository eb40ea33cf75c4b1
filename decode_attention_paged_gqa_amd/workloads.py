"""Seeded synthetic inputs for paged decode attention.

This module builds the inputs that both the HIP path and the fp64 oracle
consume: query tensors, paged K/V pools, the request -> token-slot table and
its page permutation, and (for the quantised caches) the integer codes and
their fp16 scale / zero-point tensors.  It holds none of the attention
arithmetic: no score, softmax, merge or dequantisation code lives here.  The
quantisers below only *encode* test data; both sides then decode the stored
codes independently.

Shapes follow the workloads the pages describe (LightLLM PR #1549
"feat(autotune): separate general and decode attention warmup", sections
"Covered decode kernels" and "Validation": representative KV length 32768,
concurrency 16/32/64, MTP step 3).  No dataset, prompt or model weight is
used: every value is drawn from seeded generators.

Pool layout (token-major slot pool viewed by page):
    pool[page, slot_in_page, kv_head, ...]   (contiguous)
so token slot ``p * page_size + i`` lives at ``pool[p, i]``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

# dtype codes shared with the C ABI (include/decode_attn.h)
DTYPE_FP32 = 0
DTYPE_BF16 = 1

KV_DENSE = "dense"   # bf16 / fp32 pools
KV_INT8 = "int8"     # int8 codes + one fp16 scale per (token, kv-head)
KV_INT4 = "int4"     # 2 nibbles per byte + fp16 (scale, zero) per 32-group along D

INT4_GROUP = 32


@dataclass(frozen=True)
class Workload:
    """A named decode-attention workload."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    q_per_req: int = 1
    causal: bool = False
    dtype: str = "bf16"            # query / dense-KV element type: "bf16" | "fp32"
    kv: str = KV_DENSE             # KV_DENSE | KV_INT8 | KV_INT4
    lengths: str = "fixed"         # "fixed" | "list" | "loguniform" | "uniform"
    length: int = 0                # for "fixed"
    length_list: tuple = ()        # for "list"
    length_lo: int = 0             # for "loguniform" / "uniform"
    length_hi: int = 0
    pin_max: bool = False          # pin one request at length_hi
    pool_pages: int = 0            # 0 => exactly the pages needed
    seed: int = 0
    splits: tuple = (1,)
    kv_layout: str = "NHD"         # "NHD" [P, page, Hkv, row] | "HND" [P, Hkv, page, row]
    amp: tuple = (1.0, 1.0, 1.0)   # standard deviations of the Q, K, V draws (before encoding)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def scaled(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The five workloads.  Names say what they are.
TINY_FP32 = Workload(
    name="tiny_fp32_b2_hq4_hkv1_d64_p16", batch=2, num_q_heads=4, num_kv_heads=1,
    head_dim=64, page_size=16, dtype="fp32", lengths="list", length_list=(37, 100),
    pool_pages=32, seed=1, splits=(1, 2, 4))
BF16_B16 = Workload(
    name="bf16_b16_hq32_hkv8_d128_p64_L8192", batch=16, num_q_heads=32, num_kv_heads=8,
    head_dim=128, page_size=64, lengths="fixed", length=8192, seed=2,
    splits=(1, 2, 4, 8, 16, 32), kv_layout="HND")
RAGGED_B64 = Workload(
    name="ragged_bf16_b64_hq40_hkv8_d128_p64_L1k-32k", batch=64, num_q_heads=40,
    num_kv_heads=8, head_dim=128, page_size=64, lengths="loguniform", length_lo=1024,
    length_hi=32768, pin_max=True, seed=3, splits=(1, 2, 4, 8, 16, 32), kv_layout="HND")
UNIFORM_B64 = RAGGED_B64.scaled(
    name="bf16_b64_hq40_hkv8_d128_p64_L32768", lengths="fixed", length=32768,
    pin_max=False)
INT8_B32 = Workload(
    name="int8kv_b32_hq32_hkv8_d128_p64_L32768", batch=32, num_q_heads=32, num_kv_heads=8,
    head_dim=128, page_size=64, kv=KV_INT8, lengths="fixed", length=32768, seed=4,
    splits=(1, 2, 4, 8, 16, 32), kv_layout="HND")
INT4_MTP_B64 = Workload(
    name="int4kv_mtp4_b64_hq32_hkv8_d128_p64_L8k-32k", batch=64, num_q_heads=32,
    num_kv_heads=8, head_dim=128, page_size=64, q_per_req=4, causal=True, kv=KV_INT4,
    lengths="uniform", length_lo=8192, length_hi=32768, seed=5,
    splits=(1, 2, 4, 8, 16, 32), kv_layout="HND")

# the INT4-MTP verify shape over a dense bf16 cache (16 query rows per kv-head)
BF16_MTP_B64 = INT4_MTP_B64.scaled(name="bf16_mtp4_b64_hq32_hkv8_d128_p64_L8k-32k", kv=KV_DENSE,
                                   seed=6)

# MTP verify (4 causal tokens) on the headline's heads (Hq 40, Hkv 8): 20 query
# rows per kv-head, processed as two row blocks of 10
BF16_MTP_G5_B64 = INT4_MTP_B64.scaled(name="bf16_mtp4_b64_hq40_hkv8_d128_p64_L8k-32k",
                                      kv=KV_DENSE, num_q_heads=40, seed=7)

# head dim 64: the INT4-MTP verify shape (16 query rows per kv-head)
INT4_MTP_D64_B64 = INT4_MTP_B64.scaled(name="int4kv_mtp4_b64_hq32_hkv8_d64_p64_L8k-32k",
                                       head_dim=64, seed=8)

# a dense fp32 cache (fp32 Q), B=16, G=8: 8 query rows per kv-head, on the fp32
# matrix cores
FP32_B16 = BF16_B16.scaled(name="fp32_b16_hq64_hkv8_d128_p64_L8192", dtype="fp32",
                           num_q_heads=64, seed=9)

# the same fp32 cache with G=4: 4 query rows per kv-head, on the vector ALU
FP32_G4_B16 = BF16_B16.scaled(name="fp32_b16_hq32_hkv8_d128_p64_L8192", dtype="fp32", seed=10)

WORKLOADS = {w.name: w for w in (TINY_FP32, BF16_B16, RAGGED_B64, UNIFORM_B64,
                                 INT8_B32, INT4_MTP_B64, BF16_MTP_B64, BF16_MTP_G5_B64,
                                 INT4_MTP_D64_B64, FP32_B16, FP32_G4_B16)}


def draw_lengths(w: Workload, rng: np.random.Generator) -> np.ndarray:
    """KV lengths per request (int64 numpy)."""
    B = w.batch
    if w.lengths == "fixed":
        L = np.full(B, w.length, dtype=np.int64)
    elif w.lengths == "list":
        assert len(w.length_list) == B
        L = np.asarray(w.length_list, dtype=np.int64)
    elif w.lengths == "loguniform":
        u = rng.uniform(math.log(w.length_lo), math.log(w.length_hi), size=B)
        L = np.clip(np.rint(np.exp(u)), w.length_lo, w.length_hi).astype(np.int64)
    elif w.lengths == "uniform":
        L = rng.integers(w.length_lo, w.length_hi, size=B, endpoint=True).astype(np.int64)
    else:
        raise ValueError(w.lengths)
    if w.pin_max:
        L[int(rng.integers(0, B))] = w.length_hi
    return L


@dataclass
class PagedBatch:
    """One synthetic decode batch.  Tensors live on ``device``."""

    w: Workload
    seq_lens: torch.Tensor          # [B] int32
    req_pool_indices: torch.Tensor  # [B] int64
    req_to_token: torch.Tensor      # [R, W] int32 token slots, -1 where unused
    page_table: torch.Tensor        # [B, max_pages] int32 physical page ids (0-padded)
    q: torch.Tensor                 # [B, q, Hq, D] bf16 / fp32
    k_pool: torch.Tensor            # dense [P,S,Hkv,D]; int8 [P,S,Hkv,D]; int4 u8 [P,S,Hkv,D/2]
    v_pool: torch.Tensor            # (the first three dims [P,Hkv,S] when w.kv_layout is "HND")
    k_scale: Optional[torch.Tensor] = None  # int8: fp16 [P,S,Hkv]; int4: fp16 [P,S,Hkv,D/32,2]
    v_scale: Optional[torch.Tensor] = None
    lengths: np.ndarray = field(default=None)

    @property
    def kv_layout(self) -> str:
        return self.w.kv_layout

    def nhd(self, t: torch.Tensor) -> torch.Tensor:
        """View of a pool or scale tensor of this batch in NHD order (dims 1, 2 swapped back)."""
        return t if self.w.kv_layout == "NHD" else t.transpose(1, 2)

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])


def _pages_needed(L: np.ndarray, page_size: int) -> np.ndarray:
    return (L + page_size - 1) // page_size


def build_layout(w: Workload, L: np.ndarray, rng: np.random.Generator, extra_rows: int = 3):
    """Scatter each request's logical pages over a randomly permuted pool.

    Returns (page_table [B, max_pages] int32, req_to_token [R, W] int32,
    req_pool_indices [B] int64, num_pages).
    """
    B, S = w.batch, w.page_size
    n = _pages_needed(L, S)
    total = int(n.sum())
    P = w.pool_pages if w.pool_pages else total
    assert P >= total, "pool too small"
    max_pages = max(1, int(n.max()))
    perm = rng.permutation(P)[:total]
    page_table = np.zeros((B, max_pages), dtype=np.int32)
    off = 0
    for b in range(B):
        page_table[b, : n[b]] = perm[off: off + n[b]]
        off += n[b]
    R = B + extra_rows
    W = max_pages * S
    rpi = rng.permutation(R)[:B].astype(np.int64)
    r2t = np.full((R, W), -1, dtype=np.int32)
    for b in range(B):
        t = np.arange(L[b])
        r2t[rpi[b], : L[b]] = page_table[b, t // S] * S + (t % S)
    return page_table, r2t, rpi, P


def _to_dtype(x: torch.Tensor, dtype: str) -> torch.Tensor:
    return x.to(torch.bfloat16) if dtype == "bf16" else x.to(torch.float32)


def quantize_int8(x: torch.Tensor):
    """Symmetric int8 with one fp16 scale per row of the last dim.

    s = fp16(amax / 127) (1 where that is 0), code = clamp(rne(x / s), -127, 127).
    Test-data encoder only.
    """
    xf = x.to(torch.float32)
    amax = xf.abs().amax(dim=-1)
    s = (amax / 127.0).to(torch.float16)
    s = torch.where(s == 0, torch.ones_like(s), s)
    code = torch.clamp(torch.round(xf / s.to(torch.float32).unsqueeze(-1)), -127, 127)
    return code.to(torch.int8), s


def quantize_int4(x: torch.Tensor, group: int = INT4_GROUP):
    """Asymmetric 4-bit with fp16 (scale, zero) per group of ``group`` along D.

    s = fp16((max - min) / 15) (1 where that is 0); z = fp16(clamp(rne(-min / s), 0, 15));
    nib = clamp(rne(x / s) + z, 0, 15); byte j = nib[2j] | nib[2j+1] << 4.
    Returns (packed uint8 [..., D/2], scale_zero fp16 [..., D/group, 2]).
    Test-data encoder only.
    """
    xf = x.to(torch.float32)
    D = xf.shape[-1]
    g = xf.reshape(*xf.shape[:-1], D // group, group)
    mn = g.amin(dim=-1)
    mx = g.amax(dim=-1)
    s = ((mx - mn) / 15.0).to(torch.float16)
    s = torch.where(s == 0, torch.ones_like(s), s)
    sf = s.to(torch.float32)
    z = (torch.clamp(torch.round(-mn / sf), 0, 15) + 0.0).to(torch.float16)  # -0 -> +0
    nib = torch.clamp(torch.round(g / sf.unsqueeze(-1)) + z.to(torch.float32).unsqueeze(-1), 0, 15)
    nib = nib.to(torch.uint8).reshape(*xf.shape[:-1], D)
    packed = nib[..., 0::2] | (nib[..., 1::2] << 4)
    sz = torch.stack([s, z], dim=-1)
    return packed.contiguous(), sz.contiguous()


def make_batch(w: Workload, device="cpu", seed: Optional[int] = None,
               lengths: Optional[np.ndarray] = None) -> PagedBatch:
    """Build the batch for workload ``w``.

    Lengths, the page permutation, the req-pool permutation and Q come from a
    numpy PCG64 stream seeded ``1000 + seed``; K/V come from a torch generator
    on ``device`` seeded ``2000 + seed`` (read back to the host by whoever
    needs host copies).
    """
    seed = w.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(1000 + seed))
    L = draw_lengths(w, rng) if lengths is None else np.asarray(lengths, dtype=np.int64)
    page_table, r2t, rpi, P = build_layout(w, L, rng)
    B, Hq, Hkv, D, S, qn = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size, w.q_per_req
    q = torch.from_numpy(rng.standard_normal((B, qn, Hq, D)).astype(np.float32)) * w.amp[0]
    q = _to_dtype(q, "fp32" if w.dtype == "fp32" else "bf16").to(device)

    gen = torch.Generator(device=device)
    gen.manual_seed(2000 + seed)
    shape = (P, S, Hkv, D)

    def normal(sd):
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * sd

    k_scale = v_scale = None
    ka, va = w.amp[1], w.amp[2]
    if w.kv == KV_DENSE:
        k_pool = _to_dtype(normal(ka), w.dtype)
        v_pool = _to_dtype(normal(va), w.dtype)
    elif w.kv == KV_INT8:
        k_pool, k_scale = quantize_int8(normal(ka).to(torch.bfloat16))
        v_pool, v_scale = quantize_int8(normal(va).to(torch.bfloat16))
    elif w.kv == KV_INT4:
        k_pool, k_scale = quantize_int4(normal(ka).to(torch.bfloat16))
        v_pool, v_scale = quantize_int4(normal(va).to(torch.bfloat16))
    else:
        raise ValueError(w.kv)
    if w.kv_layout == "HND":  # same values, head-major within each page
        k_pool, v_pool = to_hnd(k_pool), to_hnd(v_pool)
        if k_scale is not None:
            k_scale, v_scale = to_hnd(k_scale), to_hnd(v_scale)
    elif w.kv_layout != "NHD":
        raise ValueError(w.kv_layout)
    return PagedBatch(
        w=w,
        seq_lens=torch.from_numpy(L.astype(np.int32)).to(device),
        req_pool_indices=torch.from_numpy(rpi).to(device),
        req_to_token=torch.from_numpy(r2t).to(device),
        page_table=torch.from_numpy(page_table).to(device),
        q=q, k_pool=k_pool, v_pool=v_pool, k_scale=k_scale, v_scale=v_scale,
        lengths=L,
    )


def to_hnd(t: torch.Tensor) -> torch.Tensor:
    """[P, page, Hkv, ...] -> contiguous [P, Hkv, page, ...]."""
    return t.transpose(1, 2).contiguous()


def host_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a float tensor to a float64 numpy array on the host."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def host_int(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").numpy()


def host_u16(t: torch.Tensor) -> np.ndarray:
    """fp16 tensor -> its raw bit patterns (uint16), for decoders that widen them."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
