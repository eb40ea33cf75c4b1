"""GPU parity of stage 1 (split), stage 2 (merge) and the whole decode
against the fp64 oracle, on seeded inputs shaped like the pages' workloads.

Small cases are compared element by element (every output, every split
partial); full-size workloads in the launch configuration the benchmark uses
are compared on sampled (request, kv-head) pairs the oracle evaluates one by
one.  Gates are documented in tests/_gpu_util.py.
"""
import numpy as np
import pytest
import torch

from decode_attention_paged_gqa_amd import workloads as W
from tests import _gpu_util as U

pytestmark = pytest.mark.gpu
log = U.log

# ---------------------------------------------------------------- small cases
TINY = W.TINY_FP32
TINY_BF16 = W.TINY_FP32.scaled(name="tiny_bf16", dtype="bf16")
EDGE_LENGTHS = (0, 1, 2, 15, 16, 17, 63, 64, 65, 127, 128, 129, 1000, 2047, 3001, 5)
RAGGED_SMALL = W.RAGGED_B64.scaled(name="ragged_small_g5", batch=len(EDGE_LENGTHS),
                                   lengths="list", length_list=EDGE_LENGTHS, pin_max=False)
BF16_SMALL = W.BF16_B16.scaled(name="bf16_small_g4", batch=4, length=1500)
D64_P16 = W.RAGGED_B64.scaled(name="d64_p16_g2", batch=5, num_q_heads=8, num_kv_heads=4,
                              head_dim=64, page_size=16, lengths="list",
                              length_list=(3, 16, 40, 333, 17), pin_max=False)
# D = 64 with 6 or more query rows per kv-head: the matrix-core path
D64_G8 = W.RAGGED_B64.scaled(name="d64_g8_p16", batch=8, num_q_heads=32, num_kv_heads=4,
                             head_dim=64, page_size=16, lengths="list",
                             length_list=(0, 1, 15, 16, 17, 63, 65, 2047), pin_max=False)
D64_MTP = W.BF16_B16.scaled(name="d64_mtp4_g4_r16", batch=5, q_per_req=4, causal=True,
                            head_dim=64, lengths="list", length_list=(1, 3, 4, 70, 900))
D64_R20 = W.BF16_B16.scaled(name="d64_mtp4_g5_r20_p32", batch=3, num_q_heads=40, q_per_req=4,
                            causal=True, head_dim=64, page_size=32, lengths="list",
                            length_list=(2, 100, 1300))
D64_G6_P128 = W.BF16_B16.scaled(name="d64_g6_p128", batch=4, num_q_heads=12, num_kv_heads=2,
                                head_dim=64, page_size=128, lengths="list",
                                length_list=(127, 128, 129, 3000))
# fp32 with up to 4 query rows per kv-head: the vector-ALU kernel
FP32_G4_D128 = W.TINY_FP32.scaled(name="fp32_g4_d128_p64", batch=4, num_q_heads=8, num_kv_heads=2,
                                  head_dim=128, page_size=64, lengths="list",
                                  length_list=(1, 64, 65, 1300), pool_pages=0)
FP32_G2 = W.TINY_FP32.scaled(name="fp32_g2_d64_p16", batch=6, num_q_heads=4, num_kv_heads=2,
                             lengths="list", length_list=(0, 1, 15, 16, 17, 700), pool_pages=0)
FP32_G1_NC = W.TINY_FP32.scaled(name="fp32_mha_d64_p64", batch=3, num_q_heads=3, num_kv_heads=3,
                                page_size=64, lengths="list", length_list=(5, 64, 1000),
                                pool_pages=0)
FP32_MTP2_G2 = W.TINY_FP32.scaled(name="fp32_mtp2_g2_r4_d128", batch=4, num_q_heads=4,
                                  num_kv_heads=2, head_dim=128, page_size=64, q_per_req=2,
                                  causal=True, lengths="list", length_list=(1, 2, 65, 1300),
                                  pool_pages=0)
FP32_G3_D64 = W.TINY_FP32.scaled(name="fp32_g3_d64_p32", batch=4, num_q_heads=6, num_kv_heads=2,
                                 page_size=32, lengths="list", length_list=(7, 32, 33, 900),
                                 pool_pages=0)
# the other fp32 shapes: the fp32 matrix-core path
FP32_G5 = W.TINY_FP32.scaled(name="fp32_g5_d128_p64", batch=3, num_q_heads=10, num_kv_heads=2,
                             head_dim=128, page_size=64, lengths="list",
                             length_list=(1, 200, 1500), pool_pages=0)
FP32_G8_P16 = W.TINY_FP32.scaled(name="fp32_g8_d64_p16", batch=6, num_q_heads=8, num_kv_heads=1,
                                 lengths="list", length_list=(0, 1, 15, 16, 17, 700),
                                 pool_pages=0)
FP32_MTP = W.TINY_FP32.scaled(name="fp32_mtp4_g4_r16_d128", batch=4, num_q_heads=16,
                              num_kv_heads=4, head_dim=128, page_size=64, q_per_req=4,
                              causal=True, lengths="list", length_list=(2, 4, 90, 1100),
                              pool_pages=0)
FP32_R20 = W.TINY_FP32.scaled(name="fp32_mtp4_g5_r20_d64_p32", batch=3, num_q_heads=10,
                              num_kv_heads=2, page_size=32, q_per_req=4, causal=True,
                              lengths="list", length_list=(3, 100, 900), pool_pages=0)
MHA_P32 = W.RAGGED_B64.scaled(name="mha_p32_g1", batch=3, num_q_heads=4, num_kv_heads=4,
                              page_size=32, lengths="list", length_list=(33, 100, 1), pin_max=False)
MTP_BF16 = W.BF16_B16.scaled(name="mtp4_bf16_g4", batch=5, q_per_req=4, causal=True,
                             lengths="list", length_list=(1, 3, 4, 70, 900))
MTP_BF16_G2Q3 = W.BF16_B16.scaled(name="mtp3_bf16_g2", batch=3, num_q_heads=16, q_per_req=3,
                                  causal=True, lengths="list", length_list=(2, 66, 500))
INT8_SMALL = W.INT8_B32.scaled(name="int8_small", batch=5, lengths="list",
                               length_list=(1, 64, 65, 777, 2000))
INT8_MTP = W.INT8_B32.scaled(name="int8_mtp2_r8_small", batch=4, q_per_req=2, causal=True,
                             lengths="list", length_list=(2, 33, 500, 1500))
INT8_G8Q2 = W.INT8_B32.scaled(name="int8_g8_mtp2_r16_small", batch=3, num_q_heads=64, q_per_req=2,
                              causal=True, lengths="list", length_list=(1, 80, 900))
INT8_ODD_HKV = W.INT8_B32.scaled(name="int8_hkv3_g2_small", batch=4, num_q_heads=6,
                                 num_kv_heads=3, lengths="list", length_list=(5, 64, 129, 1100))
INT8_FP32Q = W.INT8_B32.scaled(name="int8_fp32q_small", batch=3, dtype="fp32", lengths="list",
                               length_list=(1, 100, 700))
INT8_FP32Q_MTP = W.INT8_B32.scaled(name="int8_fp32q_mtp4_r16", batch=3, dtype="fp32", q_per_req=4,
                                   causal=True, lengths="list", length_list=(2, 65, 1200))
INT8_FP32Q_D64 = W.INT8_B32.scaled(name="int8_fp32q_d64_r4", batch=3, dtype="fp32", head_dim=64,
                                   lengths="list", length_list=(1, 300, 900))
INT8_D64 = W.INT8_B32.scaled(name="int8_d64_small", batch=3, head_dim=64, lengths="list",
                             length_list=(7, 64, 1000))
INT8_D64_MTP = W.INT8_B32.scaled(name="int8_d64_mtp4_r16_p16", batch=4, q_per_req=4, causal=True,
                                 head_dim=64, page_size=16, lengths="list",
                                 length_list=(1, 17, 64, 1500))
INT8_D64_R20 = W.INT8_B32.scaled(name="int8_d64_g5_mtp4_r20_p128", batch=3, num_q_heads=40,
                                 q_per_req=4, causal=True, head_dim=64, page_size=128,
                                 lengths="list", length_list=(3, 129, 2100))
INT4_SMALL = W.INT4_MTP_B64.scaled(name="int4_mtp_small", batch=5, lengths="list",
                                   length_list=(1, 4, 65, 777, 2000))
INT4_Q1 = W.INT4_MTP_B64.scaled(name="int4_q1_small", batch=4, q_per_req=1, causal=False,
                                lengths="list", length_list=(1, 64, 300, 1500))
INT4_R12 = W.INT4_MTP_B64.scaled(name="int4_mtp3_r12_small", batch=4, q_per_req=3,
                                 lengths="list", length_list=(2, 17, 95, 1234))
INT4_D64 = W.INT4_MTP_B64.scaled(name="int4_d64_mtp4_r16_p16", batch=4, head_dim=64,
                                 page_size=16, lengths="list", length_list=(1, 4, 17, 1500))
INT4_D64_Q1 = W.INT4_MTP_B64.scaled(name="int4_d64_q1_r4", batch=4, head_dim=64, q_per_req=1,
                                    causal=False, lengths="list", length_list=(1, 64, 300, 2000))
INT4_D64_R20 = W.INT4_MTP_B64.scaled(name="int4_d64_g5_mtp4_r20_p128", batch=3, num_q_heads=40,
                                     head_dim=64, page_size=128, lengths="list",
                                     length_list=(3, 129, 2100))
INT4_FP32Q = W.INT4_MTP_B64.scaled(name="int4_fp32q_mtp4_r16", batch=4, dtype="fp32",
                                   lengths="list", length_list=(1, 5, 129, 1400))
INT4_FP32Q_Q1 = W.INT4_MTP_B64.scaled(name="int4_fp32q_q1_r4", batch=3, dtype="fp32", q_per_req=1,
                                      causal=False, lengths="list", length_list=(7, 64, 800))
INT4_FP32Q_D64 = W.INT4_MTP_B64.scaled(name="int4_fp32q_d64_r16_p32", batch=3, dtype="fp32",
                                       head_dim=64, page_size=32, lengths="list",
                                       length_list=(3, 100, 1000))
# fp32 Q over quantised caches with two row tiles per workgroup (17..32 rows)
INT4_FP32Q_R20 = W.INT4_MTP_B64.scaled(name="int4_fp32q_g5_mtp4_r20", batch=3, dtype="fp32",
                                       num_q_heads=40, lengths="list", length_list=(3, 130, 1000))
INT4_FP32Q_D64_R32 = W.INT4_MTP_B64.scaled(name="int4_fp32q_d64_g8_mtp4_r32", batch=3,
                                           dtype="fp32", num_q_heads=64, head_dim=64,
                                           lengths="list", length_list=(2, 70, 900))
INT8_FP32Q_R20 = W.INT8_B32.scaled(name="int8_fp32q_g5_mtp4_r20", batch=3, dtype="fp32",
                                   num_q_heads=40, q_per_req=4, causal=True, lengths="list",
                                   length_list=(5, 129, 1000))
INT4_G8Q2 = W.INT4_MTP_B64.scaled(name="int4_g8_mtp2_small", batch=3, num_q_heads=64, q_per_req=2,
                                  lengths="list", length_list=(1, 48, 700))
# kv-head counts that are not a multiple of 4: token-major pools take the
# one-kv-head-per-workgroup kernel (four per workgroup need a multiple of 4),
# D = 128 and 64
INT4_ODD_HKV = W.INT4_MTP_B64.scaled(name="int4_hkv3_mtp4_r16_small", batch=3, num_q_heads=12,
                                     num_kv_heads=3, lengths="list", length_list=(2, 70, 1300))
INT4_D64_MQA = W.INT4_MTP_B64.scaled(name="int4_d64_hkv1_q2_r8", batch=3, num_q_heads=4,
                                     num_kv_heads=1, head_dim=64, q_per_req=2,
                                     lengths="list", length_list=(9, 300, 1000))
# four kv-heads per workgroup (token-major INT8 / INT4, dense bf16 and fp32 at
# D = 64): one group of four (Hkv = 4), three (Hkv = 12), and two row tiles
# (20 rows) at D = 128, and four groups at Hkv = 16 (every such kernel)
QUAD = [
    W.INT4_MTP_B64.scaled(name="int4_hkv16_g2_mtp2_r4", batch=3, num_q_heads=32, num_kv_heads=16,
                          q_per_req=2, lengths="list", length_list=(1, 260, 1300)),
    W.INT4_MTP_B64.scaled(name="int4_d64_hkv16_g3_r3", batch=2, num_q_heads=48, num_kv_heads=16,
                          head_dim=64, q_per_req=1, causal=False, lengths="list",
                          length_list=(100, 2222)),
    W.INT8_B32.scaled(name="int8_hkv16_g2", batch=2, num_q_heads=32, num_kv_heads=16,
                      lengths="list", length_list=(70, 1900)),
    W.BF16_MTP_B64.scaled(name="bf16_d64_hkv16_g2_mtp4_r8", batch=2, num_q_heads=32,
                          num_kv_heads=16, head_dim=64, lengths="list", length_list=(5, 1700)),
    W.RAGGED_B64.scaled(name="bf16_d64_hkv16_g3", batch=2, num_q_heads=48, num_kv_heads=16,
                        head_dim=64, lengths="list", length_list=(1, 1200), pin_max=False),
    W.TINY_FP32.scaled(name="fp32_d64_hkv16_g2", batch=2, num_q_heads=32, num_kv_heads=16,
                       page_size=64, lengths="list", length_list=(33, 700), pool_pages=0),
    W.TINY_FP32.scaled(name="fp32_d64_hkv16_g8", batch=2, num_q_heads=128, num_kv_heads=16,
                       page_size=64, lengths="list", length_list=(2, 650), pool_pages=0),
    W.INT4_MTP_B64.scaled(name="int4_hkv4_mtp4_r16", batch=3, num_q_heads=16, num_kv_heads=4,
                          lengths="list", length_list=(2, 70, 1500)),
    W.INT4_MTP_B64.scaled(name="int4_hkv12_mtp4_r8", batch=3, num_q_heads=24, num_kv_heads=12,
                          lengths="list", length_list=(5, 200, 900)),
    W.INT4_MTP_B64.scaled(name="int4_g5_mtp4_r20", batch=3, num_q_heads=40, lengths="list",
                          length_list=(3, 129, 1100)),
    W.INT8_B32.scaled(name="int8_hkv4_g4", batch=3, num_q_heads=16, num_kv_heads=4,
                      lengths="list", length_list=(1, 65, 1400)),
    W.INT8_B32.scaled(name="int8_hkv12_g2_mtp2_r4", batch=3, num_q_heads=24, num_kv_heads=12,
                      q_per_req=2, causal=True, lengths="list", length_list=(2, 300, 800)),
    W.INT8_B32.scaled(name="int8_g5_mtp4_r20", batch=3, num_q_heads=40, q_per_req=4, causal=True,
                      lengths="list", length_list=(4, 129, 1100)),
    W.BF16_MTP_B64.scaled(name="bf16_d64_hkv4_mtp4_r16", batch=3, num_q_heads=16, num_kv_heads=4,
                          head_dim=64, lengths="list", length_list=(4, 100, 1200)),
    W.BF16_MTP_B64.scaled(name="bf16_d64_hkv12_mtp2_r8", batch=3, num_q_heads=48, num_kv_heads=12,
                          head_dim=64, q_per_req=2, lengths="list", length_list=(2, 77, 600)),
    # dense bf16 and fp32 at D = 64 on the vector ALU, fp32 on the matrix cores
    W.RAGGED_B64.scaled(name="bf16_d64_hkv4_g5", batch=3, num_q_heads=20, num_kv_heads=4,
                        head_dim=64, lengths="list", length_list=(1, 150, 1300), pin_max=False),
    W.TINY_FP32.scaled(name="fp32_d64_hkv4_g2", batch=3, num_q_heads=8, num_kv_heads=4,
                       page_size=64, lengths="list", length_list=(3, 130, 1100), pool_pages=0),
    W.TINY_FP32.scaled(name="fp32_d64_hkv4_g8", batch=3, num_q_heads=32, num_kv_heads=4,
                       page_size=64, lengths="list", length_list=(2, 90, 900), pool_pages=0),
]


def _check_out(w, out, ref, label):
    if w.kv != W.KV_DENSE:
        U.check_quant(out, ref, label)
    elif w.dtype == "fp32" and out.dtype == np.float64 and label.endswith("fp32"):
        U.check_fp32(out, ref, label)
    else:
        U.check_bf16(out, ref, label)


@pytest.mark.parametrize("S", [1, 2, 4])
def test_tiny_fp32_every_split(gpu, S):
    log(f"tiny fp32 S={S}")
    batch = W.make_batch(TINY, device="cuda")
    o_ref, l_ref = U.oracle_partials(batch, S)
    out_ref, lse_ref = U.oracle_full(batch)
    out, lse, o, l = U.run_decode(gpu, batch, S, out_dtype=torch.float32)
    U.check_partials(U.to_np(o), U.to_np(l), o_ref, l_ref, f"tiny S={S}")
    U.check_fp32(U.to_np(out), out_ref, f"tiny S={S} out fp32")
    U.check_lse(U.to_np(lse), lse_ref, f"tiny S={S} lse")
    out16, _, _, _ = U.run_decode(gpu, batch, S, out_dtype=torch.bfloat16)
    U.check_bf16(U.to_np(out16), out_ref, f"tiny S={S} out bf16")


SMALL = [TINY_BF16, RAGGED_SMALL, BF16_SMALL, D64_P16, D64_G8, D64_MTP, D64_R20, D64_G6_P128,
         FP32_G2, FP32_G1_NC, FP32_G4_D128, FP32_MTP2_G2, FP32_G3_D64, FP32_G5, FP32_G8_P16, FP32_MTP, FP32_R20, MHA_P32, MTP_BF16, MTP_BF16_G2Q3,
         INT8_SMALL, INT8_MTP, INT8_G8Q2, INT8_ODD_HKV, INT8_FP32Q, INT8_D64, INT8_D64_MTP, INT8_D64_R20,
         INT4_SMALL, INT4_Q1,
         INT4_R12, INT4_G8Q2, INT4_D64, INT4_D64_Q1, INT4_D64_R20, INT8_FP32Q_MTP, INT8_FP32Q_D64,
         INT4_FP32Q, INT4_FP32Q_Q1, INT4_FP32Q_D64, INT4_ODD_HKV, INT4_D64_MQA,
         INT4_FP32Q_R20, INT4_FP32Q_D64_R32, INT8_FP32Q_R20] + QUAD


def both_layouts(ws):
    """Every case in the token-major (NHD) and the head-major (HND) pool layout."""
    return [w.scaled(name=f"{w.name}_{lay.lower()}", kv_layout=lay) for w in ws
            for lay in ("NHD", "HND")]


@pytest.mark.parametrize("w", both_layouts(SMALL), ids=lambda w: w.name)
@pytest.mark.parametrize("S", [1, 3, 8, 32])
def test_small_elementwise(gpu, w, S):
    log(f"small {w.name} S={S}")
    batch = W.make_batch(w, device="cuda")
    o_ref, l_ref = U.oracle_partials(batch, S)
    out_ref, lse_ref = U.oracle_full(batch)
    out, lse, o, l = U.run_decode(gpu, batch, S)
    extra = U.matrix_path_o_bound(batch)
    U.check_partials(U.to_np(o), U.to_np(l), o_ref, l_ref, f"{w.name} S={S}", o_extra=extra)
    _check_out(w, U.to_np(out), out_ref, f"{w.name} S={S} out")
    U.check_lse(U.to_np(lse), lse_ref, f"{w.name} S={S} lse")


@pytest.mark.parametrize("w", both_layouts([INT4_SMALL, INT4_Q1, INT4_R12, INT4_D64]),
                         ids=lambda w: w.name)
def test_int4_fractional_zero_points(gpu, w):
    """The zero point is any fp16 value, not only a code: shift every zero by a
    fraction (different per slot) and compare with the oracle decoding the same
    bits."""
    log(f"int4 fractional zeros {w.name}")
    batch = W.make_batch(w, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(11)
    for sc in (batch.k_scale, batch.v_scale):
        frac = torch.rand(sc[..., 1].shape, generator=gen, device="cuda") * 0.9 + 0.05
        sc[..., 1] = (sc[..., 1].float() + frac).to(torch.float16)
    S = 3
    o_ref, l_ref = U.oracle_partials(batch, S)
    out_ref, lse_ref = U.oracle_full(batch)
    out, lse, o, l = U.run_decode(gpu, batch, S)
    extra = U.matrix_path_o_bound(batch)
    U.check_partials(U.to_np(o), U.to_np(l), o_ref, l_ref, f"{w.name} frac-z", o_extra=extra)
    U.check_quant(U.to_np(out), out_ref, f"{w.name} frac-z out")
    U.check_lse(U.to_np(lse), lse_ref, f"{w.name} frac-z lse")


def test_page_permutation_is_bit_identical(gpu):
    w = RAGGED_SMALL
    log("page permutation invariance")
    batch = W.make_batch(w, device="cuda")
    out1, lse1, _, _ = U.run_decode(gpu, batch, 4)
    P = batch.num_pages
    perm = torch.randperm(P, generator=torch.Generator().manual_seed(5)).cuda()
    k2 = torch.empty_like(batch.k_pool)
    v2 = torch.empty_like(batch.v_pool)
    k2[perm] = batch.k_pool
    v2[perm] = batch.v_pool
    pt2 = perm[batch.page_table.long()].to(torch.int32)
    batch.k_pool, batch.v_pool, batch.page_table = k2, v2, pt2
    out2, lse2, _, _ = U.run_decode(gpu, batch, 4)
    assert torch.equal(out1, out2)
    assert torch.equal(lse1, lse2)


def test_batch_order_is_bit_identical(gpu):
    """Scheduling requests longest-first (the metadata batch order) changes no bit."""
    for w in both_layouts([RAGGED_SMALL, INT8_SMALL, INT8_ODD_HKV, INT4_SMALL, MTP_BF16]):
        log(f"batch order {w.name}")
        batch = W.make_batch(w, device="cuda")
        md = gpu.decode_attn_metadata(batch.seq_lens, batch.req_pool_indices, batch.req_to_token,
                                      w.page_size, batch.max_pages)
        for S in (1, 4):
            o1, l1 = U.run_split(gpu, batch, S)
            o2, l2 = U.run_split(gpu, batch, S, batch_order=md["batch_order"])
            assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_num_splits_invariance(gpu):
    w = RAGGED_SMALL
    log("num_splits invariance")
    batch = W.make_batch(w, device="cuda")
    base, _, _, _ = U.run_decode(gpu, batch, 1, out_dtype=torch.float32)
    for S in (2, 5, 16, 64, 256):
        out, _, _, _ = U.run_decode(gpu, batch, S, out_dtype=torch.float32)
        d = (out - base).abs().max().item()
        log(f"  S={S}: max |out - out(S=1)| = {d:.3e}")
        assert d <= 1e-5


def test_outputs_fully_overwritten(gpu):
    """Stage 1 writes every partial slot (no clearing needed): poison first."""
    w = RAGGED_SMALL
    batch = W.make_batch(w, device="cuda")
    B, qn, Hq, D = batch.q.shape
    S = 16
    o = torch.full((B, qn, Hq, S, D), float("nan"), device="cuda")
    l = torch.full((B, qn, Hq, S), float("nan"), device="cuda")
    gpu.decode_attn_split(batch.q, batch.k_pool, batch.v_pool, batch.page_table, batch.seq_lens,
                          S, w.softmax_scale, False, o_partial=o, lse_partial=l,
                          kv_layout=w.kv_layout)
    assert not torch.isnan(o).any() and not torch.isnan(l).any()


@pytest.mark.parametrize("w", both_layouts([RAGGED_SMALL.scaled(pool_pages=200),
                                             MTP_BF16.scaled(pool_pages=80),
                                             INT8_SMALL.scaled(pool_pages=80),
                                             INT4_SMALL.scaled(pool_pages=80)]),
                         ids=lambda w: w.name)
def test_nan_in_unused_slots_does_not_leak(gpu, w):
    """Slots past a request's length (tail of its last page, unused pages) may hold
    anything: NaN in dense pools, NaN scales and arbitrary codes in quantised ones.
    Poison them and check the output is bit-identical."""
    batch = W.make_batch(w, device="cuda")
    ref, _, _, _ = U.run_decode(gpu, batch, 4)
    L = batch.lengths
    pt = batch.page_table.cpu().numpy()
    used = torch.zeros(batch.num_pages, w.page_size, dtype=torch.bool)
    for b in range(len(L)):
        t = np.arange(int(L[b]))
        used[pt[b, t // w.page_size], t % w.page_size] = True
    mask = (~used).cuda()  # [P, page] slots; nhd() views the pools in that order
    if w.kv == W.KV_DENSE:
        batch.nhd(batch.k_pool)[mask] = float("nan")
        batch.nhd(batch.v_pool)[mask] = float("nan")
    else:
        for sc in (batch.k_scale, batch.v_scale):
            batch.nhd(sc)[mask] = float("nan")
        for pool in (batch.k_pool, batch.v_pool):
            junk = torch.randint(0, 256, pool.shape, dtype=torch.uint8, device="cuda").view(pool.dtype)
            batch.nhd(pool)[mask] = batch.nhd(junk)[mask]
    out, _, _, _ = U.run_decode(gpu, batch, 4)
    assert torch.equal(out, ref)


# ---------------------------------------------------------------- full sizes
# The benchmark's launch configuration: its split count comes from the tuned
# table for the kernel variant, batch size and longest request, as bench.py
# picks it (None below); a second fixed count covers another split shape.
FULL = [
    (W.BF16_B16, None, [(0, 0), (7, 3), (15, 7)]),
    (W.RAGGED_B64, None, None),
    (W.RAGGED_B64, 16, None),
    (W.UNIFORM_B64, None, [(0, 0), (63, 7), (21, 4)]),
    (W.INT8_B32, None, [(0, 0), (31, 7), (13, 2)]),
    (W.INT4_MTP_B64, None, None),
    (W.INT4_MTP_B64, 8, None),
    (W.BF16_MTP_B64, None, None),
    (W.INT4_MTP_D64_B64, None, None),
    # the token-major pool layout of the pages, at its own tuned split counts
    (W.RAGGED_B64.scaled(name=W.RAGGED_B64.name + "_nhd", kv_layout="NHD"), None, None),
    (W.INT8_B32.scaled(name=W.INT8_B32.name + "_nhd", kv_layout="NHD"), None,
     [(0, 0), (31, 7), (13, 2)]),
    (W.INT4_MTP_B64.scaled(name=W.INT4_MTP_B64.name + "_nhd", kv_layout="NHD"), None, None),
]


def bench_splits(w, batch):
    from decode_attention_paged_gqa_amd.splits import SplitTable, kernel_key
    kv = w.dtype if w.kv == W.KV_DENSE else w.kv
    key = kernel_key(kv, w.group * w.q_per_req, w.head_dim, w.page_size, w.kv_layout)
    return SplitTable.load().pick(key, w.batch, int(batch.lengths.max()))


@pytest.mark.parametrize("w,S,pairs", FULL,
                         ids=[f"{f[0].name}-S{f[1] or 'bench'}" for f in FULL])
def test_full_size_sampled(gpu, w, S, pairs):
    batch = W.make_batch(w, device="cuda")
    S = S or bench_splits(w, batch)
    log(f"full {w.name} ({w.kv_layout}) S={S}")
    out, lse, _, _ = U.run_decode(gpu, batch, S, batch_order=gpu.decode_attn_metadata(
        batch.seq_lens, batch.req_pool_indices, batch.req_to_token, w.page_size,
        batch.max_pages, q_stride=w.q_per_req)["batch_order"])
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    L = batch.lengths
    if pairs is None:  # the longest and the shortest request, and one in between
        order = np.argsort(L)
        pairs = [(int(order[-1]), 0), (int(order[0]), w.num_kv_heads - 1),
                 (int(order[len(L) // 2]), 3)]
    res = U.oracle_sampled(batch, pairs)
    G = w.group
    for (b, g), (o_ref, l_ref) in res.items():
        got = U.to_np(out[b, :, g * G:(g + 1) * G])
        got_l = U.to_np(lse[b, :, g * G:(g + 1) * G])
        _check_out(w, got, o_ref, f"{w.name} b={b} (L={L[b]}) g={g}")
        U.check_lse(got_l, l_ref, f"{w.name} b={b} g={g} lse")
