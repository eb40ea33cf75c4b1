"""GPU parity at the edges of the supported shapes, element by element against
the fp64 oracle (gates in tests/_gpu_util.py):

* a split longer than the specialised kernels' page-id tables (1024 pages for
  the bf16 vector kernel, 512 for the matrix-core ones), which they take in
  chunks of page ids;
* page sizes 128 and 256;
* 16 query rows per kv-head from 16 MTP tokens of one head (q_per_req = 16);
* a batch much wider than one workgroup (300 requests), with both schedules;
* more than 16 query rows per kv-head (G * q_per_req up to 256), which runs
  as row blocks (of up to 32 rows, two 16-row tiles, on the matrix-core
  kernels; of up to 16 on the others), with both schedules.
"""
import numpy as np
import pytest
import torch

from decode_attention_paged_gqa_amd import workloads as W
from tests import _gpu_util as U
from tests.test_gpu_attention import _check_out, both_layouts

pytestmark = pytest.mark.gpu
log = U.log


def _run_and_check(gpu, w, S, label):
    log(f"{label}: {w.name} S={S}")
    batch = W.make_batch(w, device="cuda")
    o_ref, l_ref = U.oracle_partials(batch, S)
    out_ref, lse_ref = U.oracle_full(batch)
    out, lse, o, l = U.run_decode(gpu, batch, S)
    extra = U.matrix_path_o_bound(batch)
    U.check_partials(U.to_np(o), U.to_np(l), o_ref, l_ref, f"{w.name} S={S}", o_extra=extra)
    _check_out(w, U.to_np(out), out_ref, f"{w.name} S={S} out")
    U.check_lse(U.to_np(lse), lse_ref, f"{w.name} S={S} lse")


# one request whose single split spans more pages than the LDS page-id table
# (1024 pages for the bf16 vector kernel, 512 for the matrix-core kernels):
# two or three chunks of page ids
LONG = [
    W.RAGGED_B64.scaled(name="long_split_bf16_g5_p16", batch=2, page_size=16, lengths="list",
                        length_list=(16400, 37), pin_max=False),
    W.INT8_B32.scaled(name="long_split_int8_p16", batch=2, page_size=16, lengths="list",
                      length_list=(8250, 5)),
    W.INT4_MTP_B64.scaled(name="long_split_int4_mtp_p16", batch=2, page_size=16, lengths="list",
                          length_list=(8250, 9)),
    W.BF16_MTP_B64.scaled(name="long_split_bf16_mtp_p16", batch=2, page_size=16, lengths="list",
                          length_list=(8250, 9)),
    # fp32: the vector kernel (1024-page table; 2-stage ring at D = 128, 4 at D = 64)
    # and the matrix-core kernel (512 pages)
    W.TINY_FP32.scaled(name="long_split_fp32_g4_d128_p16", batch=2, num_q_heads=8, num_kv_heads=2,
                       head_dim=128, lengths="list", length_list=(16400, 37), pool_pages=0),
    W.TINY_FP32.scaled(name="long_split_fp32_g2_d64_p16", batch=2, num_q_heads=4, num_kv_heads=2,
                       lengths="list", length_list=(16400, 37), pool_pages=0),
    W.TINY_FP32.scaled(name="long_split_fp32_g8_d128_p16", batch=2, num_q_heads=8, num_kv_heads=1,
                       head_dim=128, lengths="list", length_list=(8250, 9), pool_pages=0),
]


@pytest.mark.parametrize("w", both_layouts(LONG), ids=lambda w: w.name)
def test_split_longer_than_the_page_id_table(gpu, w):
    _run_and_check(gpu, w, 1, "long split")


PAGES = [
    W.RAGGED_B64.scaled(name="ragged_g5_p128", batch=4, page_size=128, lengths="list",
                        length_list=(1, 127, 129, 3000), pin_max=False),
    W.RAGGED_B64.scaled(name="ragged_g5_p256", batch=3, page_size=256, lengths="list",
                        length_list=(255, 257, 2100), pin_max=False),
    W.INT8_B32.scaled(name="int8_p128", batch=3, page_size=128, lengths="list",
                      length_list=(5, 128, 1500)),
    W.INT8_B32.scaled(name="int8_p256", batch=2, page_size=256, lengths="list",
                      length_list=(300, 1100)),
    W.INT4_MTP_B64.scaled(name="int4_mtp_p128", batch=3, page_size=128, lengths="list",
                          length_list=(4, 130, 1400)),
    W.INT4_MTP_B64.scaled(name="int4_mtp_p256", batch=2, page_size=256, lengths="list",
                          length_list=(260, 900)),
]


@pytest.mark.parametrize("w", both_layouts(PAGES), ids=lambda w: w.name)
@pytest.mark.parametrize("S", [1, 3])
def test_large_pages(gpu, w, S):
    _run_and_check(gpu, w, S, "large pages")


Q16 = [
    W.BF16_B16.scaled(name="mtp16_bf16_g1", batch=3, num_q_heads=4, num_kv_heads=4, q_per_req=16,
                      causal=True, lengths="list", length_list=(16, 17, 700)),
    W.INT8_B32.scaled(name="mtp16_int8_g1", batch=3, num_q_heads=4, num_kv_heads=4, q_per_req=16,
                      causal=True, lengths="list", length_list=(16, 40, 900)),
    W.INT4_MTP_B64.scaled(name="mtp16_int4_g1", batch=3, num_q_heads=4, num_kv_heads=4,
                          q_per_req=16, lengths="list", length_list=(16, 33, 800)),
]


@pytest.mark.parametrize("w", both_layouts(Q16), ids=lambda w: w.name)
def test_sixteen_query_tokens(gpu, w):
    _run_and_check(gpu, w, 4, "q_per_req 16")


WIDE = W.RAGGED_B64.scaled(name="wide_b300_g5", batch=300, lengths="loguniform", length_lo=1,
                           length_hi=400, pin_max=True)


@pytest.mark.parametrize("w", both_layouts([WIDE]), ids=lambda w: w.name)
def test_wide_batch_both_schedules(gpu, w):
    _run_and_check(gpu, w, 2, "wide batch")
    batch = W.make_batch(w, device="cuda")
    table = [1, 2, 3, 4]
    md = U.schedule(gpu, batch, table, 128, 4)
    out, lse, o, l = U.run_decode(gpu, batch, 4, sched=md)
    out_ref, lse_ref = U.oracle_full(batch)
    U.check_bf16(U.to_np(out), out_ref, f"{w.name} per-request out")
    U.check_lse(U.to_np(lse), lse_ref, f"{w.name} per-request lse")
    counts = md["split_counts"].cpu().numpy()
    assert counts.min() >= 1 and counts.max() <= 4
    o_ref, l_ref = U.oracle_partials_per_request(batch, 4, counts)
    og, lg = U.blank_unused_slots(U.to_np(o), U.to_np(l), counts)
    U.check_partials(og, lg, o_ref, l_ref, f"{w.name} per-request")
    assert torch.isfinite(out.float()).all()
    assert np.isfinite(lse_ref).sum() == np.isfinite(U.to_np(lse)).sum()


# G * q_per_req > 16: ceil(R / 16) row blocks of ceil(R / blocks) rows each
# (blocks of up to 32 rows on the dense bf16 matrix-core kernel, which holds
# two 16-row tiles)
ROW_BLOCKS = [
    # the headline heads with 4 MTP tokens: 20 rows, one block (bf16 matrix cores, 2 tiles)
    W.RAGGED_B64.scaled(name="rows20_bf16_g5_mtp4", batch=3, q_per_req=4, causal=True,
                        lengths="list", length_list=(4, 700, 1500), pin_max=False),
    # 32 rows, one block (bf16 matrix cores, 2 tiles), with an empty request
    W.BF16_B16.scaled(name="rows32_bf16_g8_mtp4", batch=3, num_q_heads=16, num_kv_heads=2,
                      q_per_req=4, causal=True, lengths="list", length_list=(0, 130, 1100)),
    # INT4 20 rows and INT8 18 rows: one block, two row tiles (matrix cores)
    W.INT4_MTP_B64.scaled(name="rows20_int4_g5_mtp4", batch=3, num_q_heads=40, lengths="list",
                          length_list=(5, 333, 1200)),
    W.INT8_B32.scaled(name="rows18_int8_g6_mtp3", batch=2, num_q_heads=12, num_kv_heads=2,
                      q_per_req=3, causal=True, lengths="list", length_list=(77, 900)),
    # INT4 32 rows (one full block of two tiles), INT8 64 rows (2 x 32)
    W.INT4_MTP_B64.scaled(name="rows32_int4_g8_mtp4", batch=2, num_q_heads=16, num_kv_heads=2,
                          lengths="list", length_list=(40, 1000)),
    W.INT8_B32.scaled(name="rows64_int8_mqa", batch=2, num_q_heads=64, num_kv_heads=1,
                      lengths="list", length_list=(3, 700)),
    # vector-ALU kernel: fp32 18 rows = 2 x 9; bf16 D = 64, 17 rows = 2 x 9
    W.TINY_FP32.scaled(name="rows18_fp32_g6_mtp3", batch=2, num_q_heads=12, num_kv_heads=2,
                       q_per_req=3, causal=True, lengths="list", length_list=(50, 600),
                       pool_pages=0),
    W.BF16_B16.scaled(name="rows17_bf16_d64_g17", batch=2, num_q_heads=17, num_kv_heads=1,
                      head_dim=64, page_size=32, lengths="list", length_list=(3, 800)),
    # one kv-head for 64 query heads: 64 rows = 2 x 32
    W.BF16_B16.scaled(name="rows64_bf16_mqa", batch=2, num_q_heads=64, num_kv_heads=1,
                      lengths="list", length_list=(1, 900)),
    # four kv-heads per workgroup (token-major, Hkv = 4) with two row blocks of 32:
    # INT8, INT4 and bf16 at D = 64 on the matrix cores, 64 rows each
    W.INT8_B32.scaled(name="rows64_int8_hkv4_g8_mtp8", batch=2, num_q_heads=32, num_kv_heads=4,
                      q_per_req=8, causal=True, lengths="list", length_list=(9, 700)),
    W.INT4_MTP_B64.scaled(name="rows64_int4_hkv4_g4_mtp16", batch=2, num_q_heads=16,
                          num_kv_heads=4, q_per_req=16, lengths="list", length_list=(17, 600)),
    W.BF16_B16.scaled(name="rows64_bf16_d64_hkv4_g8_mtp8", batch=2, num_q_heads=32, num_kv_heads=4,
                      head_dim=64, q_per_req=8, causal=True, lengths="list", length_list=(9, 500)),
    # INT4 at the common Hkv = 8 (two groups of four kv-heads when token-major),
    # two row blocks of 32
    W.INT4_MTP_B64.scaled(name="rows64_int4_hkv8_g4_mtp16", batch=2, q_per_req=16,
                          lengths="list", length_list=(11, 520)),
    # 16 heads x 16 MTP tokens on one kv-head: 256 rows = 8 x 32
    W.BF16_B16.scaled(name="rows256_bf16_g16_mtp16", batch=2, num_q_heads=16, num_kv_heads=1,
                      q_per_req=16, causal=True, lengths="list", length_list=(16, 500)),
]


@pytest.mark.parametrize("w", both_layouts(ROW_BLOCKS), ids=lambda w: w.name)
@pytest.mark.parametrize("S", [1, 3])
def test_row_blocks(gpu, w, S):
    _run_and_check(gpu, w, S, "row blocks")


@pytest.mark.parametrize("w", [ROW_BLOCKS[0], ROW_BLOCKS[2]], ids=lambda w: w.name)
def test_row_blocks_per_request_schedule(gpu, w):
    log(f"row blocks, per-request schedule: {w.name}")
    batch = W.make_batch(w, device="cuda")
    md = U.schedule(gpu, batch, [1, 2, 4], 256, 4)
    counts = md["split_counts"].cpu().numpy()
    out, lse, o, l = U.run_decode(gpu, batch, 4, sched=md)
    o_ref, l_ref = U.oracle_partials_per_request(batch, 4, counts)
    og, lg = U.blank_unused_slots(U.to_np(o), U.to_np(l), counts)
    U.check_partials(og, lg, o_ref, l_ref, f"{w.name} per-request",
                     o_extra=U.matrix_path_o_bound(batch))
    out_ref, lse_ref = U.oracle_full(batch)
    _check_out(w, U.to_np(out), out_ref, f"{w.name} per-request out")
    U.check_lse(U.to_np(lse), lse_ref, f"{w.name} per-request lse")
