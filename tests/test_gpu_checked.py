"""The checked build (libdecode_attn_checked.so, compiled with -DDA_CHECKED).

On valid inputs it records no contract violation and its results are
bit-identical to the plain library's, on every stage-1 kernel.  Each kind of
device-data violation the kernels clamp (the DA_CHECK_* bits of
decode_attn.h) is recorded, and the outputs still equal the plain
library's: both builds give the clamped meaning the header states (an
out-of-range page id reads page 0, a length is clamped to the page table, a
bad batch_order entry is replaced by its slot, a bad work-list entry is
skipped, a split count is clamped to [1, num_splits], a row past
req_to_token reads as empty).  Every bad value here is one the kernels' own
bounds checks turn into an in-bounds access.
"""
import contextlib
import copy

import pytest
import torch

import decode_attention_paged_gqa_amd as da
from decode_attention_paged_gqa_amd import _binding as B
from decode_attention_paged_gqa_amd import workloads as W
from tests import _gpu_util as U

pytestmark = pytest.mark.gpu
log = U.log


@contextlib.contextmanager
def checked_library():
    prev = B._lib
    B.load(B.CHECKED_LIB_PATH, reload=True)
    try:
        da.decode_attn_checks(reset=True)
        yield
    finally:
        torch.cuda.synchronize()
        B._lib = prev


def _both(fn):
    """fn() under the plain library, then under the checked one; returns
    (plain result, checked result, (flags, count))."""
    plain = fn()
    torch.cuda.synchronize()
    with checked_library():
        chk = fn()
        flags = da.decode_attn_checks(reset=True)
    return plain, chk, flags


def _same(a, b, label):
    for x, y in zip(a, b):
        assert x.shape == y.shape and torch.equal(x, y), label


# one workload per stage-1 kernel
PATHS = [
    W.RAGGED_B64.scaled(name="chk_bf16_g5", batch=3, lengths="list", length_list=(1, 300, 900),
                        pin_max=False),                                     # bf16 vector
    W.BF16_MTP_B64.scaled(name="chk_bf16_mtp", batch=3, lengths="list",
                          length_list=(4, 300, 900)),                      # bf16 matrix cores
    W.INT8_B32.scaled(name="chk_int8", batch=3, lengths="list", length_list=(1, 300, 900)),
    W.INT4_MTP_B64.scaled(name="chk_int4_mtp", batch=3, lengths="list",
                          length_list=(4, 300, 900)),                      # INT4 matrix cores
    W.TINY_FP32.scaled(name="chk_fp32_g2", batch=3, num_q_heads=2, lengths="list",
                       length_list=(1, 300, 900), pool_pages=0),          # fp32 vector ALU
    # the head-dim-64 and fp32-query instances of the matrix-core kernels
    W.BF16_MTP_B64.scaled(name="chk_bf16_mtp_d64", batch=3, head_dim=64, lengths="list",
                          length_list=(4, 300, 900)),
    W.INT8_B32.scaled(name="chk_int8_d64", batch=3, head_dim=64, lengths="list",
                      length_list=(1, 300, 900)),
    W.INT4_MTP_B64.scaled(name="chk_int4_mtp_d64", batch=3, head_dim=64, lengths="list",
                          length_list=(4, 300, 900)),
    W.INT8_B32.scaled(name="chk_int8_fp32q", batch=3, dtype="fp32", lengths="list",
                      length_list=(1, 300, 900)),
    W.INT4_MTP_B64.scaled(name="chk_int4_mtp_fp32q", batch=3, dtype="fp32", lengths="list",
                          length_list=(4, 300, 900)),
    W.TINY_FP32.scaled(name="chk_fp32_g8", batch=3, num_q_heads=8, num_kv_heads=1,
                       lengths="list", length_list=(1, 300, 900), pool_pages=0),  # fp32 matrix cores
    # token-major pools: the quantised kernels (and bf16 on the matrix cores at
    # D = 64) take four kv-heads per workgroup there
    W.INT8_B32.scaled(name="chk_int8_nhd", batch=3, lengths="list", length_list=(1, 300, 900),
                      kv_layout="NHD"),
    W.INT4_MTP_B64.scaled(name="chk_int4_mtp_nhd", batch=3, lengths="list",
                          length_list=(4, 300, 900), kv_layout="NHD"),
    W.BF16_MTP_B64.scaled(name="chk_bf16_mtp_d64_nhd", batch=3, head_dim=64, lengths="list",
                          length_list=(4, 300, 900), kv_layout="NHD"),
]


def _decode(batch, S, **kw):
    def run():
        out, lse, o, l = U.run_decode(da, batch, S, **kw)
        sched = kw.get("sched")
        if sched is not None:
            # with per-request counts, slots from the (clamped) count on are never written
            counts = sched["split_counts"].cpu().clamp(1, S).tolist()
            o, l = o.clone(), l.clone()
            for b, c in enumerate(counts):
                o[b, :, :, c:] = 0
                l[b, :, :, c:] = float("-inf")
        return o, l, out, lse
    return run


@pytest.mark.parametrize("w", PATHS, ids=lambda w: w.name)
def test_valid_inputs_record_nothing_and_match(gpu, w):
    log(f"checked build, valid inputs: {w.name}")
    batch = W.make_batch(w, device="cuda")
    plain, chk, (flags, count) = _both(_decode(batch, 3))
    assert (flags, count) == (0, 0)
    _same(plain, chk, w.name)


@pytest.mark.parametrize("w", PATHS, ids=lambda w: w.name)
def test_bad_page_ids_and_lengths(gpu, w):
    log(f"checked build, bad page ids and lengths: {w.name}")
    batch = copy.copy(W.make_batch(w, device="cuda"))
    pt = batch.page_table.clone()
    pt[1, 0] = batch.num_pages + 3   # past the pool
    pt[2, 1] = -2                    # negative
    batch.page_table = pt
    plain, chk, (flags, count) = _both(_decode(batch, 2))
    assert flags == da.DA_CHECK_PAGE_ID and count >= 2, (hex(flags), count)
    _same(plain, chk, w.name)

    batch.page_table = W.make_batch(w, device="cuda").page_table
    sl = batch.seq_lens.clone()
    sl[0] = batch.max_pages * w.page_size + 50  # longer than the page table
    sl[1] = -5
    batch.seq_lens = sl
    plain, chk, (flags, count) = _both(_decode(batch, 2))
    assert flags == da.DA_CHECK_SEQLEN and count >= 2, (hex(flags), count)
    _same(plain, chk, w.name)


def test_bad_batch_order(gpu):
    w = PATHS[0]
    batch = W.make_batch(w, device="cuda")
    order = torch.tensor([2, 7, 0], dtype=torch.int32, device="cuda")  # 7 is no request
    plain, chk, (flags, count) = _both(_decode(batch, 2, batch_order=order))
    assert flags == da.DA_CHECK_ORDER and count >= 1, (hex(flags), count)
    _same(plain, chk, "batch order")


@pytest.mark.parametrize("w", [PATHS[0], PATHS[3]], ids=lambda w: w.name)
def test_bad_work_list_and_counts(gpu, w):
    log(f"checked build, bad work list and counts: {w.name}")
    batch = W.make_batch(w, device="cuda")
    md = U.schedule(da, batch, [1, 2, 3], 256, 3)
    bad = dict(md)
    work = md["work_list"].clone()
    work[-1] = (5 << 8) | 0          # no request 5 (the list's last slot is padding)
    bad["work_list"] = work
    plain, chk, (flags, count) = _both(_decode(batch, 3, sched=bad))
    assert flags == da.DA_CHECK_WORK and count >= 1, (hex(flags), count)
    _same(plain, chk, f"{w.name} work list")

    counts = md["split_counts"].clone()
    counts[0] = 0                    # clamped to 1 by stage 1 and by the merge
    counts[2] = 9                    # clamped to num_splits
    bad = dict(md, split_counts=counts)
    plain, chk, (flags, count) = _both(_decode(batch, 3, sched=bad))
    assert flags & da.DA_CHECK_COUNTS and not flags & ~(da.DA_CHECK_COUNTS | da.DA_CHECK_WORK), \
        hex(flags)
    _same(plain, chk, f"{w.name} counts")


def test_metadata_rows_and_lengths(gpu):
    w = PATHS[0]
    batch = W.make_batch(w, device="cuda")
    rows, cols = batch.req_to_token.shape
    rpi = batch.req_pool_indices.clone()
    rpi[1] = rows + 3                # past req_to_token
    sl = batch.seq_lens.clone()
    sl[2] = batch.max_pages * w.page_size + 1  # one page more than the table holds

    def meta():
        md = da.decode_attn_metadata(sl, rpi, batch.req_to_token, w.page_size, batch.max_pages)
        return [md[k] for k in ("cache_seqlens", "cu_seqlens_k", "cu_seqlens_q", "page_table")]

    plain, chk, (flags, count) = _both(meta)
    assert flags == da.DA_CHECK_REQ_ROW | da.DA_CHECK_TOO_LONG and count == 2, (hex(flags), count)
    _same(plain, chk, "metadata")
    assert int(plain[3][1].abs().sum()) == 0  # a row past the table reads as empty


def test_valid_metadata_with_schedule_records_nothing(gpu):
    w = PATHS[3]
    batch = W.make_batch(w, device="cuda")

    def meta():
        md = da.decode_attn_metadata(batch.seq_lens, batch.req_pool_indices, batch.req_to_token,
                                     w.page_size, batch.max_pages, split_table=[1, 2],
                                     bucket_tokens=256, max_splits=2)
        return [md[k] for k in ("cache_seqlens", "page_table", "split_counts", "work_list")]

    plain, chk, (flags, count) = _both(meta)
    assert (flags, count) == (0, 0)
    _same(plain, chk, "metadata with schedule")
