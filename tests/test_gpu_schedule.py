"""GPU: per-request split counts and the flattened stage-1 work list.

The metadata prelude's schedule outputs (split_counts, work_list) must equal
oracle/schedule.py bit for bit; stage 1 driven by the work list must match
the oracle's per-request partials on every written slot, and the merged
output the un-split oracle.  With a table holding one value S, the schedule
is the batch-wide split and every output bit must be unchanged.
"""
import json
import os

import numpy as np
import pytest
import torch

from decode_attention_paged_gqa_amd import workloads as W
from oracle import schedule as OS
from tests import _gpu_util as U
from tests.test_gpu_attention import (INT4_G8Q2, INT4_SMALL, INT8_MTP, INT8_ODD_HKV, INT8_SMALL,
                                      MTP_BF16, QUAD, RAGGED_SMALL, TINY, D64_P16, INT8_FP32Q,
                                      _check_out, both_layouts)

pytestmark = pytest.mark.gpu
log = U.log
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _i32(x):
    return torch.as_tensor(np.asarray(x), dtype=torch.int32, device="cuda")


def _sched_md(gpu, seq, table, bt, smax, ps=16, cap=None):
    """Metadata with a schedule for bare lengths (page table not used here)."""
    B = len(seq)
    rpi = torch.arange(B, dtype=torch.int64, device="cuda")
    r2t = torch.zeros((B, 64), dtype=torch.int32, device="cuda")
    return gpu.decode_attn_metadata(_i32(seq), rpi, r2t, ps, 4, split_table=table,
                                    bucket_tokens=bt, max_splits=smax, work_capacity=cap)


def test_schedule_hand_built(gpu):
    """The library asks for room for every request's largest possible count
    (batch * min(max(table), max_splits) = 54 here), more than the fixture's
    28; past the fixture's items the list is -1."""
    g = json.load(open(os.path.join(GOLDEN, "schedule_hand.json")))
    B = len(g["seq_lens"])
    cap = B * min(max(g["table"]), g["max_splits"])
    md = _sched_md(gpu, g["seq_lens"], g["table"], g["bucket_tokens"], g["max_splits"],
                   ps=g["page_size"], cap=cap)
    items = [x for x in g["expect"]["work_list"] if x >= 0]
    assert md["split_counts"].tolist() == g["expect"]["split_counts"]
    assert md["work_list"].tolist() == items + [-1] * (cap - len(items))
    with pytest.raises(gpu.DecodeAttnError):  # one entry short of that room
        _sched_md(gpu, g["seq_lens"], g["table"], g["bucket_tokens"], g["max_splits"],
                  ps=g["page_size"], cap=cap - 1)


@pytest.mark.parametrize("seed,B", [(0, 1), (1, 7), (2, 64), (3, 300), (4, 1000)])
def test_schedule_generated_bit_exact(gpu, seed, B):
    """Random lengths (sentinels, zeros, ties, more rows than one workgroup's
    threads), random tables: split_counts and work_list equal the oracle's."""
    rng = np.random.default_rng(seed)
    seq = rng.integers(-2, 40000, size=B)
    seq[rng.random(B) < 0.2] = 0
    if B > 3:
        seq[1] = seq[2] = seq[3]  # a tie
    nb = int(rng.integers(1, 17))
    table = rng.integers(1, 40, size=nb).tolist()
    smax = int(rng.integers(1, 64))
    ps = int(rng.choice([16, 32, 64]))
    bt = int(rng.choice([512, 4096]))
    cap = B * min(smax, max(table)) + int(rng.integers(0, 50))
    log(f"schedule seed={seed} B={B} n_buckets={nb} max_splits={smax} cap={cap}")
    md = _sched_md(gpu, seq, table, bt, smax, ps=ps, cap=cap)
    want_c = OS.request_splits(seq, ps, table, bt, smax)
    want_w = OS.work_list(seq, want_c, cap)
    assert np.array_equal(md["split_counts"].cpu().numpy().astype(np.int64), want_c)
    assert np.array_equal(md["work_list"].cpu().numpy().astype(np.int64), want_w)


def test_schedule_rewrites_a_stale_list(gpu):
    """The list is fully rewritten each launch (it may hold a previous batch)."""
    md = _sched_md(gpu, [5000, 10, 700], [1, 2, 4], 1024, 8, cap=24)
    stale = {"work_list": torch.full((24,), 12345, dtype=torch.int32, device="cuda"),
             "split_counts": torch.full((3,), 77, dtype=torch.int32, device="cuda")}
    B = 3
    md2 = gpu.decode_attn_metadata(_i32([5000, 10, 700]), torch.arange(B, device="cuda"),
                                   torch.zeros((B, 64), dtype=torch.int32, device="cuda"), 16, 4,
                                   split_table=[1, 2, 4], bucket_tokens=1024, max_splits=8,
                                   work_capacity=24, out=stale)
    assert torch.equal(md2["work_list"], md["work_list"])
    assert torch.equal(md2["split_counts"], md["split_counts"])


def test_reused_out_dict_with_other_options(gpu):
    """An `out` dict that also holds another option's buffers (here the SWA
    table) passes only the buffers of the options requested."""
    seq = [5000, 10, 700]
    ref = _sched_md(gpu, seq, [1, 2, 4], 1024, 8, cap=24)
    out = dict(ref)
    out["swa_page_table"] = torch.zeros((3, 4), dtype=torch.int32, device="cuda")
    md = gpu.decode_attn_metadata(_i32(seq), torch.arange(3, device="cuda"),
                                  torch.zeros((3, 64), dtype=torch.int32, device="cuda"), 16, 4,
                                  split_table=[1, 2, 4], bucket_tokens=1024, max_splits=8,
                                  work_capacity=24, out=out)
    assert torch.equal(md["work_list"], ref["work_list"])
    plain = gpu.decode_attn_metadata(_i32(seq), torch.arange(3, device="cuda"),
                                     torch.zeros((3, 64), dtype=torch.int32, device="cuda"), 16, 4,
                                     out=out)
    assert torch.equal(plain["page_table"], ref["page_table"])


# ---------------------------------------------------------------- attention
SMALL_TABLE = [1, 2, 3, 5, 8, 13, 21, 32]
SMALL_BUCKET = 256
# the kernels that take four kv-heads per workgroup on token-major pools: bf16
# at D = 64 on the matrix cores, fp32 at D = 64 on the vector ALU and on the
# matrix cores, INT4 with Hkv = 16
_QUAD_SCHED = [w for w in QUAD if w.name in ("bf16_d64_hkv4_mtp4_r16", "fp32_d64_hkv4_g2",
                                             "fp32_d64_hkv4_g8", "int4_hkv16_g2_mtp2_r4")]
assert len(_QUAD_SCHED) == 4
SCHED_CASES = both_layouts([RAGGED_SMALL, D64_P16, MTP_BF16, INT8_SMALL, INT8_MTP, INT8_ODD_HKV,
                            INT8_FP32Q, INT4_SMALL, INT4_G8Q2] + _QUAD_SCHED) + [TINY]


@pytest.mark.parametrize("w", SCHED_CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("smax", [32, 5])
def test_per_request_splits_elementwise(gpu, w, smax):
    log(f"per-request splits {w.name} max_splits={smax}")
    batch = W.make_batch(w, device="cuda")
    md = U.schedule(gpu, batch, SMALL_TABLE, SMALL_BUCKET, smax)
    counts = md["split_counts"].cpu().numpy()
    want = OS.request_splits(batch.lengths, w.page_size, SMALL_TABLE, SMALL_BUCKET, smax)
    assert np.array_equal(counts.astype(np.int64), want)
    log(f"  split counts {counts.tolist()}")
    out_dtype = torch.float32 if w.dtype == "fp32" and w.kv == W.KV_DENSE else torch.bfloat16
    out, lse, o, l = U.run_decode(gpu, batch, smax, out_dtype=out_dtype, sched=md)
    o_ref, l_ref = U.oracle_partials_per_request(batch, smax, counts)
    out_ref, lse_ref = U.oracle_full(batch)
    og, lg = U.blank_unused_slots(U.to_np(o), U.to_np(l), counts)
    extra = U.matrix_path_o_bound(batch)
    U.check_partials(og, lg, o_ref, l_ref, f"{w.name} per-request", o_extra=extra)
    if out_dtype == torch.float32:
        U.check_fp32(U.to_np(out), out_ref, f"{w.name} per-request out fp32")
    else:
        _check_out(w, U.to_np(out), out_ref, f"{w.name} per-request out")
    U.check_lse(U.to_np(lse), lse_ref, f"{w.name} per-request lse")


@pytest.mark.parametrize("w", both_layouts([RAGGED_SMALL, INT8_SMALL, INT4_SMALL, MTP_BF16]),
                         ids=lambda w: w.name)
@pytest.mark.parametrize("S", [1, 4, 16])
def test_constant_table_is_bit_identical_to_batch_wide(gpu, w, S):
    """Table [S]*8: each request gets min(S, its pages) splits over the same
    page ranges as a batch-wide S (whose extra splits are empty), so stage 1
    writes the same bits in those slots and the merge returns the same bits."""
    batch = W.make_batch(w, device="cuda")
    md = U.schedule(gpu, batch, [S] * 8, 4096, S)
    out1, lse1, o1, l1 = U.run_decode(gpu, batch, S)
    out2, lse2, o2, l2 = U.run_decode(gpu, batch, S, sched=md)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
    counts = md["split_counts"].tolist()
    for b, c in enumerate(counts):
        assert torch.equal(o1[b, :, :, :c], o2[b, :, :, :c])
        assert torch.equal(l1[b, :, :, :c], l2[b, :, :, :c])


def test_unused_slots_are_not_read(gpu):
    """NaN in the slots past each request's count must not reach the output."""
    w = RAGGED_SMALL
    batch = W.make_batch(w, device="cuda")
    smax = 32
    md = U.schedule(gpu, batch, SMALL_TABLE, SMALL_BUCKET, smax)
    B, qn, Hq, D = batch.q.shape
    o = torch.full((B, qn, Hq, smax, D), float("nan"), device="cuda")
    l = torch.full((B, qn, Hq, smax), float("nan"), device="cuda")
    gpu.decode_attn_split(batch.q, batch.k_pool, batch.v_pool, batch.page_table, batch.seq_lens,
                          smax, w.softmax_scale, False, o_partial=o, lse_partial=l,
                          kv_layout=w.kv_layout, split_counts=md["split_counts"],
                          work_list=md["work_list"])
    out = gpu.decode_attn_merge(o, l, split_counts=md["split_counts"])
    assert torch.isfinite(out.float()).all()
    ref, _, _, _ = U.run_decode(gpu, batch, smax, sched=md)
    assert torch.equal(out, ref)


# ---------------------------------------------------------------- full size
def chunk_table(chunk_pages, page_size=64, bucket_tokens=4096, n_buckets=8):
    """Per-bucket counts giving splits of about ``chunk_pages`` pages at each bucket's top."""
    per = bucket_tokens // page_size
    return [max(1, -(-(k + 1) * per // chunk_pages)) for k in range(n_buckets)]


FULL_SCHED = [
    (W.RAGGED_B64, chunk_table(32)),
    (W.INT4_MTP_B64, chunk_table(64)),
]


@pytest.mark.parametrize("w,table", FULL_SCHED, ids=[f[0].name for f in FULL_SCHED])
def test_full_size_per_request_sampled(gpu, w, table):
    log(f"full {w.name} per-request table {table}")
    batch = W.make_batch(w, device="cuda")
    smax = max(table)
    md = U.schedule(gpu, batch, table, 4096, smax)
    out, lse, _, _ = U.run_decode(gpu, batch, smax, sched=md)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    L = batch.lengths
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
