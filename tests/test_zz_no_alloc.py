"""decode_attn_decode_static -- stage 1 and the merge in one call, the split
partials in the library's per-GPU scratch array, for callers that cannot
allocate device memory -- against the two calls it stands in for:
decode_attn_split / _int8 / _int4 into caller-allocated partials, then
decode_attn_merge.  Both run the same kernels on the same inputs, so the
outputs and LSEs must be bit-identical.

Every format is called twice in a row on one GPU, the second time with a
smaller batch, fewer splits and other lengths, so the second call runs over
the scratch the first one left behind (nothing in it needs clearing: stage 1
writes every slot the merge reads).  The per-request schedule (split counts
and a work list) goes through it as well, and a call whose partials would
exceed the scratch is refused before anything is enqueued.
"""
import pytest
import torch

import decode_attention_paged_gqa_amd as da_mod
from decode_attention_paged_gqa_amd import workloads as W
from tests import _gpu_util as U

pytestmark = pytest.mark.gpu
log = U.log

BIG_SMALL = {
    "bf16_g5_hnd": (
        W.RAGGED_B64.scaled(name="static_bf16_g5_big", batch=9, lengths="list",
                            length_list=(1, 64, 65, 700, 3001, 0, 129, 2048, 17), pin_max=False),
        8,
        W.RAGGED_B64.scaled(name="static_bf16_g5_small", batch=3, lengths="list",
                            length_list=(300, 5, 1100), pin_max=False, seed=11),
        3),
    "int8_g4_nhd": (
        W.INT8_B32.scaled(name="static_int8_big", batch=5, kv_layout="NHD", lengths="list",
                          length_list=(1, 64, 65, 777, 2000)),
        6,
        W.INT8_B32.scaled(name="static_int8_small", batch=2, kv_layout="NHD", lengths="list",
                          length_list=(33, 400), seed=12),
        2),
    "int4_mtp4_hnd": (
        W.INT4_MTP_B64.scaled(name="static_int4_mtp_big", batch=4, lengths="list",
                          length_list=(4, 90, 700, 1500)),
        5,
        W.INT4_MTP_B64.scaled(name="static_int4_mtp_small", batch=2, lengths="list",
                          length_list=(70, 300), seed=13),
        2),
    "fp32_tiny": (W.TINY_FP32, 4, W.TINY_FP32.scaled(name="static_tiny_small", batch=1,
                                                     lengths="list", length_list=(50,),
                                                     seed=14), 1),
}


def _static(da, batch, S, out_dtype, sched=None):
    w = batch.w
    kw = dict(batch_order=None, kv_layout=w.kv_layout, causal=w.causal,
              softmax_scale=w.softmax_scale, out_dtype=out_dtype, want_lse=True)
    if sched is not None:
        kw.update(split_counts=sched["split_counts"], work_list=sched["work_list"])
    if w.kv != W.KV_DENSE:
        kw.update(k_scale=batch.k_scale, v_scale=batch.v_scale,
                  cache_format="int8" if w.kv == W.KV_INT8 else "int4")
    return da.decode_attn_decode_static(batch.q, batch.k_pool, batch.v_pool, batch.page_table,
                                        batch.seq_lens, S, **kw)


def _same(a, b, label):
    assert a.dtype == b.dtype and a.shape == b.shape, label
    ok = torch.equal(a, b)
    if not ok:
        d = (a.float() - b.float()).abs()
        log(f"  {label}: max |diff| {float(d[torch.isfinite(d)].max()) if d.numel() else 0}")
    assert ok, f"{label}: not bit-identical to the two-call path"


@pytest.mark.parametrize("case", list(BIG_SMALL), ids=list(BIG_SMALL))
def test_static_matches_split_then_merge_twice(gpu, case):
    da = gpu
    w1, s1, w2, s2 = BIG_SMALL[case]
    out_dtype = torch.float32 if w1.dtype == "fp32" else torch.bfloat16
    b1 = W.make_batch(w1, device="cuda:0")
    b2 = W.make_batch(w2, device="cuda:0")
    for n, (b, S) in enumerate(((b1, s1), (b2, s2))):
        log(f"  call {n + 1}: {b.w.name} B={b.w.batch} S={S}")
        out, lse = _static(da, b, S, out_dtype)
        ref_out, ref_lse, _, _ = U.run_decode(da, b, S, out_dtype=out_dtype)
        torch.cuda.synchronize()
        _same(out, ref_out, f"{case} call {n + 1} out")
        _same(lse, ref_lse, f"{case} call {n + 1} lse")


def test_static_per_request_schedule_twice(gpu):
    da = gpu
    w1 = W.RAGGED_B64.scaled(name="static_sched_big", batch=7, lengths="list",
                             length_list=(5000, 1, 64, 9000, 300, 0, 2500), pin_max=False)
    w2 = W.RAGGED_B64.scaled(name="static_sched_small", batch=3, lengths="list",
                             length_list=(800, 4100, 2), pin_max=False, seed=15)
    for n, (w, table, smax) in enumerate(((w1, [2, 3, 5], 6), (w2, [1, 2], 2))):
        b = W.make_batch(w, device="cuda:0")
        sched = U.schedule(da, b, table, 4096, smax)
        out, lse = _static(da, b, smax, torch.bfloat16, sched=sched)
        ref_out, ref_lse, _, _ = U.run_decode(da, b, smax, sched=sched)
        torch.cuda.synchronize()
        _same(out, ref_out, f"schedule call {n + 1} out")
        _same(lse, ref_lse, f"schedule call {n + 1} lse")


def test_static_refuses_partials_beyond_the_scratch(gpu):
    da = gpu
    w = W.RAGGED_B64.scaled(name="static_too_big", batch=2, lengths="list",
                            length_list=(64, 64), pin_max=False)
    b = W.make_batch(w, device="cuda:0")
    # 2 requests x 40 heads x 256 splits x 129 floats fit the 64 MiB scratch ...
    _static(da, b, 256, torch.bfloat16)
    # ... 64 requests x 40 heads x 64 splits do not
    big = W.RAGGED_B64.scaled(name="static_too_big2", batch=64, lengths="list",
                              length_list=(64,) * 64, pin_max=False)
    bb = W.make_batch(big, device="cuda:0")
    out = torch.full((64, 1, 40, 128), 7.0, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(da_mod.DecodeAttnError, match="status 4"):
        da.decode_attn_decode_static(bb.q, bb.k_pool, bb.v_pool, bb.page_table, bb.seq_lens, 64,
                                     out=out, kv_layout=big.kv_layout)
    torch.cuda.synchronize()
    assert bool((out.float() == 7.0).all())  # nothing was enqueued
