"""GPU: the whole step (metadata -> stage 1 -> merge) captured once in a HIP
graph and replayed, with the split count fixed at capture (LightLLM PR #1549
deploys its tuned decode kernels under CUDA graphs, "Covered decode kernels";
SGLang PR #29843 digest rebuilds the decode metadata inside the captured
graph, "Features and motivation").

Between replays the test changes the inputs in place (shorter KV lengths, new
queries), runs the same calls eagerly on separate buffers, synchronises, and
requires every replay to match the eager result bit for bit.  With a
per-request split table the schedule (split counts, work list) is rebuilt
on the device at every replay from the new lengths, so the captured graph
follows them; the table itself is part of the captured launch.  No call in the
step records a memset (stage 1 overwrites every partial slot), so nothing in
the graph depends on one.
"""
import pytest
import torch

from decode_attention_paged_gqa_amd import workloads as W
from tests import _gpu_util as U

pytestmark = pytest.mark.gpu
log = U.log

CASES = [
    W.RAGGED_B64.scaled(name="graph_ragged_bf16", batch=7, lengths="list",
                        length_list=(1, 64, 65, 700, 2000, 3100, 0), pin_max=False),
    W.INT8_B32.scaled(name="graph_int8", batch=4, lengths="list", length_list=(33, 640, 1500, 2)),
    W.INT4_MTP_B64.scaled(name="graph_int4_mtp", batch=4, lengths="list",
                          length_list=(4, 100, 1300, 2500)),
    W.INT4_MTP_B64.scaled(name="graph_int4_mtp_nhd", batch=3, lengths="list",
                          length_list=(9, 400, 1800), kv_layout="NHD"),
    W.BF16_MTP_B64.scaled(name="graph_bf16_mtp", batch=4, lengths="list",
                          length_list=(3, 90, 1200, 2600)),
    # 20 query rows per kv-head: the matrix-core kernels with two row tiles
    W.BF16_MTP_G5_B64.scaled(name="graph_bf16_mtp_20rows", batch=3, lengths="list",
                             length_list=(4, 700, 2100)),
    W.INT4_MTP_B64.scaled(name="graph_int4_mtp_20rows", batch=3, num_q_heads=40, lengths="list",
                          length_list=(6, 500, 1900)),
    # head dim 64, and the fp32 matrix-core kernel
    W.INT8_B32.scaled(name="graph_int8_d64", batch=3, head_dim=64, lengths="list",
                      length_list=(5, 900, 2300)),
    W.BF16_MTP_B64.scaled(name="graph_bf16_mtp_d64", batch=3, head_dim=64, lengths="list",
                          length_list=(2, 333, 2000)),
    W.FP32_B16.scaled(name="graph_fp32_8rows", batch=3, lengths="list",
                      length_list=(7, 640, 1800)),
]


class Step:
    """Buffers and calls of one decode step; every output is caller-owned."""

    def __init__(self, da, batch, S, table=None):
        self.da, self.batch, self.S, self.table = da, batch, S, table
        w = batch.w
        B, qn, Hq, D = batch.q.shape
        dev = batch.q.device
        i32 = dict(dtype=torch.int32, device=dev)
        self.md = {"cache_seqlens": torch.empty(B, **i32), "cu_seqlens_k": torch.empty(B + 1, **i32),
                   "cu_seqlens_q": torch.empty(B + 1, **i32),
                   "page_table": torch.empty(B, batch.max_pages, **i32),
                   "batch_order": torch.empty(B, **i32)}
        if table is not None:
            self.md["split_counts"] = torch.empty(B, **i32)
            self.md["work_list"] = torch.empty(B * S, **i32)
        self.o = torch.empty((B, qn, Hq, S, D), dtype=torch.float32, device=dev)
        self.l = torch.empty((B, qn, Hq, S), dtype=torch.float32, device=dev)
        self.out = torch.empty((B, qn, Hq, D), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, qn, Hq), dtype=torch.float32, device=dev)
        self.w = w

    def __call__(self):
        da, b, w, md = self.da, self.batch, self.w, self.md
        sched = {}
        if self.table is not None:
            sched = dict(split_table=self.table, bucket_tokens=512, max_splits=self.S,
                         work_capacity=md["work_list"].shape[0])
        da.decode_attn_metadata(b.seq_lens, b.req_pool_indices, b.req_to_token, w.page_size,
                                b.max_pages, q_stride=w.q_per_req, out=md, **sched)
        kw = dict(o_partial=self.o, lse_partial=self.l, batch_order=md["batch_order"],
                  kv_layout=w.kv_layout)
        if self.table is not None:
            kw.update(split_counts=md["split_counts"], work_list=md["work_list"])
        args = (md["page_table"], md["cache_seqlens"], self.S, w.softmax_scale, w.causal)
        if w.kv == W.KV_DENSE:
            da.decode_attn_split(b.q, b.k_pool, b.v_pool, *args, **kw)
        elif w.kv == W.KV_INT8:
            da.decode_attn_split_int8(b.q, b.k_pool, b.v_pool, b.k_scale, b.v_scale, *args, **kw)
        else:
            da.decode_attn_split_int4(b.q, b.k_pool, b.v_pool, b.k_scale, b.v_scale, *args, **kw)
        da.decode_attn_merge(self.o, self.l, out=self.out, lse_out=self.lse,
                             split_counts=md.get("split_counts"))


TABLE = [1, 2, 3, 4, 6, 8, 8, 8]  # per 512-token bucket


@pytest.mark.parametrize("table", [None, TABLE], ids=["batch_wide_S", "per_request"])
@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_graph_replay_matches_eager(gpu, w, table):
    log(f"graph {w.name} table={table}")
    batch = W.make_batch(w, device="cuda")
    S = 4 if table is None else 8
    step = Step(gpu, batch, S, table)
    ref = Step(gpu, batch, S, table)  # eager twin on its own buffers

    step()  # warm up outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    gen = torch.Generator(device="cuda").manual_seed(17)
    L0 = batch.seq_lens.clone()
    for rep in range(4):
        if rep:  # new inputs in the captured buffers: shorter lengths, fresh queries
            cut = torch.randint(0, 3, L0.shape, generator=gen, device="cuda", dtype=torch.int32)
            batch.seq_lens.copy_(torch.clamp(L0 - cut * 37 * rep, min=0))
            batch.q.copy_(torch.randn(batch.q.shape, generator=gen, device="cuda").to(batch.q.dtype))
        ref()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in ref.md:
            assert torch.equal(step.md[k], ref.md[k]), (rep, k)
        assert torch.equal(step.out, ref.out), rep
        assert torch.equal(step.lse, ref.lse), rep
        log(f"  replay {rep}: bit-identical to eager (L={batch.seq_lens.tolist()})")
    # and the eager result itself against the oracle on the last inputs
    batch.lengths = batch.seq_lens.cpu().numpy()
    out_ref, lse_ref = U.oracle_full(batch)
    if w.kv == W.KV_DENSE:
        U.check_bf16(U.to_np(step.out), out_ref, f"{w.name} graph out")
    else:
        U.check_quant(U.to_np(step.out), out_ref, f"{w.name} graph out")
    U.check_lse(U.to_np(step.lse), lse_ref, f"{w.name} graph lse")


class StaticStep(Step):
    """The same step through decode_attn_decode_static: the split partials live
    in the library's per-GPU scratch array, so the captured graph holds no
    caller-allocated intermediate at all."""

    def __call__(self):
        da, b, w, md = self.da, self.batch, self.w, self.md
        sched = {}
        if self.table is not None:
            sched = dict(split_table=self.table, bucket_tokens=512, max_splits=self.S,
                         work_capacity=md["work_list"].shape[0])
        da.decode_attn_metadata(b.seq_lens, b.req_pool_indices, b.req_to_token, w.page_size,
                                b.max_pages, q_stride=w.q_per_req, out=md, **sched)
        kw = dict(batch_order=md["batch_order"], kv_layout=w.kv_layout, causal=w.causal,
                  softmax_scale=w.softmax_scale, out=self.out, lse_out=self.lse)
        if self.table is not None:
            kw.update(split_counts=md["split_counts"], work_list=md["work_list"])
        if w.kv != W.KV_DENSE:
            kw.update(k_scale=b.k_scale, v_scale=b.v_scale,
                      cache_format="int8" if w.kv == W.KV_INT8 else "int4")
        da.decode_attn_decode_static(b.q, b.k_pool, b.v_pool, md["page_table"],
                                     md["cache_seqlens"], self.S, **kw)


@pytest.mark.parametrize("table", [None, TABLE], ids=["batch_wide_S", "per_request"])
@pytest.mark.parametrize("w", CASES[:4], ids=lambda w: w.name)
def test_static_entry_point_replays_like_split_and_merge(gpu, w, table):
    """Metadata and decode_attn_decode_static captured in one graph; every
    replay, after the inputs change, must equal the eager split + merge path
    (other buffers) bit for bit."""
    log(f"graph static {w.name} table={table}")
    batch = W.make_batch(w, device="cuda")
    S = 4 if table is None else 8
    step = StaticStep(gpu, batch, S, table)
    ref = Step(gpu, batch, S, table)
    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(23)
    L0 = batch.seq_lens.clone()
    for rep in range(4):
        if rep:
            cut = torch.randint(0, 3, L0.shape, generator=gen, device="cuda", dtype=torch.int32)
            batch.seq_lens.copy_(torch.clamp(L0 - cut * 41 * rep, min=0))
            batch.q.copy_(torch.randn(batch.q.shape, generator=gen, device="cuda").to(batch.q.dtype))
        ref()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out, ref.out), rep
        assert torch.equal(step.lse, ref.lse), rep
        log(f"  replay {rep}: static entry point bit-identical to split + merge")
