"""Decode-attention benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--splits S]
                    [--sched batch|request] [--chunk PAGES] [--no-cpu-baseline]
                    [--tune [FORMATS]] [--tune-chunks [FORMATS]]

One step is the whole hot path over one synthetic batch: the metadata
prelude (cache_seqlens / cu_seqlens_k/q / page_table in one launch), the
split-count lookup, stage 1 (split) and stage 2 (LSE merge).  Inputs are
resident in HBM before the timed region.  Prints ONE JSON line.

value      = algorithmic bytes of one step / measured step time (GB/s), the K
             steps launched eagerly on one stream; the same step captured once
             in a HIP graph (num_splits fixed at capture) and replayed K times
             is reported beside it as graph_ms_per_step

roofline   = the stage-1 kernel: algorithmic bytes per launch / its average
             launch time from HIP events on the launch stream, against
             MI355X's 8 TB/s HBM peak.  The timed launches are the stage-1
             dispatches [warmup + steps, warmup + 2 steps) of the run
             (roofline.dispatch_window), so a kernel trace of the same command
             averages exactly those (--profile-report does).
variants   = the other workloads of the pages' matrix (B=16 at 8K, the
             uniform 32K batch, INT8 at 32K, INT4 MTP verify), each timed the
             same way at its tuned split count: stage-1 and whole-step us,
             algorithmic GB/s and the fraction of 8 TB/s.
pool copies: a pool smaller than 2 GB is built in several independent
             copies (same shape, other draws) that consecutive steps rotate
             through, so that no launch finds its K/V in the 256 MB
             Infinity Cache left there by the previous one.
schedule   = how stage 1 is split: "batch" (one tuned num_splits for every
             request, the default) or "request" (the metadata prelude picks
             each request's split count from its own length through a
             per-bucket table derived from a tuned split size); the other
             schedule's stage-1 time is reported beside it (alt_schedule).
Algorithmic bytes: every attended K/V byte once per (request, kv-head)
(plus quantisation scales), Q, the output, the page-table entries read and
the lengths.  Split partials are method overhead and are not counted.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BUCKET_TOKENS = 4096  # KV-length bucket of the split tables
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="ragged_bf16_b64_hq40_hkv8_d128_p64_L1k-32k")
    p.add_argument("--kv-layout", choices=("HND", "NHD"), default=None,
                   help="override the workload's pool layout (head-major HND, token-major NHD)")
    p.add_argument("--splits", type=int, default=0, help="override num_splits (0 = table)")
    p.add_argument("--sched", choices=("batch", "request"), default="batch",
                   help="batch-wide num_splits, or per-request counts from the metadata prelude")
    p.add_argument("--chunk", type=int, default=0,
                   help="per-request split size in pages (0 = tuned table)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-alt", action="store_true",
                   help="skip timing the other schedule and the auxiliary rows (KV append, SWA "
                        "and schedule metadata), keeping a kernel trace to one configuration")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--no-variants", action="store_true",
                   help="skip the other workloads' timings (the variants object)")
    p.add_argument("--pool-copies", type=int, default=0,
                   help="independent copies of the batch that steps rotate through "
                        "(0 = enough for 2 GB of K/V)")
    p.add_argument("--tune", nargs="?", const="all", default=None,
                   help="sweep num_splits per bucket and write the table (optionally a comma list "
                        "of cache formats -- bf16,int8,int4 -- and workload names)")
    p.add_argument("--tune-chunks", nargs="?", const="all", default=None,
                   help="sweep the per-request split size per batch key and write it to the table")
    p.add_argument("--profile-only", action="store_true",
                   help="for rocprofv3 --pmc runs: one 1 GiB copy (the byte-count reference), "
                        "then --steps whole steps, no timing")
    p.add_argument("--rocprof-summary", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                   help="print per-kernel stats and HBM bytes from rocprofv3 CSV output (no GPU)")
    p.add_argument("--profile-report", metavar="RUN_PREFIX",
                   help="write profiles/<kernel>_<workload>.md and update profiles/traffic.json "
                        "from the rocprofv3 runs RUN_PREFIX_{trace,fetch,write[,sq]} (no GPU)")
    return p.parse_args()


def kv_bytes_per_token_head(w) -> int:
    from decode_attention_paged_gqa_amd import workloads as W

    D = w.head_dim
    if w.kv == W.KV_DENSE:
        e = 2 if w.dtype == "bf16" else 4
        return 2 * D * e
    if w.kv == W.KV_INT8:
        return 2 * (D + 2)
    return 2 * (D // 2 + 4 * (D // 32))


def algorithmic_bytes(w, lengths, out_elem=2):
    L = np.asarray(lengths, dtype=np.int64)
    qe = 2 if w.dtype == "bf16" else 4
    n_pages = int(((L + w.page_size - 1) // w.page_size).sum())
    q_bytes = w.batch * w.q_per_req * w.num_q_heads * w.head_dim * qe
    out_bytes = w.batch * w.q_per_req * w.num_q_heads * w.head_dim * out_elem
    kv = int(L.sum()) * w.num_kv_heads * kv_bytes_per_token_head(w)
    return dict(kv=kv, q=q_bytes, out=out_bytes, pt=4 * n_pages, lens=4 * w.batch,
                split=kv + q_bytes + 4 * n_pages + 4 * w.batch,
                step=kv + q_bytes + out_bytes + 4 * n_pages + 4 * w.batch)


def stage1_kernel(w):
    """(kernel name, source files) of the stage-1 kernel a workload runs on,
    as the library dispatches it; traffic counters taken on a kernel stay
    valid only while its sources are unchanged."""
    from decode_attention_paged_gqa_amd import workloads as W

    rows = w.group * w.q_per_req
    bf16_q = w.dtype == "bf16"
    if bf16_q and w.kv == W.KV_DENSE:
        if rows <= 5:
            return "split_bf16_kernel", ["split_bf16.hip", "split_vec.h", "common.h"]
        return "split_bf16_mfma_kernel", ["split_bf16_mfma.hip", "mfma_util.h", "common.h"]
    if w.kv == W.KV_INT8:
        return "split_int8_mfma_kernel", ["split_int8.hip", "mfma_util.h", "common.h"]
    if w.kv == W.KV_INT4:
        return "split_int4_mfma_kernel", ["split_int4.hip", "mfma_util.h", "common.h"]
    if rows >= 5:  # fp32 cache
        return "split_f32_mfma_kernel", ["split_f32_mfma.hip", "mfma_util.h", "common.h"]
    return "split_fma_kernel", ["split_fma.hip", "split_vec.h", "common.h"]


def kernel_hash(w) -> str:
    """Hash of the code (comments and blank space removed) of the kernel's sources."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decode_attention_paged_gqa_amd", "csrc")
    for f in stage1_kernel(w)[1]:
        path = os.path.join(csrc, f)
        if os.path.exists(path):
            src = open(path).read()
            src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
            src = re.sub(r"//[^\n]*", " ", src)
            h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def stage1(da, batch, S, o, l, md=None, sched=False):
    """Stage 1 of the batch; with ``sched`` the metadata's per-request split
    counts and work list drive it (S is then the slots per query row)."""
    from decode_attention_paged_gqa_amd import workloads as W

    w = batch.w
    md = batch.md if md is None else md
    kw = dict(kv_layout=w.kv_layout)
    if sched:
        kw.update(split_counts=md["split_counts"], work_list=md["work_list"])
    else:
        kw.update(batch_order=md["batch_order"])
    if w.kv == W.KV_DENSE:
        return da.decode_attn_split(batch.q, batch.k_pool, batch.v_pool, md["page_table"],
                                    md["cache_seqlens"], S, w.softmax_scale, w.causal, o, l, **kw)
    if w.kv == W.KV_INT8:
        return da.decode_attn_split_int8(batch.q, batch.k_pool, batch.v_pool, batch.k_scale,
                                         batch.v_scale, md["page_table"], md["cache_seqlens"], S,
                                         w.softmax_scale, w.causal, o, l, **kw)
    return da.decode_attn_split_int4(batch.q, batch.k_pool, batch.v_pool, batch.k_scale,
                                     batch.v_scale, md["page_table"], md["cache_seqlens"], S,
                                     w.softmax_scale, w.causal, o, l, **kw)


class Step:
    """Caller-owned buffers and the three calls of one whole step.

    table=None: every request has S splits.  table=[per-bucket counts]: the
    metadata prelude also writes split_counts and the work list, stage 1 and
    the merge follow them, and S = max(table) slots per query row."""

    def __init__(self, da, batch, torch, S=None, table=None):
        w = batch.w
        self.da, self.batch, self.table = da, batch, table
        self.S = max(table) if table is not None else S
        B, qn, Hq, D = batch.q.shape
        self.o = torch.empty((B, qn, Hq, self.S, D), dtype=torch.float32, device="cuda")
        self.l = torch.empty((B, qn, Hq, self.S), dtype=torch.float32, device="cuda")
        self.out = torch.empty((B, qn, Hq, D), dtype=torch.bfloat16, device="cuda")
        self.md = {k: torch.empty_like(v) for k, v in batch.md.items()}
        self.sched_kw = {}
        if table is not None:
            self.md["split_counts"] = torch.empty(B, dtype=torch.int32, device="cuda")
            self.md["work_list"] = torch.empty(B * self.S, dtype=torch.int32, device="cuda")
            self.sched_kw = dict(split_table=table, bucket_tokens=BUCKET_TOKENS,
                                 max_splits=self.S, work_capacity=B * self.S)

    def meta(self):
        b, w = self.batch, self.batch.w
        self.da.decode_attn_metadata(b.seq_lens, b.req_pool_indices, b.req_to_token, w.page_size,
                                     b.max_pages, q_stride=w.q_per_req, out=self.md,
                                     **self.sched_kw)

    def split(self):
        stage1(self.da, self.batch, self.S, self.o, self.l, md=self.md,
               sched=self.table is not None)

    def merge(self):
        self.da.decode_attn_merge(self.o, self.l, out=self.out,
                                  split_counts=self.md.get("split_counts"))

    def __call__(self):
        self.meta()
        self.split()
        self.merge()

    def describe(self):
        if self.table is None:
            return {"mode": "batch", "num_splits": self.S}
        items = int(self.md["split_counts"].sum().item())
        return {"mode": "request", "table": list(self.table), "bucket_tokens": BUCKET_TOKENS,
                "max_splits": self.S, "work_items": items}


def rows_per_kv_head(w):
    return w.group * w.q_per_req


def kv_name(w):
    from decode_attention_paged_gqa_amd import workloads as W

    return w.dtype if w.kv == W.KV_DENSE else w.kv


def time_config(step_list, steps, warmup, torch, settle_ms=0.0):
    """Times `steps` whole steps back to back (host clock, synchronised on both
    sides); then the same number again with events between the three calls for
    the per-kernel breakdown and percentiles (an event record between steps
    costs the stream ~12 us here, so the timed steps carry none).  Step i runs
    on copy i % len(step_list) of the batch.  Returns (ms_per_step,
    split_ms_avg, merge_ms_avg, meta_ms_avg, percentiles); the stage-1 average
    is over the launches [warmup + steps, warmup + 2 steps) of the run.
    settle_ms > 0 (the variants): after the `warmup` steps, more untimed steps
    until the warm-up has kept the GPU busy that long, so that short launches
    are timed once the clocks have settled (10-20 ms after idle)."""
    stream = torch.cuda.current_stream()
    n = len(step_list)

    def run(i, ev=None):
        step = step_list[i % n]
        if ev is not None:
            ev[0].record(stream)
        step.meta()
        if ev is not None:
            ev[1].record(stream)
        step.split()
        if ev is not None:
            ev[2].record(stream)
        step.merge()
        if ev is not None:
            ev[3].record(stream)

    tw = time.perf_counter()
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    if settle_ms > 0:  # back to back, no synchronisation between the steps
        per_ms = (time.perf_counter() - tw) * 1e3 / max(warmup, 1)
        for i in range(int(math.ceil(settle_ms / max(per_ms, 1e-3)))):
            run(i)
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        run(i)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        run(i, evs[i])
    torch.cuda.synchronize()
    meta = np.mean([e[0].elapsed_time(e[1]) for e in evs])
    splits = [e[1].elapsed_time(e[2]) for e in evs]
    merge = np.mean([e[2].elapsed_time(e[3]) for e in evs])
    steps_ms = [e[0].elapsed_time(e[3]) for e in evs]
    pct = {"split_us": [round(float(np.percentile(splits, p)) * 1e3, 2) for p in (10, 50, 90)],
           "step_us": [round(float(np.percentile(steps_ms, p)) * 1e3, 2) for p in (10, 50, 90)]}
    return wall_ms, float(np.mean(splits)), float(merge), float(meta), pct


def time_graph(step, steps, warmup, torch):
    """The same step captured once in a HIP graph (the schedule fixed at capture, as
    the pages deploy their tuned kernels) and replayed; returns ms per replayed step."""
    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def time_calls(fn, iters, torch):
    """Average device time (us) of one call of fn: `iters` calls captured in a
    HIP graph and replayed, so that host launch cost does not leave the GPU
    idle between these few-microsecond kernels."""
    fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(iters):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * iters) * 1e3


def aux_timings(da, batch, iters, torch):
    """The rows around the attention step, timed on the same batch shape:
    * append: the step's B*q new tokens written (encoded for INT8 / INT4
      caches) into a scratch pool of the workload's format and layout at
      distinct random slots -- the benchmarked pools are left untouched;
    * metadata with SWA translation (a page-permuted SWA pool, a quarter of
      its pages not resident), and with the per-request split schedule.
    Bytes are the algorithmic ones: new rows read, codes/scales written."""
    from decode_attention_paged_gqa_amd import workloads as W

    w = batch.w
    B, qn, Hq, D = batch.q.shape
    Hkv, ps = w.num_kv_heads, w.page_size
    N = B * qn
    gen = torch.Generator(device="cuda").manual_seed(99)
    P = max(4 * ((N + ps - 1) // ps), 64)
    shape = (P, ps, Hkv) if w.kv_layout == "NHD" else (P, Hkv, ps)
    fmt = "dense" if w.kv == W.KV_DENSE else w.kv
    new_dtype = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    k_new = torch.randn((N, Hkv, D), generator=gen, device="cuda").to(new_dtype)
    v_new = torch.randn((N, Hkv, D), generator=gen, device="cuda").to(new_dtype)
    if fmt == "dense":
        pools = [torch.empty(shape + (D,), dtype=new_dtype, device="cuda") for _ in range(2)]
        scales = [None, None]
        row_out = D * new_dtype.itemsize
    elif fmt == "int8":
        pools = [torch.empty(shape + (D,), dtype=torch.int8, device="cuda") for _ in range(2)]
        scales = [torch.empty(shape, dtype=torch.float16, device="cuda") for _ in range(2)]
        row_out = D + 2
    else:
        pools = [torch.empty(shape + (D // 2,), dtype=torch.uint8, device="cuda") for _ in range(2)]
        scales = [torch.empty(shape + (D // 32, 2), dtype=torch.float16, device="cuda")
                  for _ in range(2)]
        row_out = D // 2 + 4 * (D // 32)
    loc = torch.randperm(P * ps, generator=gen, device="cuda")[:N].to(torch.int64)
    us = time_calls(lambda: da.decode_attn_append_kv(k_new, v_new, loc, pools[0], pools[1],
                                                      scales[0], scales[1], cache_format=fmt,
                                                      kv_layout=w.kv_layout), iters, torch)
    append_bytes = 2 * N * Hkv * (D * new_dtype.itemsize + row_out) + 8 * N
    out = {"append": {"us": round(us, 2), "tokens": N, "format": fmt,
                      "algorithmic_bytes": append_bytes,
                      "GB_per_s": round(append_bytes / (us * 1e-6) / 1e9, 1)}}

    slots = int(batch.req_to_token.max().item()) + 1
    pages = (slots + ps - 1) // ps
    perm = torch.randperm(pages + 7, generator=gen, device="cuda")[:pages]
    f2s = (perm[:, None] * ps + torch.arange(ps, device="cuda")[None, :]).to(torch.int64)
    f2s[torch.rand(pages, generator=gen, device="cuda") < 0.25] = -1
    f2s = f2s.reshape(-1).contiguous()
    md = {k: torch.empty_like(v) for k, v in batch.md.items()}
    md["swa_page_table"] = torch.empty_like(batch.md["page_table"])
    args = (batch.seq_lens, batch.req_pool_indices, batch.req_to_token, ps, batch.max_pages)
    out["metadata"] = {"us": round(time_calls(lambda: da.decode_attn_metadata(
        *args, q_stride=qn, out=md), iters, torch), 2)}
    out["metadata_swa"] = {"us": round(time_calls(lambda: da.decode_attn_metadata(
        *args, q_stride=qn, out=md, full_to_swa=f2s), iters, torch), 2)}
    table = [1, 2, 3, 4, 5, 6, 7, 8]
    md2 = dict(md, split_counts=torch.empty(B, dtype=torch.int32, device="cuda"),
               work_list=torch.empty(B * 8, dtype=torch.int32, device="cuda"))
    out["metadata_schedule"] = {"us": round(time_calls(lambda: da.decode_attn_metadata(
        *args, q_stride=qn, out=md2, split_table=table, bucket_tokens=BUCKET_TOKENS,
        max_splits=8), iters, torch), 2)}
    return out


def time_split_merge(step, iters, torch):
    """Average time (ms) of stage 1 + merge over `iters` back-to-back pairs (the
    part of a step that depends on the split count)."""
    step.meta()
    for _ in range(3):
        step.split()
        step.merge()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        step.split()
        step.merge()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def settle(step, torch, ms=60.0):
    """Stage 1 + merge back to back for about `ms` (untimed): building a batch
    leaves the GPU idle, and its clocks settle 10-20 ms after it is busy again,
    so candidates timed right away would be timed at other clocks than the
    later ones."""
    step.meta()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step.split()
    step.merge()
    torch.cuda.synchronize()
    per_ms = max((time.perf_counter() - t0) * 1e3, 1e-3)
    for _ in range(int(math.ceil(ms / per_ms))):
        step.split()
        step.merge()
    torch.cuda.synchronize()


def time_split_only(step, iters, torch):
    """Average stage-1 time (ms) over `iters` back-to-back launches."""
    step.meta()
    for _ in range(3):
        step.split()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        step.split()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(batch, seconds):
    """The fp64 oracle on a bounded sample of the same batch, on the host cores.

    Requests are taken in batch order until `seconds` of oracle time are spent;
    each one's host copy is prepared outside the timer, the oracle is run once
    warm, then timed three times, and the median counts."""
    import torch
    from decode_attention_paged_gqa_amd import workloads as W
    from oracle import attention as OA
    from oracle import quant as OQ

    w = batch.w
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    done_bytes = 0
    done = []
    elapsed = 0.0
    pt_all = batch.page_table.cpu().numpy()
    for b in range(w.batch):
        L = int(batch.lengths[b])
        n = -(-L // w.page_size)
        pages = torch.from_numpy(pt_all[b, :n].astype(np.int64)).cuda()
        q = W.host_f64(batch.q[b:b + 1])

        def take(t):  # this request's pages, in the oracle's [P, page, Hkv, ...] order
            return batch.nhd(t).index_select(0, pages)

        if w.kv == W.KV_DENSE:
            k = W.host_f64(take(batch.k_pool))
            v = W.host_f64(take(batch.v_pool))
        else:
            k = (W.host_int(take(batch.k_pool)), W.host_u16(take(batch.k_scale)))
            v = (W.host_int(take(batch.v_pool)), W.host_u16(take(batch.v_scale)))
        pt = np.arange(n, dtype=np.int64)[None, :]

        def run():
            kk, vv = k, v
            if w.kv == W.KV_INT8:
                kk, vv = OQ.dequant_int8(*k), OQ.dequant_int8(*v)
            elif w.kv == W.KV_INT4:
                kk, vv = OQ.dequant_int4(*k), OQ.dequant_int4(*v)
            OA.decode_attention(q, kk, vv, pt, np.array([L]), w.page_size, w.softmax_scale,
                                w.causal)

        run()  # warm
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            run()
            ts.append(time.perf_counter() - t0)
        elapsed += sorted(ts)[1]
        done.append(b)
        done_bytes += L * w.num_kv_heads * kv_bytes_per_token_head(w)
        if elapsed >= seconds:
            break
    gbs = done_bytes / elapsed / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 oracle over {len(done)} of {w.batch} requests (all heads), "
                      f"{done_bytes / 1e9:.3f} GB of algorithmic K/V bytes in {elapsed:.1f} s "
                      f"(per request: one warm run, median of three timed runs; host copies "
                      f"prepared outside the timed region)",
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": _cpu_model()}


def make_resident(da, w, torch, seed=None, lengths=None):
    from decode_attention_paged_gqa_amd import workloads as W

    batch = W.make_batch(w, device="cuda", seed=seed, lengths=lengths)
    batch.md = da.decode_attn_metadata(batch.seq_lens, batch.req_pool_indices, batch.req_to_token,
                                       w.page_size, batch.max_pages, q_stride=w.q_per_req)
    torch.cuda.synchronize()
    return batch


ROTATE_BYTES = 2 << 30  # K/V footprint the rotated copies add up to at least


def pool_bytes(batch) -> int:
    t = [batch.k_pool, batch.v_pool, batch.k_scale, batch.v_scale]
    return sum(x.numel() * x.element_size() for x in t if x is not None)


def resident_copies(da, w, torch, copies=0):
    """The batch, plus independent copies (same lengths and shape, other draws
    and page permutations) until the pools add up to ROTATE_BYTES; ``copies``
    > 0 fixes the number."""
    first = make_resident(da, w, torch)
    n = copies or max(1, -(-ROTATE_BYTES // max(1, pool_bytes(first))))
    return [first] + [make_resident(da, w, torch, seed=w.seed + 1000 * i, lengths=first.lengths)
                      for i in range(1, n)]


# workload names; "@NHD" runs the workload over the token-major pool layout
VARIANT_WORKLOADS = ("bf16_b16_hq32_hkv8_d128_p64_L8192", "bf16_b64_hq40_hkv8_d128_p64_L32768",
                     "int8kv_b32_hq32_hkv8_d128_p64_L32768",
                     "int4kv_mtp4_b64_hq32_hkv8_d128_p64_L8k-32k",
                     "int8kv_b32_hq32_hkv8_d128_p64_L32768@NHD",
                     "int4kv_mtp4_b64_hq32_hkv8_d128_p64_L8k-32k@NHD")


# untimed warm-up of every variant, at least: the clocks settle 10-20 ms after
# the GPU leaves idle (building a variant's pools leaves it idle)
VARIANT_SETTLE_MS = 60.0


def variant_timings(da, torch, steps, warmup):
    """The pages' other decode shapes, each at its tuned split count and timed
    as the main line is (HIP events per call; pools under 2 GB rotated); the
    quantised ones also over the token-major pool layout."""
    from decode_attention_paged_gqa_amd import workloads as W
    from decode_attention_paged_gqa_amd.splits import SplitTable, kernel_key

    tables = SplitTable.load()
    out = {}
    for entry in VARIANT_WORKLOADS:
        name, _, layout = entry.partition("@")
        w = W.WORKLOADS[name]
        if layout:
            w = w.scaled(kv_layout=layout)
        batches = resident_copies(da, w, torch)
        key = kernel_key(kv_name(w), rows_per_kv_head(w), w.head_dim, w.page_size, w.kv_layout)
        S = tables.pick(key, w.batch, int(batches[0].lengths.max()))
        step_list = [Step(da, b, torch, S=S) for b in batches]
        ms, split_ms, merge_ms, meta_ms, _ = time_config(step_list, steps, warmup, torch,
                                                         settle_ms=VARIANT_SETTLE_MS)
        ab = algorithmic_bytes(w, batches[0].lengths)
        gbs = ab["split"] / (split_ms * 1e-3) / 1e9
        out[entry] = {"kernel": stage1_kernel(w)[0], "kv": kv_name(w), "kv_layout": w.kv_layout,
                      "batch": w.batch, "q_per_req": w.q_per_req, "num_q_heads": w.num_q_heads,
                      "kv_tokens": int(batches[0].lengths.sum()), "num_splits": S,
                      "pool_copies": len(batches), "split_us": round(split_ms * 1e3, 2),
                      "step_us": round(ms * 1e3, 2), "split_GBps": round(gbs, 1),
                      "frac": round(gbs / HBM_PEAK_GBS, 4),
                      "step_frac": round(ab["step"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "algorithmic_bytes_per_launch": ab["split"]}
        del step_list, batches
        torch.cuda.empty_cache()
    return out


def tune_variants(which):
    """Workloads whose kernel variants a sweep covers: all, or a comma list of
    cache formats (bf16, int8, int4) and workload names."""
    from decode_attention_paged_gqa_amd import workloads as W

    variants = [W.RAGGED_B64, W.BF16_B16, W.INT8_B32, W.INT4_MTP_B64, W.BF16_MTP_B64,
                W.BF16_MTP_G5_B64]
    # the same shapes at head dim 64 (one per stage-1 kernel)
    variants += [v.scaled(name=v.name.replace("_d128_", "_d64_"), head_dim=64)
                 for v in (W.RAGGED_B64, W.INT8_B32, W.INT4_MTP_B64, W.BF16_MTP_B64)]
    # the token-major pool layout: the bf16 vector kernel, and one shape per
    # matrix-core kernel (INT4 at both head dims)
    variants += [v.scaled(name=v.name + "_nhd", kv_layout="NHD")
                 for v in (W.RAGGED_B64, W.BF16_B16, W.INT8_B32, W.INT4_MTP_B64, W.BF16_MTP_B64,
                           W.INT4_MTP_D64_B64)]
    # token-major at head dim 64 where the kernel takes four kv-heads per workgroup
    variants += [v.scaled(name=v.name.replace("_d128_", "_d64_") + "_nhd", head_dim=64,
                          kv_layout="NHD")
                 for v in (W.INT8_B32, W.BF16_MTP_B64, W.RAGGED_B64, W.BF16_B16, W.FP32_G4_B16,
                           W.FP32_B16)]
    # the dense fp32 cache: vector kernel (G = 4) and matrix cores (G = 8)
    variants += [W.FP32_G4_B16, W.FP32_B16]
    if which == "all":
        return variants
    keep = set(which.split(","))
    return [v for v in variants if kv_name(v) in keep or v.name in keep]


def tune(da, torch, which="all", old_keys=None):
    """Sweep num_splits per KV-length bucket and batch key; write splits_table.json.
    A variant's row for a batch key of ``old_keys`` (the batch keys the table's
    rows were tuned for; default: those of the loaded table) is kept (set
    DECODE_ATTN_RETUNE=1 to sweep every key again)."""
    from decode_attention_paged_gqa_amd import workloads as W
    from decode_attention_paged_gqa_amd.splits import (BATCH_KEYS, BUCKET_TOKENS, CANDIDATES,
                                                       N_BUCKETS, SplitTable, kernel_key)

    table = SplitTable.load()
    old_keys = list(table.batch_keys) if old_keys is None else list(old_keys)
    retune = os.environ.get("DECODE_ATTN_RETUNE") == "1"
    # DECODE_ATTN_RETUNE_KEYS=1,4: sweep those batch keys again, keep the other rows
    only = {int(x) for x in os.environ.get("DECODE_ATTN_RETUNE_KEYS", "").split(",") if x}
    table.batch_keys = list(BATCH_KEYS)  # rows of variants not swept here stop matching
    variants = tune_variants(which)
    for base in variants:
        key = kernel_key(kv_name(base), rows_per_kv_head(base), base.head_dim, base.page_size,
                         base.kv_layout)
        old = table.tables.get(key)
        old = old if old is not None and len(old) == len(old_keys) else None
        rows = []
        for bk in BATCH_KEYS:
            if old is not None and bk in old_keys and not retune and bk not in only:
                rows.append(old[old_keys.index(bk)])
                continue
            row = []
            for k in range(1, N_BUCKETS + 1):
                # representative batches: the bucket's upper length for one request, the
                # rest log-uniform below it (ragged, like the pages' serving batches).
                # Candidates stop at the longest request's page count (more splits
                # would be empty); each is timed as stage 1 + merge, twice per seed,
                # and the smallest split count within the measured noise of the
                # fastest wins
                Lmax = k * BUCKET_TOKENS
                cands = [S for S in CANDIDATES if S <= max(1, -(-Lmax // base.page_size))]
                tot = {S: 0.0 for S in cands}
                rel = []  # relative differences between the two timings of one configuration
                for rep in range(3):
                    w = base.scaled(batch=bk, lengths="loguniform", length_lo=max(64, Lmax // 32),
                                    length_hi=Lmax, pin_max=True, seed=100 + 10 * k + rep)
                    batch = make_resident(da, w, torch)
                    settle(Step(da, batch, torch, S=cands[len(cands) // 2]), torch)
                    for S in cands:
                        step = Step(da, batch, torch, S=S)
                        t1 = time_split_merge(step, 10, torch)
                        t2 = time_split_merge(step, 10, torch)
                        tot[S] += t1 + t2
                        rel.append(abs(t1 - t2) / max(min(t1, t2), 1e-9))
                    del batch
                    torch.cuda.empty_cache()
                fastest = min(tot.values())
                tol = max(0.01, 2.0 * float(np.median(rel)))
                best = min(S for S in cands if tot[S] <= fastest * (1.0 + tol))
                row.append(best)
                print(f"tune {key} B={bk} bucket={k} -> S={best} (noise tol {100 * tol:.1f} %) "
                      + " ".join(f"{S}:{tot[S] / 6 * 1e3:.1f}" for S in cands), flush=True)
            rows.append(row)
        table.tables[key] = rows
        table.save()  # after every variant, so a long sweep keeps what it has done
    table.save()
    print(json.dumps({"tuned": list(table.tables)}), flush=True)


def tune_chunks(da, torch, which="all", old_keys=None):
    """Sweep the per-request split size (pages) per batch key over ragged batches
    whose longest request sits in buckets 2, 4 and 8 (the 32K representative
    length); write the best size per batch key into splits_table.json.  Sizes
    already tuned for a batch key of ``old_keys`` are kept, as in tune()."""
    from decode_attention_paged_gqa_amd import workloads as W
    from decode_attention_paged_gqa_amd.splits import (BATCH_KEYS, CHUNK_CANDIDATES, SplitTable,
                                                       kernel_key, per_request_table)

    table = SplitTable.load()
    old_keys = list(table.batch_keys) if old_keys is None else list(old_keys)
    retune = os.environ.get("DECODE_ATTN_RETUNE") == "1"
    table.batch_keys = list(BATCH_KEYS)
    variants = tune_variants(which)
    for base in variants:
        key = kernel_key(kv_name(base), rows_per_kv_head(base), base.head_dim, base.page_size,
                         base.kv_layout)
        old = table.chunk_pages.get(key)
        old = old if old is not None and len(old) == len(old_keys) else None
        row = []
        for bk in BATCH_KEYS:
            if old is not None and bk in old_keys and not retune:
                row.append(old[old_keys.index(bk)])
                continue
            tot = {c: 0.0 for c in CHUNK_CANDIDATES}
            for k in (2, 4, 8):
                Lmax = k * BUCKET_TOKENS
                w = base.scaled(batch=bk, lengths="loguniform", length_lo=max(64, Lmax // 32),
                                length_hi=Lmax, pin_max=True, seed=200 + k)
                batch = make_resident(da, w, torch)
                mid = CHUNK_CANDIDATES[len(CHUNK_CANDIDATES) // 2]
                settle(Step(da, batch, torch,
                            table=per_request_table(mid, w.page_size, BUCKET_TOKENS)), torch)
                for c in CHUNK_CANDIDATES:
                    t = per_request_table(c, w.page_size, BUCKET_TOKENS)
                    tot[c] += time_split_only(Step(da, batch, torch, table=t), 10, torch)
                del batch
                torch.cuda.empty_cache()
            best = min(CHUNK_CANDIDATES, key=lambda c: (tot[c], -c))
            row.append(best)
            print(f"tune-chunks {key} B={bk} -> {best} pages "
                  + " ".join(f"{c}:{tot[c] * 1e3:.1f}" for c in CHUNK_CANDIDATES), flush=True)
        table.chunk_pages[key] = row
    table.save()
    print(json.dumps({"tuned_chunks": table.chunk_pages}), flush=True)


COPY_BYTES = 1 << 30


def profile_only(step_list, steps, torch):
    """Dispatches for counter collection: a plain 1 GiB device copy whose byte
    count is known (it calibrates FETCH_SIZE / WRITE_SIZE), then whole steps
    (rotating over the batch copies)."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    for i in range(steps):
        step_list[i % len(step_list)]()
    torch.cuda.synchronize()
    step = step_list[0]
    w = step.batch.w
    ab = algorithmic_bytes(w, step.batch.lengths)
    print(json.dumps({"profile_only": w.name, "schedule": step.describe(), "copy_bytes": COPY_BYTES,
                      "split_algorithmic_bytes": ab["split"], "kernel_hash": kernel_hash(w)}),
          flush=True)


def _read_csv(d, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def rocprof_summary(trace_dir, fetch_dir, write_dir):
    """Per-kernel stats from the kernel trace, HBM bytes per dispatch from the
    two counter runs, calibrated by the 1 GiB copy (read 1 GiB, write 1 GiB)."""
    stats = _read_csv(trace_dir, "kernel_stats.csv")
    def counters(d, name):
        rows = _read_csv(d, "counter_collection.csv")
        per = {}
        for r in rows:
            if r.get("Counter_Name") != name:
                continue
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        return per
    fetch = counters(fetch_dir, "FETCH_SIZE")
    write = counters(write_dir, "WRITE_SIZE")

    def by_kernel(per, pat):
        vals = [v for (d, k), v in sorted(per.items(), key=lambda x: int(x[0][0])) if pat in k]
        return vals
    # the reference copy is the largest copyBuffer dispatch (1 GiB read, 1 GiB written)
    copy_fetch_kib = sorted(by_kernel(fetch, "copyBuffer"))[-1:]
    copy_write_kib = sorted(by_kernel(write, "copyBuffer"))[-1:]
    split_fetch = by_kernel(fetch, "split_")
    split_write = by_kernel(write, "split_")
    f_scale = (COPY_BYTES / 1024) / max(copy_fetch_kib[-1], 1e-9) if copy_fetch_kib else None
    w_scale = (COPY_BYTES / 1024) / max(copy_write_kib[-1], 1e-9) if copy_write_kib else None
    lines = ["| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | "
                     f"{float(r['MinNs'])/1e3:.2f} | {float(r['MaxNs'])/1e3:.2f} |")
    sf = float(np.mean(split_fetch)) * 1024 * f_scale if split_fetch and f_scale else None
    sw = float(np.mean(split_write)) * 1024 * w_scale if split_write and w_scale else None
    return "\n".join(lines), dict(copy_fetch_kib=copy_fetch_kib[-1] if copy_fetch_kib else None,
                                   copy_write_kib=copy_write_kib[-1] if copy_write_kib else None,
                                   fetch_scale=f_scale, write_scale=w_scale,
                                   split_fetch_kib=split_fetch, split_write_kib=split_write,
                                   split_fetch_bytes=sf, split_write_bytes=sw)


def window_us(trace_dir, kname, window):
    """Mean duration (us) of dispatches [first, first + count) of kernel `kname`
    in a rocprofv3 kernel trace, in launch order, and the number averaged."""
    rows = [r for r in _read_csv(trace_dir, "kernel_trace.csv")
            if kname + "<" in r["Kernel_Name"] or kname + "(" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    first, count = window
    sel = rows[first:first + count]
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in sel]
    return (float(np.mean(durs)) if durs else float("nan")), len(durs), len(rows)


SQ_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE")


def sq_summary(sq_dir, pat):
    """MFMA and VALU busy of the kernel named `pat` (mean over its dispatches):
    sum over SIMDs of SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE of one XCC x 1024
    SIMDs), and sum of SQ_ACTIVE_INST_VALU / (GRBM_GUI_ACTIVE x 256 CUs)."""
    rows = _read_csv(sq_dir, "counter_collection.csv")
    per, grbm = {}, {}
    for r in rows:
        if pat + "<" not in r["Kernel_Name"] and pat + "(" not in r["Kernel_Name"]:
            continue
        d = per.setdefault(r["Dispatch_Id"], {})
        name = r["Counter_Name"]
        v = float(r["Counter_Value"])
        if name == "GRBM_GUI_ACTIVE":
            grbm.setdefault(r["Dispatch_Id"], []).append(v)
        else:
            d[name] = d.get(name, 0.0) + v
    for k, vals in grbm.items():
        # one row per XCC -> the largest; one row summed over the 8 XCCs -> / 8
        per[k]["GRBM_GUI_ACTIVE"] = max(vals) if len(vals) > 1 else vals[0] / 8
    mfma = [d["SQ_VALU_MFMA_BUSY_CYCLES"] / (d["GRBM_GUI_ACTIVE"] * 1024) for d in per.values()]
    valu = [d["SQ_ACTIVE_INST_VALU"] / (d["GRBM_GUI_ACTIVE"] * 256) for d in per.values()]
    return dict(dispatches=len(per), mfma_busy=float(np.mean(mfma)), valu_busy=float(np.mean(valu)),
                gui_active_cycles=float(np.mean([d["GRBM_GUI_ACTIVE"] for d in per.values()])))


def profile_report(prefix):
    """Summary of the rocprofv3 runs of one workload: writes
    profiles/<kernel>_<workload>_<layout>.md and its entry in profiles/traffic.json."""
    import re
    from decode_attention_paged_gqa_amd import workloads as W

    trace_log = prefix + "_trace.log"
    line = [ln for ln in open(trace_log) if ln.startswith('{"metric"')][-1]
    res = json.loads(line)
    w = W.WORKLOADS[res["config"]["workload"]]
    w = w.scaled(kv_layout=res["config"].get("kv_layout", w.kv_layout))
    wl = w.name
    kv = kv_name(w)
    sched = res["schedule"]
    S = res["config"]["num_splits"]
    ab = res["roofline"]["algorithmic_bytes_per_launch"]
    table, tr = rocprof_summary(prefix + "_trace", prefix + "_fetch", prefix + "_write")
    stats = _read_csv(prefix + "_trace", "kernel_stats.csv")
    kname = stage1_kernel(w)[0]
    srow = [r for r in stats if kname + "<" in r["Name"] or kname + "(" in r["Name"]][0]
    all_avg_us = float(srow["AverageNs"]) / 1e3
    calls = int(srow["Calls"])
    # the launches the bench line's roofline was timed on (HIP events), from the trace
    window = res["roofline"].get("dispatch_window")
    avg_us, n_win, n_all = window_us(prefix + "_trace", kname, window)
    kern = re.sub(r"^(void )?\(anonymous namespace\)::", "", srow["Name"]).split("(")[0]
    fetch, write = tr["split_fetch_bytes"], tr["split_write_bytes"]
    hbm = fetch + write
    cfg = res["config"]
    short = wl.replace("_p64", "")
    fn = f"profiles/{kname}_{short}_{w.kv_layout.lower()}.md"
    rel = os.path.relpath(prefix, ROOT)
    lens = (f"{w.lengths} {w.length}" if w.lengths == "fixed"
            else f"{w.lengths} in [{w.length_lo}, {w.length_hi}]")
    wdesc = (f"B={w.batch}, Hq={w.num_q_heads}, Hkv={w.num_kv_heads} (G={w.group}), "
             f"q_per_req={w.q_per_req}{' causal' if w.causal else ''}, D={w.head_dim}, "
             f"page_size {w.page_size}, {kv} cache, {w.kv_layout} pool layout; KV lengths {lens}"
             + (" with one request at the maximum" if w.pin_max else "")
             + f" (seed {w.seed}): {cfg['kv_tokens']:,} tokens, {ab:,} algorithmic bytes per "
             f"stage-1 launch")
    copies = int(cfg.get("pool_copies", 1))
    if copies > 1:
        wdesc += (f"; consecutive steps rotate over {copies} independent copies of the pools "
                  f"(K/V and scales under 2 GB otherwise), so no launch finds the previous "
                  f"one's K/V in the 256 MB Infinity Cache")
    run = f"python3 $R/bench.py --workload {wl} --sched {sched['mode']}"
    if w.kv_layout != W.WORKLOADS[wl].kv_layout:
        run += f" --kv-layout {w.kv_layout}"
    cmds = ["cd /tmp && export TMPDIR=/tmp",
            f"rocprofv3 --kernel-trace --stats --output-format csv -d $R/{rel}_trace -o run -- "
            f"{run} --steps {res['steps']} --warmup {res['warmup']} --no-cpu-baseline --no-alt "
            f"--no-variants",
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d $R/{rel}_fetch -o run -- "
            f"{run} --profile-only --steps 3",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d $R/{rel}_write -o run -- "
            f"{run} --profile-only --steps 3"]
    sq = None
    if os.path.isdir(prefix + "_sq"):
        sq = sq_summary(prefix + "_sq", kname)
        cmds.append(f"rocprofv3 --pmc {' '.join(SQ_COUNTERS)} --output-format csv -d $R/{rel}_sq "
                    f"-o run -- {run} --profile-only --steps 3")
    cmds.append(f"cd $R && python3 bench.py --profile-report {rel}")
    rows = "\n".join(f"| {i} | {f:.1f} | {wv:.1f} |" for i, (f, wv) in
                     enumerate(zip(tr["split_fetch_kib"], tr["split_write_kib"])))
    partial_bytes = w.batch * w.q_per_req * w.num_q_heads * S * (w.head_dim + 1) * 4
    sched_txt = (f"num_splits {S} from the tuned split table" if sched["mode"] == "batch" else
                 f"per-request split counts (table {sched['table']} per {sched['bucket_tokens']}"
                 f"-token bucket, {sched['work_items']} work items)")
    units = ""
    if sq is not None:
        units = f"""
## Compute units (`--pmc {' '.join(SQ_COUNTERS)}`, {sq['dispatches']} dispatches)

MFMA busy = sum of SQ_VALU_MFMA_BUSY_CYCLES over the 1024 SIMDs / (GRBM_GUI_ACTIVE x 1024),
GRBM_GUI_ACTIVE being the busy cycles of one XCC (the counter row is the sum over the 8 XCCs):
**{100 * sq['mfma_busy']:.1f} %**.  VALU busy = sum of SQ_ACTIVE_INST_VALU / (GRBM_GUI_ACTIVE x 256 CUs):
**{100 * sq['valu_busy']:.1f} %**.  (GRBM_GUI_ACTIVE {sq['gui_active_cycles']:,.0f} cycles of one XCC
per dispatch; counters run with the profiler's serialised dispatches.)
"""
    md = f"""# {kern} on {wl} ({w.kv_layout}), {sched['mode']} schedule

Workload: {wdesc}.  MI355X (gfx950), one GPU, rocprofv3 from ROCm 7.2; {sched_txt}.
`$R` is the repository root.

Commands:

```
{chr(10).join(cmds)}
```

## Kernel trace (`--kernel-trace --stats`, {calls} stage-1 calls in all)

{table}

The bench line's roofline times stage-1 launches {window[0]} .. {window[0] + window[1] - 1} of the
run with HIP events (after {window[0]} warm-up and wall-clock launches).  Those {n_win} launches in
the kernel trace ({n_all} stage-1 dispatches traced): average **{avg_us:.2f} us** ->
{ab / (avg_us * 1e-6) / 1e9:.1f} GB/s algorithmic, **{ab / (avg_us * 1e-6) / 1e9 / HBM_PEAK_GBS * 100:.1f} %** of 8 TB/s.
bench.py's HIP-event average over the same launches: {res['kernels_us']['split']:.2f} us
({res['roofline']['achieved']:.1f} GB/s, {100 * res['roofline']['frac']:.1f} %).  The average over all
{calls} calls in the stats table (warm-up, graph replays included) is {all_avg_us:.2f} us.

## HBM traffic (`--pmc FETCH_SIZE`, `--pmc WRITE_SIZE`, per stage-1 dispatch)

Calibration: a 1 GiB device-to-device copy (`__amd_rocclr_copyBuffer`) reads
FETCH_SIZE = {tr['copy_fetch_kib']:.1f} KiB and writes WRITE_SIZE = {tr['copy_write_kib']:.1f} KiB,
so FETCH_SIZE is scaled by {tr['fetch_scale']:.4f} and WRITE_SIZE by {tr['write_scale']:.4f} to give bytes.

| stage-1 dispatch | FETCH_SIZE KiB | WRITE_SIZE KiB |
|---|---|---|
{rows}

Mean: {fetch / 1e9:.4f} GB read + {write / 1e6:.2f} MB written = {hbm / 1e9:.4f} GB per launch,
{hbm / ab:.4f} x the algorithmic bytes (the writes are the fp32 split partials, at most
{w.batch}*{w.q_per_req}*{w.num_q_heads}*{S}*({w.head_dim}+1)*4 B = {partial_bytes / 1e6:.2f} MB).
{units}"""
    with open(os.path.join(ROOT, fn), "w") as f:
        f.write(md)
    traffic = json.load(open(TRAFFIC_FILE)) if os.path.exists(TRAFFIC_FILE) else {}
    ent = {"kernel": kern, "kernel_hash": kernel_hash(w),
           "schedule": {k: sched[k] for k in ("mode", "num_splits") if k in sched},
           "num_splits": S, "hbm_bytes_per_launch": int(round(hbm)),
           "fetch_bytes": int(round(fetch)), "write_bytes": int(round(write)),
           "fetch_scale": tr["fetch_scale"], "write_scale": tr["write_scale"],
           "rocprof_avg_us": round(avg_us, 2), "rocprof_all_calls_avg_us": round(all_avg_us, 2),
           "summary": fn}
    if sq is not None:
        ent["mfma_busy"] = round(sq["mfma_busy"], 4)
        ent["valu_busy"] = round(sq["valu_busy"], 4)
    traffic[f"{wl}/{w.kv_layout}"] = ent
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(traffic, f, indent=1)
        f.write("\n")
    print(fn, f"{avg_us:.1f} us (window; HIP events {res['kernels_us']['split']:.1f} us)",
          f"traffic {hbm / ab:.4f}x",
          "" if sq is None else f"mfma {100 * sq['mfma_busy']:.1f}% valu {100 * sq['valu_busy']:.1f}%")


def main():
    args = parse()
    if args.profile_report:
        profile_report(os.path.join(ROOT, args.profile_report))
        return
    if args.rocprof_summary:
        table, tr = rocprof_summary(*args.rocprof_summary)
        print(table)
        print(json.dumps(tr))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the path runs on one GPU; sharding it by kv-head, by request or by "
              "KV sequence is a design note only and nothing here launches it. Use --gpus 1.",
              file=sys.stderr, flush=True)
        sys.exit(2)
    import torch

    import decode_attention_paged_gqa_amd as da
    from decode_attention_paged_gqa_amd import workloads as W
    from decode_attention_paged_gqa_amd.splits import SplitTable, kernel_key, per_request_table

    da.load()
    if args.tune or args.tune_chunks:
        from decode_attention_paged_gqa_amd.splits import SplitTable
        old_keys = SplitTable.load().batch_keys  # what the stored rows were tuned for
        if args.tune:
            tune(da, torch, args.tune, old_keys)
        if args.tune_chunks:
            tune_chunks(da, torch, args.tune_chunks, old_keys)
        return
    w = W.WORKLOADS[args.workload]
    if args.kv_layout:
        w = w.scaled(kv_layout=args.kv_layout)
    batches = resident_copies(da, w, torch, args.pool_copies)
    batch = batches[0]
    key = kernel_key(kv_name(w), rows_per_kv_head(w), w.head_dim, w.page_size, w.kv_layout)
    tables = SplitTable.load()
    S = args.splits or tables.pick(key, w.batch, int(batch.lengths.max()))
    chunk = args.chunk or tables.chunk_for(key, w.batch)
    req_table = per_request_table(chunk, w.page_size, tables.bucket_tokens)
    if args.sched == "batch":
        steps_main = [Step(da, b, torch, S=S) for b in batches]
        alt = Step(da, batch, torch, table=req_table)
    else:
        steps_main = [Step(da, b, torch, table=req_table) for b in batches]
        alt = Step(da, batch, torch, S=S)
    step = steps_main[0]
    if args.profile_only:
        profile_only(steps_main, args.steps, torch)
        return
    ms, split_ms, merge_ms, meta_ms, pct = time_config(steps_main, args.steps, args.warmup, torch)
    # the same step captured once in a HIP graph and replayed (reported beside it)
    try:
        graph_ms = time_graph(step, args.steps, args.warmup, torch)
    except Exception as e:
        print(f"bench.py: graph capture failed ({e})", file=sys.stderr)
        graph_ms = None
    alt_split_ms = None if args.no_alt else time_split_only(alt, args.steps, torch)
    aux = None if args.no_alt else aux_timings(da, batch, args.steps, torch)
    schedule, alt_schedule = step.describe(), alt.describe()
    if args.sched == "request":
        schedule["chunk_pages"] = chunk
    else:
        alt_schedule["chunk_pages"] = chunk
    ab = algorithmic_bytes(w, batch.lengths)
    value = ab["step"] / (ms * 1e-3) / 1e9
    achieved = ab["split"] / (split_ms * 1e-3) / 1e9
    traffic = None
    counters = {}
    if os.path.exists(TRAFFIC_FILE):
        t = json.load(open(TRAFFIC_FILE))
        ent = t.get(f"{w.name}/{w.kv_layout}")
        if ent and ent.get("kernel_hash") == kernel_hash(w) \
                and ent.get("schedule", {"mode": "batch", "num_splits": ent.get("num_splits")}) \
                == {k: schedule[k] for k in ("mode", "num_splits") if k in schedule}:
            traffic = ent.get("hbm_bytes_per_launch")
            counters = {k: ent[k] for k in ("mfma_busy", "valu_busy") if k in ent}
    res = {
        "metric": "decode-attn achieved HBM GB/s (% of peak) + us/call, B=64 KV=32K bf16",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_call": round(ms * 1e3, 2),
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if (w.kv == W.KV_DENSE and w.dtype == "bf16") else kv_name(w),
        "data": "synthetic",
        "config": {"workload": w.name, "pool_copies": len(batches), "batch": w.batch,
                   "q_per_req": w.q_per_req,
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "page_size": w.page_size, "kv_layout": w.kv_layout,
                   "kv_len_max": int(batch.lengths.max()), "kv_len_mean": float(batch.lengths.mean()),
                   "kv_tokens": int(batch.lengths.sum()), "num_splits": step.S, "seed": w.seed,
                   "parallelism": "single-gpu"},
        "schedule": schedule,
        "alt_schedule": None if alt_split_ms is None else dict(
            alt_schedule, split_us=round(alt_split_ms * 1e3, 2),
            frac=round(ab["split"] / (alt_split_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)),
        "kernels_us": {"metadata": round(meta_ms * 1e3, 2), "split": round(split_ms * 1e3, 2),
                       "merge": round(merge_ms * 1e3, 2)},
        "percentiles_p10_p50_p90": pct,
        "roofline": {"bound": "hbm", "kernel": "split (stage 1)", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": ab["split"],
                     "dispatch_window": [args.warmup + args.steps, args.steps], **counters},
        "aux_us": aux,
        "step_frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": ab["step"],
    }
    if not args.no_variants:
        del alt
        res["variants"] = variant_timings(da, torch, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(batch, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
