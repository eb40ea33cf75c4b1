"""CPU checks of bench.py's bookkeeping: the one-GPU contract, the algorithmic
byte count of a stage-1 launch written out from its definition (every K/V byte
of every request's tokens, the queries, the page ids and the lengths), and the
stage-1 kernel each workload runs on, which names the rocprofv3 summaries and
keys their traffic counters."""
import os
import subprocess
import sys

import bench as B
from decode_attention_paged_gqa_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr


def test_algorithmic_bytes_by_cache_format():
    L = [1, 63, 64, 65, 1000]
    pages = 1 + 1 + 1 + 2 + 16  # ceil(L / 64)
    # bytes of one token's K row for one kv-head (V the same)
    per_row = {("dense", "bf16"): lambda D: 2 * D, ("dense", "fp32"): lambda D: 4 * D,
               (W.KV_INT8, "bf16"): lambda D: D + 2,             # codes + fp16 scale
               (W.KV_INT4, "bf16"): lambda D: D // 2 + 4 * (D // 32)}  # nibbles + (s, z) pairs
    for (kv, dtype), row in per_row.items():
        for D in (64, 128):
            w = W.BF16_B16.scaled(name="t", batch=5, num_q_heads=8, num_kv_heads=2, head_dim=D,
                                  q_per_req=2, kv=W.KV_DENSE if kv == "dense" else kv,
                                  dtype=dtype, lengths="list", length_list=tuple(L))
            q_elem = 2 if dtype == "bf16" else 4
            want = (sum(L) * 2 * 2 * row(D)          # tokens x kv-heads x (K + V)
                    + 5 * 2 * 8 * D * q_elem         # queries [B, q, Hq, D]
                    + 4 * pages + 4 * 5)             # page ids, lengths
            got = B.algorithmic_bytes(w, L)
            assert got["split"] == want, (kv, dtype, D)
            assert got["step"] == want + 5 * 2 * 8 * D * 2  # + the bf16 output


def test_headline_bytes_per_launch():
    """The headline batch's lengths (the batch builder's PCG64 stream, seed
    1000 + workload seed) and the byte count quoted for it."""
    import numpy as np

    w = W.RAGGED_B64
    L = W.draw_lengths(w, np.random.Generator(np.random.PCG64(1000 + w.seed)))
    assert int(L.sum()) == 646_338 and int(L.max()) == 32_768
    assert B.algorithmic_bytes(w, L)["split"] == 2_648_096_572


def test_stage1_kernel_follows_the_dispatch_rules():
    base = W.BF16_B16  # Hq 32, Hkv 8: 4 query rows per kv-head
    cases = [
        (dict(), "split_bf16_kernel"),
        (dict(num_q_heads=40), "split_bf16_kernel"),              # 5 rows
        (dict(num_q_heads=48), "split_bf16_mfma_kernel"),         # 6 rows
        (dict(q_per_req=4, causal=True), "split_bf16_mfma_kernel"),
        (dict(dtype="fp32"), "split_fma_kernel"),                 # fp32, 4 rows
        (dict(dtype="fp32", num_q_heads=40), "split_f32_mfma_kernel"),
        (dict(kv=W.KV_INT8), "split_int8_mfma_kernel"),
        (dict(kv=W.KV_INT8, dtype="fp32", head_dim=64), "split_int8_mfma_kernel"),
        (dict(kv=W.KV_INT4, q_per_req=1), "split_int4_mfma_kernel"),
    ]
    for kw, kernel in cases:
        assert B.stage1_kernel(base.scaled(name="t", **kw))[0] == kernel, kw
