"""GPU parity on seeded random configurations: cache format (bf16, fp32,
INT8, INT4), pool layout, head dim, page size, kv-heads, GQA group, query
tokens (causal or not), ragged lengths with empty requests, split count, and
the batch-wide or per-request schedule, drawn together so that combinations
the hand-picked cases do not name are compared against the fp64 oracle too.
Gates as in tests/_gpu_util.py; every stage-1 slot and every output element
is checked.  N_WIDE more cases draw 17..64 query rows per kv-head.
"""
import numpy as np
import pytest
import torch

from decode_attention_paged_gqa_amd import workloads as W
from tests import _gpu_util as U
from tests.test_gpu_attention import _check_out

pytestmark = pytest.mark.gpu
log = U.log

N_CASES = 64
N_WIDE = 16


def random_case(i):
    rng = np.random.default_rng(9000 + i)
    fmt = ["bf16", "fp32", "int8", "int4"][i % 4]  # every format in turn
    kv = {"bf16": W.KV_DENSE, "fp32": W.KV_DENSE, "int8": W.KV_INT8, "int4": W.KV_INT4}[fmt]
    dtype = fmt if kv == W.KV_DENSE else str(rng.choice(["bf16", "bf16", "bf16", "fp32"]))
    D = int(rng.choice([64, 128, 128]))
    ps = int(rng.choice([16, 32, 64, 128, 256]))
    Hkv = int(rng.choice([1, 2, 3, 4, 8]))
    qn = int(rng.choice([1, 1, 2, 3, 4, 4]))
    G = int(rng.integers(1, min(16 // qn, 8) + 1))
    if fmt == "int4" and (i // 4) % 2 == 0:  # every other INT4 case: an MTP-verify shape
        dtype, D, qn, G = "bf16", 128, 4, int(rng.choice([3, 4]))  # 12 or 16 rows
    while G * Hkv > 32:
        G -= 1
    causal = bool(qn > 1 and rng.random() < 0.8)
    B = int(rng.integers(1, 9))
    L = rng.integers(0, 2500, size=B)
    L[rng.random(B) < 0.15] = 0
    short = rng.random(B) < 0.15
    L[short] = rng.integers(1, 6, size=int(short.sum()))
    L[0] = max(int(L[0]), 1)
    pages = int(((L + ps - 1) // ps).sum())
    layout = str(rng.choice(["NHD", "HND"]))
    S = int(rng.choice([1, 2, 3, 5, 8, 13, 32]))
    table = None
    if rng.random() < 0.4:
        table = sorted(int(x) for x in rng.integers(1, S + 1, size=int(rng.integers(1, 9))))
    w = W.Workload(name=f"rand{i}_{fmt}_{dtype}q_{layout.lower()}_d{D}_p{ps}_hkv{Hkv}_g{G}_q{qn}"
                        f"{'c' if causal else ''}_b{B}_s{S}{'_sched' if table else ''}",
                   batch=B, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D, page_size=ps,
                   q_per_req=qn, causal=causal, dtype=dtype, kv=kv, lengths="list",
                   length_list=tuple(int(x) for x in L),
                   pool_pages=pages + int(rng.integers(1, 6)), seed=100 + i, kv_layout=layout)
    return w, S, table


def wide_case(i):
    """More than 16 query rows per kv-head (row blocks; two row tiles on the
    matrix-core kernels): G * q in 17..64, every format in turn."""
    rng = np.random.default_rng(9500 + i)
    fmt = ["bf16", "int8", "int4", "fp32"][i % 4]
    kv = {"bf16": W.KV_DENSE, "fp32": W.KV_DENSE, "int8": W.KV_INT8, "int4": W.KV_INT4}[fmt]
    dtype = "fp32" if fmt == "fp32" else "bf16"
    D = int(rng.choice([64, 128]))
    qn = int(rng.choice([1, 2, 3, 4, 8]))
    rows = int(rng.integers(17, 65))
    G = max(1, rows // qn)
    Hkv = int(rng.choice([1, 2]))
    ps = int(rng.choice([16, 64, 128]))
    causal = bool(qn > 1)
    B = int(rng.integers(1, 5))
    L = rng.integers(1, 1500, size=B)
    L[rng.random(B) < 0.2] = 0
    L[0] = max(int(L[0]), 1)
    pages = int(((L + ps - 1) // ps).sum())
    layout = str(rng.choice(["NHD", "HND"]))
    S = int(rng.choice([1, 2, 3, 5]))
    table = None
    if rng.random() < 0.4:
        table = sorted(int(x) for x in rng.integers(1, S + 1, size=int(rng.integers(1, 5))))
    w = W.Workload(name=f"wide{i}_{fmt}_{layout.lower()}_d{D}_p{ps}_hkv{Hkv}_g{G}_q{qn}"
                        f"_b{B}_s{S}{'_sched' if table else ''}",
                   batch=B, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D, page_size=ps,
                   q_per_req=qn, causal=causal, dtype=dtype, kv=kv, lengths="list",
                   length_list=tuple(int(x) for x in L), pool_pages=pages + 2, seed=300 + i,
                   kv_layout=layout)
    return w, S, table


CASES = [random_case(i) for i in range(N_CASES)] + [wide_case(i) for i in range(N_WIDE)]


@pytest.mark.parametrize("w,S,table", CASES, ids=[c[0].name for c in CASES])
def test_random_configuration(gpu, w, S, table):
    log(f"{w.name}: L={list(w.length_list)} table={table}")
    batch = W.make_batch(w, device="cuda")
    fp32_out = w.kv == W.KV_DENSE and w.dtype == "fp32"
    out_dtype = torch.float32 if fp32_out else torch.bfloat16
    counts = None
    md = None
    if table is not None:
        md = U.schedule(gpu, batch, table, 256, S)
        counts = md["split_counts"].cpu().numpy()
    out, lse, o, l = U.run_decode(gpu, batch, S, out_dtype=out_dtype, sched=md)
    if counts is None:
        o_ref, l_ref = U.oracle_partials(batch, S)
        og, lg = U.to_np(o), U.to_np(l)
    else:
        o_ref, l_ref = U.oracle_partials_per_request(batch, S, counts)
        og, lg = U.blank_unused_slots(U.to_np(o), U.to_np(l), counts)
    out_ref, lse_ref = U.oracle_full(batch)
    extra = U.matrix_path_o_bound(batch)
    U.check_partials(og, lg, o_ref, l_ref, w.name, o_extra=extra)
    if fp32_out:
        U.check_fp32(U.to_np(out), out_ref, f"{w.name} out fp32")
    else:
        _check_out(w, U.to_np(out), out_ref, f"{w.name} out")
    U.check_lse(U.to_np(lse), lse_ref, f"{w.name} lse")
