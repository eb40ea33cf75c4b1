"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and its host-side argument validation and split-count
lookup behave as documented (no call here reaches a kernel launch)."""
import ctypes
import os
import re
import subprocess

import pytest

import decode_attention_paged_gqa_amd as da
from decode_attention_paged_gqa_amd import _binding as B
from decode_attention_paged_gqa_amd.splits import SplitTable, kernel_key

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "decode_attn.h")

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails before any launch


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(decode_attn_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libdecode_attn.so not built (run __graft_entry__.build())")
    return da.load()


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(B.EXPORTS)


@pytest.mark.parametrize("path", [B.LIB_PATH, B.CHECKED_LIB_PATH], ids=["plain", "checked"])
def test_library_exports_every_declared_symbol(lib, path):
    if not os.path.exists(path):
        pytest.fail(f"{path} not built (run __graft_entry__.build())")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(decode_attn_\w+)", out))
    for name in _declared():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_checks_need_the_checked_build(lib):
    # the plain library has no contract checks: the query says so without touching a device
    flags, count = ctypes.c_uint32(7), ctypes.c_uint64(7)
    assert lib.decode_attn_checks(ctypes.byref(flags), ctypes.byref(count), 0) == 2
    assert (flags.value, count.value) == (7, 7)
    with pytest.raises(da.DecodeAttnError):
        da.decode_attn_checks()


def test_checked_build_flag_bits_match_the_header():
    src = open(HEADER).read()
    bits = {m[0]: int(m[1], 16) for m in re.findall(r"#define (DA_CHECK_\w+) (0x[0-9a-f]+)u", src)}
    assert bits == {k: getattr(B, k) for k in bits} and len(bits) == 7


def test_strerror_and_version(lib):
    assert lib.decode_attn_strerror(0) == b"ok"
    assert lib.decode_attn_strerror(1) == b"invalid argument"
    assert lib.decode_attn_strerror(2) == b"unsupported shape or dtype"
    assert lib.decode_attn_strerror(3) == b"kernel launch failed"
    assert lib.decode_attn_strerror(4) == b"partials exceed the static scratch buffer"
    assert lib.decode_attn_strerror(99) == b"unknown status"
    assert lib.decode_attn_version() == 300


def _split_args(**kw):
    a = dict(q=FAKE, dtype=B.DA_BF16, k=FAKE, v=FAKE, pt=FAKE, pt_stride=8, max_pages=8,
             seqlens=FAKE, order=None, batch=4, qn=1, Hq=32, Hkv=8, D=128, ps=64, num_pages=100,
             layout=B.DA_KV_NHD, S=4, counts=None, work=None, cap=0, scale=0.1, causal=0,
             o=FAKE, lse=FAKE, stream=None)
    a.update(kw)
    return [a[k] for k in ("q", "dtype", "k", "v", "pt", "pt_stride", "max_pages", "seqlens",
                           "order", "batch", "qn", "Hq", "Hkv", "D", "ps", "num_pages", "layout",
                           "S", "counts", "work", "cap", "scale",
                           "causal", "o", "lse", "stream")]


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(batch=0), 1), (dict(Hq=30), 1),
    (dict(S=0), 1), (dict(S=257), 1), (dict(qn=17), 1), (dict(pt_stride=4), 1),
    (dict(num_pages=0), 1), (dict(D=96), 2), (dict(ps=48), 2), (dict(ps=8), 2),
    (dict(dtype=7), 2), (dict(Hq=2 ** 21, Hkv=1), 1),
    # one page of 2^31 bytes (64 slots x 2^16 kv-heads x 4 D bytes): beyond 32-bit offsets
    (dict(Hq=2 ** 16, Hkv=2 ** 16), 2),
    # 16-byte vector accesses: q, pools and o_partial must be 16-byte aligned
    (dict(q=ctypes.c_void_p(0x1008)), 1), (dict(k=ctypes.c_void_p(0x1004)), 1),
    (dict(o=ctypes.c_void_p(0x1008)), 1),
    # 65535 * 256 units * 8 kv-heads * 32 row blocks: more workgroups than a 1-D grid holds
    (dict(batch=65535, S=256, Hq=4096, Hkv=8), 1), (dict(layout=2), 1), (dict(layout=-1), 1),
    # work lists: counts required, 1 <= capacity <= batch * S
    (dict(work=FAKE, cap=8), 1), (dict(work=FAKE, counts=FAKE, cap=0), 1),
    (dict(work=FAKE, counts=FAKE, cap=17), 1),
])
def test_split_validation(lib, kw, status):
    assert lib.decode_attn_split(*_split_args(**kw)) == status


def test_static_decode_refuses_before_touching_a_device(lib):
    # (q, q_dtype, format, k, v, ks, vs, pt, pt_stride, max_pages, seqlens, order, batch, q, Hq,
    #  Hkv, D, ps, P, layout, S, counts, work, cap, scale, causal, out, out_dtype, lse, stream)
    a = [FAKE, B.DA_BF16, B.DA_CACHE_DENSE, FAKE, FAKE, None, None, FAKE, 8, 8, FAKE, None,
         64, 1, 40, 8, 128, 64, 100, B.DA_KV_HND, 64, None, None, 0, 0.1, 0, FAKE, B.DA_BF16,
         None, None]
    assert lib.decode_attn_decode_static(*a) == 4  # 64 x 40 x 64 split rows: beyond the scratch
    for i, v, st in ((26, None, 1), (26, ctypes.c_void_p(0x1002), 1), (27, 9, 2), (2, 3, 1),
                     (12, 0, 1), (20, 0, 1), (28, ctypes.c_void_p(0x1001), 1)):
        b = list(a); b[i] = v
        assert lib.decode_attn_decode_static(*b) == st, (i, v)
    # sizes whose product would wrap 64 bits (2^30 rows x 2^31 - 1 splits x 2^31 D) are refused
    # as too large, not sized modulo 2^64
    b = list(a)
    b[12], b[13], b[14], b[15], b[16], b[20] = 2 ** 22, 16, 16, 16, 2 ** 31 - 1, 2 ** 31 - 1
    assert lib.decode_attn_decode_static(*b) == 4
    b[12], b[20], b[16] = 1, 1, 2 ** 31 - 1  # one row, one split, absurd D: still beyond the scratch
    b[13] = b[14] = 1
    b[15] = 1
    assert lib.decode_attn_decode_static(*b) == 4


@pytest.mark.parametrize("scale", [float("nan"), float("inf"), float("-inf"), 0.0, -0.125,
                                   -0.0])
def test_softmax_scale_must_be_finite_and_positive(lib, scale):
    base = _split_args(scale=scale)
    assert lib.decode_attn_split(*base) == 1
    q8 = base[:2] + [FAKE, FAKE, FAKE, FAKE] + base[4:]
    assert lib.decode_attn_split_int8(*q8) == 1
    assert lib.decode_attn_split_int4(*q8) == 1


def test_int8_int4_validation(lib):
    base = _split_args()
    # (q, q_dtype, k, v, k_scale, v_scale, ...) -- null scales are invalid
    args8 = base[:2] + [FAKE, FAKE, None, FAKE] + base[4:]
    assert lib.decode_attn_split_int8(*args8) == 1
    args4 = base[:2] + [FAKE, FAKE, FAKE, None] + base[4:]
    assert lib.decode_attn_split_int4(*args4) == 1
    args4 = base[:2] + [FAKE, FAKE, FAKE, FAKE] + base[4:13] + [80] + base[14:]
    assert lib.decode_attn_split_int4(*args4) == 2
    args8 = base[:2] + [FAKE, FAKE, FAKE, FAKE] + _split_args(work=FAKE, cap=4)[4:]
    assert lib.decode_attn_split_int8(*args8) == 1  # work list without counts


def test_merge_and_metadata_and_gather_validation(lib):
    # (o, lse, batch, q, Hq, D, S, split_counts, out, out_dtype, lse_out, stream)
    assert lib.decode_attn_merge(None, FAKE, 1, 1, 8, 128, 4, None, FAKE, B.DA_BF16, None, None) == 1
    assert lib.decode_attn_merge(FAKE, FAKE, 1, 1, 8, 96, 4, None, FAKE, B.DA_BF16, None, None) == 2
    assert lib.decode_attn_merge(FAKE, FAKE, 1, 1, 8, 128, 4, FAKE, FAKE, 5, None, None) == 2
    assert lib.decode_attn_merge(FAKE, FAKE, 1, 1, 8, 128, 0, None, FAKE, B.DA_BF16, None, None) == 1
    # bf16 outputs are written in pairs: out must be 4-byte aligned
    odd = ctypes.c_void_p(0x1002)
    assert lib.decode_attn_merge(FAKE, FAKE, 1, 1, 8, 128, 4, None, odd, B.DA_BF16, None, None) == 1
    md = [FAKE, FAKE, FAKE, 4, 64, 64, 2, 16, 4, B.DA_Q_STRIDED, None, 1, FAKE, FAKE, FAKE, FAKE,
          None, None]
    bad = list(md); bad[0] = None
    assert lib.decode_attn_metadata(*bad) == 1
    bad = list(md); bad[9] = 7
    assert lib.decode_attn_metadata(*bad) == 1
    bad = list(md); bad[9] = B.DA_Q_CUMSUM  # cumsum needs q_in
    assert lib.decode_attn_metadata(*bad) == 1
    bad = list(md); bad[5] = 32  # stride < cols
    assert lib.decode_attn_metadata(*bad) == 1
    # metadata_ex: (..., batch_order, f2s, f2s_len, swa_pt, table, n_buckets, bucket_tokens,
    #               max_splits, split_counts, work_list, capacity, stream)
    table = (ctypes.c_int32 * 3)(1, 4, 8)
    ex = md[:17] + [None, 0, None, table, 3, 4096, 8, FAKE, FAKE, 16, None]
    def bad_ex(i, v):
        b = list(ex); b[i] = v
        return lib.decode_attn_metadata_ex(*b)
    assert bad_ex(17, FAKE) == 1                    # mapping without its output table
    assert bad_ex(19, FAKE) == 1                    # output without a mapping
    assert bad_ex(25, None) == 1                    # table without a work list
    assert bad_ex(24, None) == 1                    # ... or without counts
    assert bad_ex(21, 0) == 1 and bad_ex(21, 17) == 1  # bucket count
    assert bad_ex(22, 0) == 1                       # bucket width
    assert bad_ex(23, 0) == 1 and bad_ex(23, 257) == 1  # max_splits
    assert bad_ex(26, 15) == 1                      # capacity < batch * min(max(table), max_splits)
    zero = (ctypes.c_int32 * 3)(1, 0, 8)
    assert bad_ex(20, zero) == 1                    # a table entry out of range
    b = list(ex); b[17], b[18], b[19] = FAKE, 0, FAKE
    assert lib.decode_attn_metadata_ex(*b) == 1     # empty mapping
    # (pool, row_bytes, Hkv, layout, page_size, num_pages, pt, pt_stride, max_pages, seqlens,
    #  cu_k, batch, out, stream)
    g = [FAKE, 6, 2, B.DA_KV_NHD, 16, 10, FAKE, 4, 4, FAKE, FAKE, 2, FAKE, None]
    bad = list(g); bad[1] = 5
    assert lib.decode_attn_gather_kv(*bad) == 1  # odd row_bytes
    bad = list(g); bad[3] = 2
    assert lib.decode_attn_gather_kv(*bad) == 1  # unknown layout
    bad = list(g); bad[2] = 0
    assert lib.decode_attn_gather_kv(*bad) == 1  # no heads


def test_append_validation(lib):
    # (k_new, v_new, new_dtype, loc, N, Hkv, D, fmt, k_pool, v_pool, k_scale, v_scale,
    #  page_size, num_pages, layout, stream)
    a = [FAKE, FAKE, B.DA_BF16, FAKE, 4, 8, 128, B.DA_CACHE_INT8, FAKE, FAKE, FAKE, FAKE, 64, 10,
         B.DA_KV_HND, None]
    def bad(i, v):
        b = list(a); b[i] = v
        return lib.decode_attn_append_kv(*b)
    assert bad(4, -1) == 1       # negative token count
    assert bad(5, 0) == 1        # no heads
    assert bad(2, 9) == 2        # dtype
    assert bad(6, 96) == 2       # head_dim
    assert bad(7, 3) == 1        # cache format
    assert bad(14, 5) == 1       # layout
    assert bad(10, None) == 1    # int8 needs scales
    assert bad(3, None) == 1     # no slots
    assert bad(4, 0) == 0        # nothing to do: OK, nothing enqueued


def test_pick_splits_buckets_and_nearest_key(lib):
    table = [[1, 2, 3, 4, 5, 6, 7, 8], [11, 12, 13, 14, 15, 16, 17, 18], [21, 22, 23, 24, 25, 26, 27, 28]]
    keys = [16, 32, 64]
    pick = lambda b, L: da.decode_attn_pick_splits(table, keys, 4096, b, L)
    assert pick(16, 1) == 1
    assert pick(16, 4096) == 1
    assert pick(16, 4097) == 2
    assert pick(16, 32768) == 8
    assert pick(16, 10 ** 6) == 8        # clamped to the last bucket
    assert pick(16, 0) == 1 and pick(16, -5) == 1
    assert pick(64, 8192) == 22
    assert pick(1, 8192) == 2            # nearest key 16
    assert pick(24, 8192) == 2           # tie 16 / 32 -> smaller
    assert pick(25, 8192) == 12
    assert pick(48, 8192) == 12          # tie 32 / 64 -> smaller
    assert pick(1000, 8192) == 22
    with pytest.raises(da.DecodeAttnError):
        da.decode_attn_pick_splits(table, [32, 16, 64], 4096, 16, 100)   # keys not ascending
    with pytest.raises(da.DecodeAttnError):
        da.decode_attn_pick_splits([[0] * 8] * 3, keys, 4096, 16, 100)   # split count 0


def test_split_table_roundtrip(tmp_path, lib):
    assert kernel_key("int4", 16, 128, 64, "HND") == "int4_r16_d128_p64_hnd"
    t = SplitTable()
    key = kernel_key("bf16", 5, 128, 64)
    t.tables[key] = [[1, 2, 4, 4, 8, 8, 16, 16]] * len(t.batch_keys)
    p = tmp_path / "t.json"
    t.save(str(p))
    t2 = SplitTable.load(str(p))
    assert t2.tables == t.tables
    assert t2.pick(key, 64, 32768) == 16
    assert t2.pick(key, 64, 5000) == 2
    # untuned variants fall back to a heuristic in range
    s = t2.pick(kernel_key("int8", 4, 128, 64), 32, 32768)
    assert 1 <= s <= 32
    # a kernel that covers four kv-heads per workgroup (token-major quantised
    # caches) takes four times the splits for the same number of workgroups
    from decode_attention_paged_gqa_amd.splits import heads_per_workgroup
    nhd, hnd = kernel_key("int4", 16, 128, 64, "NHD"), kernel_key("int4", 16, 128, 64, "HND")
    assert heads_per_workgroup(nhd) == 4 and heads_per_workgroup(hnd) == 1
    nhd8, hnd8 = kernel_key("int8", 4, 128, 64, "NHD"), kernel_key("int8", 4, 128, 64, "HND")
    assert heads_per_workgroup(nhd8) == 4 and heads_per_workgroup(hnd8) == 1
    assert heads_per_workgroup(kernel_key("int4", 16, 64, 64, "NHD")) == 4
    assert heads_per_workgroup(kernel_key("bf16", 16, 64, 64, "NHD")) == 4
    assert heads_per_workgroup(kernel_key("bf16", 16, 128, 64, "NHD")) == 1
    assert heads_per_workgroup(kernel_key("bf16", 5, 64, 64, "NHD")) == 4
    assert heads_per_workgroup(kernel_key("bf16", 5, 128, 64, "NHD")) == 1
    assert heads_per_workgroup(kernel_key("fp32", 4, 64, 64, "NHD")) == 4
    assert heads_per_workgroup(kernel_key("fp32", 8, 128, 64, "NHD")) == 1
    fresh = SplitTable()
    assert fresh.pick(nhd, 64, 32768) == 4 * fresh.pick(hnd, 64, 32768)
    assert fresh.pick(nhd8, 64, 32768) == 4 * fresh.pick(hnd8, 64, 32768)
    # rows tuned for another set of batch keys are not read (heuristic / default instead)
    t2.tables[key] = [[7] * 8] * (len(t2.batch_keys) - 2)
    t2.chunk_pages[key] = [40] * (len(t2.batch_keys) + 1)
    assert t2.table_for(key) != t2.tables[key]
    assert 1 <= t2.pick(key, 64, 32768) <= 32
    assert t2.chunk_for(key, 64) == 64  # the default split size


def test_binding_rejects_host_tensors(lib):
    import torch
    q = torch.zeros(2, 1, 4, 64)
    kp = torch.zeros(4, 16, 1, 64)
    pt = torch.zeros(2, 4, dtype=torch.int32)
    sl = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        da.decode_attn_split(q, kp, kp, pt, sl, 2)


def test_binding_checks_shapes_before_any_pointer_is_passed(lib):
    """Every size the kernels rely on is checked in the binding, so a wrongly
    sized tensor is a ValueError, never an out-of-bounds device access.  Host
    tensors are used: the shape checks come before the GPU-residency check,
    which then rejects the correctly shaped call."""
    import torch
    nb, Hq, Hkv, D, P, ps, S = 2, 8, 2, 128, 6, 16, 3
    pt = torch.zeros(nb, 4, dtype=torch.int32)
    sl = torch.zeros(nb, dtype=torch.int32)
    # INT8: q's head dim must be the pool's
    k8 = torch.zeros(P, ps, Hkv, D, dtype=torch.int8)
    sc = torch.zeros(P, ps, Hkv, dtype=torch.float16)
    with pytest.raises(ValueError, match="head_dim"):
        da.decode_attn_split_int8(torch.zeros(nb, 1, Hq, 64), k8, k8, sc, sc, pt, sl, S)
    with pytest.raises(ValueError, match="GPU"):
        da.decode_attn_split_int8(torch.zeros(nb, 1, Hq, D), k8, k8, sc, sc, pt, sl, S)
    # caller-supplied partials must match (nb, q, Hq, S, D) exactly
    q = torch.zeros(nb, 1, Hq, D, dtype=torch.bfloat16)
    kb = torch.zeros(P, ps, Hkv, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="o_partial must have shape"):
        da.decode_attn_split(q, kb, kb, pt, sl, S, o_partial=torch.zeros(nb, 1, Hq, D, S))
    # merge: out (nb, q, Hq, D), lse_out (nb, q, Hq), split_counts (nb,)
    o = torch.zeros(nb, 1, Hq, S, D)
    lse = torch.zeros(nb, 1, Hq, S)
    with pytest.raises(ValueError, match="out must have shape"):
        da.decode_attn_merge(o, lse, out=torch.zeros(nb, 1, Hq, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="lse_out must have shape"):
        da.decode_attn_merge(o, lse, lse_out=torch.zeros(nb * Hq))
    with pytest.raises(ValueError, match="split_counts must have shape"):
        da.decode_attn_merge(o, lse, split_counts=torch.ones(nb + 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU"):
        da.decode_attn_merge(o, lse, out=torch.zeros(nb, 1, Hq, D), lse_out=torch.zeros(nb, 1, Hq))
    # metadata: outputs of length nb / nb + 1, and q_in long enough for its mode
    seq = torch.zeros(nb, dtype=torch.int32)
    rpi = torch.zeros(nb, dtype=torch.int64)
    r2t = torch.zeros(nb, 64, dtype=torch.int32)
    bad_out = {"cu_seqlens_k": torch.zeros(nb, dtype=torch.int32)}
    with pytest.raises(ValueError, match="cu_seqlens_k must have shape"):
        da.decode_attn_metadata(seq, rpi, r2t, ps, 4, out=bad_out)
    with pytest.raises(ValueError, match="batch_order must have shape"):
        da.decode_attn_metadata(seq, rpi, r2t, ps, 4,
                                out={"batch_order": torch.zeros(nb + 1, dtype=torch.int32)})
    with pytest.raises(ValueError, match="q_in needs at least 2"):
        da.decode_attn_metadata(seq, rpi, r2t, ps, 4, q_mode=B.DA_Q_CUMSUM)
    with pytest.raises(ValueError, match="q_in needs at least 3"):
        da.decode_attn_metadata(seq, rpi, r2t, ps, 4, q_mode=B.DA_Q_PRESET,
                                q_in=torch.zeros(nb, dtype=torch.int32))
    with pytest.raises(ValueError, match="unknown q_mode"):
        da.decode_attn_metadata(seq, rpi, r2t, ps, 4, q_mode=5)
    with pytest.raises(ValueError, match="GPU"):
        da.decode_attn_metadata(seq, rpi, r2t, ps, 4, q_mode=B.DA_Q_PRESET,
                                q_in=torch.zeros(nb + 1, dtype=torch.int32))
    # gather: per-request arrays sized by the page table's batch
    with pytest.raises(ValueError, match="cu_seqlens_k must have shape"):
        da.decode_attn_gather_kv(kb, pt, sl, torch.zeros(nb, dtype=torch.int32), 10)
