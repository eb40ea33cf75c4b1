"""GPU parity of the KV append with quantise-on-write against oracle/kvcache.py.

Pools start with arbitrary content; a batch of new rows is appended at
distinct random slots plus a -1 sentinel and a slot past the pool.  The whole
pools and scale arrays must then equal the oracle's, bit for bit: the written
rows (codes, scales, zero points) and every untouched byte.  Rows include the
edge cases of the encoders: all zero, all equal, tiny and large magnitudes,
and INT4 groups whose small positive minimum rounds the zero point to -0.
"""
import numpy as np
import pytest
import torch

from oracle import kvcache as OK
from tests import _gpu_util as U

pytestmark = pytest.mark.gpu
log = U.log


def _new_rows(N, Hkv, D, dtype, gen):
    x = torch.randn((N, Hkv, D), generator=gen, device="cuda")
    x[0, 0] = 0.0                                   # all zero row
    x[1, 0] = 1.25                                  # all equal row
    x[2] *= 1e-3                                    # tiny
    x[3] *= 100.0                                   # large
    x[4, 0] = torch.linspace(0.01, 3.0, D, device="cuda")  # small positive minimum per group
    x[5, 0, : D // 2] = -2.5                        # one constant negative half
    return x.to(dtype)


def _host(t):
    """Host copy; bf16 as its raw 16-bit patterns (numpy has no bf16; dense appends copy bits)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy()


def _swap_layout(a, layout):
    """NHD <-> HND of a pool or scale array (swapping axes 1 and 2 is its own inverse)."""
    return a if layout == "NHD" else np.ascontiguousarray(np.swapaxes(a, 1, 2))


CASES = [(fmt, dt, lay, D) for fmt, dt in (("dense", torch.bfloat16), ("dense", torch.float32),
                                           ("int8", torch.bfloat16), ("int8", torch.float32),
                                           ("int4", torch.bfloat16), ("int4", torch.float32))
         for lay in ("NHD", "HND") for D in (128, 64)]


@pytest.mark.parametrize("fmt,dtype,layout,D", CASES,
                         ids=[f"{c[0]}-{str(c[1])[6:]}-{c[2]}-d{c[3]}" for c in CASES])
def test_append_bit_exact(gpu, fmt, dtype, layout, D):
    log(f"append {fmt} {dtype} {layout} D={D}")
    P, ps, Hkv, N = 12, 16, 3, 20
    gen = torch.Generator(device="cuda").manual_seed(7)
    lay_shape = (P, ps, Hkv) if layout == "NHD" else (P, Hkv, ps)
    if fmt == "dense":
        k_pool = torch.randn(lay_shape + (D,), generator=gen, device="cuda").to(dtype)
        v_pool = torch.randn(lay_shape + (D,), generator=gen, device="cuda").to(dtype)
        k_sc = v_sc = None
    elif fmt == "int8":
        k_pool = torch.randint(-127, 128, lay_shape + (D,), generator=gen, device="cuda").to(torch.int8)
        v_pool = torch.randint(-127, 128, lay_shape + (D,), generator=gen, device="cuda").to(torch.int8)
        k_sc = torch.rand(lay_shape, generator=gen, device="cuda").to(torch.float16)
        v_sc = torch.rand(lay_shape, generator=gen, device="cuda").to(torch.float16)
    else:
        k_pool = torch.randint(0, 256, lay_shape + (D // 2,), generator=gen, device="cuda").to(torch.uint8)
        v_pool = torch.randint(0, 256, lay_shape + (D // 2,), generator=gen, device="cuda").to(torch.uint8)
        k_sc = torch.rand(lay_shape + (D // 32, 2), generator=gen, device="cuda").to(torch.float16)
        v_sc = torch.rand(lay_shape + (D // 32, 2), generator=gen, device="cuda").to(torch.float16)
    k_new = _new_rows(N, Hkv, D, dtype, gen)
    v_new = _new_rows(N, Hkv, D, dtype, gen)
    slots = torch.randperm(P * ps, generator=torch.Generator().manual_seed(3))[: N - 2].tolist()
    slots = slots[:7] + [-1] + slots[7:] + [P * ps]  # sentinel and past-the-pool slots
    loc = torch.tensor(slots, dtype=torch.int64, device="cuda")

    want = {}
    for name, pool, sc, new in (("k", k_pool, k_sc, k_new), ("v", v_pool, v_sc, v_new)):
        p = _swap_layout(_host(pool), layout).copy()
        s = None if sc is None else _swap_layout(_host(sc), layout).copy()
        nw = _host(new.float()) if fmt != "dense" else _host(new)
        OK.append_kv(p, nw, slots, ps, fmt, s)
        want[name] = (_swap_layout(p, layout), None if s is None else _swap_layout(s, layout))

    gpu.decode_attn_append_kv(k_new, v_new, loc, k_pool, v_pool, k_sc, v_sc, cache_format=fmt,
                              kv_layout=layout)
    torch.cuda.synchronize()
    for name, pool, sc in (("k", k_pool, k_sc), ("v", v_pool, v_sc)):
        wp, ws = want[name]
        got = _host(pool)
        assert np.array_equal(got.view(np.uint8), wp.view(np.uint8)), f"{name} pool differs"
        if ws is not None:
            assert np.array_equal(_host(sc).view(np.uint16), ws.view(np.uint16)), f"{name} scales differ"
    log(f"  {fmt} {layout} D={D}: pools and scales bit-identical to the oracle")


def test_append_full_size_int4_mtp(gpu):
    """The INT4-MTP decode step's append: 64 requests x 4 new tokens x 8 kv-heads,
    HND, into a 4096-page pool; every written row and scale checked against the
    oracle, every other byte checked unchanged."""
    P, ps, Hkv, D, N = 4096, 64, 8, 128, 256
    gen = torch.Generator(device="cuda").manual_seed(11)
    shape = (P, Hkv, ps)
    k_pool = torch.randint(0, 256, shape + (D // 2,), generator=gen, device="cuda").to(torch.uint8)
    v_pool = torch.randint(0, 256, shape + (D // 2,), generator=gen, device="cuda").to(torch.uint8)
    k_sc = torch.rand(shape + (D // 32, 2), generator=gen, device="cuda").to(torch.float16)
    v_sc = torch.rand(shape + (D // 32, 2), generator=gen, device="cuda").to(torch.float16)
    before = [t.clone() for t in (k_pool, v_pool, k_sc, v_sc)]
    k_new = _new_rows(N, Hkv, D, torch.bfloat16, gen)
    v_new = _new_rows(N, Hkv, D, torch.bfloat16, gen)
    slots = torch.randperm(P * ps, generator=torch.Generator().manual_seed(5))[:N]
    loc = slots.to(torch.int64).cuda()
    gpu.decode_attn_append_kv(k_new, v_new, loc, k_pool, v_pool, k_sc, v_sc, cache_format="int4",
                              kv_layout="HND")
    torch.cuda.synchronize()
    written = torch.zeros(P, Hkv, ps, dtype=torch.bool, device="cuda")
    pg, off = (loc // ps), (loc % ps)
    written[pg, :, off] = True
    for t, b in zip((k_pool, v_pool, k_sc, v_sc), before):
        assert torch.equal(t[~written], b[~written])
    for new, pool, sc in ((k_new, k_pool, k_sc), (v_new, v_pool, v_sc)):
        p, s = OK.quantize_int4(_host(new.float()))  # [N, Hkv, D/2], [N, Hkv, D/32, 2]
        got_p = _host(pool[pg, :, off])
        got_s = _host(sc[pg, :, off])
        assert np.array_equal(got_p, p)
        assert np.array_equal(got_s.view(np.uint16), s.view(np.uint16))
    log("  full-size int4 append: 2048 rows bit-identical, the rest untouched")
